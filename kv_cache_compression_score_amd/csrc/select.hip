// Per-head budgeted top-k over fp32 scores (radix select + ordered emit).
//
// Importance-based eviction keeps each head's high scorers and drops the
// rest ("A Simple Plug-in for Improving Eviction-Based KV Cache Compression",
// section "Enonce du Probleme"); the budget is a count, a kept fraction, a
// fixed threshold tau ("KVzap: Fast, Adaptive, and Faithful KV Cache
// Pruning", section 2.3) or a score-mass fraction, per head ("KVSculpt: KV
// Cache Compression as Distillation", section 2.D, allocates budgets per KV
// head).
//
// One 1024-thread workgroup owns one (sequence, KV head).  Scores become
// order-preserving uint32 keys (-0.0 folded onto +0.0).  The k-th key T of
// the order "higher score first, lower index first among equals" is found by
// three digit passes (11 + 11 + 10 bits) of LDS histograms; the keep rule is
// then key > T, or key == T and among the first q such tokens.  The emit is
// two sweeps over wave-contiguous token segments with ballot/popcount
// prefixes, so indices come out ascending.  Heads of up to 32768 tokens keep
// their keys in LDS; longer heads re-read the scores from global memory.
//
// The mass budget sums scores in 64-bit fixed point (scale 2^F with F picked
// from the head's total so the sum stays below 2^62), which makes every
// histogram sum exact and order independent.
#include <math.h>

#include "common.hpp"

namespace kvcc {
namespace {

constexpr int NT = 1024;
constexpr int NWV = NT / WAVE;
constexpr int LDS_KEYS = 32768;
constexpr int NBINS = 2048;

struct SelectArgs {
  const float* scores;
  const int32_t* ctx;
  int B, Hkv, N_max;
  kv_budget bud;
  int32_t* kept_idx;
  int32_t* kept_count;
};

__device__ __forceinline__ uint32_t to_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

struct Smem {
  uint32_t hist[NBINS];
  unsigned long long hmass[NBINS];
  unsigned long long wtot[NWV];
  double wsum[NWV];
  uint32_t wcnt_gt[NWV], wcnt_eq[NWV], keep_before[NWV], eq_before[NWV];
  uint32_t bin, cnt_above;
  unsigned long long mass_above;
  int found;
};

// Exclusive prefix over the 1024 threads (block order); wtot is scratch.
template <typename I>
__device__ I block_excl_scan(I v, unsigned long long* wtot) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const I inc = wave_incl_scan<I>(v);
  if (lane == WAVE - 1) wtot[wave] = (unsigned long long)inc;
  __syncthreads();
  if (wave == 0) {
    const I x = lane < NWV ? (I)wtot[lane] : (I)0;
    const I xi = wave_incl_scan<I>(x);
    if (lane < NWV) wtot[lane] = (unsigned long long)(xi - x);
  }
  __syncthreads();
  const I r = inc - v + (I)wtot[wave];
  __syncthreads();
  return r;
}

template <bool IN_LDS>
struct Keys {
  const uint32_t* lds;
  const float* g;
  __device__ __forceinline__ uint32_t operator()(int t) const {
    return IN_LDS ? lds[t] : to_key(g[t]);
  }
};

// Top key bits shared by every token of the head (min/max reduction): the
// digit passes start below them, so the first histogram spreads over the
// bits that actually vary.
template <class KF>
__device__ int common_prefix(const KF& key, int n, Smem& sm, uint32_t* lo_key) {
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int t = tid; t < n; t += NT) {
    const uint32_t kk = key(t);
    mn = min(mn, kk);
    mx = max(mx, kk);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, WAVE));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, WAVE));
  }
  if (lane == 0) { sm.wcnt_gt[wave] = mn; sm.wcnt_eq[wave] = mx; }
  __syncthreads();
  mn = 0xffffffffu; mx = 0u;
  for (int w = 0; w < NWV; ++w) { mn = min(mn, sm.wcnt_gt[w]); mx = max(mx, sm.wcnt_eq[w]); }
  __syncthreads();
  *lo_key = mn;
  return mn == mx ? 32 : __clz(mn ^ mx);
}

// Radix descent for the k-th key (1 <= k <= n).  Returns T; *quota = number
// of tokens with key == T that are kept.
template <class KF>
__device__ uint32_t kth_key(const KF& key, int n, int k, int cp, uint32_t lo_key, Smem& sm,
                            uint32_t* quota) {
  if (cp >= 32) { *quota = (uint32_t)k; return lo_key; }   // every key equal
  uint32_t pmask = cp == 0 ? 0u : ~0u << (32 - cp);
  uint32_t prefix = lo_key & pmask, rem = (uint32_t)k;
  const int tid = threadIdx.x;
  int left = 32 - cp;
#pragma unroll 1
  while (left > 0) {
    const int bits = min(11, left);
    const int shift = left - bits;
    const int nb = 1 << bits;
    for (int i = tid; i < nb; i += NT) sm.hist[i] = 0;
    __syncthreads();
    for (int t = tid; t < n; t += NT) {
      const uint32_t kk = key(t);
      if ((kk & pmask) == prefix) atomicAdd(&sm.hist[(kk >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    // positions in descending bin order: thread owns positions 2*tid, 2*tid+1
    const int p0 = 2 * tid, p1 = 2 * tid + 1;
    const uint32_t h0 = p0 < nb ? sm.hist[nb - 1 - p0] : 0u;
    const uint32_t h1 = p1 < nb ? sm.hist[nb - 1 - p1] : 0u;
    const uint32_t above = block_excl_scan<uint32_t>(h0 + h1, sm.wtot);
    if (p0 < nb && above < rem && rem <= above + h0) {
      sm.bin = (uint32_t)(nb - 1 - p0); sm.cnt_above = above;
    } else if (p1 < nb && above + h0 < rem && rem <= above + h0 + h1) {
      sm.bin = (uint32_t)(nb - 1 - p1); sm.cnt_above = above + h0;
    }
    __syncthreads();
    rem -= sm.cnt_above;
    prefix |= sm.bin << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    left -= bits;
    __syncthreads();
  }
  *quota = rem;
  return prefix;
}

// Mass budget: fewest top tokens whose fixed-point score sum reaches
// ceil(f * total).  Returns k >= 1 (before clamping).
template <class KF>
__device__ int mass_count(const KF& key, int n, float f, int cp, uint32_t lo_key, Smem& sm) {
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  // exponent of the total (fixed-order fp64 reduction; only picks F)
  double part = 0.0;
  for (int t = tid; t < n; t += NT) part += (double)from_key(key(t));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, WAVE);
  if (lane == 0) sm.wsum[wave] = part;
  __syncthreads();
  double total = 0.0;
  for (int w = 0; w < NWV; ++w) total += sm.wsum[w];
  __syncthreads();
  if (!(total > 0.0)) return 1;
  const double scale = ldexp(1.0, 61 - ilogb(total));
  auto fx = [&](uint32_t kk) -> unsigned long long {
    const double v = (double)from_key(kk) * scale;
    return v > 0.0 ? (unsigned long long)v : 0ull;
  };
  // exact fixed-point total
  unsigned long long tp = 0;
  for (int t = tid; t < n; t += NT) tp += fx(key(t));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tp += __shfl_xor(tp, o, WAVE);
  if (lane == 0) sm.wtot[wave] = tp;
  __syncthreads();
  unsigned long long tot_fx = 0;
  for (int w = 0; w < NWV; ++w) tot_fx += sm.wtot[w];
  __syncthreads();
  unsigned long long target = (unsigned long long)ceil((double)f * (double)tot_fx);
  if (target > tot_fx) target = tot_fx;   // double rounding of f * total
  if (target == 0) return 1;

  uint32_t pmask = cp == 0 ? 0u : (cp >= 32 ? ~0u : ~0u << (32 - cp));
  uint32_t prefix = lo_key & pmask, cnt_above = 0;
  unsigned long long rem = target;
  int left = cp >= 32 ? 0 : 32 - cp;
#pragma unroll 1
  while (left > 0) {
    const int bits = min(11, left);
    const int shift = left - bits;
    const int nb = 1 << bits;
    for (int i = tid; i < nb; i += NT) { sm.hist[i] = 0; sm.hmass[i] = 0; }
    __syncthreads();
    for (int t = tid; t < n; t += NT) {
      const uint32_t kk = key(t);
      if ((kk & pmask) == prefix) {
        const int bin = (kk >> shift) & (nb - 1);
        atomicAdd(&sm.hist[bin], 1u);
        atomicAdd(&sm.hmass[bin], fx(kk));
      }
    }
    __syncthreads();
    const int p0 = 2 * tid, p1 = 2 * tid + 1;
    const unsigned long long m0 = p0 < nb ? sm.hmass[nb - 1 - p0] : 0ull;
    const unsigned long long m1 = p1 < nb ? sm.hmass[nb - 1 - p1] : 0ull;
    const uint32_t c0 = p0 < nb ? sm.hist[nb - 1 - p0] : 0u;
    const uint32_t c1 = p1 < nb ? sm.hist[nb - 1 - p1] : 0u;
    const unsigned long long mab = block_excl_scan<unsigned long long>(m0 + m1, sm.wtot);
    const uint32_t cab = block_excl_scan<uint32_t>(c0 + c1, sm.wtot);
    if (p0 < nb && mab < rem && rem <= mab + m0) {
      sm.bin = (uint32_t)(nb - 1 - p0); sm.mass_above = mab; sm.cnt_above = cab;
    } else if (p1 < nb && mab + m0 < rem && rem <= mab + m0 + m1) {
      sm.bin = (uint32_t)(nb - 1 - p1); sm.mass_above = mab + m0; sm.cnt_above = cab + c0;
    }
    __syncthreads();
    rem -= sm.mass_above;
    cnt_above += sm.cnt_above;
    prefix |= sm.bin << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    left -= bits;
    __syncthreads();
  }
  const unsigned long long fv = fx(prefix);   // > 0: the bin holds mass
  const unsigned long long j = fv ? (rem + fv - 1) / fv : 1ull;
  return (int)(cnt_above + (uint32_t)j);
}

template <bool IN_LDS>
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a) {
  __shared__ uint32_t keys_lds[IN_LDS ? LDS_KEYS : 1];
  __shared__ Smem sm;
  const int head = blockIdx.x, b = head / a.Hkv;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int n = a.ctx ? min(max(a.ctx[b], 0), a.N_max) : a.N_max;
  if (n == 0) {
    if (tid == 0) a.kept_count[head] = 0;
    return;
  }
  const float* src = a.scores + (size_t)head * a.N_max;
  if (IN_LDS) {
    // 16-byte loads, all in flight before the first LDS store.
    constexpr int PER = LDS_KEYS / 4 / NT;
    const int n4 = ((a.N_max & 3) == 0) ? n >> 2 : 0;
    const float4* src4 = reinterpret_cast<const float4*>(src);
    float4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * NT;
      v[u] = i < n4 ? src4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * NT;
      if (i < n4) {
        keys_lds[4 * i + 0] = to_key(v[u].x);
        keys_lds[4 * i + 1] = to_key(v[u].y);
        keys_lds[4 * i + 2] = to_key(v[u].z);
        keys_lds[4 * i + 3] = to_key(v[u].w);
      }
    }
    for (int t = 4 * n4 + tid; t < n; t += NT) keys_lds[t] = to_key(src[t]);
    __syncthreads();
  }
  Keys<IN_LDS> key{keys_lds, src};

  // Budget -> k.
  const kv_budget& bu = a.bud;
  const double nd = (double)n;
  int lo = (int)floor((double)bu.min_ratio * nd + 0.5);
  int hi = (int)floor((double)bu.max_ratio * nd + 0.5);
  lo = max(lo, 1);
  hi = min(max(hi, 1), n);
  lo = min(lo, hi);
  int k = 1;
  if (bu.mode == KV_BUDGET_K) {
    k = bu.k ? bu.k[head] : bu.k_scalar;
    k = min(max(k, 1), n);
  } else if (bu.mode == KV_BUDGET_RATIO) {
    const float r = bu.ratio ? bu.ratio[head] : bu.ratio_scalar;
    const double x = floor((double)r * nd + 0.5);
    k = x >= 1.0 ? (x >= nd ? n : (int)x) : 1;
  } else if (bu.mode == KV_BUDGET_THRESHOLD) {
    const uint32_t tk = to_key(bu.tau);
    uint32_t c = 0;
    for (int t = tid; t < n; t += NT) c += key(t) >= tk ? 1u : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, WAVE);
    if (lane == 0) sm.wcnt_gt[wave] = c;
    __syncthreads();
    uint32_t tot = 0;
    for (int w = 0; w < NWV; ++w) tot += sm.wcnt_gt[w];
    __syncthreads();
    k = min(max((int)tot, lo), hi);
  }
  uint32_t lo_key;
  const int cp = common_prefix(key, n, sm, &lo_key);
  if (bu.mode == KV_BUDGET_MASS) {
    k = mass_count(key, n, bu.mass, cp, lo_key, sm);
    k = min(max(k, lo), hi);
  }

  uint32_t quota;
  const uint32_t T = kth_key(key, n, k, cp, lo_key, sm, &quota);

  // Emit.  Wave w owns tokens [w*seg, min((w+1)*seg, n)), seg a multiple of 64.
  const int seg = ((n + NWV - 1) / NWV + WAVE - 1) / WAVE * WAVE;
  const int s0 = wave * seg, s1 = min(s0 + seg, n);
  uint32_t gt = 0, eq = 0;
  for (int base = s0; base < s1; base += WAVE) {
    const int t = base + lane;
    const uint32_t kk = t < s1 ? key(t) : 0u;
    gt += __popcll(__ballot(t < s1 && kk > T));
    eq += __popcll(__ballot(t < s1 && kk == T));
  }
  if (lane == 0) { sm.wcnt_gt[wave] = gt; sm.wcnt_eq[wave] = eq; }
  __syncthreads();
  if (tid == 0) {
    uint32_t eb = 0, kb = 0;
    for (int w = 0; w < NWV; ++w) {
      sm.eq_before[w] = eb;
      sm.keep_before[w] = kb;
      const uint32_t left = quota > eb ? quota - eb : 0u;
      kb += sm.wcnt_gt[w] + min(left, sm.wcnt_eq[w]);
      eb += sm.wcnt_eq[w];
    }
    a.kept_count[head] = k;
  }
  __syncthreads();
  uint32_t eqr = sm.eq_before[wave], slot = sm.keep_before[wave];
  int32_t* dst = a.kept_idx + (size_t)head * a.N_max;
  const uint64_t lt = lanemask_lt();
  for (int base = s0; base < s1; base += WAVE) {
    const int t = base + lane;
    const uint32_t kk = t < s1 ? key(t) : 0u;
    const bool is_eq = t < s1 && kk == T;
    const uint64_t eqm = __ballot(is_eq);
    const uint32_t my_eq_rank = eqr + (uint32_t)__popcll(eqm & lt);
    const bool keep = t < s1 && (kk > T || (is_eq && my_eq_rank < quota));
    const uint64_t km = __ballot(keep);
    const uint32_t at = slot + (uint32_t)__popcll(km & lt);
    if (keep && at < (uint32_t)n) dst[at] = t;
    slot += (uint32_t)__popcll(km);
    eqr += (uint32_t)__popcll(eqm);
  }
}

}  // namespace
}  // namespace kvcc

using namespace kvcc;

extern "C" size_t kv_select_workspace_size(int B, int Hkv, int N_max) {
  (void)B; (void)Hkv; (void)N_max;
  return 0;
}

extern "C" int kv_select(const float* scores, const int32_t* ctx_len,
                         int B, int Hkv, int N_max, const kv_budget* budget,
                         int32_t* kept_idx, int32_t* kept_count,
                         void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace; (void)workspace_bytes;
  if (!scores || !budget || !kept_idx || !kept_count) return KV_ERR_NULL;
  if (!aligned16(scores) || !aligned16(ctx_len) || !aligned16(kept_idx) ||
      !aligned16(kept_count) || !aligned16(budget->k) || !aligned16(budget->ratio))
    return KV_ERR_ALIGN;
  if (B < 1 || Hkv < 1 || N_max < 1 || (int64_t)B * Hkv * N_max >= (int64_t(1) << 31))
    return KV_ERR_SHAPE;
  const kv_budget& bu = *budget;
  if (bu.mode < KV_BUDGET_K || bu.mode > KV_BUDGET_MASS) return KV_ERR_MODE;
  if (!(bu.min_ratio >= 0.f && bu.min_ratio <= 1.f && bu.max_ratio >= 0.f && bu.max_ratio <= 1.f))
    return KV_ERR_MODE;
  if (bu.mode == KV_BUDGET_RATIO && !bu.ratio && !(bu.ratio_scalar >= 0.f && bu.ratio_scalar <= 1.f))
    return KV_ERR_MODE;
  if (bu.mode == KV_BUDGET_MASS && !(bu.mass >= 0.f && bu.mass <= 1.f)) return KV_ERR_MODE;
  if (bu.mode == KV_BUDGET_THRESHOLD && isnan(bu.tau)) return KV_ERR_MODE;

  SelectArgs a;
  a.scores = scores; a.ctx = ctx_len; a.B = B; a.Hkv = Hkv; a.N_max = N_max;
  a.bud = bu; a.kept_idx = kept_idx; a.kept_count = kept_count;
  hipStream_t st = static_cast<hipStream_t>(stream);
  TimedLaunch t("select", st);
  if (N_max <= LDS_KEYS)
    select_kernel<true><<<B * Hkv, NT, 0, st>>>(a);
  else
    select_kernel<false><<<B * Hkv, NT, 0, st>>>(a);
  return launch_status();
}
