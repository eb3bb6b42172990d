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
// a radix descent over the key bits below the prefix every token shares
// (min/max from the staging pass), 11 bits per digit: all waves build an LDS
// histogram, then every thread takes two bins (descending), a DPP wave scan
// and the sixteen wave totals locate the digit, and each owner clears its
// bins for the next digit.  Sweeps over LDS-resident keys read four
// consecutive keys per lane.  The keep rule is key > T, or key == T and among
// the first q such tokens; the emit walks wave-contiguous token segments with
// ballot/mbcnt prefixes, so indices come out ascending.  Heads of up to 32768
// tokens keep their keys in LDS (and a wave's segment in registers for the
// emit); longer heads re-read the scores, or, under a count budget with the
// workspace given, are split over several workgroups (the part path below).
//
// Protected tokens (the first n_sink and last n_recent of a head) get the
// largest key, 0xffffffff, above every finite score: they lead the order,
// pass any threshold and, with k raised to at least their number, are always
// kept.  In the mass budget their key carries no mass; their real scores are
// summed separately and count first.
//
// The mass budget sums scores in 64-bit fixed point (scale 2^F with F picked
// from the head's total so the sum stays below 2^62), which makes every
// histogram sum exact and independent of the order of the atomic adds.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace kvcc {
namespace {

constexpr int NT = 1024;
constexpr int NWV = NT / WAVE;
constexpr int LDS_KEYS = 32768;
constexpr int NBINS = 2048;
constexpr int DIGIT = 11;

struct SelectArgs {
  const float* scores;
  const int32_t* ctx;
  const int32_t* n_head;   // per-head lengths (overrides ctx), or null
  int B, Hkv, N_max;
  int k_zero_ok;           // BUDGET_K with k <= 0 keeps nothing (else k >= 1)
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
  uint32_t w_min[NWV], w_max[NWV], w_cnt[NWV], w_gt[NWV], w_eq[NWV];
  double w_sum[NWV];
  unsigned long long w_fx[NWV];
  unsigned long long f_m[NWV];   // bin search: per-wave totals
  uint32_t f_c[NWV];
  uint32_t bin, cnt_above, bin_cnt;
  unsigned long long mass_above;
};

constexpr uint32_t PROTECTED_KEY = 0xffffffffu;

template <bool IN_LDS>
struct Keys {
  const uint32_t* lds;
  const float* g;
  int p_end, r_begin;   // protected: t < p_end or t >= r_begin
  __device__ __forceinline__ uint32_t of(float x, int t) const {
    return (t < p_end || t >= r_begin) ? PROTECTED_KEY : to_key(x);
  }
  __device__ __forceinline__ uint32_t operator()(int t) const {
    if (IN_LDS) return lds[t];
    return of(g[t], t);
  }
  // keys of tokens t .. t+3 from their four scores
  __device__ __forceinline__ uint4 four(const float4& v, int t) const {
    return make_uint4(of(v.x, t), of(v.y, t + 1), of(v.z, t + 2), of(v.w, t + 3));
  }
};

// Heads whose keys do not fit in LDS re-read the scores on every sweep: GU
// 16-byte loads per thread are issued before any is used, so a sweep waits
// for memory about once per GU * 4 * NT tokens instead of once per NT.
constexpr int GU = 8;

// Apply f(score, t) to the scores of tokens [0, n) read from global memory.
template <class F>
__device__ __forceinline__ void for_scores(const float* g, int n, const F& f) {
  const int tid = threadIdx.x;
  const int n4 = (reinterpret_cast<uintptr_t>(g) & 15) == 0 ? n >> 2 : 0;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  for (int i0 = 0; i0 < n4; i0 += GU * NT) {
    float4 v[GU];
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int i = i0 + tid + u * NT;
      v[u] = i < n4 ? g4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int i = i0 + tid + u * NT;
      if (i < n4) { f(v[u].x, 4 * i); f(v[u].y, 4 * i + 1); f(v[u].z, 4 * i + 2); f(v[u].w, 4 * i + 3); }
    }
  }
  for (int t = 4 * n4 + tid; t < n; t += NT) f(g[t], t);
}

template <typename I>
__device__ __forceinline__ I wave_sum_i(I v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Apply f to every key of the head.  With the keys in LDS a lane takes four
// consecutive keys per step (one 16-byte read).
template <bool IN_LDS, class F>
__device__ __forceinline__ void for_keys(const Keys<IN_LDS>& key, int n, const F& f) {
  const int tid = threadIdx.x;
  if (IN_LDS) {
    constexpr int PER = LDS_KEYS / 4 / NT;   // n <= LDS_KEYS
    const int n4 = n >> 2;
    const uint4* k4 = reinterpret_cast<const uint4*>(key.lds);
    uint4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * NT;
      v[u] = i < n4 ? k4[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if (tid + u * NT < n4) { f(v[u].x); f(v[u].y); f(v[u].z); f(v[u].w); }
    }
    for (int t = 4 * n4 + tid; t < n; t += NT) f(key.lds[t]);
  } else {
    for_scores(key.g, n, [&](float x, int t) { f(key.of(x, t)); });
  }
}

// One digit of a radix descent: sm.hist (and, with MASS, sm.hmass) hold the
// digit's nb bins (nb even, at most 2 * NT).  Finds the bin at which the
// top-down total (counts, or masses with MASS) reaches rem (1 <= rem <= the
// total) and leaves it in sm.bin, with the count and mass of the bins above
// it (sm.cnt_above, sm.mass_above) and its own count (sm.bin_cnt).  Clears
// the bins.  Thread t owns descending positions 2t and 2t+1 (bins nb-1-2t,
// nb-2-2t): it reads and clears them; a DPP wave scan and the wave totals
// locate the bin.  All threads must call it.
template <bool MASS>
__device__ void resolve_digit(Smem& sm, int nb, unsigned long long rem) {
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int p0 = 2 * tid;
  uint32_t c0 = 0, c1 = 0;
  unsigned long long m0 = 0, m1 = 0;
  if (p0 < nb) {
    const int b0 = nb - 1 - p0, b1 = b0 - 1;
    c0 = sm.hist[b0]; c1 = sm.hist[b1];
    sm.hist[b0] = 0; sm.hist[b1] = 0;
    if (MASS) {
      m0 = sm.hmass[b0]; m1 = sm.hmass[b1];
      sm.hmass[b0] = 0; sm.hmass[b1] = 0;
    }
  }
  if (!MASS) { m0 = c0; m1 = c1; }
  const unsigned long long own = m0 + m1;
  const uint32_t own_c = c0 + c1;
  unsigned long long incl;
  uint32_t incl_c;
  if (MASS) {
    incl = wave_scan_add_u64(own);
    incl_c = wave_scan_u32(own_c, 0u, OpAdd());
  } else {
    incl_c = wave_scan_u32(own_c, 0u, OpAdd());
    incl = incl_c;
  }
  if (lane == WAVE - 1) { sm.f_m[wave] = incl; sm.f_c[wave] = incl_c; }
  __syncthreads();
  unsigned long long wb = 0;
  uint32_t wbc = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    if (w < wave) { wb += sm.f_m[w]; wbc += sm.f_c[w]; }
  }
  const unsigned long long before = wb + incl - own;
  if (before < rem && rem <= before + own) {   // exactly one thread
    const bool first = before + m0 >= rem;      // then m0 > 0
    sm.bin = (uint32_t)(first ? nb - 1 - p0 : nb - 2 - p0);
    sm.cnt_above = wbc + incl_c - own_c + (first ? 0u : c0);
    sm.mass_above = first ? before : before + m0;
    sm.bin_cnt = first ? c0 : c1;
  }
  __syncthreads();
}

// Radix descent.  Without MASS: the k-th key T (rem = k, 1 <= k <= n) and,
// in *rem_out, the quota of keys equal to T that are kept.  With MASS: the
// key T at which the top-down fixed-point mass reaches rem, the count of
// keys above it and the mass still missing at T.
// On entry sm.hist (and, with MASS, sm.hmass) are zero; on exit too.  The
// sm.bin/cnt_above/mass_above reads of one digit all precede the next
// digit's first barrier, so one set of fields serves every digit.
template <bool MASS, bool IN_LDS, class FX>
__device__ uint32_t descend(const Keys<IN_LDS>& key, int n, int cp, uint32_t lo_key,
                            unsigned long long rem, Smem& sm, const FX& fx,
                            uint32_t* cnt_above_out, unsigned long long* rem_out,
                            bool top_ready = false, uint32_t* eq_out = nullptr) {
  if (top_ready) cp = 0;   // sm.hist already holds the top DIGIT bits of every key
  uint32_t pmask = cp <= 0 ? 0u : (cp >= 32 ? ~0u : ~0u << (32 - cp));
  uint32_t prefix = lo_key & pmask, cnt_above = 0;
  int left = cp >= 32 ? 0 : 32 - cp;
  bool ready = top_ready;
  uint32_t pref_cnt = (uint32_t)n;   // keys matching the current prefix
#pragma unroll 1
  while (left > 0) {
    const int bits = min(DIGIT, left);
    const int shift = left - bits;
    const int nb = 1 << bits;
    if (!ready) {
      for_keys(key, n, [&](uint32_t kk) {
        if ((kk & pmask) == prefix) {
          const int bin = (kk >> shift) & (nb - 1);
          atomicAdd(&sm.hist[bin], 1u);
          if (MASS) atomicAdd(&sm.hmass[bin], fx(kk));
        }
      });
    }
    ready = false;
    __syncthreads();
    resolve_digit<MASS>(sm, nb, rem);
    rem -= MASS ? sm.mass_above : (unsigned long long)sm.cnt_above;
    cnt_above += sm.cnt_above;
    pref_cnt = sm.bin_cnt;
    prefix |= sm.bin << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    left -= bits;
  }
  *cnt_above_out = cnt_above;
  *rem_out = rem;
  if (eq_out) *eq_out = cp >= 32 ? (uint32_t)n : pref_cnt;   // keys equal to the result
  return prefix;
}

// The clamp range [lo, hi] of the threshold and mass budgets for a head of
// n >= 1 tokens.
__device__ __forceinline__ void budget_clamps(const kv_budget& bu, int n, int* lo, int* hi) {
  const double nd = (double)n;
  int l = (int)floor((double)bu.min_ratio * nd + 0.5);
  int h = (int)floor((double)bu.max_ratio * nd + 0.5);
  l = max(l, 1);
  h = min(max(h, 1), n);
  *lo = min(l, h);
  *hi = h;
}

// k of the count budgets (explicit k, kept fraction, threshold with cnt
// scores at or above tau), before the protected tokens raise it.
__device__ __forceinline__ int count_budget(const kv_budget& bu, int head, int n, uint32_t cnt,
                                            int lo, int hi) {
  if (bu.mode == KV_BUDGET_K) {
    const int k = bu.k ? bu.k[head] : bu.k_scalar;
    return min(max(k, 1), n);
  }
  if (bu.mode == KV_BUDGET_RATIO) {
    const float r = bu.ratio ? bu.ratio[head] : bu.ratio_scalar;
    const double nd = (double)n;
    const double x = floor((double)r * nd + 0.5);
    return x >= 1.0 ? (x >= nd ? n : (int)x) : 1;
  }
  return min(max((int)cnt, lo), hi);   // threshold
}

template <bool IN_LDS>
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t keys_lds[IN_LDS ? LDS_KEYS : 4];
  __shared__ Smem sm;
  const int head = blockIdx.x, b = head / a.Hkv;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int n = a.n_head ? min(max(a.n_head[head], 0), a.N_max)
                        : (a.ctx ? min(max(a.ctx[b], 0), a.N_max) : a.N_max);
  const bool none = a.k_zero_ok && a.bud.mode == KV_BUDGET_K &&
                    (a.bud.k ? a.bud.k[head] : a.bud.k_scalar) <= 0;
  if (n == 0 || none) {
    if (tid == 0) a.kept_count[head] = 0;
    return;
  }
  const float* src = a.scores + (size_t)head * a.N_max;
  const kv_budget& bu = a.bud;
  const bool mass = bu.mode == KV_BUDGET_MASS;
  const uint32_t tk = to_key(bu.tau);
  // protected tokens: [0, p_end) and [r_begin, n)
  const int p_end = min(max(bu.n_sink, 0), n);
  const int r_begin = n - min(max(bu.n_recent, 0), n);
  const int n_prot = min(n, p_end + (n - r_begin));
  auto is_prot = [&](int t) { return t < p_end || t >= r_begin; };

  // Staging pass: keys (to LDS), min/max key, threshold count, fp64 total
  // of the real scores.
  uint32_t mn = 0xffffffffu, mx = 0u, cnt = 0u;
  double tot = 0.0;
  // Count budgets also histogram the top DIGIT key bits here (the first digit
  // of the descent), which saves one sweep over the keys.
  auto visit = [&](uint32_t kr, bool prot) -> uint32_t {
    const uint32_t kk = prot ? PROTECTED_KEY : kr;
    mn = min(mn, kk);
    mx = max(mx, kk);
    cnt += kk >= tk ? 1u : 0u;
    if (mass) tot += (double)from_key(kr);
    else atomicAdd(&sm.hist[kk >> (32 - DIGIT)], 1u);
    return kk;
  };
  for (int i = tid; i < NBINS; i += NT) { sm.hist[i] = 0; sm.hmass[i] = 0; }
  if (IN_LDS) {
    constexpr int PER = LDS_KEYS / 4 / NT;
    const int n4 = ((a.N_max & 3) == 0) ? n >> 2 : 0;
    const float4* src4 = reinterpret_cast<const float4*>(src);
    float4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * NT;
      v[u] = i < n4 ? src4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();   // histogram cleared before the first count (loads in flight)
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * NT;
      if (i < n4) {
        const int t = 4 * i;
        const uint32_t k0 = visit(to_key(v[u].x), is_prot(t));
        const uint32_t k1 = visit(to_key(v[u].y), is_prot(t + 1));
        const uint32_t k2 = visit(to_key(v[u].z), is_prot(t + 2));
        const uint32_t k3 = visit(to_key(v[u].w), is_prot(t + 3));
        *reinterpret_cast<uint4*>(&keys_lds[t]) = make_uint4(k0, k1, k2, k3);
      }
    }
    for (int t = 4 * n4 + tid; t < n; t += NT) keys_lds[t] = visit(to_key(src[t]), is_prot(t));
  } else {
    __syncthreads();
    for_scores(src, n, [&](float x, int t) { visit(to_key(x), is_prot(t)); });
  }
  mn = last_lane(wave_scan_u32(mn, 0xffffffffu, OpMin()));
  mx = last_lane(wave_scan_u32(mx, 0u, OpMax()));
  cnt = last_lane(wave_scan_u32(cnt, 0u, OpAdd()));
  if (mass) tot = wave_sum_i<double>(tot);
  if (lane == 0) {
    sm.w_min[wave] = mn; sm.w_max[wave] = mx; sm.w_cnt[wave] = cnt; sm.w_sum[wave] = tot;
  }
  __syncthreads();
  mn = 0xffffffffu; mx = 0u; cnt = 0u; tot = 0.0;
  for (int w = 0; w < NWV; ++w) {
    mn = min(mn, sm.w_min[w]); mx = max(mx, sm.w_max[w]);
    cnt += sm.w_cnt[w]; tot += sm.w_sum[w];
  }
  const int cp = mn == mx ? 32 : __clz(mn ^ mx);   // top key bits every token shares
  Keys<IN_LDS> key{keys_lds, src, p_end, r_begin};

  // Budget -> k.
  int lo, hi;
  budget_clamps(bu, n, &lo, &hi);
  int k = 1;
  if (bu.mode != KV_BUDGET_MASS) {
    k = count_budget(bu, head, n, cnt, lo, hi);
  } else if (tot > 0.0) {
    // mass: fixed point with 2^(61 - floor(log2 total)) so every sum < 2^62
    const double scale = ldexp(1.0, 61 - ilogb(tot));
    auto fx = [&](uint32_t kk) -> unsigned long long {   // protected keys: no mass
      const double v = kk == PROTECTED_KEY ? 0.0 : (double)from_key(kk) * scale;
      return v > 0.0 ? (unsigned long long)v : 0ull;
    };
    unsigned long long tp = 0, pm = 0;
    for_keys(key, n, [&](uint32_t kk) { tp += fx(kk); });
    if (n_prot > 0) {   // real mass of the protected tokens
      for (int t = tid; t < p_end; t += NT) pm += fx(to_key(src[t]));
      for (int t = max(r_begin, p_end) + tid; t < n; t += NT) pm += fx(to_key(src[t]));
    }
    tp = last_lane(wave_scan_add_u64(tp));
    pm = last_lane(wave_scan_add_u64(pm));
    if (lane == 0) { sm.w_fx[wave] = tp; sm.f_m[wave] = pm; }
    __syncthreads();
    unsigned long long pm_fx = 0, tot_fx = 0;
    for (int w = 0; w < NWV; ++w) { tot_fx += sm.w_fx[w]; pm_fx += sm.f_m[w]; }
    __syncthreads();   // sm.f_m is reused by the descent
    tot_fx += pm_fx;
    unsigned long long target = (unsigned long long)ceil((double)bu.mass * (double)tot_fx);
    if (target > tot_fx) target = tot_fx;   // double rounding of f * total
    if (target > pm_fx) {
      // the protected tokens come first (their bin holds no mass and only
      // adds to the count above); descend for the mass still missing
      uint32_t above;
      unsigned long long rem;
      const uint32_t Tm = descend<true>(key, n, cp, mn, target - pm_fx, sm, fx, &above, &rem);
      const unsigned long long fv = fx(Tm);   // > 0: its bin holds mass
      const unsigned long long j = fv ? (rem + fv - 1) / fv : 1ull;
      k = (int)(above + (uint32_t)j);
    } else if (target > 0) {
      k = n_prot;
    }
    k = min(max(k, lo), hi);
  } else {
    k = lo;
  }
  k = min(max(k, n_prot), n);

  // The k-th key and the tie quota.
  uint32_t T, quota, eq_total = 0;
  {
    uint32_t above;
    unsigned long long rem;
    auto nofx = [](uint32_t) { return 0ull; };
    T = descend<false>(key, n, cp, mn, (unsigned long long)k, sm, nofx, &above, &rem, !mass,
                       &eq_total);
    quota = (uint32_t)rem;
  }

  // Emit.  Wave w owns tokens [w*seg, min((w+1)*seg, n)), seg a multiple of
  // 256, and walks it in steps of 256 (four consecutive tokens per lane).
  // Lane order is token order, so per-step ballots give each lane the tie
  // rank of its first equal key and the output slot of its first kept key.
  const int seg = ((n + NWV - 1) / NWV + 4 * WAVE - 1) / (4 * WAVE) * (4 * WAVE);
  const int s0 = wave * seg, s1 = min(s0 + seg, n);
  int32_t* dst = a.kept_idx + (size_t)head * a.N_max;
  uint32_t gt = 0, eq = 0, slot = 0, eqr = 0;
  auto count4 = [&](int t, const uint32_t* kk) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool valid = t + u < s1;
      gt += (uint32_t)__popcll(__ballot(valid && kk[u] > T));
      eq += (uint32_t)__popcll(__ballot(valid && kk[u] == T));
    }
  };
  auto prefix_of_waves = [&]() __attribute__((always_inline)) {
    if (lane == 0) { sm.w_gt[wave] = gt; sm.w_eq[wave] = eq; }
    __syncthreads();
    for (int w = 0; w < wave; ++w) {
      const uint32_t left = quota > eqr ? quota - eqr : 0u;
      slot += sm.w_gt[w] + min(left, sm.w_eq[w]);
      eqr += sm.w_eq[w];
    }
  };
  auto write4 = [&](int t, const uint32_t* kk) __attribute__((always_inline)) {
    bool is_gt[4], is_eq[4], keep[4];
    uint64_t be[4], bk[4];
    uint32_t r = eqr;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool valid = t + u < s1;
      is_gt[u] = valid && kk[u] > T;
      is_eq[u] = valid && kk[u] == T;
      be[u] = __ballot(is_eq[u]);
      r += mbcnt(be[u]);
    }
    uint32_t at = slot;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      keep[u] = is_gt[u] || (is_eq[u] && r < quota);
      r += is_eq[u] ? 1u : 0u;
      bk[u] = __ballot(keep[u]);
      at += mbcnt(bk[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (keep[u]) {
        if (at < (uint32_t)n) dst[at] = t + u;
        ++at;
      }
      slot += (uint32_t)__popcll(bk[u]);
      eqr += (uint32_t)__popcll(be[u]);
    }
  };
  if (tid == 0) a.kept_count[head] = k;
  if (IN_LDS) {
    constexpr int EPI = LDS_KEYS / NWV / (4 * WAVE);   // seg <= EPI * 256
    uint4 ek[EPI];
#pragma unroll
    for (int j = 0; j < EPI; ++j) {
      const int t = s0 + j * 4 * WAVE + 4 * lane;
      ek[j] = t < s1 ? *reinterpret_cast<const uint4*>(&keys_lds[t]) : make_uint4(0u, 0u, 0u, 0u);
    }
    // Every wave holds its segment's keys in registers, so after one barrier
    // the key area of LDS is free: each wave compacts its kept indices into
    // its own key range [s0, s1), then copies them out contiguously.
    // When every key equal to T is kept (no tie to rank) the keep rule is
    // key >= T; otherwise waves first count their equal keys for the ranks.
    const bool all_ties = quota >= eq_total;
    if (!all_ties) {
      uint32_t eqw = 0;
#pragma unroll
      for (int j = 0; j < EPI; ++j) {
        if (s0 + j * 4 * WAVE < s1) {
          const int t = s0 + j * 4 * WAVE + 4 * lane;
          const uint32_t kk[4] = {ek[j].x, ek[j].y, ek[j].z, ek[j].w};
#pragma unroll
          for (int u = 0; u < 4; ++u)
            eqw += (uint32_t)__popcll(__ballot(t + u < s1 && kk[u] == T));
        }
      }
      if (lane == 0) sm.w_eq[wave] = eqw;
    }
    __syncthreads();   // also: every wave holds its keys in registers now
    if (!all_ties)
      for (int w = 0; w < wave; ++w) eqr += sm.w_eq[w];   // ties before this wave
    uint32_t* stage = keys_lds + s0;
    uint32_t nk = 0;
#pragma unroll
    for (int j = 0; j < EPI; ++j) {
      if (all_ties && s0 + j * 4 * WAVE < s1) {
        const int t = s0 + j * 4 * WAVE + 4 * lane;
        const uint32_t kk[4] = {ek[j].x, ek[j].y, ek[j].z, ek[j].w};
        uint32_t at = nk;
        bool keep[4];
        uint64_t bk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          keep[u] = t + u < s1 && kk[u] >= T;
          bk[u] = __ballot(keep[u]);
          at += mbcnt(bk[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (keep[u]) stage[at++] = (uint32_t)(t + u);
          nk += (uint32_t)__popcll(bk[u]);
        }
      } else if (s0 + j * 4 * WAVE < s1) {
        const int t = s0 + j * 4 * WAVE + 4 * lane;
        const uint32_t kk[4] = {ek[j].x, ek[j].y, ek[j].z, ek[j].w};
        bool is_gt[4], is_eq[4], keep[4];
        uint64_t be[4], bk[4];
        uint32_t r = eqr;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool valid = t + u < s1;
          is_gt[u] = valid && kk[u] > T;
          is_eq[u] = valid && kk[u] == T;
          be[u] = __ballot(is_eq[u]);
          r += mbcnt(be[u]);
        }
        uint32_t at = nk;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          keep[u] = is_gt[u] || (is_eq[u] && r < quota);
          r += is_eq[u] ? 1u : 0u;
          bk[u] = __ballot(keep[u]);
          at += mbcnt(bk[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (keep[u]) stage[at++] = (uint32_t)(t + u);
          nk += (uint32_t)__popcll(bk[u]);
          eqr += (uint32_t)__popcll(be[u]);
        }
      }
    }
    if (lane == 0) sm.w_gt[wave] = nk;
    __syncthreads();
    for (int w = 0; w < wave; ++w) slot += sm.w_gt[w];
    for (uint32_t i = lane; i < nk; i += WAVE)
      if (slot + i < (uint32_t)n) dst[slot + i] = (int32_t)stage[i];
  } else {
    // GU steps of the segment are loaded (16 bytes per lane each) before the
    // first is counted or written; s0 is a multiple of 256, so a lane's four
    // tokens start on a 16-byte boundary whenever the head's scores do.
    const bool vec = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
    const float4* g4 = reinterpret_cast<const float4*>(src);
    auto load = [&](int b0, uint32_t (*kk)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        const int t = b0 + u * 4 * WAVE + 4 * lane;
        if (vec && t + 3 < s1) {
          const uint4 k = key.four(g4[t >> 2], t);
          kk[u][0] = k.x; kk[u][1] = k.y; kk[u][2] = k.z; kk[u][3] = k.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) kk[u][e] = t + e < s1 ? key(t + e) : 0u;
        }
      }
    };
    for (int b0 = s0; b0 < s1; b0 += GU * 4 * WAVE) {
      uint32_t kk[GU][4];
      load(b0, kk);
#pragma unroll
      for (int u = 0; u < GU; ++u)
        if (b0 + u * 4 * WAVE < s1) count4(b0 + u * 4 * WAVE + 4 * lane, kk[u]);
    }
    prefix_of_waves();
    for (int b0 = s0; b0 < s1; b0 += GU * 4 * WAVE) {
      uint32_t kk[GU][4];
      load(b0, kk);
#pragma unroll
      for (int u = 0; u < GU; ++u)
        if (b0 + u * 4 * WAVE < s1) write4(b0 + u * 4 * WAVE + 4 * lane, kk[u]);
    }
  }
}


// ---------------------------------------------------------------------------
// Heads longer than LDS_KEYS tokens under a count budget.  One workgroup per
// head would leave most CUs idle and re-read the head on every sweep, so the
// head is cut into parts of PT tokens, one workgroup each, and the descent
// runs as five launches over the (part, head) grid with fixed digits of 11,
// 11 and 10 key bits:
//   0: each part histograms the top digit of its keys and counts keys >= tau;
//   1, 2: every workgroup of a head sums the parts' histograms of the last
//         digit, resolves it exactly as resolve_digit does for one workgroup
//         (so all of them agree), and histograms the next digit of its part;
//   3: the last digit gives T and the number of keys equal to T to keep;
//         each part counts its keys above T and equal to T;
//   4: each part writes its kept indices at the offset the earlier parts
//      leave, ties going to the earliest tokens.
// Part 0 of a head publishes the resolved state of each launch.
constexpr int PT = 16384;             // tokens per part
constexpr int PQ = PT / (4 * NT);     // float4 loads per thread (4)

struct PartState {
  int k;
  uint32_t prefix;   // resolved key bits
  uint32_t rem;      // keys still to take among those matching prefix
  uint32_t pad;
};

struct PartArgs {
  SelectArgs s;
  int P;                 // parts per head
  uint32_t* hist;        // [H][3][P][NBINS]
  uint32_t* pstat;       // [H][P][4]: count >= tau, count > T, count == T
  PartState* state;      // [H][4]: after launches 0..3
};

size_t part_workspace(int H, int P) {
  const size_t hist = (size_t)H * 3 * P * NBINS * sizeof(uint32_t);
  const size_t pstat = (size_t)H * P * 4 * sizeof(uint32_t);
  const size_t state = (size_t)H * 4 * sizeof(PartState);
  return hist + pstat + state;
}

// Sum over the block of one value per thread (every thread gets it).
__device__ __forceinline__ uint32_t block_sum(uint32_t v, Smem& sm) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  v = last_lane(wave_scan_u32(v, 0u, OpAdd()));
  if (lane == 0) sm.f_c[wave] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) t += sm.f_c[w];
  __syncthreads();
  return t;
}

template <int PHASE>
__global__ __launch_bounds__(NT) void select_part_kernel(PartArgs pa) {
  __shared__ Smem sm;
  const SelectArgs& a = pa.s;
  const int part = blockIdx.x, head = blockIdx.y, b = head / a.Hkv;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int n = a.ctx ? min(max(a.ctx[b], 0), a.N_max) : a.N_max;
  if (n == 0) {
    if (PHASE == 4 && part == 0 && tid == 0) a.kept_count[head] = 0;
    return;
  }
  const kv_budget& bu = a.bud;
  const int p_end = min(max(bu.n_sink, 0), n);
  const int r_begin = n - min(max(bu.n_recent, 0), n);
  const int n_prot = min(n, p_end + (n - r_begin));
  const int P = pa.P;
  uint32_t* hist_h = pa.hist + (size_t)head * 3 * P * NBINS;
  uint32_t* pstat_h = pa.pstat + (size_t)head * P * 4;
  PartState* st_h = pa.state + (size_t)head * 4;

  // This thread's keys: tokens t0 + 4 (tid + u NT) + e, valid below t1.
  const int t0 = part * PT, t1 = min(t0 + PT, n);
  const float* src = a.scores + (size_t)head * a.N_max;
  const bool vec = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  Keys<false> key{nullptr, src, p_end, r_begin};
  uint32_t kk[PQ][4];
#pragma unroll
  for (int u = 0; u < PQ; ++u) {
    const int t = t0 + 4 * (tid + u * NT);
    if (vec && t + 3 < t1) {
      const uint4 k4 = key.four(reinterpret_cast<const float4*>(src)[t >> 2], t);
      kk[u][0] = k4.x; kk[u][1] = k4.y; kk[u][2] = k4.z; kk[u][3] = k4.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) kk[u][e] = t + e < t1 ? key(t + e) : 0u;
    }
  }
  auto valid = [&](int u, int e) { return t0 + 4 * (tid + u * NT) + e < t1; };
  auto sum_parts = [&](int d, int nb) {   // sm.hist = sum over parts of digit d
    for (int i = tid; i < nb; i += NT) {
      uint32_t c = 0;
      for (int q = 0; q < P; ++q) c += hist_h[((size_t)d * P + q) * NBINS + i];
      sm.hist[i] = c;
    }
    __syncthreads();
  };
  auto publish = [&](int d, int nb) {     // this part's histogram of digit d
    __syncthreads();
    for (int i = tid; i < nb; i += NT) {
      hist_h[((size_t)d * P + part) * NBINS + i] = sm.hist[i];
    }
  };

  if (PHASE == 0) {
    for (int i = tid; i < NBINS; i += NT) sm.hist[i] = 0;
    __syncthreads();
    const uint32_t tk = to_key(bu.tau);
    uint32_t cnt = 0;
#pragma unroll
    for (int u = 0; u < PQ; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (valid(u, e)) {
          cnt += kk[u][e] >= tk ? 1u : 0u;
          atomicAdd(&sm.hist[kk[u][e] >> 21], 1u);
        }
    cnt = block_sum(cnt, sm);
    if (tid == 0) pstat_h[part * 4 + 0] = cnt;
    publish(0, NBINS);
    return;
  }

  if (PHASE == 1) {
    uint32_t cnt = 0;
    for (int q = 0; q < P; ++q) cnt += pstat_h[q * 4 + 0];
    int lo, hi;
    budget_clamps(bu, n, &lo, &hi);
    int k = count_budget(bu, head, n, cnt, lo, hi);
    k = min(max(k, n_prot), n);
    sum_parts(0, NBINS);
    resolve_digit<false>(sm, NBINS, (unsigned long long)k);
    const uint32_t bin = sm.bin;
    const uint32_t rem = (uint32_t)k - sm.cnt_above;
    if (part == 0 && tid == 0) st_h[1] = PartState{k, bin << 21, rem, 0u};
#pragma unroll
    for (int u = 0; u < PQ; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (valid(u, e) && (kk[u][e] >> 21) == bin) atomicAdd(&sm.hist[(kk[u][e] >> 10) & 2047], 1u);
    publish(1, NBINS);
    return;
  }

  if (PHASE == 2) {
    const PartState ps = st_h[1];
    sum_parts(1, NBINS);
    resolve_digit<false>(sm, NBINS, (unsigned long long)ps.rem);
    const uint32_t prefix = ps.prefix | (sm.bin << 10);
    const uint32_t rem = ps.rem - sm.cnt_above;
    if (part == 0 && tid == 0) st_h[2] = PartState{ps.k, prefix, rem, 0u};
#pragma unroll
    for (int u = 0; u < PQ; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (valid(u, e) && (kk[u][e] >> 10) == (prefix >> 10)) atomicAdd(&sm.hist[kk[u][e] & 1023], 1u);
    publish(2, 1024);
    return;
  }

  if (PHASE == 3) {
    const PartState ps = st_h[2];
    sum_parts(2, 1024);
    resolve_digit<false>(sm, 1024, (unsigned long long)ps.rem);
    const uint32_t T = ps.prefix | sm.bin;
    const uint32_t quota = ps.rem - sm.cnt_above;
    if (part == 0 && tid == 0) st_h[3] = PartState{ps.k, T, quota, 0u};
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int u = 0; u < PQ; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (valid(u, e)) { gt += kk[u][e] > T ? 1u : 0u; eq += kk[u][e] == T ? 1u : 0u; }
    gt = block_sum(gt, sm);
    eq = block_sum(eq, sm);
    if (tid == 0) { pstat_h[part * 4 + 1] = gt; pstat_h[part * 4 + 2] = eq; }
    return;
  }

  // PHASE 4: emit.  The part's tokens form PQ * NWV chunks of 4 * WAVE
  // consecutive tokens, chunk (u, w) = lanes of wave w at load u, in token
  // order u-major; each chunk's kept tokens go out in lane order.
  const PartState ps = st_h[3];
  const uint32_t T = ps.prefix, quota = ps.rem;
  uint32_t off = 0, eqb = 0;   // kept by, and ties in, the earlier parts
  for (int q = 0; q < part; ++q) {
    const uint32_t g = pstat_h[q * 4 + 1], e = pstat_h[q * 4 + 2];
    const uint32_t left = quota > eqb ? quota - eqb : 0u;
    off += g + min(left, e);
    eqb += e;
  }
  if (part == 0 && tid == 0) a.kept_count[head] = ps.k;
  __shared__ uint32_t cg[PQ][NWV], ce[PQ][NWV];
#pragma unroll
  for (int u = 0; u < PQ; ++u) {
    uint32_t g = 0, e = 0;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      g += (uint32_t)__popcll(__ballot(valid(u, x) && kk[u][x] > T));
      e += (uint32_t)__popcll(__ballot(valid(u, x) && kk[u][x] == T));
    }
    if (lane == 0) { cg[u][wave] = g; ce[u][wave] = e; }
  }
  __syncthreads();
  int32_t* dst = a.kept_idx + (size_t)head * a.N_max;
#pragma unroll
  for (int u = 0; u < PQ; ++u) {
    // slot and tie rank at the start of chunk (u, wave)
    uint32_t slot = off, r = eqb;
    for (int c = 0; c < u * NWV + wave; ++c) {
      const uint32_t g = cg[c / NWV][c % NWV], e = ce[c / NWV][c % NWV];
      const uint32_t left = quota > r ? quota - r : 0u;
      slot += g + min(left, e);
      r += e;
    }
    bool is_gt[4], is_eq[4], keep[4];
    uint64_t be[4], bk[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      is_gt[x] = valid(u, x) && kk[u][x] > T;
      is_eq[x] = valid(u, x) && kk[u][x] == T;
      be[x] = __ballot(is_eq[x]);
      r += mbcnt(be[x]);
    }
    uint32_t at = slot;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      keep[x] = is_gt[x] || (is_eq[x] && r < quota);
      r += is_eq[x] ? 1u : 0u;
      bk[x] = __ballot(keep[x]);
      at += mbcnt(bk[x]);
    }
    const int t = t0 + 4 * (tid + u * NT);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      if (keep[x]) {
        if (at < (uint32_t)n) dst[at] = t + x;
        ++at;
      }
    }
  }
}

// The five launches of the part path; per-kernel timing sees them as one
// "select" (start stamped by the first dispatch, stop by the last).
void select_parts(const SelectArgs& s, int P, void* ws, hipStream_t st) {
  PartArgs pa;
  pa.s = s;
  pa.P = P;
  const int H = s.B * s.Hkv;
  pa.hist = static_cast<uint32_t*>(ws);
  pa.pstat = pa.hist + (size_t)H * 3 * P * NBINS;
  pa.state = reinterpret_cast<PartState*>(pa.pstat + (size_t)H * P * 4);
  const dim3 grid(P, H), block(NT);
  hipEvent_t e0, e1;
  const bool timed = timing_events("select", &e0, &e1);
  if (timed)
    hipExtLaunchKernelGGL(select_part_kernel<0>, grid, block, 0, st, e0, nullptr, 0, pa);
  else
    hipLaunchKernelGGL(select_part_kernel<0>, grid, block, 0, st, pa);
  hipLaunchKernelGGL(select_part_kernel<1>, grid, block, 0, st, pa);
  hipLaunchKernelGGL(select_part_kernel<2>, grid, block, 0, st, pa);
  hipLaunchKernelGGL(select_part_kernel<3>, grid, block, 0, st, pa);
  if (timed) {
    hipExtLaunchKernelGGL(select_part_kernel<4>, grid, block, 0, st, nullptr, e1, 0, pa);
    timing_done("select", e0, e1);
  } else {
    hipLaunchKernelGGL(select_part_kernel<4>, grid, block, 0, st, pa);
  }
}

}  // namespace
}  // namespace kvcc

using namespace kvcc;

extern "C" size_t kv_select_workspace_size(int B, int Hkv, int N_max) {
  if (B < 1 || Hkv < 1 || N_max <= LDS_KEYS) return 0;
  return part_workspace(B * Hkv, ceil_div(N_max, PT));
}

extern "C" int kv_select(const float* scores, const int32_t* ctx_len,
                         int B, int Hkv, int N_max, const kv_budget* budget,
                         int32_t* kept_idx, int32_t* kept_count,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!scores || !budget || !kept_idx || !kept_count) return KV_ERR_NULL;
  if (!aligned16(scores) || !aligned16(ctx_len) || !aligned16(kept_idx) ||
      !aligned16(kept_count) || !aligned16(budget->k) || !aligned16(budget->ratio) ||
      !aligned16(workspace))
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
  if (bu.n_sink < 0 || bu.n_recent < 0) return KV_ERR_MODE;

  // Long heads under a count budget take the part path when the workspace
  // is there (its size covers it whenever N_max > LDS_KEYS).
  const int P = ceil_div(N_max, PT);
  if (N_max > LDS_KEYS && bu.mode != KV_BUDGET_MASS && workspace &&
      workspace_bytes >= part_workspace(B * Hkv, P)) {
    SelectArgs a;
    a.scores = scores; a.ctx = ctx_len; a.n_head = nullptr; a.B = B; a.Hkv = Hkv; a.N_max = N_max;
    a.k_zero_ok = 0;
    a.bud = bu; a.kept_idx = kept_idx; a.kept_count = kept_count;
    select_parts(a, P, workspace, static_cast<hipStream_t>(stream));
    return launch_status();
  }
  select_launch(scores, ctx_len, nullptr, B, Hkv, N_max, bu, false, kept_idx, kept_count,
                static_cast<hipStream_t>(stream), "select");
  return launch_status();
}

void kvcc::select_launch(const float* scores, const int32_t* ctx, const int32_t* n_head, int B,
                         int Hkv, int N_max, const kv_budget& bud, bool k_zero_ok,
                         int32_t* kept_idx, int32_t* kept_count, hipStream_t st,
                         const char* timer_name) {
  SelectArgs a;
  a.scores = scores; a.ctx = ctx; a.n_head = n_head; a.B = B; a.Hkv = Hkv; a.N_max = N_max;
  a.k_zero_ok = k_zero_ok ? 1 : 0;
  a.bud = bud; a.kept_idx = kept_idx; a.kept_count = kept_count;
  if (N_max <= LDS_KEYS)
    launch(timer_name, select_kernel<true>, dim3(B * Hkv), dim3(NT), 0, st, a);
  else
    launch(timer_name, select_kernel<false>, dim3(B * Hkv), dim3(NT), 0, st, a);
}
