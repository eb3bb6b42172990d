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

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace kvcc {
namespace {

constexpr int NT = 1024;
constexpr int NWV = NT / WAVE;

// The calling thread's wave as a wave-uniform value (an SGPR), so that
// conditions on it and on what derives from it branch instead of masking lanes.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)threadIdx.x / WAVE);
}
constexpr int LDS_KEYS = 32768;
constexpr int NBINS = KEY_BINS;
constexpr int DIGIT = KEY_DIGIT;

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

// Adds one key to the LDS histogram (its bin, and with MASS its fixed-point
// mass) for every lane with `active`.  All lanes of the wave call it together.
// Score keys can crowd into one bin (a Zipf key-norm profile puts 98% of a
// head's keys in one top-digit bin), and LDS atomics that hit one address
// serialise, so when at least AGG_MIN active lanes share the first active
// lane's bin, one lane adds their count (and summed mass) for all of them.
// The sums are integers, so the result does not depend on the grouping.
constexpr int AGG_MIN = 8;
template <bool MASS>
__device__ __forceinline__ void hist_add(Smem& sm, bool active, int bin, unsigned long long m) {
  const uint64_t act = __ballot(active);
  if (act == 0) return;
  const int lead = __builtin_ctzll(act);
  const int b0 = __builtin_amdgcn_readlane(bin, lead);
  const bool same = active && bin == b0;
  const uint64_t ms = __ballot(same);
  const uint32_t c = (uint32_t)__popcll(ms);
  const int lane = threadIdx.x & (WAVE - 1);
  if (c >= (uint32_t)AGG_MIN) {
    if (MASS) {
      const unsigned long long tot = last_lane(wave_scan_add_u64(same ? m : 0ull));
      if (lane == lead) atomicAdd(&sm.hmass[b0], tot);
    }
    if (lane == lead) atomicAdd(&sm.hist[b0], c);
    if (active && !same) {
      atomicAdd(&sm.hist[bin], 1u);
      if (MASS) atomicAdd(&sm.hmass[bin], m);
    }
  } else if (active) {
    atomicAdd(&sm.hist[bin], 1u);
    if (MASS) atomicAdd(&sm.hmass[bin], m);
  }
}

// A wave's histogram adds over one pass when its keys crowd into one bin
// (see crowded below): the bin of the wave's first key (hb, wave-uniform) is
// counted in registers, lane by lane, and added once at the end (flush);
// other bins go through hist_add.  With one bin holding most keys this
// leaves that bin no LDS atomic and no wave reduction per step.  With MASS a
// second bin (hb2) is kept in registers too, the first that AGG_MIN lanes of
// a step share outside hb: a head whose keys split between two bins would
// otherwise pay a 64-bit wave reduction per step.  Every lane calls add at
// every step and flush once.
template <bool MASS>
struct HistAcc {
  int hb = -1, hb2 = -1;
  uint32_t c = 0, c2 = 0;
  unsigned long long m = 0, m2 = 0;
  __device__ __forceinline__ void add(Smem& sm, bool active, int bin, unsigned long long mass) {
    if (hb < 0) {
      const uint64_t act = __ballot(active);
      if (act == 0) return;
      hb = __builtin_amdgcn_readlane(bin, __builtin_ctzll(act));
    }
    const bool hot = active && bin == hb;
    if (hot) {
      ++c;
      if (MASS) m += mass;
    }
    bool rest = active && !hot;
    if (MASS) {
      if (hb2 < 0) {
        const uint64_t r = __ballot(rest);
        if (r != 0) {
          const int b = __builtin_amdgcn_readlane(bin, __builtin_ctzll(r));
          if (__popcll(__ballot(rest && bin == b)) >= AGG_MIN) hb2 = b;
        }
      }
      const bool hot2 = rest && bin == hb2;
      if (hot2) {
        ++c2;
        m2 += mass;
      }
      rest = rest && !hot2;
    }
    hist_add<MASS>(sm, rest, bin, mass);
  }
  __device__ __forceinline__ void flush(Smem& sm) {
    if (hb < 0) return;
    const uint32_t cs = last_lane(wave_scan_u32(c, 0u, OpAdd()));
    const unsigned long long ms = MASS ? last_lane(wave_scan_add_u64(m)) : 0ull;
    uint32_t cs2 = 0;
    unsigned long long ms2 = 0;
    if (MASS && hb2 >= 0) {
      cs2 = last_lane(wave_scan_u32(c2, 0u, OpAdd()));
      ms2 = last_lane(wave_scan_add_u64(m2));
    }
    if ((threadIdx.x & (WAVE - 1)) == 0) {
      if (cs) atomicAdd(&sm.hist[hb], cs);
      if (MASS && ms) atomicAdd(&sm.hmass[hb], ms);
      if (MASS && cs2) atomicAdd(&sm.hist[hb2], cs2);
      if (MASS && ms2) atomicAdd(&sm.hmass[hb2], ms2);
    }
  }
};

// Whether a wave's keys crowd into one bin: at least AGG_MODE of the 64
// sampled keys (one per lane, `in` marking those that take part) share the
// first one's bin.  Wave-uniform; decides, per wave and pass, between one
// LDS atomic per key (diverse bins: nothing else is as cheap) and the
// aggregating adds above.
constexpr int AGG_MODE = 24;
__device__ __forceinline__ bool crowded(bool in, int bin) {
  const uint64_t act = __ballot(in);
  if (act == 0) return false;
  const int b0 = __builtin_amdgcn_readlane(bin, __builtin_ctzll(act));
  return __popcll(__ballot(in && bin == b0)) >= AGG_MODE;
}

// As for_keys, but every lane calls f(key, valid) at every step (no branch
// around the call), so f may use wave-wide operations such as hist_add.
template <bool IN_LDS, class F>
__device__ __forceinline__ void for_keys_all(const Keys<IN_LDS>& key, int n, const F& f) {
  const int tid = threadIdx.x;
  const int n4 = n >> 2;
  if (IN_LDS) {
    constexpr int PER = LDS_KEYS / 4 / NT;   // n <= LDS_KEYS
    const uint4* k4 = reinterpret_cast<const uint4*>(key.lds);
    uint4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * NT;
      v[u] = i < n4 ? k4[i] : make_uint4(0u, 0u, 0u, 0u);
    }
    const int wbase = tid & ~(WAVE - 1);   // the wave's first thread
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if (wbase + u * NT >= n4) break;   // no lane of this wave has a key left (uniform)
      const bool ok = tid + u * NT < n4;
      f(v[u].x, ok); f(v[u].y, ok); f(v[u].z, ok); f(v[u].w, ok);
    }
    const int t = 4 * n4 + tid;   // the last n % 4 keys (fewer than NT)
    if (wbase + 4 * n4 < n) f(t < n ? key.lds[t] : 0u, t < n);
  } else {
    const float* g = key.g;
    const int m4 = (reinterpret_cast<uintptr_t>(g) & 15) == 0 ? n4 : 0;
    const float4* g4 = reinterpret_cast<const float4*>(g);
    for (int i0 = 0; i0 < m4; i0 += GU * NT) {
      float4 v[GU];
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        const int i = i0 + tid + u * NT;
        v[u] = i < m4 ? g4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < GU; ++u) {
        const int i = i0 + tid + u * NT;
        const bool ok = i < m4;
        const uint4 k = key.four(v[u], 4 * i);
        f(k.x, ok); f(k.y, ok); f(k.z, ok); f(k.w, ok);
      }
    }
    for (int t0 = 4 * m4; t0 < n; t0 += NT) {   // uniform trip count
      const int t = t0 + tid;
      f(t < n ? key(t) : 0u, t < n);
    }
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
// RF (optional): rem = rf(total), the digit's total (masses with MASS,
// else counts) worked out from the wave totals before the search, for a
// first digit whose target depends on the total of every key.
struct KeepRem {
  __device__ unsigned long long operator()(unsigned long long) const { return 0ull; }
};
// save (optional): each count also goes to save[bin] as it is read.
template <bool MASS, class RF = KeepRem>
__device__ __forceinline__ void resolve_digit(Smem& sm, int nb, unsigned long long rem,
                                              RF rf = RF(), uint16_t* save = nullptr) {
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = wave_index();
  const int p0 = 2 * tid;
  uint32_t c0 = 0, c1 = 0;
  unsigned long long m0 = 0, m1 = 0;
  if (p0 < nb) {
    const int b0 = nb - 1 - p0, b1 = b0 - 1;
    c0 = sm.hist[b0]; c1 = sm.hist[b1];
    sm.hist[b0] = 0; sm.hist[b1] = 0;
    if (save) { save[b0] = (uint16_t)c0; save[b1] = (uint16_t)c1; }
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
  if (lane == WAVE - 1) {
    if (MASS) sm.f_m[wave] = incl;
    sm.f_c[wave] = incl_c;
  }
  __syncthreads();
  unsigned long long wb = 0;
  uint32_t wbc = 0;
  if constexpr (!std::is_same<RF, KeepRem>::value) {
    unsigned long long total = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) total += MASS ? sm.f_m[w] : (unsigned long long)sm.f_c[w];
    rem = rf(total);
  }
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    if (w < wave) {
      if (MASS) wb += sm.f_m[w];
      wbc += sm.f_c[w];
    }
  }
  if (!MASS) wb = wbc;
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
// REG: count the wave's first-key bin in registers (HistAcc), for key sets
// that may crowd into one bin; otherwise every key goes through hist_add.
// RF: as resolve_digit's, for the first digit (rem is then ignored).
// EX: after each digit, ex(keys above the prefix found so far, keys that
// carry it) may end the descent early (returns true; the result is then
// not the key the full descent gives).
struct NoExit {
  __device__ bool operator()(uint32_t, uint32_t) const { return false; }
};
template <bool MASS, bool IN_LDS, class FX, bool REG = true, class RF = KeepRem,
          class EX = NoExit>
__device__ __forceinline__ uint32_t descend(const Keys<IN_LDS>& key, int n, int cp, uint32_t lo_key,
                            unsigned long long rem, Smem& sm, const FX& fx,
                            uint32_t* cnt_above_out, unsigned long long* rem_out,
                            bool top_ready = false, uint32_t* eq_out = nullptr, RF first_rf = RF(),
                            EX ex = EX(), uint16_t* save_first = nullptr,
                            bool first_ready = false) {
  // top_ready: sm.hist already holds the top DIGIT bits of every key;
  // first_ready: it holds the first digit below the shared prefix (as
  // save_first keeps it, counts below 2^16) of every key
  if (top_ready) cp = 0;
  uint32_t pmask = cp <= 0 ? 0u : (cp >= 32 ? ~0u : ~0u << (32 - cp));
  uint32_t prefix = lo_key & pmask, cnt_above = 0;
  int left = cp >= 32 ? 0 : 32 - cp;
  bool ready = top_ready || first_ready;
  uint32_t pref_cnt = (uint32_t)n;   // keys matching the current prefix
  bool first = true;
#pragma unroll 1
  while (left > 0) {
    const int bits = min(DIGIT, left);
    const int shift = left - bits;
    const int nb = 1 << bits;
    bool crowd = false;
    if (!ready && REG) {   // sample: each lane's first key of the pass
      const int t = 4 * (int)threadIdx.x;
      const uint32_t kk = t < n ? key(t) : 0u;
      const bool in = t < n && (kk & pmask) == prefix;
      crowd = crowded(in, (int)((kk >> shift) & (uint32_t)(nb - 1)));
    }
    if (!ready && crowd) {
      HistAcc<MASS> acc;
      for_keys_all(key, n, [&](uint32_t kk, bool valid) {
        const bool in = valid && (kk & pmask) == prefix;
        acc.add(sm, in, (int)((kk >> shift) & (uint32_t)(nb - 1)), MASS && in ? fx(kk) : 0ull);
      });
      acc.flush(sm);
    } else if (!ready && REG) {
      for_keys(key, n, [&](uint32_t kk) {
        if ((kk & pmask) == prefix) {
          const int bin = (kk >> shift) & (nb - 1);
          atomicAdd(&sm.hist[bin], 1u);
          if (MASS) atomicAdd(&sm.hmass[bin], fx(kk));
        }
      });
    } else if (!ready) {
      for_keys_all(key, n, [&](uint32_t kk, bool valid) {
        const bool in = valid && (kk & pmask) == prefix;
        hist_add<MASS>(sm, in, (int)((kk >> shift) & (uint32_t)(nb - 1)),
                       MASS && in ? fx(kk) : 0ull);
      });
    }
    __syncthreads();
    bool plain = true;
    if constexpr (!std::is_same<RF, KeepRem>::value) {
      if (first) {   // the first digit's target from its total
        resolve_digit<MASS>(sm, nb, rem, [&](unsigned long long total) {
          rem = first_rf(total);
          return rem;
        }, save_first);
        plain = false;
      }
    }
    if (plain) resolve_digit<MASS>(sm, nb, rem, KeepRem(), first ? save_first : nullptr);
    first = false;
    ready = false;
    rem -= MASS ? sm.mass_above : (unsigned long long)sm.cnt_above;
    cnt_above += sm.cnt_above;
    pref_cnt = sm.bin_cnt;
    prefix |= sm.bin << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    left -= bits;
    if (left > 0 && ex(cnt_above, pref_cnt)) break;   // uniform
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

constexpr int EPI = LDS_KEYS / NWV / (4 * WAVE);   // register steps per lane (seg <= EPI * 256)

// Of e keys equal to T that follow `before` earlier ones (in token order),
// how many are kept when the first `quota` of them are: min(max(quota -
// before, 0), e), in signed 64-bit arithmetic (the unsigned form
// `quota > before ? min(quota - before, e) : 0` once compiled to an
// unguarded subtraction).
__device__ __forceinline__ uint32_t ties_kept(uint32_t quota, uint32_t before, uint32_t e) {
  const int64_t avail = (int64_t)quota - (int64_t)before;
  return (uint32_t)(avail <= 0 ? 0 : (avail < (int64_t)e ? avail : (int64_t)e));
}

// Bit b of the result: key b of the lane's run (token tl + b) is valid
// (below s1, or the whole wave is: `full`) and satisfies pred.  The keys are
// taken last to first, each doubling the mask and adding its predicate, an
// add with the compare's carry; full waves skip the bounds.
template <class P>
__device__ __forceinline__ uint32_t run_mask(const uint4 (&ek)[EPI], int tl, int s1, int JR,
                                             bool full, const P& pred) {
  uint32_t mm = 0u;
  if (full) {
#pragma unroll
    for (int j = EPI - 1; j >= 0; --j) {
      if (j >= JR) continue;   // uniform
      mm = mm + mm + (pred(ek[j].w) ? 1u : 0u);
      mm = mm + mm + (pred(ek[j].z) ? 1u : 0u);
      mm = mm + mm + (pred(ek[j].y) ? 1u : 0u);
      mm = mm + mm + (pred(ek[j].x) ? 1u : 0u);
    }
  } else {
    const int left = s1 - tl;   // this lane's keys in the segment
#pragma unroll
    for (int j = EPI - 1; j >= 0; --j) {
      if (j >= JR) continue;   // uniform
      mm = mm + mm + (4 * j + 3 < left && pred(ek[j].w) ? 1u : 0u);
      mm = mm + mm + (4 * j + 2 < left && pred(ek[j].z) ? 1u : 0u);
      mm = mm + mm + (4 * j + 1 < left && pred(ek[j].y) ? 1u : 0u);
      mm = mm + mm + (4 * j < left && pred(ek[j].x) ? 1u : 0u);
    }
  }
  return mm;
}

// One digit's histogram over a wave's register-held keys, each lane holding
// a run of R = 4 * JR consecutive tokens (key 4 j + u of the lane is token
// tl + 4 j + u, valid below s1; `full`: every key of the wave is valid; the
// same keys sit in the wave's LDS stretch): keys whose bits from `hi` up
// equal `prefix` add one to bin (key >> lo) of the bits below `hi`.  A wave
// whose sampled keys crowd into one bin aggregates its adds.
__device__ __forceinline__ void count_runs(const uint4 (&ek)[EPI], int tl, int s1, int JR, bool full,
                                           int hi, int lo, uint32_t prefix, Smem& sm,
                                           const uint32_t* stretch) {
  const uint32_t bmask = (1u << (hi - lo)) - 1u;
  const bool in0 = tl < s1 && (ek[0].x >> hi) == prefix;
  if (crowded(in0, (int)((ek[0].x >> lo) & bmask))) {
    HistAcc<false> acc;
#pragma unroll
    for (int j = 0; j < EPI; ++j) {
      if (j >= JR) break;   // uniform
      const int t = tl + 4 * j;
      const uint32_t kk[4] = {ek[j].x, ek[j].y, ek[j].z, ek[j].w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc.add(sm, t + u < s1 && (kk[u] >> hi) == prefix, (int)((kk[u] >> lo) & bmask), 0ull);
    }
    acc.flush(sm);
    return;
  }
  // Otherwise each lane marks its keys that carry the prefix in a bit mask
  // and adds them one by one (a few per lane: the lower digits match a few
  // keys of a head), reading each key back from the wave's stretch of LDS
  // (16-byte chunk c at slot c ^ ((c >> 3) & 7)): one LDS atomic per
  // matching key of the busiest lane instead of one per four keys.
  uint32_t mm = run_mask(ek, tl, s1, JR, full, [&](uint32_t kk) { return (kk >> hi) == prefix; });
  const int lane = threadIdx.x & (WAVE - 1);
  while (mm) {
    const int bit = __builtin_ctz(mm);
    mm &= mm - 1u;
    const int c = lane * JR + (bit >> 2);
    const uint32_t key = stretch[4 * (c ^ ((c >> 3) & 7)) + (bit & 3)];
    atomicAdd(&sm.hist[(key >> lo) & bmask], 1u);
  }
}

// Emit from register-held runs (the layout of count_runs; the wave's
// segment starts at s0): keeps key > T, and the first `quota` keys equal to
// T (eq_total of them in the head), ascending.  Each lane gathers its kept
// keys into a bit mask (bit b: token tl + b), a wave scan of the masks'
// popcounts places each lane's tokens in the wave's stretch of keys_lds
// (free LDS of at least n words), and the wave copies its stretch out
// contiguously at the offset the earlier waves leave.  Ties: the equal keys
// before each lane (a wave scan plus the earlier waves' counts) decide how
// many of the lane's equal keys, lowest tokens first, are kept.
__device__ __forceinline__ void emit_runs(const uint4 (&ek)[EPI], int s0, int tl, int s1, int JR,
                                          bool full, int n, uint32_t T, uint32_t quota,
                                          uint32_t eq_total, uint32_t* keys_lds, Smem& sm,
                                          int32_t* dst) {
  const int lane = threadIdx.x & (WAVE - 1), wave = wave_index();
  const bool all_ties = quota >= eq_total;   // then the keep rule is key >= T
  uint32_t keep, eqm = 0u;
  if (all_ties) {
    keep = run_mask(ek, tl, s1, JR, full, [&](uint32_t kk) { return kk >= T; });
  } else {
    keep = run_mask(ek, tl, s1, JR, full, [&](uint32_t kk) { return kk > T; });
    eqm = run_mask(ek, tl, s1, JR, full, [&](uint32_t kk) { return kk == T; });
  }
  if (!all_ties) {
    const uint32_t ne = (uint32_t)__popc(eqm);
    const uint32_t incl = wave_scan_u32(ne, 0u, OpAdd());
    if (lane == WAVE - 1) sm.w_eq[wave] = incl;
    __syncthreads();
    uint32_t before = incl - ne;
    for (int w = 0; w < wave; ++w) before += sm.w_eq[w];
    // the lane keeps the first ties_kept(...) of its equal keys
    const uint32_t m = ties_kept(quota, before, ne);
    uint32_t rest = eqm;
    for (uint32_t i = 0; i < m; ++i) rest &= rest - 1u;   // drop the lowest m
    keep |= eqm ^ rest;
  }
  const uint32_t nk = (uint32_t)__popc(keep);
  const uint32_t incl = wave_scan_u32(nk, 0u, OpAdd());
  const uint32_t wave_nk = last_lane(incl);
  if (lane == 0) sm.w_gt[wave] = wave_nk;
  uint32_t* stage = keys_lds + s0;
  uint32_t at = incl - nk;
  while (keep) {
    stage[at++] = (uint32_t)(tl + __builtin_ctz(keep));
    keep &= keep - 1u;
  }
  __syncthreads();
  uint32_t slot = 0;
  for (int w = 0; w < wave; ++w) slot += sm.w_gt[w];
  for (uint32_t i = lane; i < wave_nk; i += WAVE)
    if (slot + i < (uint32_t)n) dst[slot + i] = (int32_t)stage[i];
}

// Emit of the kept indices from keys held in registers: wave w holds the
// keys of its segment [s0, s1) (seg a multiple of 256, four consecutive
// tokens per lane per step) in ek.  keys_lds is free LDS of at least n words
// once every wave holds its keys; LDS_BUSY: other waves may still read it
// on entry (then a barrier comes first).  Keeps key > T, and the first
// `quota` keys equal to T (eq_total of them in the head), ascending.
// Each step ranks its kept keys with one ballot per key and chained
// v_mbcnt; a full step (all 256 keys in the segment) takes its own copy of
// the step, whose masks are plain compares.
template <bool LDS_BUSY>
__device__ __forceinline__ void emit_regs(const uint4 (&ek)[EPI], int s0, int s1, int n, uint32_t T,
                                          uint32_t quota, uint32_t eq_total, uint32_t* keys_lds,
                                          Smem& sm, int32_t* dst) {
  const int lane = threadIdx.x & (WAVE - 1), wave = wave_index();
  // When every key equal to T is kept (no tie to rank) the keep rule is
  // key >= T; otherwise waves first count their equal keys for the ranks.
  const bool all_ties = quota >= eq_total;
  uint32_t eqr = 0;   // keys equal to T before this wave's next step
  if (!all_ties) {
    uint32_t eqw = 0;
#pragma unroll
    for (int j = 0; j < EPI; ++j) {
      const int base = s0 + j * 4 * WAVE;
      if (base >= s1) break;   // uniform
      const int left = s1 - base - 4 * lane;
      eqw += (uint32_t)__popcll(__ballot(left > 0 && ek[j].x == T)) +
             (uint32_t)__popcll(__ballot(left > 1 && ek[j].y == T)) +
             (uint32_t)__popcll(__ballot(left > 2 && ek[j].z == T)) +
             (uint32_t)__popcll(__ballot(left > 3 && ek[j].w == T));
    }
    if (lane == 0) sm.w_eq[wave] = eqw;
  }
  if (LDS_BUSY || !all_ties) __syncthreads();
  if (!all_ties)
    for (int w = 0; w < wave; ++w) eqr += sm.w_eq[w];
  uint32_t* stage = keys_lds + s0;
  // one spare word per thread in sm.hmass, which no caller reads after the
  // emit (the mass sums are done by then, and its first barrier, with
  // LDS_BUSY, orders this after their last reads)
  uint32_t* const spare = reinterpret_cast<uint32_t*>(sm.hmass) + threadIdx.x;
  uint32_t nk = 0;   // kept keys of this wave so far (uniform)
  // stage the kept ones of 4 keys per lane (token t + u), in token order
  auto put = [&](int t, bool k0, bool k1, bool k2, bool k3) {
    const uint64_t b0 = __ballot(k0), b1 = __ballot(k1), b2 = __ballot(k2), b3 = __ballot(k3);
    uint32_t at = __builtin_amdgcn_mbcnt_lo((uint32_t)b0, nk);
    at = __builtin_amdgcn_mbcnt_hi((uint32_t)(b0 >> 32), at);
    at = __builtin_amdgcn_mbcnt_lo((uint32_t)b1, at);
    at = __builtin_amdgcn_mbcnt_hi((uint32_t)(b1 >> 32), at);
    at = __builtin_amdgcn_mbcnt_lo((uint32_t)b2, at);
    at = __builtin_amdgcn_mbcnt_hi((uint32_t)(b2 >> 32), at);
    at = __builtin_amdgcn_mbcnt_lo((uint32_t)b3, at);
    at = __builtin_amdgcn_mbcnt_hi((uint32_t)(b3 >> 32), at);
    // a key not kept writes its token to the lane's own spare word instead
    // (no branch and no exec-mask change per key)
    *(k0 ? stage + at : spare) = (uint32_t)t;
    at += k0 ? 1u : 0u;
    *(k1 ? stage + at : spare) = (uint32_t)(t + 1);
    at += k1 ? 1u : 0u;
    *(k2 ? stage + at : spare) = (uint32_t)(t + 2);
    at += k2 ? 1u : 0u;
    *(k3 ? stage + at : spare) = (uint32_t)(t + 3);
    nk += (uint32_t)(__popcll(b0) + __popcll(b1) + __popcll(b2) + __popcll(b3));
  };
#pragma unroll
  for (int j = 0; j < EPI; ++j) {
    const int base = s0 + j * 4 * WAVE;
    if (base >= s1) break;   // uniform
    const int t = base + 4 * lane;
    const uint32_t kk[4] = {ek[j].x, ek[j].y, ek[j].z, ek[j].w};
    if (all_ties) {
      if (base + 4 * WAVE <= s1) {
        put(t, kk[0] >= T, kk[1] >= T, kk[2] >= T, kk[3] >= T);
      } else {
        const int left = s1 - t;
        put(t, left > 0 && kk[0] >= T, left > 1 && kk[1] >= T, left > 2 && kk[2] >= T,
            left > 3 && kk[3] >= T);
      }
    } else {
      // rank of each key equal to T among those of the head, in token order
      const int left = s1 - t;
      bool gt[4], eq[4];
      uint64_t be[4];
      uint32_t r = eqr;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        gt[u] = left > u && kk[u] > T;
        eq[u] = left > u && kk[u] == T;
        be[u] = __ballot(eq[u]);
        r += mbcnt(be[u]);
      }
      bool keep[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        keep[u] = gt[u] || (eq[u] && r < quota);
        r += eq[u] ? 1u : 0u;
      }
      put(t, keep[0], keep[1], keep[2], keep[3]);
      eqr += (uint32_t)(__popcll(be[0]) + __popcll(be[1]) + __popcll(be[2]) + __popcll(be[3]));
    }
  }
  if (lane == 0) sm.w_gt[wave] = nk;
  __syncthreads();
  uint32_t slot = 0;
  for (int w = 0; w < wave; ++w) slot += sm.w_gt[w];
  for (uint32_t i = lane; i < nk; i += WAVE)
    if (slot + i < (uint32_t)n) dst[slot + i] = (int32_t)stage[i];
}

template <bool IN_LDS>
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t keys_lds[IN_LDS ? LDS_KEYS : 4];
  __shared__ Smem sm;
  // the mass descent's first-digit counts, for the count descent that may
  // follow (counts of at most 65535 keys)
  __shared__ uint16_t save16[NBINS];
  const int head = blockIdx.x, b = head / a.Hkv;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = wave_index();
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
  // of the descent), which saves one sweep over the keys.  A wave whose keys
  // crowd into one bin (sampled from its first keys) aggregates its adds
  // (HistAcc, every lane calling visit at every step); other waves take one
  // LDS atomic per key.
  for (int i = tid; i < NBINS; i += NT) { sm.hist[i] = 0; sm.hmass[i] = 0; }
  HistAcc<false> acc;
  auto stats = [&](uint32_t kr, bool prot) -> uint32_t {
    const uint32_t kk = prot ? PROTECTED_KEY : kr;
    mn = min(mn, kk);
    mx = max(mx, kk);
    cnt += kk >= tk ? 1u : 0u;
    if (mass) tot += (double)from_key(kr);
    return kk;
  };
  auto visit = [&](uint32_t kr, bool prot) -> uint32_t {   // one atomic per key
    const uint32_t kk = stats(kr, prot);
    if (!mass) atomicAdd(&sm.hist[kk >> (32 - DIGIT)], 1u);
    return kk;
  };
  auto visit_all = [&](uint32_t kr, bool prot, bool valid) -> uint32_t {   // aggregating
    const uint32_t kk = prot ? PROTECTED_KEY : kr;
    if (valid) stats(kr, prot);
    acc.add(sm, valid && !mass, (int)(kk >> (32 - DIGIT)), 0ull);
    return kk;
  };
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
    const bool crowd = !mass && crowded(tid < n4, (int)(to_key(v[0].x) >> (32 - DIGIT)));
    __syncthreads();   // histogram cleared before the first count (loads in flight)
    if (crowd) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int i = tid + u * NT;
        const bool ok = i < n4;
        const int t = 4 * i;
        const uint32_t k0 = visit_all(to_key(v[u].x), is_prot(t), ok);
        const uint32_t k1 = visit_all(to_key(v[u].y), is_prot(t + 1), ok);
        const uint32_t k2 = visit_all(to_key(v[u].z), is_prot(t + 2), ok);
        const uint32_t k3 = visit_all(to_key(v[u].w), is_prot(t + 3), ok);
        if (ok) *reinterpret_cast<uint4*>(&keys_lds[t]) = make_uint4(k0, k1, k2, k3);
      }
      for (int t0 = 4 * n4; t0 < n; t0 += NT) {   // uniform trip count
        const int t = t0 + tid;
        const bool ok = t < n;
        const uint32_t kk = visit_all(to_key(ok ? src[t] : 0.f), is_prot(t), ok);
        if (ok) keys_lds[t] = kk;
      }
      acc.flush(sm);
    } else {
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
    }
  } else {
    const bool crowd = !mass && crowded(4 * tid < n, (int)(to_key(4 * tid < n ? src[4 * tid] : 0.f) >>
                                                        (32 - DIGIT)));
    __syncthreads();
    if (crowd) {
      const int m4 = (reinterpret_cast<uintptr_t>(src) & 15) == 0 ? n >> 2 : 0;
      const float4* g4 = reinterpret_cast<const float4*>(src);
      for (int i0 = 0; i0 < m4; i0 += GU * NT) {
        float4 v[GU];
#pragma unroll
        for (int u = 0; u < GU; ++u) {
          const int i = i0 + tid + u * NT;
          v[u] = i < m4 ? g4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < GU; ++u) {
          const int i = i0 + tid + u * NT;
          const bool ok = i < m4;
          visit_all(to_key(v[u].x), is_prot(4 * i), ok);
          visit_all(to_key(v[u].y), is_prot(4 * i + 1), ok);
          visit_all(to_key(v[u].z), is_prot(4 * i + 2), ok);
          visit_all(to_key(v[u].w), is_prot(4 * i + 3), ok);
        }
      }
      for (int t0 = 4 * m4; t0 < n; t0 += NT) {   // uniform trip count
        const int t = t0 + tid;
        const bool ok = t < n;
        visit_all(to_key(ok ? src[t] : 0.f), is_prot(t), ok);
      }
      acc.flush(sm);
    } else {
      for_scores(src, n, [&](float x, int t) { visit(to_key(x), is_prot(t)); });
    }
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
  bool saved_first = false;   // save16 holds the first digit's counts of every key
  bool mass_done = false;   // the mass descent gave the k-th key and the quota
  uint32_t mass_T = 0, mass_quota = 0, mass_eq = 0;
  if (bu.mode != KV_BUDGET_MASS) {
    k = count_budget(bu, head, n, cnt, lo, hi);
  } else if (tot > 0.0) {
    // mass: fixed point with 2^(61 - floor(log2 total)) so every sum < 2^62
    const double scale = ldexp(1.0, 61 - ilogb(tot));
    auto fx = [&](uint32_t kk) -> unsigned long long {   // protected keys: no mass
      const double v = kk == PROTECTED_KEY ? 0.0 : (double)from_key(kk) * scale;
      return v > 0.0 ? (unsigned long long)v : 0ull;
    };
    if (n_prot == 0 && cp < 32) {
      // No protected tokens: the first digit's histogram of the mass descent
      // sums every key's mass, so the target f * total comes from that sum
      // (no sweep of its own).  An unclamped count leaves the k-th key and
      // the tie quota known (the count descent below is skipped).
      unsigned long long tgt = 0;
      auto rf = [&](unsigned long long total) -> unsigned long long {
        unsigned long long t = (unsigned long long)ceil((double)bu.mass * (double)total);
        if (t > total) t = total;   // double rounding of f * total
        tgt = t;
        return t ? t : 1ull;        // no target: the descent's result goes unused
      };
      // After each digit the count lies in [above + 1, above + keys in the
      // chosen bin]; once that range is at or below lo (at or above hi) the
      // clamp decides k and the descent stops.
      int clamped = 0;   // -1: k = lo, +1: k = hi
      auto ex = [&](uint32_t ab, uint32_t in_bin) -> bool {
        if (tgt == 0) return false;
        if ((long long)ab + in_bin <= (long long)lo) clamped = -1;
        else if ((long long)ab + 1 >= (long long)hi) clamped = 1;
        return clamped != 0;
      };
      uint32_t above, eqm;
      unsigned long long rem;
      saved_first = n < 65536;
      const uint32_t Tm = descend<true>(key, n, cp, mn, 1ull, sm, fx, &above, &rem, false, &eqm,
                                        rf, ex, saved_first ? save16 : nullptr);
      if (clamped != 0) {
        k = clamped < 0 ? lo : hi;
      } else if (tgt > 0) {
        const unsigned long long fv = fx(Tm);   // > 0: its bin holds mass
        const unsigned long long j = fv ? (rem + fv - 1) / fv : 1ull;
        k = (int)(above + (uint32_t)j);
        if (k >= lo && k <= hi) {
          mass_T = Tm;
          mass_quota = (uint32_t)j;
          mass_eq = eqm;
          mass_done = true;
        }
      }
      k = min(max(k, lo), hi);
      goto budget_done;
    }
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
budget_done:
  k = min(max(k, n_prot), n);

  // The k-th key and the tie quota.
  uint32_t T, quota, eq_total = 0;
  if (mass_done) {
    T = mass_T;
    quota = mass_quota;
    eq_total = mass_eq;
  } else {
    uint32_t above;
    unsigned long long rem;
    auto nofx = [](uint32_t) { return 0ull; };
    if (saved_first) {   // the first digit is the mass descent's: its counts come back
      const int nb1 = 1 << min(DIGIT, 32 - cp);
      for (int i = tid; i < nb1; i += NT) sm.hist[i] = save16[i];
      __syncthreads();
    }
    T = descend<false>(key, n, cp, mn, (unsigned long long)k, sm, nofx, &above, &rem, !mass,
                       &eq_total, KeepRem(), NoExit(), nullptr, saved_first);
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
    uint4 ek[EPI];
#pragma unroll
    for (int j = 0; j < EPI; ++j) {
      const int t = s0 + j * 4 * WAVE + 4 * lane;
      ek[j] = t < s1 ? *reinterpret_cast<const uint4*>(&keys_lds[t]) : make_uint4(0u, 0u, 0u, 0u);
    }
    emit_regs<true>(ek, s0, s1, n, T, quota, eq_total, keys_lds, sm, dst);
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
// Selection from a precomputed top-digit histogram (kv_score_select): the
// score kernel has counted the top DIGIT key bits of every score of the
// head into hist[head][NBINS].  Count budgets (k, kept fraction) without
// protected tokens, heads of at most LDS_KEYS tokens.  One workgroup per
// head:
//   1. the histogram gives the top digit b1 of the k-th key and the count of
//      keys above it (the same scan as resolve_digit);
//   2. each wave loads its segment's scores into registers as keys, each
//      lane a run of consecutive tokens (the loads are issued before the
//      scan above and land during it);
//   3. the second and third digits are counted straight from the registers
//      (count_runs: only keys that carry the prefix found so far add);
//   4. the emit runs from the registers (emit_runs: per-lane bit masks of
//      the kept tokens, placed by one wave scan).
// The k-th key T and the tie quota are those of select_kernel, so the kept
// indices are the same.
template <bool VEC>   // VEC: 16-byte aligned scores with N_max a multiple of 4
__global__ __launch_bounds__(NT) void select_hist_kernel(SelectArgs a, const uint32_t* hist) {
  __shared__ __attribute__((aligned(16))) uint32_t keys_lds[LDS_KEYS];
  __shared__ Smem sm;
  const int head = blockIdx.x, b = head / a.Hkv;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = wave_index();
  const int n = a.ctx ? min(max(a.ctx[b], 0), a.N_max) : a.N_max;
  if (n == 0) {
    if (tid == 0) a.kept_count[head] = 0;
    return;
  }
  const int k = count_budget(a.bud, head, n, 0u, 1, n);
  const float* src = a.scores + (size_t)head * a.N_max;
  const uint32_t* hh = hist + (size_t)head * NBINS;
  // Every load below is issued before any is used (no branch between them:
  // indices past the head are clamped onto it and the keys masked later).
  static_assert(NBINS == 2 * NT, "two bins per thread");
  const uint32_t h0 = hh[tid], h1 = hh[tid + NT];
  const int seg = ((n + NWV - 1) / NWV + 4 * WAVE - 1) / (4 * WAVE) * (4 * WAVE);
  const int s0 = wave * seg, s1 = min(s0 + seg, n);
  // Lane l ends up holding the run of R = seg / 64 consecutive tokens from
  // tl = s0 + l R (R a multiple of 4, at most 4 EPI): key 4 j + u is token
  // tl + 4 j + u.  The scores are loaded coalesced (step j of lane l: the 16
  // bytes of tokens s0 + 256 j + 4 l) and turned into runs through the
  // wave's own stretch of keys_lds (below).
  const int JR = seg / (4 * WAVE);   // 16-byte steps per lane (uniform)
  const int tl = s0 + lane * (4 * JR);
  const bool full = s0 + seg <= n;   // every key of the wave is in the head
  // this wave's segment, loaded while the histogram is scanned: whole 16-byte
  // loads clamped onto the head's row (N_max - 4 is aligned) when the row
  // allows, else scalar loads clamped onto the head; tokens at or past n are
  // masked by their index, and steps past the segment go unused
  uint4 v4[VEC ? EPI : 1];
  float v1[VEC ? 1 : EPI][4];
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < EPI; ++j) v4[j] = ld16(src + min(s0 + j * 4 * WAVE + 4 * lane, a.N_max - 4));
  } else {
#pragma unroll
    for (int j = 0; j < EPI; ++j)
#pragma unroll
      for (int u = 0; u < 4; ++u) v1[j][u] = src[min(s0 + j * 4 * WAVE + 4 * lane + u, n - 1)];
  }
  sm.hist[tid] = h0;
  sm.hist[tid + NT] = h1;
  __syncthreads();
  resolve_digit<false>(sm, NBINS, (unsigned long long)k);   // leaves sm.hist cleared
  // keys as the score pass histogrammed them (score_key: scores written by
  // the score pass are never negative, so these order them as to_key does)
  // Coalesced steps to runs through the wave's stretch of keys_lds (only
  // this wave touches it, so no barrier): 16-byte chunk c of the stretch
  // (tokens s0 + 4 c .. + 3) sits at slot c ^ ((c >> 3) & 7), so that the
  // chunk writes (lane l: c = 64 j + l) and the run reads (lane l: c = JR l
  // + j) of eight consecutive lanes fall on eight different 16-byte bank
  // groups.
  uint4 ek[EPI];
  {
    uint4* stretch = reinterpret_cast<uint4*>(keys_lds + s0);
    auto slot = [](int c) { return c ^ ((c >> 3) & 7); };
#pragma unroll
    for (int j = 0; j < EPI; ++j) {
      if (j * 4 * WAVE >= seg) break;   // uniform
      uint4 key;
      if constexpr (VEC)
        key = make_uint4(score_key(__uint_as_float(v4[j].x)), score_key(__uint_as_float(v4[j].y)),
                         score_key(__uint_as_float(v4[j].z)), score_key(__uint_as_float(v4[j].w)));
      else
        key = make_uint4(score_key(v1[j][0]), score_key(v1[j][1]), score_key(v1[j][2]),
                         score_key(v1[j][3]));
      stretch[slot(j * WAVE + lane)] = key;
    }
#pragma unroll
    for (int j = 0; j < EPI; ++j)   // steps past the run (j >= JR, uniform) are never read
      ek[j] = j < JR ? stretch[slot(lane * JR + j)] : make_uint4(0u, 0u, 0u, 0u);
  }
  // The lower digits count straight from the registers: a key takes part
  // when its bits above the digit equal the prefix found so far.
  unsigned long long rem = (unsigned long long)(k - sm.cnt_above);
  uint32_t prefix = sm.bin;   // the top DIGIT bits of the k-th largest key
  count_runs(ek, tl, s1, JR, full, 32 - DIGIT, 32 - 2 * DIGIT, prefix, sm, keys_lds + s0);
  __syncthreads();
  resolve_digit<false>(sm, NBINS, rem);
  rem -= sm.cnt_above;
  prefix = prefix << DIGIT | sm.bin;   // the top 2 * DIGIT bits
  count_runs(ek, tl, s1, JR, full, 32 - 2 * DIGIT, 0, prefix, sm, keys_lds + s0);
  __syncthreads();
  resolve_digit<false>(sm, 1 << (32 - 2 * DIGIT), rem);
  rem -= sm.cnt_above;
  const uint32_t T = prefix << (32 - 2 * DIGIT) | sm.bin;   // the k-th largest key
  const uint32_t quota = (uint32_t)rem;                    // keys equal to T to keep
  const uint32_t eq_total = sm.bin_cnt;                    // keys equal to T in the head
  if (tid == 0) a.kept_count[head] = k;
  // keys_lds serves only as the emit's staging area here (no barrier needed)
  emit_runs(ek, s0, tl, s1, JR, full, n, T, quota, eq_total, keys_lds, sm,
            a.kept_idx + (size_t)head * a.N_max);
}

// ---------------------------------------------------------------------------
// Heads longer than LDS_KEYS tokens under a count budget.  One workgroup per
// head would leave most CUs idle and re-read the head on every sweep, so the
// head is cut into parts of PT tokens, one workgroup each, and the descent
// runs as four launches over the (part, head) grid with fixed digits of 11,
// 11 and 10 key bits:
//   0: each part histograms the top digit of its keys and counts keys >= tau
//      (skipped when the score pass has counted the head's top digits:
//      launch 1 then starts from that histogram);
//   1, 2: every workgroup of a head sums the parts' histograms of the last
//         digit, resolves it exactly as resolve_digit does for one workgroup
//         (so all of them agree), and histograms the next digit of its part;
//   3: the last digit gives T and the number of keys equal to T to keep;
//      each part writes its kept indices at the offset the earlier parts
//      leave (their counts above T and equal to T come from what launch 2
//      published: keys above the 22-bit prefix and the last digit's bins),
//      ties going to the earliest tokens.
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
  const uint32_t* head_hist;   // [H][NBINS] top-digit histogram of each head's keys from the
                               // score pass (count budgets, no protected tokens), or null
  int P;                 // parts per head
  uint32_t* hist;        // [H][3][P][NBINS]
  uint32_t* pstat;       // [H][P][4]: count >= tau, (unused), (unused), count above the
                         // 22-bit prefix
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
  const int lane = threadIdx.x & (WAVE - 1), wave = wave_index();
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
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = wave_index();
  const int n = a.ctx ? min(max(a.ctx[b], 0), a.N_max) : a.N_max;
  if (n == 0) {
    if (PHASE == 3 && part == 0 && tid == 0) a.kept_count[head] = 0;
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
    // bins tid and tid + NT (nb <= 2 NT), the parts' loads issued eight at a
    // time before any is added
    static_assert(NBINS <= 2 * NT, "two bins per thread");
    const uint32_t* hd = hist_h + (size_t)d * P * NBINS;
    const bool two = tid + NT < nb;
    uint32_t c0 = 0, c1 = 0;
    for (int q0 = 0; q0 < P; q0 += 8) {
      uint32_t v0[8], v1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const size_t row = (size_t)min(q0 + u, P - 1) * NBINS;
        v0[u] = hd[row + tid];
        v1[u] = two ? hd[row + tid + NT] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        c0 += q0 + u < P ? v0[u] : 0u;
        c1 += q0 + u < P ? v1[u] : 0u;
      }
    }
    if (tid < nb) sm.hist[tid] = c0;
    if (two) sm.hist[tid + NT] = c1;
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
    uint32_t cnt = 0;   // keys >= tau (threshold budgets; launch 0 counted them)
    if (!pa.head_hist)
      for (int q = 0; q < P; ++q) cnt += pstat_h[q * 4 + 0];
    int lo, hi;
    budget_clamps(bu, n, &lo, &hi);
    int k = count_budget(bu, head, n, cnt, lo, hi);
    k = min(max(k, n_prot), n);
    if (pa.head_hist) {   // the head's top digits as the score pass counted them
      const uint32_t* hh = pa.head_hist + (size_t)head * NBINS;
      for (int i = tid; i < NBINS; i += NT) sm.hist[i] = hh[i];
      __syncthreads();
    } else {
      sum_parts(0, NBINS);
    }
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
    uint32_t above = 0;   // keys above every key that carries the prefix
#pragma unroll
    for (int u = 0; u < PQ; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (valid(u, e) && (kk[u][e] >> 10) == (prefix >> 10)) atomicAdd(&sm.hist[kk[u][e] & 1023], 1u);
        above += valid(u, e) && (kk[u][e] >> 10) > (prefix >> 10) ? 1u : 0u;
      }
    above = block_sum(above, sm);
    if (tid == 0) pstat_h[part * 4 + 3] = above;
    publish(2, 1024);
    return;
  }

  // PHASE 3: the last digit gives T and the number of keys equal to T to
  // keep; then the emit.  Part q keeps its keys above T, g_q = (its keys
  // above the 22-bit prefix, counted in launch 2) + (its digit-3 bins above
  // T's), and its share of the ties, e_q = its bin of T: the earlier parts'
  // (g_q, e_q) place this part's kept tokens, ties going to the earliest.
  // The part's tokens form PQ * NWV chunks of 4 * WAVE consecutive tokens,
  // chunk (u, w) = lanes of wave w at load u, in token order u-major; each
  // chunk's kept tokens go out in lane order.
  const PartState ps = st_h[2];
  sum_parts(2, 1024);
  resolve_digit<false>(sm, 1024, (unsigned long long)ps.rem);
  const uint32_t b3 = sm.bin;
  const uint32_t T = ps.prefix | b3;
  const uint32_t quota = ps.rem - sm.cnt_above;
  __shared__ uint32_t pg[NWV], pe[NWV];
  uint32_t off = 0, eqb = 0;   // kept by, and ties in, the earlier parts
  for (int q0 = 0; q0 < part; q0 += NWV) {   // sixteen earlier parts per round, one per wave
    const int q = q0 + wave;
    if (q < part) {
      const uint32_t* h3 = hist_h + ((size_t)2 * P + q) * NBINS;
      uint32_t g = 0;
#pragma unroll
      for (int i = lane; i < 1024; i += WAVE) g += i > (int)b3 ? h3[i] : 0u;
      g = last_lane(wave_scan_u32(g, 0u, OpAdd()));
      if (lane == 0) { pg[wave] = g + pstat_h[q * 4 + 3]; pe[wave] = h3[b3]; }
    }
    __syncthreads();
    for (int w = 0; w < NWV && q0 + w < part; ++w) {   // in part order (uniform)
      off += pg[w] + ties_kept(quota, eqb, pe[w]);
      eqb += pe[w];
    }
    __syncthreads();
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
  // Exclusive prefix sums over the part's chunks in token order (chunk c =
  // (c / NWV, c % NWV), one lane each): G_c keys above T and E_c keys equal
  // to T before chunk c.  The ties kept before it are the first of the
  // part's eqb + E_c, i.e. ties_kept(quota, eqb, E_c) of the part's own.
  static_assert(PQ * NWV == WAVE, "one lane per chunk");
  __shared__ uint32_t gx[PQ * NWV], ex[PQ * NWV];
  if (wave == 0) {
    const uint32_t g = cg[lane / NWV][lane % NWV], e = ce[lane / NWV][lane % NWV];
    gx[lane] = wave_scan_u32(g, 0u, OpAdd()) - g;
    ex[lane] = wave_scan_u32(e, 0u, OpAdd()) - e;
  }
  __syncthreads();
  int32_t* dst = a.kept_idx + (size_t)head * a.N_max;
#pragma unroll
  for (int u = 0; u < PQ; ++u) {
    // slot and tie rank at the start of chunk (u, wave)
    const int c = u * NWV + wave;
    uint32_t slot = off + gx[c] + ties_kept(quota, eqb, ex[c]), r = eqb + ex[c];
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

// The launches of the part path (four, or three when the score pass gave the
// top-digit histogram); per-kernel timing sees them as one "select" (start
// stamped by the first dispatch, stop by the last).
void select_parts(const SelectArgs& s, int P, void* ws, const uint32_t* head_hist,
                  hipStream_t st) {
  PartArgs pa;
  pa.s = s;
  pa.head_hist = head_hist;
  pa.P = P;
  const int H = s.B * s.Hkv;
  pa.hist = static_cast<uint32_t*>(ws);
  pa.pstat = pa.hist + (size_t)H * 3 * P * NBINS;
  pa.state = reinterpret_cast<PartState*>(pa.pstat + (size_t)H * P * 4);
  const dim3 grid(P, H), block(NT);
  hipEvent_t e0, e1;
  const bool timed = timing_events("select", &e0, &e1);
  if (!head_hist) {
    if (timed)
      hipExtLaunchKernelGGL(select_part_kernel<0>, grid, block, 0, st, e0, nullptr, 0, pa);
    else
      hipLaunchKernelGGL(select_part_kernel<0>, grid, block, 0, st, pa);
  }
  if (timed && head_hist)
    hipExtLaunchKernelGGL(select_part_kernel<1>, grid, block, 0, st, e0, nullptr, 0, pa);
  else
    hipLaunchKernelGGL(select_part_kernel<1>, grid, block, 0, st, pa);
  hipLaunchKernelGGL(select_part_kernel<2>, grid, block, 0, st, pa);
  if (timed) {
    hipExtLaunchKernelGGL(select_part_kernel<3>, grid, block, 0, st, nullptr, e1, 0, pa);
    timing_done("select", e0, e1, grid, block);   // three or four launches of this shape
  } else {
    hipLaunchKernelGGL(select_part_kernel<3>, grid, block, 0, st, pa);
  }
}

}  // namespace
}  // namespace kvcc

using namespace kvcc;

extern "C" size_t kv_select_workspace_size(int B, int Hkv, int N_max) {
  return select_part_workspace(B, Hkv, N_max);
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
  if (const int st = check_budget(bu)) return st;

  // Long heads under a count budget take the part path when the workspace
  // is there (its size covers it whenever N_max > LDS_KEYS).
  if (select_parts_launch(scores, ctx_len, B, Hkv, N_max, bu, kept_idx, kept_count, workspace,
                          workspace_bytes, static_cast<hipStream_t>(stream)))
    return launch_status();
  select_launch(scores, ctx_len, nullptr, B, Hkv, N_max, bu, false, kept_idx, kept_count,
                static_cast<hipStream_t>(stream), "select");
  return launch_status();
}

int kvcc::check_budget(const kv_budget& bu) {
  if (bu.mode < KV_BUDGET_K || bu.mode > KV_BUDGET_MASS) return KV_ERR_MODE;
  if (!(bu.min_ratio >= 0.f && bu.min_ratio <= 1.f && bu.max_ratio >= 0.f && bu.max_ratio <= 1.f))
    return KV_ERR_MODE;
  if (bu.mode == KV_BUDGET_RATIO && !bu.ratio && !(bu.ratio_scalar >= 0.f && bu.ratio_scalar <= 1.f))
    return KV_ERR_MODE;
  if (bu.mode == KV_BUDGET_MASS && !(bu.mass >= 0.f && bu.mass <= 1.f)) return KV_ERR_MODE;
  if (bu.mode == KV_BUDGET_THRESHOLD && isnan(bu.tau)) return KV_ERR_MODE;
  if (bu.n_sink < 0 || bu.n_recent < 0) return KV_ERR_MODE;
  if (!aligned16(bu.k) || !aligned16(bu.ratio)) return KV_ERR_ALIGN;
  return KV_OK;
}

size_t kvcc::select_part_workspace(int B, int Hkv, int N_max) {
  if (B < 1 || Hkv < 1 || N_max <= LDS_KEYS) return 0;
  return part_workspace(B * Hkv, ceil_div(N_max, PT));
}

bool kvcc::select_parts_launch(const float* scores, const int32_t* ctx, int B, int Hkv, int N_max,
                               const kv_budget& bud, int32_t* kept_idx, int32_t* kept_count,
                               void* workspace, size_t workspace_bytes, hipStream_t st,
                               const uint32_t* head_hist) {
  const int P = ceil_div(N_max, PT);
  if (N_max <= LDS_KEYS || bud.mode == KV_BUDGET_MASS || !workspace ||
      workspace_bytes < part_workspace(B * Hkv, P))
    return false;
  SelectArgs a;
  a.scores = scores; a.ctx = ctx; a.n_head = nullptr; a.B = B; a.Hkv = Hkv; a.N_max = N_max;
  a.k_zero_ok = 0;
  a.bud = bud; a.kept_idx = kept_idx; a.kept_count = kept_count;
  select_parts(a, P, workspace, head_hist, st);
  return true;
}

bool kvcc::select_hist_budget(const kv_budget& bud) {
  return (bud.mode == KV_BUDGET_K || bud.mode == KV_BUDGET_RATIO) && bud.n_sink == 0 &&
         bud.n_recent == 0;
}

bool kvcc::select_hist_eligible(const kv_budget& bud, int N_max) {
  return N_max <= LDS_KEYS && select_hist_budget(bud);
}

void kvcc::select_hist_launch(const float* scores, const int32_t* ctx, const uint32_t* hist, int B,
                              int Hkv, int N_max, const kv_budget& bud, int32_t* kept_idx,
                              int32_t* kept_count, hipStream_t st) {
  SelectArgs a;
  a.scores = scores; a.ctx = ctx; a.n_head = nullptr; a.B = B; a.Hkv = Hkv; a.N_max = N_max;
  a.k_zero_ok = 0;
  a.bud = bud; a.kept_idx = kept_idx; a.kept_count = kept_count;
  if (aligned16(scores) && N_max % 4 == 0)
    launch("select", select_hist_kernel<true>, dim3(B * Hkv), dim3(NT), 0, st, a, hist);
  else
    launch("select", select_hist_kernel<false>, dim3(B * Hkv), dim3(NT), 0, st, a, hist);
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
