// Split-K decode attention over the packed, ragged compacted cache.
//
// One fresh query per query head reads its KV head's kept rows with plain
// softmax attention; the step is bandwidth-bound ("KVzap: Fast, Adaptive,
// and Faithful KV Cache Pruning", section 4, on decode cycles otherwise lost
// to memory bandwidth), so the kernel is organised around streaming each K/V
// row from HBM exactly once for all G query heads of its group.
//
// Work items are chunks of CH consecutive rows of one head; every workgroup
// rebuilds the item list from the offsets in LDS and walks it grid-stride,
// so ragged heads balance by rows, not by head count.  Inside an item a group
// of d*sizeof(T)/16 lanes owns one row at a time (16 bytes of K and of V per
// lane; RPS rows per stage, the next stage in flight while one is computed),
// forms the G dot products (bf16: v_dot2 against
// the packed query) with a DPP reduction inside the group, and keeps a
// base-2 (max, sum, o) per query head.  Groups merge through LDS in a fixed
// order into one partial per item; a second kernel merges each head's items
// in item order, so the result is deterministic.  A routed (VECTOR) cache has
// its own split kernel, which first sorts an item's rows into an exact and a
// rebuilt list, and the merge adds W_h times the rebuilt rows' sum.
#include <math.h>

#include <mutex>

#include "common.hpp"

namespace kvcc {
namespace {

constexpr int DT = 256;
constexpr int CH = 256;          // rows per work item
constexpr int RPG = 8;           // rows per lane group per pass (routed cache)
constexpr int RPS = 4;           // rows per lane group per stage (plain and fused split)
constexpr int MAX_HEADS = 4096;
constexpr int GRID_MAX = 1024;   // most split workgroups per query-head group

struct DecodeArgs {
  const void* q;
  const char* kc;
  const char* vc;
  const int64_t* offsets;
  int B, Hq, Hkv, G, n_sub, items_max;
  int64_t cap;
  float c;                 // scale * log2(e)
  float* part_o;           // [n_sub][items_max][GT][D]
  float2* part_ml;         // [n_sub][items_max][GT]
  int* item_start;         // [B*Hkv+1] first item of every head (written by the split kernel)
  float* out;
  float* lse;
  // routed cache (VECTOR): value row of key row r is vc[vmap[r]], or, when
  // vmap[r] < 0, W RoPE^-1(k_c[r]) at position pos[r]
  const int32_t* vmap;
  const int32_t* pos;
  const float* w;          // [Hkv][D][D]
  float rope_base;
  int64_t vcap;
  float* part_u;           // [n_sub][items_max][GT][D]: sum of p * RoPE^-1(k) of rebuilt rows
  // fused compaction (kv_compact_decode): the offsets are the exclusive scan
  // of cnt, and row r of head h is token idx[h][r - off[h]] of ksrc / vsrc,
  // copied to kc_w / vc_w (position to pos_w) as the split kernel reads it
  const int32_t* cnt;      // [B*Hkv] kept counts (NULL: plain decode over kc / vc)
  const int32_t* idx;      // [B*Hkv][N_max]
  const char* ksrc;
  const char* vsrc;
  int N_max;
  char* kc_w;
  char* vc_w;
  int32_t* pos_w;
  int64_t* off_w;          // [B*Hkv+1] the unclipped offsets, written by workgroup 0
};

// Row offsets clipped to the capacity, and the first item of every head.
__device__ void build_items(const DecodeArgs& a, long long* off, int* ist, int* wtot) {
  const int H = a.B * a.Hkv;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  constexpr int NWV = DT / WAVE;
  if (a.cnt) {   // fused compaction: exclusive scan of the kept counts
    __shared__ long long wl[DT / WAVE];
    long long carry = 0;
    for (int base = 0; base < H; base += DT) {
      const int i = base + tid;
      const long long c = i < H ? (long long)max(a.cnt[i], 0) : 0ll;
      const long long inc = wave_incl_scan<long long>(c);
      if (lane == WAVE - 1) wl[wave] = inc;
      __syncthreads();
      long long before = 0, chunk = 0;
      for (int w = 0; w < NWV; ++w) {
        if (w < wave) before += wl[w];
        chunk += wl[w];
      }
      if (i < H) off[i] = carry + before + inc - c;
      carry += chunk;
      __syncthreads();
    }
    if (tid == 0) off[H] = carry;
    __syncthreads();
    if (blockIdx.x == 0 && blockIdx.y == 0)
      for (int i = tid; i <= H; i += DT) a.off_w[i] = off[i];
    __syncthreads();
    for (int i = tid; i <= H; i += DT) off[i] = min(off[i], (long long)a.cap);
  } else {
    for (int i = tid; i <= H; i += DT) {
      const long long o = a.offsets[i];
      off[i] = o < 0 ? 0 : (o > a.cap ? a.cap : o);
    }
  }
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < H; base += DT) {
    const int i = base + tid;
    const int ni = i < H ? (int)(max(off[i + 1] - off[i], 0ll) + CH - 1) / CH : 0;
    const int inc = wave_incl_scan<int>(ni);
    if (lane == WAVE - 1) wtot[wave] = inc;
    __syncthreads();
    int before = 0, chunk = 0;
    for (int w = 0; w < NWV; ++w) {
      if (w < wave) before += wtot[w];
      chunk += wtot[w];
    }
    if (i < H) ist[i] = carry + before + inc - ni;
    carry += chunk;
    __syncthreads();
  }
  if (tid == 0) ist[H] = carry;
  __syncthreads();
}

__device__ __forceinline__ int find_item_head(const int* ist, int H, int it) {
  int lo = 0, hi = H - 1;   // largest i with ist[i] <= it
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ist[mid] <= it) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <typename T>
__device__ __forceinline__ void unpack16(const uint4 w, float* x);
template <>
__device__ __forceinline__ void unpack16<__bf16>(const uint4 w, float* x) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}
template <>
__device__ __forceinline__ void unpack16<float>(const uint4 w, float* x) {
  x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
  x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
}

// One lane's slice (EPL elements) of the query of each of the GT heads of a
// group.  bf16 slices stay packed: the lane's 16 bytes of a key row enter
// v_dot2 against them directly (a bf16 product is exact in fp32) and the
// scale multiplies the reduced sum.  fp32 slices are scaled up front.
template <typename T, int GT> struct QSlices;

template <int GT> struct QSlices<__bf16, GT> {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  uint4 q[GT];
  template <int D>
  __device__ void load(const DecodeArgs& a, int b, int h, int qsub, int sub) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const int jg = qsub * GT + g;
      q[g] = make_uint4(0, 0, 0, 0);
      if (jg < a.G)
        q[g] = ld16(static_cast<const char*>(a.q) +
                    (((size_t)b * a.Hq + h * a.G + jg) * D + (size_t)sub * 8) * sizeof(__bf16));
    }
  }
  static __device__ __forceinline__ float d2(uint32_t x, uint32_t y, float s) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, x), __builtin_bit_cast(bf2, y), s,
                                           false);
  }
  __device__ __forceinline__ float score(int g, const uint4 k, float c) const {
    return d2(q[g].w, k.w, d2(q[g].z, k.z, d2(q[g].y, k.y, d2(q[g].x, k.x, 0.f))));
  }
  static constexpr bool kScaled = false;
};

template <int GT> struct QSlices<float, GT> {
  float q[GT][4];
  template <int D>
  __device__ void load(const DecodeArgs& a, int b, int h, int qsub, int sub) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const int jg = qsub * GT + g;
      uint4 w = make_uint4(0, 0, 0, 0);
      if (jg < a.G)
        w = ld16(static_cast<const char*>(a.q) +
                 (((size_t)b * a.Hq + h * a.G + jg) * D + (size_t)sub * 4) * sizeof(float));
      q[g][0] = __uint_as_float(w.x) * a.c; q[g][1] = __uint_as_float(w.y) * a.c;
      q[g][2] = __uint_as_float(w.z) * a.c; q[g][3] = __uint_as_float(w.w) * a.c;
    }
  }
  __device__ __forceinline__ float score(int g, const uint4 k, float) const {
    float s = q[g][0] * __uint_as_float(k.x);
    s = fmaf(q[g][1], __uint_as_float(k.y), s);
    s = fmaf(q[g][2], __uint_as_float(k.z), s);
    return fmaf(q[g][3], __uint_as_float(k.w), s);
  }
  static constexpr bool kScaled = true;
};

// A lane group's running base-2 softmax state for the GT query heads over
// the rows it has seen: maximum m, sum l, and o = sum of weight * row.
template <int GT, int EPL> struct RowState {
  float m[GT], l[GT], o[GT][EPL];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] = 0.f;
    }
  }
  // raise the maximum to cover a pass's scores (rows with ok[u]), rescaling
  template <int R>
  __device__ __forceinline__ void cover(const float (&sc)[R][GT], const bool (&ok)[R]) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float mm = m[g];
#pragma unroll
      for (int u = 0; u < R; ++u)
        if (ok[u]) mm = fmaxf(mm, sc[u][g]);
      if (mm != -INFINITY && mm != m[g]) {
        const float w = fast_exp2(m[g] - mm);   // 0 when m was -inf
        l[g] *= w;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] *= w;
        m[g] = mm;
      }
    }
  }
  __device__ __forceinline__ void add(const float (&sc)[GT], const float (&x)[EPL]) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float p = fast_exp2(sc[g] - m[g]);
      l[g] += p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] = fmaf(p, x[e], o[g][e]);
    }
  }
  // park this lane group's state in LDS for the group merge
  template <int NG, int D>
  __device__ __forceinline__ void park(float (&sm)[NG][GT][D], float (&sm_m)[NG][GT],
                                       float (&sm_l)[NG][GT], int grp, int sub) const {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      if (sub == 0) { sm_m[grp][g] = m[g]; sm_l[grp][g] = l[g]; }
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm[grp][g][sub * EPL + e] = o[g][e];
    }
  }
};

// Fixed-order merge of the NG parked lane-group states.  Slot k of this
// thread is x = tid + k * DT, i.e. (g, e) = (x / D, x % D), when x < GT * D.
template <int NG, int GT, int D>
struct GroupMerge {
  static constexpr int S = (GT * D + DT - 1) / DT;
  float M[S], L[S], O[S];
  __device__ __forceinline__ void run(const float (&sm)[NG][GT][D], const float (&sm_m)[NG][GT],
                                      const float (&sm_l)[NG][GT], int tid) {
#pragma unroll
    for (int k = 0; k < S; ++k) {
      const int x = tid + k * DT;
      M[k] = -INFINITY; L[k] = 0.f; O[k] = 0.f;
      if (GT * D % DT != 0 && x >= GT * D) continue;
      const int g = x / D, e = x % D;
      float mx = -INFINITY;
      for (int r = 0; r < NG; ++r) mx = fmaxf(mx, sm_m[r][g]);
      if (mx == -INFINITY) continue;
      float l = 0.f, o = 0.f;
      for (int r = 0; r < NG; ++r) {
        const float w = fast_exp2(sm_m[r][g] - mx);
        l = fmaf(sm_l[r][g], w, l);
        o = fmaf(sm[r][g][e], w, o);
      }
      M[k] = mx; L[k] = l; O[k] = o;
    }
  }
};

// FUSED: the rows come from the full cache through the kept indices and are
// written to the packed cache on the way (kv_compact_decode); the arithmetic
// is the same, so the result equals kv_compact followed by kv_decode_attn.
// An item is walked in stages of NG * RPS rows, two register sets deep: the
// next stage's loads go out once this stage's rows have landed (and, fused,
// been stored) and stay in flight while this stage is computed.  Every load
// is branch-free and every stage issues the next one (a row past the item
// re-reads the item's last row, an index outside [0, N_max) reads token 0;
// both are masked or zeroed afterwards), so the wait for a stage's rows never
// covers the next stage's.
template <typename T, int D, int GT, bool FUSED>
__global__ __launch_bounds__(DT) void decode_split(DecodeArgs a) {
  constexpr int EPL = 16 / (int)sizeof(T);     // elements per lane
  constexpr int LPR = D / EPL;                 // lanes per row (power of two, <= 32)
  constexpr int NG = DT / LPR;                 // row groups per workgroup
  constexpr int PS = NG * RPS;                 // rows per stage
  constexpr int ROWB = D * (int)sizeof(T);
  static_assert(CH % (2 * PS) == 0, "an item is a whole number of stage pairs");
  typedef GroupMerge<NG, GT, D> Merge;

  __shared__ int wtot[DT / WAVE];
  __shared__ float sm_m[NG][GT], sm_l[NG][GT];
  __shared__ float sm_o[NG][GT][D];
  __shared__ int sidx[CH];             // fused: the item's kept indices (-1 past its end)
  extern __shared__ long long dyn[];   // off[H+1] (int64) then ist[H+1] (int32)
  const int H = a.B * a.Hkv;
  long long* off = dyn;
  int* ist = reinterpret_cast<int*>(dyn + H + 1);

  build_items(a, off, ist, wtot);
  const int n_items = ist[H];
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i <= H; i += DT) a.item_start[i] = ist[i];
  const int tid = threadIdx.x, grp = tid / LPR, sub = tid % LPR;
  const int qsub = blockIdx.y;

  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int head = find_item_head(ist, H, it);
    const int b = head / a.Hkv, h = head % a.Hkv;
    const long long r0 = off[head] + (long long)(it - ist[head]) * CH;
    const long long r1 = min(r0 + CH, off[head + 1]);

    QSlices<T, GT> qs;
    qs.template load<D>(a, b, h, qsub, sub);
    RowState<GT, EPL> st;
    st.reset();
    if constexpr (FUSED) {   // one round trip for the item's indices
      for (int i = tid; i < CH; i += DT) {
        const long long row = r0 + i;
        const long long r = row - off[head];
        sidx[i] = row < r1 && r < a.N_max ? a.idx[(size_t)head * a.N_max + r] : -1;
      }
      __syncthreads();
    }
    // row u of a stage at `base` is base + grp + u * NG
    auto issue = [&](uint4 (&kr)[RPS], uint4 (&vr)[RPS], long long base)
        __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < RPS; ++u) {
        const long long row = min(base + grp + (long long)u * NG, r1 - 1);
        size_t src;
        if constexpr (FUSED) {
          const int t = sidx[(int)(row - r0)];
          src = ((size_t)head * a.N_max + ((unsigned)t < (unsigned)a.N_max ? t : 0)) * ROWB;
        } else {
          src = (size_t)row * ROWB;
        }
        const char* kb = FUSED ? a.ksrc : a.kc;
        const char* vb = FUSED ? a.vsrc : a.vc;
        kr[u] = ld16(kb + src + sub * 16);
        vr[u] = ld16(vb + src + sub * 16);
      }
    };
    auto process = [&](uint4 (&kr)[RPS], uint4 (&vr)[RPS], long long base, auto&& next)
        __attribute__((always_inline)) {
      bool ok[RPS];
#pragma unroll
      for (int u = 0; u < RPS; ++u) ok[u] = base + grp + (long long)u * NG < r1;
      if constexpr (FUSED) {
        int t[RPS];
#pragma unroll
        for (int u = 0; u < RPS; ++u) {
          t[u] = sidx[(int)(base + grp + (long long)u * NG - r0)];
          // an index outside [0, N_max) packs a zero K/V row (as kv_compact
          // does), which the attention then reads like any other row
          if ((unsigned)t[u] >= (unsigned)a.N_max) {
            kr[u] = make_uint4(0, 0, 0, 0);
            vr[u] = make_uint4(0, 0, 0, 0);
          }
        }
        if (qsub == 0) {
#pragma unroll
          for (int u = 0; u < RPS; ++u) {
            const long long row = base + grp + (long long)u * NG;
            if (ok[u]) {
              st16(a.kc_w + (size_t)row * ROWB + sub * 16, kr[u]);
              st16(a.vc_w + (size_t)row * ROWB + sub * 16, vr[u]);
              if (sub == 0) a.pos_w[row] = t[u];
            }
          }
        }
      }
      next();
      float sc[RPS][GT];
#pragma unroll
      for (int u = 0; u < RPS; ++u)
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          sc[u][g] = group_sum<LPR>(qs.score(g, kr[u], a.c));
          if (!QSlices<T, GT>::kScaled) sc[u][g] *= a.c;
        }
      st.cover(sc, ok);
#pragma unroll
      for (int u = 0; u < RPS; ++u) {
        if (ok[u]) {
          float vx[EPL];
          unpack16<T>(vr[u], vx);
          st.add(sc[u], vx);
        }
      }
    };
    uint4 kr0[RPS], vr0[RPS], kr1[RPS], vr1[RPS];
    issue(kr0, vr0, r0);
    for (long long base = r0; base < r1; base += 2 * PS) {
      const long long b1 = base + PS;
      process(kr0, vr0, base, [&]() __attribute__((always_inline)) { issue(kr1, vr1, b1); });
      if (b1 >= r1) break;
      process(kr1, vr1, b1, [&]() __attribute__((always_inline)) { issue(kr0, vr0, b1 + PS); });
    }

    // merge the row groups (fixed order) into this item's partial
    st.park(sm_o, sm_m, sm_l, grp, sub);
    __syncthreads();
    Merge mg;
    mg.run(sm_o, sm_m, sm_l, tid);
    const size_t pbase = ((size_t)qsub * a.items_max + it) * GT;
#pragma unroll
    for (int k = 0; k < Merge::S; ++k) {
      const int x = tid + k * DT;
      if (GT * D % DT != 0 && x >= GT * D) continue;
      const int g = x / D, e = x % D;
      a.part_o[(pbase + g) * D + e] = mg.O[k];
      if (e == 0) a.part_ml[pbase + g] = make_float2(mg.M[k], mg.L[k]);
    }
    __syncthreads();
  }
}

// Split kernel over a routed cache.  Each item first sorts its rows into two
// lists in LDS, in row order within each: exact rows (value row vmap[r]) and
// rebuilt rows (position pos[r]).  The lane groups walk the exact rows (key
// and value loads, no per-row branch), merge, then walk the rebuilt rows:
// the key row is turned back by RoPE^-1 and accumulated as U, the sum that
// the merge kernel multiplies by W_h once per query head.  The two phases'
// states meet in the item's partial under one maximum.
template <typename T, int D, int GT>
__global__ __launch_bounds__(DT) void vector_decode_split(DecodeArgs a) {
  constexpr int EPL = 16 / (int)sizeof(T);
  constexpr int LPR = D / EPL;
  constexpr int NG = DT / LPR;
  constexpr int PASS = NG * RPG;
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int NWV = DT / WAVE;
  static_assert(CH == DT, "one row of an item per thread when routing it");
  typedef GroupMerge<NG, GT, D> Merge;

  __shared__ int wtot[NWV];
  __shared__ int wcnt[2][NWV];
  __shared__ int2 lst[CH];
  __shared__ float sm_m[NG][GT], sm_l[NG][GT];
  __shared__ float sm_o[NG][GT][D];
  extern __shared__ long long dyn[];
  const int H = a.B * a.Hkv;
  long long* off = dyn;
  int* ist = reinterpret_cast<int*>(dyn + H + 1);

  build_items(a, off, ist, wtot);
  const int n_items = ist[H];
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i <= H; i += DT) a.item_start[i] = ist[i];
  const int tid = threadIdx.x, grp = tid / LPR, sub = tid % LPR;
  const int lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int qsub = blockIdx.y;
  // revolutions per position of this lane's rotary pairs
  double rope_g[EPL / 2];
  {
    const double l2b = a.rope_base > 0.f ? log2((double)a.rope_base) : 0.0;
#pragma unroll
    for (int m2 = 0; m2 < EPL / 2; ++m2)
      rope_g[m2] = exp2(-(2.0 * (sub * EPL / 2 + m2) / D) * l2b) * 0.15915494309189535;
  }

  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int head = find_item_head(ist, H, it);
    const int b = head / a.Hkv, h = head % a.Hkv;
    const long long r0 = off[head] + (long long)(it - ist[head]) * CH;
    const long long r1 = min(r0 + CH, off[head + 1]);

    // route the item's rows: lst = [exact (row, vmap) ... | rebuilt (row, pos) ...]
    {
      const bool in = r0 + tid < r1;
      int vm = 0, ps = 0;
      if (in) { vm = a.vmap[r0 + tid]; ps = a.pos[r0 + tid]; }
      const bool ex = in && vm >= 0, rb = in && vm < 0;
      const uint64_t be = __ballot(ex), bb = __ballot(rb);
      if (lane == 0) { wcnt[0][wave] = __popcll(be); wcnt[1][wave] = __popcll(bb); }
      __syncthreads();
      int ne = 0, pe = 0, pb = 0;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        ne += wcnt[0][w];
        if (w < wave) { pe += wcnt[0][w]; pb += wcnt[1][w]; }
      }
      if (ex) lst[pe + (int)mbcnt(be)] = make_int2(tid, vm);
      if (rb) lst[ne + pb + (int)mbcnt(bb)] = make_int2(tid, ps);
      __syncthreads();
    }
    int n_ex = 0, n_all = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) { n_ex += wcnt[0][w]; n_all += wcnt[0][w] + wcnt[1][w]; }

    QSlices<T, GT> qs;
    qs.template load<D>(a, b, h, qsub, sub);
    RowState<GT, EPL> st;
    st.reset();
    // exact rows
    for (int base = 0; base < n_ex; base += PASS) {
      uint4 kr[RPG], vr[RPG];
      bool ok[RPG];
#pragma unroll
      for (int u = 0; u < RPG; ++u) {
        const int idx = base + grp + u * NG;
        ok[u] = idx < n_ex;
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
        if (ok[u]) {
          const int2 e = lst[idx];
          kr[u] = ld16(a.kc + (size_t)(r0 + e.x) * ROWB + sub * 16);
          if (e.y < a.vcap) vr[u] = ld16(a.vc + (size_t)e.y * ROWB + sub * 16);
        }
      }
      float sc[RPG][GT];
#pragma unroll
      for (int u = 0; u < RPG; ++u)
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          sc[u][g] = group_sum<LPR>(qs.score(g, kr[u], a.c));
          if (!QSlices<T, GT>::kScaled) sc[u][g] *= a.c;
        }
      st.cover(sc, ok);
#pragma unroll
      for (int u = 0; u < RPG; ++u) {
        if (ok[u]) {
          float vx[EPL];
          unpack16<T>(vr[u], vx);
          st.add(sc[u], vx);
        }
      }
    }
    st.park(sm_o, sm_m, sm_l, grp, sub);
    __syncthreads();
    Merge ex;
    ex.run(sm_o, sm_m, sm_l, tid);
    __syncthreads();

    // rebuilt rows
    st.reset();
    for (int base = n_ex; base < n_all; base += PASS) {
      uint4 kr[RPG];
      int pp[RPG];
      bool ok[RPG];
#pragma unroll
      for (int u = 0; u < RPG; ++u) {
        const int idx = base + grp + u * NG;
        ok[u] = idx < n_all;
        kr[u] = make_uint4(0, 0, 0, 0);
        pp[u] = 0;
        if (ok[u]) {
          const int2 e = lst[idx];
          kr[u] = ld16(a.kc + (size_t)(r0 + e.x) * ROWB + sub * 16);
          pp[u] = e.y;
        }
      }
      float sc[RPG][GT];
#pragma unroll
      for (int u = 0; u < RPG; ++u)
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          sc[u][g] = group_sum<LPR>(qs.score(g, kr[u], a.c));
          if (!QSlices<T, GT>::kScaled) sc[u][g] *= a.c;
        }
      st.cover(sc, ok);
#pragma unroll
      for (int u = 0; u < RPG; ++u) {
        if (ok[u]) {
          // RoPE^-1: pairs (2i, 2i+1) of this lane's elements turn back by
          // the angle of position pp (revolutions reduced in double)
          float kx[EPL];
          unpack16<T>(kr[u], kx);
          if (a.rope_base > 0.f) {
#pragma unroll
            for (int m2 = 0; m2 < EPL / 2; ++m2) {
              double r = (double)pp[u] * rope_g[m2];
              r -= floor(r);
              const float rv = (float)r;
              const float s = __builtin_amdgcn_sinf(rv), c = __builtin_amdgcn_cosf(rv);
              const float x = kx[2 * m2], y = kx[2 * m2 + 1];
              kx[2 * m2] = x * c + y * s;
              kx[2 * m2 + 1] = y * c - x * s;
            }
          }
          st.add(sc[u], kx);
        }
      }
    }
    st.park(sm_o, sm_m, sm_l, grp, sub);
    __syncthreads();
    Merge rb;
    rb.run(sm_o, sm_m, sm_l, tid);

    // the item's partial: both phases under one maximum
    const size_t pbase = ((size_t)qsub * a.items_max + it) * GT;
#pragma unroll
    for (int k = 0; k < Merge::S; ++k) {
      const int x = tid + k * DT;
      if (GT * D % DT != 0 && x >= GT * D) continue;
      const int g = x / D, e = x % D;
      const float M = fmaxf(ex.M[k], rb.M[k]);
      float L = 0.f, O = 0.f, U = 0.f;
      if (M != -INFINITY) {
        const float we = fast_exp2(ex.M[k] - M), wr = fast_exp2(rb.M[k] - M);
        L = fmaf(ex.L[k], we, rb.L[k] * wr);
        O = ex.O[k] * we;
        U = rb.O[k] * wr;
      }
      a.part_o[(pbase + g) * D + e] = O;
      a.part_u[(pbase + g) * D + e] = U;
      if (e == 0) a.part_ml[pbase + g] = make_float2(M, L);
    }
    __syncthreads();
  }
}

// Per (head, query sub-group): merge the head's items in item order, loads
// batched 32 items at a time (the batch maximum first, then the weights).  A
// routed cache also merges the rebuilt-row sums U and adds W U (one d x d
// product per query head) before dividing.
template <int D, int GT, bool VEC>
__global__ __launch_bounds__(GT * D) void decode_merge(DecodeArgs a) {
  constexpr int U = VEC && GT * D > 512 ? 16 : 32;   // partials per batch (registers)
  __shared__ __attribute__((aligned(16))) float su[VEC ? GT : 1][VEC ? D : 1];
  __shared__ float wu[VEC ? GT : 1][VEC ? D : 1];
  const int head = blockIdx.x, qsub = blockIdx.y;
  const int b = head / a.Hkv, h = head % a.Hkv;
  const int i0 = a.item_start[head], i1 = a.item_start[head + 1];
  const size_t base = (size_t)qsub * a.items_max;
  const int x = threadIdx.x;
  const int g = x / D, e = x % D, jg = qsub * GT + g;
  const bool live = jg < a.G;
  float M = -INFINITY, L = 0.f, O = 0.f, Uv = 0.f;
  // Routed cache: O += (W_h U)[e] at the end.  A group of D/4 lanes takes one
  // row of W_h at a time (16 bytes per lane, so a wave reads whole rows
  // contiguously), dots it with every query head's U from LDS and sums over
  // the group.  The rows are requested here, ahead of the partials.
  constexpr int LW = D / 4, RPP = GT * D / LW, NP = D / RPP;   // lanes per row, rows per pass
  float4 wv[VEC ? NP : 1];
  if constexpr (VEC) {
#pragma unroll
    for (int pz = 0; pz < NP; ++pz)
      wv[pz] = reinterpret_cast<const float4*>(a.w + ((size_t)h * D + x / LW + pz * RPP) * D)[x % LW];
  }
  if (live) {
    for (int it0 = i0; it0 < i1; it0 += U) {
      float2 ml[U];
      float ov[U], uv[VEC ? U : 1];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t p = (base + it0 + u) * GT + g;
        const bool ok = it0 + u < i1;
        ml[u] = ok ? a.part_ml[p] : make_float2(-INFINITY, 0.f);
        ov[u] = ok ? a.part_o[p * D + e] : 0.f;
        if constexpr (VEC) uv[u] = ok ? a.part_u[p * D + e] : 0.f;
      }
      // batch maximum first, then independent weights (hardware exp2)
      float mb = M;
#pragma unroll
      for (int u = 0; u < U; ++u) mb = fmaxf(mb, ml[u].x);
      if (mb == -INFINITY) continue;
      const float wa = fast_exp2(M - mb);   // 0 while M is -inf
      L *= wa;
      O *= wa;
      if constexpr (VEC) Uv *= wa;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wb = fast_exp2(ml[u].x - mb);   // 0 for empty items (-inf)
        L = fmaf(ml[u].y, wb, L);
        O = fmaf(ov[u], wb, O);
        if constexpr (VEC) Uv = fmaf(uv[u], wb, Uv);
      }
      M = mb;
    }
  }
  if constexpr (VEC) {
    su[g][e] = Uv;
    __syncthreads();
    const int j = x % LW;
#pragma unroll
    for (int pz = 0; pz < NP; ++pz) {
      const int r = x / LW + pz * RPP;
#pragma unroll
      for (int g2 = 0; g2 < GT; ++g2) {
        const float4 uv4 = *reinterpret_cast<const float4*>(&su[g2][4 * j]);
        float t = wv[pz].x * uv4.x;
        t = fmaf(wv[pz].y, uv4.y, t);
        t = fmaf(wv[pz].z, uv4.z, t);
        t = fmaf(wv[pz].w, uv4.w, t);
        t = group_sum<LW>(t);
        if (j == 0) wu[g2][r] = t;
      }
    }
    __syncthreads();
    O += wu[g][e];
  }
  if (!live) return;
  const size_t bj = (size_t)b * a.Hq + h * a.G + jg;
  const bool any = L > 0.f;
  a.out[bj * D + e] = any ? O / L : 0.f;
  if (a.lse && e == 0) a.lse[bj] = any ? (M + log2f(L)) * LN2_F : -INFINITY;
}

// Merge of a plain (not routed) cache's partials: one wave per (head, query
// head, 64-element slice of the output).  M is the largest item maximum; item
// i weighs 2^(m_i - M).  A head of at most 64 items takes one round trip
// (every load issued at once, the weights broadcast from LDS); longer heads
// walk their items 64 at a time,
// lane i turning item c + i's maximum into its weight (kept in LDS) while
// every lane sums its output element over the 64 items.  The sums run in
// item order (the normaliser's lane sums by a fixed butterfly), so the
// result is deterministic.
template <int D, int GT>
__global__ __launch_bounds__(WAVE) void decode_merge_w(DecodeArgs a) {
  constexpr int UB = 16;   // item loads in flight per lane (heads of more than 64 items)
  __shared__ __attribute__((aligned(16))) float wts[WAVE];
  const int head = blockIdx.x, jg = blockIdx.y, ds = blockIdx.z;
  const int qsub = jg / GT, g = jg % GT;
  const int lane = threadIdx.x;
  const int i0 = a.item_start[head], i1 = a.item_start[head + 1];
  const int n = i1 - i0;
  const size_t base = (size_t)qsub * a.items_max;
  const float2* ml = a.part_ml + base * GT + g;              // item it: ml[it * GT]
  const int e = ds * WAVE + lane;
  const float* po = a.part_o + (base * GT + g) * D + e;     // item it: po[it * GT * D]
  float M = -INFINITY, O = 0.f, L = 0.f;
  if (n <= 0) {
    // a head with no rows: out = 0, lse = -inf
  } else if (n <= WAVE) {
    // One round trip: lane i loads item i's (m, l) while every lane loads its
    // element of all n items (indices past the last item re-read it, so the
    // loads need no branch); then the maximum, the weights and the sums, in
    // item order.
    float2 p = make_float2(-INFINITY, 0.f);
    if (lane < n) p = ml[(size_t)(i0 + lane) * GT];
    float ov[WAVE];
#pragma unroll
    for (int v = 0; v < WAVE; ++v) ov[v] = po[(size_t)(i0 + min(v, n - 1)) * GT * D];
    M = wave_max(p.x);
    if (M != -INFINITY) {
      const float w = lane < n ? fast_exp2(p.x - M) : 0.f;   // 0 for an item with no rows
      L = wave_sum(p.y * w);
      wts[lane] = w;   // one wave: its LDS reads below follow this write
#pragma unroll
      for (int v = 0; v < WAVE; v += 4) {
        const float4 w4 = *reinterpret_cast<const float4*>(&wts[v]);   // broadcast read
        if (v < n) O = fmaf(ov[v], w4.x, O);
        if (v + 1 < n) O = fmaf(ov[v + 1], w4.y, O);
        if (v + 2 < n) O = fmaf(ov[v + 2], w4.z, O);
        if (v + 3 < n) O = fmaf(ov[v + 3], w4.w, O);
      }
    }
  } else {
    for (int it = i0 + lane; it < i1; it += WAVE) M = fmaxf(M, ml[(size_t)it * GT].x);
    M = wave_max(M);
    if (M != -INFINITY) {
      for (int c0 = i0; c0 < i1; c0 += WAVE) {
        const int it = c0 + lane;
        float w = 0.f;
        if (it < i1) {
          const float2 p = ml[(size_t)it * GT];
          w = fast_exp2(p.x - M);
          L = fmaf(p.y, w, L);
        }
        wts[lane] = w;   // one wave: its LDS reads below follow this write
        const int nc = min(WAVE, i1 - c0);
        for (int u = 0; u < nc; u += UB) {
          float ov[UB];
#pragma unroll
          for (int v = 0; v < UB; ++v)
            ov[v] = u + v < nc ? po[(size_t)(c0 + u + v) * GT * D] : 0.f;
#pragma unroll
          for (int v = 0; v < UB; ++v) O = fmaf(ov[v], wts[u + v], O);
        }
      }
      L = wave_sum(L);
    }
  }
  const size_t bj = (size_t)(head / a.Hkv) * a.Hq + (head % a.Hkv) * a.G + jg;
  const bool any = L > 0.f;
  a.out[bj * D + e] = any ? O / L : 0.f;
  if (a.lse && ds == 0 && lane == 0) a.lse[bj] = any ? (M + log2f(L)) * LN2_F : -INFINITY;
}

struct DecodePlan {
  int GT, n_sub, items_max;
  size_t off_ml, off_ist, off_u, bytes;
};

bool plan_decode(int B, int Hq, int Hkv, int d, int64_t cap, DecodePlan* p, bool vec = false) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || (d != 64 && d != 128) || cap < 0 ||
      cap >= (int64_t(1) << 31) || (int64_t)B * Hkv > MAX_HEADS)
    return false;
  const int G = Hq / Hkv;
  p->GT = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
  p->n_sub = ceil_div(G, p->GT);
  const int64_t items = ceil_div64(cap, CH) + (int64_t)B * Hkv;
  if (items >= (int64_t(1) << 31)) return false;
  p->items_max = (int)std::max<int64_t>(items, 1);
  const size_t slots = (size_t)p->n_sub * p->items_max * p->GT;
  const size_t po = slots * d * sizeof(float);
  p->off_ml = (po + 255) & ~size_t(255);
  p->off_ist = (p->off_ml + slots * sizeof(float2) + 255) & ~size_t(255);
  p->bytes = p->off_ist + ((size_t)B * Hkv + 1) * sizeof(int);
  p->off_u = (p->bytes + 255) & ~size_t(255);
  if (vec) p->bytes = p->off_u + po;
  return true;
}

template <typename T, int D, int GT, bool VEC>
void launch_decode(const DecodeArgs& a, hipStream_t st) {
  const size_t dyn = (size_t)(a.B * a.Hkv + 1) * (sizeof(long long) + sizeof(int));
  // items_max bounds the items from the capacity; the real count (from the
  // offsets, on the device) can be far smaller, so the grid stops at
  // GRID_MAX workgroups (four per CU on 256 CUs) that stride over the items.
  const dim3 grid((unsigned)std::min(a.items_max, GRID_MAX), a.n_sub);
  if constexpr (VEC) {
    launch("vector_decode_split", vector_decode_split<T, D, GT>, grid, dim3(DT), (uint32_t)dyn, st, a);
  } else {
    if (a.cnt)
      launch("compact_decode", decode_split<T, D, GT, true>, grid, dim3(DT), (uint32_t)dyn, st, a);
    else
      launch("decode_split", decode_split<T, D, GT, false>, grid, dim3(DT), (uint32_t)dyn, st, a);
  }
  if constexpr (VEC)
    launch("vector_decode_merge", decode_merge<D, GT, true>, dim3(a.B * a.Hkv, a.n_sub),
           dim3(GT * D), 0, st, a);
  else
    launch("decode_merge", decode_merge_w<D, GT>, dim3(a.B * a.Hkv, a.G, D / WAVE), dim3(WAVE),
           0, st, a);
}

template <typename T, int D, bool VEC>
void launch_decode_g(const DecodeArgs& a, int GT, hipStream_t st) {
  switch (GT) {
    case 1: launch_decode<T, D, 1, VEC>(a, st); break;
    case 2: launch_decode<T, D, 2, VEC>(a, st); break;
    case 4: launch_decode<T, D, 4, VEC>(a, st); break;
    default: launch_decode<T, D, 8, VEC>(a, st); break;
  }
}

template <bool VEC>
void launch_decode_any(const DecodeArgs& a, int dtype, int d, int GT, hipStream_t st) {
  if (dtype == KV_BF16) {
    if (d == 128) launch_decode_g<__bf16, 128, VEC>(a, GT, st);
    else launch_decode_g<__bf16, 64, VEC>(a, GT, st);
  } else {
    if (d == 128) launch_decode_g<float, 128, VEC>(a, GT, st);
    else launch_decode_g<float, 64, VEC>(a, GT, st);
  }
}

}  // namespace
}  // namespace kvcc

using namespace kvcc;

extern "C" size_t kv_decode_workspace_size(int B, int Hq, int Hkv, int d, int64_t capacity_rows) {
  DecodePlan p;
  return plan_decode(B, Hq, Hkv, d, capacity_rows, &p) ? p.bytes : 0;
}

extern "C" int kv_decode_attn(const void* q, const void* k_c, const void* v_c,
                              const int64_t* offsets, int B, int Hq, int Hkv, int d, int dtype,
                              float scale, int64_t capacity_rows, float* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !offsets || !out) return KV_ERR_NULL;
  if (capacity_rows > 0 && (!k_c || !v_c)) return KV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_c) || !aligned16(v_c) || !aligned16(offsets) ||
      !aligned16(out) || !aligned16(lse) || !aligned16(workspace))
    return KV_ERR_ALIGN;
  if (dtype != KV_F32 && dtype != KV_BF16) return KV_ERR_DTYPE;
  DecodePlan p;
  if (!plan_decode(B, Hq, Hkv, d, capacity_rows, &p)) return KV_ERR_SHAPE;
  if (!workspace || workspace_bytes < p.bytes) return KV_ERR_WORKSPACE;

  DecodeArgs a;
  a.q = q; a.kc = static_cast<const char*>(k_c); a.vc = static_cast<const char*>(v_c);
  a.offsets = offsets; a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.n_sub = p.n_sub; a.items_max = p.items_max; a.cap = capacity_rows;
  a.c = (float)((scale > 0.f ? (double)scale : 1.0 / sqrt((double)d)) * LOG2E_D);
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + p.off_ml);
  a.item_start = reinterpret_cast<int*>(static_cast<char*>(workspace) + p.off_ist);
  a.out = out; a.lse = lse;
  a.vmap = nullptr; a.pos = nullptr; a.w = nullptr; a.rope_base = 0.f; a.vcap = 0;
  a.part_u = nullptr;
  a.cnt = nullptr; a.idx = nullptr; a.ksrc = nullptr; a.vsrc = nullptr; a.N_max = 0;
  a.kc_w = nullptr; a.vc_w = nullptr; a.pos_w = nullptr; a.off_w = nullptr;

  launch_decode_any<false>(a, dtype, d, p.GT, static_cast<hipStream_t>(stream));
  return launch_status();
}

// Scratch of kv_decode_attn_noalloc: the split partials live in this
// file-scope device array instead of a caller workspace.  Each GPU holds its
// own copy at its own address; host code never passes the array's name to a
// kernel (on the host it is only a stand-in), but the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept per device.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace kvcc {
namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::once_flag scratch_once[NOALLOC_MAX_DEVICES];
void* scratch_ptr[NOALLOC_MAX_DEVICES];   // written once per device under its once_flag

// The scratch array's device address on the current device, or null.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return nullptr;
  std::call_once(scratch_once[dev], [dev] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) scratch_ptr[dev] = ptr;
  });
  return scratch_ptr[dev];
}
}  // namespace
}  // namespace kvcc

extern "C" int kv_decode_attn_noalloc(const void* q, const void* k_c, const void* v_c,
                                      const int64_t* offsets, int B, int Hq, int Hkv, int d,
                                      int dtype, float scale, int64_t capacity_rows, float* out,
                                      float* lse, void* stream) {
  if (!q || !offsets || !out) return KV_ERR_NULL;
  if (capacity_rows > 0 && (!k_c || !v_c)) return KV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_c) || !aligned16(v_c) || !aligned16(offsets) ||
      !aligned16(out) || !aligned16(lse))
    return KV_ERR_ALIGN;
  if (dtype != KV_F32 && dtype != KV_BF16) return KV_ERR_DTYPE;
  DecodePlan p;
  if (!plan_decode(B, Hq, Hkv, d, capacity_rows, &p)) return KV_ERR_SHAPE;
  if (p.bytes > NOALLOC_SCRATCH_BYTES) return KV_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return KV_ERR_LAUNCH;
  return kv_decode_attn(q, k_c, v_c, offsets, B, Hq, Hkv, d, dtype, scale, capacity_rows, out,
                        lse, ws, NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" size_t kv_vector_decode_workspace_size(int B, int Hq, int Hkv, int d,
                                                  int64_t capacity_rows) {
  DecodePlan p;
  return plan_decode(B, Hq, Hkv, d, capacity_rows, &p, true) ? p.bytes : 0;
}

extern "C" int kv_vector_decode(const void* q, const void* k_c, const void* v_c,
                                const int32_t* vmap, const int32_t* pos, const int64_t* offsets,
                                const float* w, float rope_base, int B, int Hq, int Hkv, int d,
                                int dtype, float scale, int64_t capacity_rows,
                                int64_t v_capacity_rows, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !offsets || !out || !w) return KV_ERR_NULL;
  if (capacity_rows > 0 && (!k_c || !vmap || !pos)) return KV_ERR_NULL;
  if (v_capacity_rows > 0 && !v_c) return KV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_c) || !aligned16(v_c) || !aligned16(vmap) ||
      !aligned16(pos) || !aligned16(offsets) || !aligned16(w) || !aligned16(out) ||
      !aligned16(lse) || !aligned16(workspace))
    return KV_ERR_ALIGN;
  if (dtype != KV_F32 && dtype != KV_BF16) return KV_ERR_DTYPE;
  if (!(rope_base >= 0.f) || v_capacity_rows < 0 || v_capacity_rows >= (int64_t(1) << 31))
    return KV_ERR_SHAPE;
  DecodePlan p;
  if (!plan_decode(B, Hq, Hkv, d, capacity_rows, &p, true)) return KV_ERR_SHAPE;
  if (!workspace || workspace_bytes < p.bytes) return KV_ERR_WORKSPACE;

  DecodeArgs a;
  a.q = q; a.kc = static_cast<const char*>(k_c); a.vc = static_cast<const char*>(v_c);
  a.offsets = offsets; a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.n_sub = p.n_sub; a.items_max = p.items_max; a.cap = capacity_rows;
  a.c = (float)((scale > 0.f ? (double)scale : 1.0 / sqrt((double)d)) * LOG2E_D);
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + p.off_ml);
  a.item_start = reinterpret_cast<int*>(static_cast<char*>(workspace) + p.off_ist);
  a.part_u = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.off_u);
  a.out = out; a.lse = lse;
  a.vmap = vmap; a.pos = pos; a.w = w; a.rope_base = rope_base; a.vcap = v_capacity_rows;
  a.cnt = nullptr; a.idx = nullptr; a.ksrc = nullptr; a.vsrc = nullptr; a.N_max = 0;
  a.kc_w = nullptr; a.vc_w = nullptr; a.pos_w = nullptr; a.off_w = nullptr;

  launch_decode_any<true>(a, dtype, d, p.GT, static_cast<hipStream_t>(stream));
  return launch_status();
}

extern "C" int kv_compact_decode(const void* k, const void* v, const int32_t* kept_idx,
                                 const int32_t* kept_count, int B, int Hq, int Hkv, int N_max,
                                 int d, int dtype, int64_t capacity_rows, const void* q,
                                 float scale, void* k_c, void* v_c, int32_t* pos,
                                 int64_t* offsets, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!k || !v || !kept_idx || !kept_count || !q || !offsets || !out) return KV_ERR_NULL;
  if (capacity_rows > 0 && (!k_c || !v_c || !pos)) return KV_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(kept_idx) || !aligned16(kept_count) ||
      !aligned16(q) || !aligned16(k_c) || !aligned16(v_c) || !aligned16(pos) ||
      !aligned16(offsets) || !aligned16(out) || !aligned16(lse) || !aligned16(workspace))
    return KV_ERR_ALIGN;
  if (dtype != KV_F32 && dtype != KV_BF16) return KV_ERR_DTYPE;
  if (N_max < 1 || (int64_t)B * Hkv * N_max >= (int64_t(1) << 31)) return KV_ERR_SHAPE;
  DecodePlan p;
  if (!plan_decode(B, Hq, Hkv, d, capacity_rows, &p)) return KV_ERR_SHAPE;
  if (!workspace || workspace_bytes < p.bytes) return KV_ERR_WORKSPACE;

  DecodeArgs a;
  a.q = q; a.kc = static_cast<const char*>(k_c); a.vc = static_cast<const char*>(v_c);
  a.offsets = offsets; a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.n_sub = p.n_sub; a.items_max = p.items_max; a.cap = capacity_rows;
  a.c = (float)((scale > 0.f ? (double)scale : 1.0 / sqrt((double)d)) * LOG2E_D);
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + p.off_ml);
  a.item_start = reinterpret_cast<int*>(static_cast<char*>(workspace) + p.off_ist);
  a.out = out; a.lse = lse;
  a.vmap = nullptr; a.pos = nullptr; a.w = nullptr; a.rope_base = 0.f; a.vcap = 0;
  a.part_u = nullptr;
  a.cnt = kept_count; a.idx = kept_idx;
  a.ksrc = static_cast<const char*>(k); a.vsrc = static_cast<const char*>(v); a.N_max = N_max;
  a.kc_w = static_cast<char*>(k_c); a.vc_w = static_cast<char*>(v_c);
  a.pos_w = pos; a.off_w = offsets;

  launch_decode_any<false>(a, dtype, d, p.GT, static_cast<hipStream_t>(stream));
  return launch_status();
}
