// VECTOR three-way routing: retain, approximate or evict per token.
//
// "A Simple Plug-in for Improving Eviction-Based KV Cache Compression"
// (VECTOR), section "Methodologie: VECTOR": the base eviction score selects
// an enlarged pool of 1 - p_c + p_a of the tokens; each pool token's
// reconstruction residual eps = ||V - W RoPE^-1(K)||^2 is computed with an
// offline linear map W (keys rotated back to position 0 first); keys stay
// for the whole pool, the 2 p_a lowest-residual tokens drop their values
// (rebuilt from their keys when read) and the rest keep K and V exactly.
//
// kv_vector_route: pool (radix select on the scores), residuals (fp32 MFMA:
// the 64 pool rows of a workgroup, de-rotated, times W^T, with W, the rows
// and the values staged in LDS), then a second radix select on -eps inside
// the pool.  kv_vector_compact: the packed cache keeps a key row per pool
// token and a value row per exact token, with vmap telling, per key row,
// where its value is (-1: rebuilt).  The decode side lives with the other
// decode kernels.
//
// Rotary positions: adjacent pairs (2i, 2i+1) turn by pos * base^(-2i/d)
// (base 0: no rotation).  The angle is reduced to revolutions in float64
// (exact for any position) before the hardware sine/cosine.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace kvcc {
namespace {

constexpr int VT = 256;
constexpr int RPW = 64;          // pool entries per residual workgroup
constexpr int VMC = 8192;        // pool entries per window of the value-map kernel
constexpr int MAX_HEADS = 4096;
constexpr double INV_TWO_PI = 0.15915494309189535;

__global__ void vector_counts_kernel(const int32_t* ctx, int B, int Hkv, int N_max, float p_c,
                                     float p_a, int32_t* k_pool, int32_t* k_apx) {
  const int head = blockIdx.x * blockDim.x + threadIdx.x;
  if (head >= B * Hkv) return;
  const int n = ctx ? min(max(ctx[head / Hkv], 0), N_max) : N_max;
  const double pc = (double)p_c, pa = (double)p_a;
  long long kp = (long long)floor((1.0 - pc + pa) * (double)n + 0.5);
  kp = min(max(kp, 1ll), (long long)n);
  long long ka = (long long)floor(2.0 * pa * (double)n + 0.5);
  ka = min(max(ka, 0ll), kp);
  k_pool[head] = (int)kp;
  k_apx[head] = (int)ka;
}

// Revolutions per position of pair i of a d-wide row, for base > 0.
__device__ __forceinline__ double rope_freq(int i, int d, double log2_base) {
  return exp2(-(2.0 * i / d) * log2_base) * INV_TWO_PI;
}

// The angle of position pos at frequency g, reduced to [0, 1) revolutions.
__device__ __forceinline__ float rope_rev(int pos, double g) {
  double r = (double)pos * g;
  r -= floor(r);
  return (float)r;
}

// N elements of a row as raw 16-byte words (converted later by unpack_elems).
template <typename T, int N> struct RawElems { uint4 w[N * (int)sizeof(T) / 16]; };
template <typename T, int N>
__device__ __forceinline__ void raw_load(const char* row, int e0, RawElems<T, N>& r) {
#pragma unroll
  for (int c = 0; c < N * (int)sizeof(T) / 16; ++c) r.w[c] = ld16(row + (size_t)e0 * sizeof(T) + 16 * c);
}
template <typename T, int N>
__device__ __forceinline__ void unpack_elems(const RawElems<T, N>& r, float* x) {
#pragma unroll
  for (int c = 0; c < N * (int)sizeof(T) / 16; ++c) {
    const uint4 w = r.w[c];
    if constexpr (sizeof(T) == 2) {
      x[8 * c + 0] = bf16_lo(w.x); x[8 * c + 1] = bf16_hi(w.x);
      x[8 * c + 2] = bf16_lo(w.y); x[8 * c + 3] = bf16_hi(w.y);
      x[8 * c + 4] = bf16_lo(w.z); x[8 * c + 5] = bf16_hi(w.z);
      x[8 * c + 6] = bf16_lo(w.w); x[8 * c + 7] = bf16_hi(w.w);
    } else {
      x[4 * c + 0] = __uint_as_float(w.x); x[4 * c + 1] = __uint_as_float(w.y);
      x[4 * c + 2] = __uint_as_float(w.z); x[4 * c + 3] = __uint_as_float(w.w);
    }
  }
}

struct ResidualArgs {
  const char* k;
  const char* v;
  const float* w;          // [Hkv][d][d], out = w @ in
  const int32_t* pool_idx;
  const int32_t* pool_count;
  float* neg_eps;          // [B][Hkv][N_max]
  int B, Hkv, N_max;
  float rope_base;
};

// A few workgroups per head stage W_h once, then walk the head's pool in
// tiles of 64 entries, 4 waves each.  Wave w owns row block w/2 and the
// column blocks of half w%2; each 32x32 output block is
// K~ W^T over d/2 steps of v_mfma_f32_32x32x2f32, and the squared residual
// is summed over the columns in-lane, across the 32 lanes of a half-wave
// (DPP), then over the two halves through LDS.
template <typename T, int D>
__global__ __launch_bounds__(VT) void vector_residual_kernel(ResidualArgs a) {
  constexpr int LD = D + 1;                  // padded LDS rows
  constexpr int NCB = D / 32, CPW = NCB / 2; // column blocks, per wave
  constexpr int EQ = D / 4;                  // staged elements per thread
  constexpr int ROWB = D * (int)sizeof(T);
  __shared__ float Wl[D][LD];
  __shared__ float Kt[RPW][LD];
  __shared__ float Vt[RPW][LD];
  __shared__ float part[2][RPW];
  __shared__ double gfreq[D / 2];   // revolutions per position of every rotary pair

  const int h = blockIdx.y, b = blockIdx.z, head = b * a.Hkv + h;
  const int tid = threadIdx.x;
  const int cnt = min(max(a.pool_count[head], 0), a.N_max);
  float* ne = a.neg_eps + (size_t)head * a.N_max;
  // entries past the pool
  for (int j = cnt + (int)blockIdx.x * VT + tid; j < a.N_max; j += (int)gridDim.x * VT)
    ne[j] = -INFINITY;
  if ((int)blockIdx.x * RPW >= cnt) return;

  // W_h once per workgroup; the workgroup then walks its tiles of 64 entries
  const float4* w4 = reinterpret_cast<const float4*>(a.w + (size_t)h * D * D);
  for (int i = tid; i < D * D / 4; i += VT) {
    const float4 x = w4[i];
    const int o = (4 * i) / D, c = (4 * i) % D;
    Wl[o][c] = x.x; Wl[o][c + 1] = x.y; Wl[o][c + 2] = x.z; Wl[o][c + 3] = x.w;
  }
  // Thread tid stages quarter tid%4 of row tid/4 of a tile.  The next tile's
  // rows are requested before this tile's MFMAs, so their gather overlaps
  // the matrix work; only the unpacking and RoPE^-1 sit between barriers.
  const int sr = tid / 4, q4 = tid % 4;
  RawElems<T, EQ> pk, pv;
  int pt = -1;
  auto fetch = [&](int jt) __attribute__((always_inline)) {
    const int j = jt + sr;
    pt = -1;
    if (j < cnt) {
      pt = a.pool_idx[(size_t)head * a.N_max + j];
      const size_t roff = ((size_t)head * a.N_max + pt) * ROWB;
      raw_load<T, EQ>(a.k + roff, q4 * EQ, pk);
      raw_load<T, EQ>(a.v + roff, q4 * EQ, pv);
    }
  };
  fetch((int)blockIdx.x * RPW);
  if (a.rope_base > 0.f && tid < D / 2) gfreq[tid] = rope_freq(tid, D, log2((double)a.rope_base));
#pragma unroll 1
  for (int j0 = (int)blockIdx.x * RPW; j0 < cnt; j0 += (int)gridDim.x * RPW) {
  const int jend = min(j0 + RPW, a.N_max);
  __syncthreads();   // the previous tile's rows are no longer read
  {
    float kx[EQ], vx[EQ];
    if (pt >= 0) {
      unpack_elems<T, EQ>(pk, kx);
      unpack_elems<T, EQ>(pv, vx);
      if (a.rope_base > 0.f) {
#pragma unroll
        for (int m = 0; m < EQ / 2; ++m) {
          const float rv = rope_rev(pt, gfreq[q4 * EQ / 2 + m]);
          const float s = __builtin_amdgcn_sinf(rv), c = __builtin_amdgcn_cosf(rv);
          const float x = kx[2 * m], y = kx[2 * m + 1];
          kx[2 * m] = x * c + y * s;
          kx[2 * m + 1] = y * c - x * s;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < EQ; ++e) { kx[e] = 0.f; vx[e] = 0.f; }
    }
#pragma unroll
    for (int e = 0; e < EQ; ++e) { Kt[sr][q4 * EQ + e] = kx[e]; Vt[sr][q4 * EQ + e] = vx[e]; }
  }
  __syncthreads();
  if (j0 + (int)gridDim.x * RPW < cnt) fetch(j0 + (int)gridDim.x * RPW);

  const int lane = tid & (WAVE - 1), wave = tid / WAVE, l32 = lane & 31, hf = lane >> 5;
  const int rb = wave >> 1;
  float rs[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) rs[e] = 0.f;
  // the wave's column blocks are independent accumulator chains: interleave them
  f32x16 acc[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) acc[c] = f32x16{};
  // operands of KB k-steps are read from LDS one batch ahead of their MFMAs
  constexpr int KB = 4, NKB = D / 2 / KB;
  float av[2][KB], bv[2][CPW][KB];
  auto ld_ops = [&](int buf, int ks0) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      av[buf][kk] = Kt[rb * 32 + l32][2 * (ks0 + kk) + hf];
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        bv[buf][c][kk] = Wl[((wave & 1) * CPW + c) * 32 + l32][2 * (ks0 + kk) + hf];
    }
  };
  ld_ops(0, 0);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    if (kb + 1 < NKB) ld_ops((kb + 1) & 1, (kb + 1) * KB);
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[kb & 1][kk], bv[kb & 1][c][kk], acc[c],
                                                      0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int cb = (wave & 1) * CPW + c;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = rb * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
      const float r = Vt[row][cb * 32 + l32] - acc[c][e];
      rs[e] = fmaf(r, r, rs[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) rs[e] = group_sum<32>(rs[e]);
  if (l32 == 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) part[wave & 1][rb * 32 + 8 * (e >> 2) + 4 * hf + (e & 3)] = rs[e];
  }
  __syncthreads();
  if (tid < RPW) {
    const int j = j0 + tid;
    if (j < min(jend, cnt)) ne[j] = -(part[0][tid] + part[1][tid]);
  }
  }
}

// ---- compaction -------------------------------------------------------------

struct VCompactArgs {
  const char* k;
  const char* v;
  int B, Hkv, N_max, rowb;
  const int32_t* pool_idx;
  const int32_t* pool_count;
  const int32_t* apx_pos;
  const int32_t* apx_count;
  char* kc;
  char* vc;
  int32_t* pos;
  int32_t* vmap;
  int64_t* offsets;
  int64_t* voffsets;
  int64_t cap, vcap;
};

__device__ __forceinline__ int clamp_cnt(const int32_t* c, int i, int hi) {
  return min(max(c[i], 0), hi);
}

// Exclusive scans of the key-row counts (pool) and value-row counts (pool -
// approximated) over the heads, into LDS.
__device__ void scan_two(const VCompactArgs& a, int H, long long* off, long long* voff,
                         long long* wtot) {
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  constexpr int NWV = VT / WAVE;
  long long carry = 0, vcarry = 0;
  for (int base = 0; base < H; base += VT) {
    const int i = base + tid;
    long long c = 0, vc = 0;
    if (i < H) {
      c = clamp_cnt(a.pool_count, i, a.N_max);
      vc = c - clamp_cnt(a.apx_count, i, (int)c);
    }
    const long long inc = wave_incl_scan<long long>(c);
    const long long vinc = wave_incl_scan<long long>(vc);
    if (lane == WAVE - 1) { wtot[wave] = inc; wtot[NWV + wave] = vinc; }
    __syncthreads();
    long long before = 0, chunk = 0, vbefore = 0, vchunk = 0;
    for (int w = 0; w < NWV; ++w) {
      if (w < wave) { before += wtot[w]; vbefore += wtot[NWV + w]; }
      chunk += wtot[w];
      vchunk += wtot[NWV + w];
    }
    if (i < H) { off[i] = carry + before + inc - c; voff[i] = vcarry + vbefore + vinc - vc; }
    carry += chunk;
    vcarry += vchunk;
    __syncthreads();
  }
  if (tid == 0) { off[H] = carry; voff[H] = vcarry; }
  __syncthreads();
}

// One workgroup per head, over windows of VMC pool entries: the window's
// approximated entries (the next run of the ascending apx_pos list, read in
// parallel) are flagged in LDS, every thread counts the exact entries among
// its 32 consecutive ones, and one block scan gives each exact entry its
// packed value row.
__global__ __launch_bounds__(VT) void vector_vmap_kernel(VCompactArgs a) {
  constexpr int E = VMC / VT;          // pool entries per thread in a window
  extern __shared__ long long dyn[];   // off[H+1], voff[H+1]
  __shared__ long long wtot[2 * (VT / WAVE)];
  __shared__ __attribute__((aligned(16))) unsigned char flag[VMC];
  __shared__ int wsum[VT / WAVE];
  const int H = a.B * a.Hkv;
  long long* off = dyn;
  long long* voff = dyn + H + 1;
  scan_two(a, H, off, voff, wtot);
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  if (blockIdx.x == 0)
    for (int i = tid; i <= H; i += VT) { a.offsets[i] = off[i]; a.voffsets[i] = voff[i]; }
  const int head = blockIdx.x;
  const int cnt = clamp_cnt(a.pool_count, head, a.N_max);
  const int acnt = clamp_cnt(a.apx_count, head, cnt);
  const int32_t* ap = a.apx_pos + (size_t)head * a.N_max;
  const long long base = off[head], vbase = voff[head];
  int aptr = 0, vrank = 0;
  for (int J = 0; J < cnt; J += VMC) {
    // flag the approximated entries of the window [J, J + VMC): they are the
    // next entries of the ascending list (at most VMC of them)
    for (int i = tid; i < VMC / 16; i += VT) reinterpret_cast<uint4*>(flag)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    const int lim = min(acnt, aptr + VMC);
    int inwin = 0;
#pragma unroll 8
    for (int i = aptr + tid; i < lim; i += VT) {
      const int x = ap[i];
      if (x >= J && x < J + VMC) { flag[x - J] = 1; ++inwin; }
    }
    inwin = wave_incl_scan<int>(inwin);
    if (lane == WAVE - 1) wsum[wave] = inwin;
    __syncthreads();
    inwin = 0;
#pragma unroll
    for (int w = 0; w < VT / WAVE; ++w) inwin += wsum[w];
    __syncthreads();
    // exact entries among this thread's E consecutive ones, ranked by a block scan
    const int j0 = J + E * tid;
    const uint4* f4 = reinterpret_cast<const uint4*>(flag + E * tid);
    uint32_t fw[E / 4];
#pragma unroll
    for (int q = 0; q < E / 16; ++q) {
      const uint4 v = f4[q];
      fw[4 * q] = v.x; fw[4 * q + 1] = v.y; fw[4 * q + 2] = v.z; fw[4 * q + 3] = v.w;
    }
    int ex = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      ex += (j0 + e < cnt && ((fw[e / 4] >> (8 * (e % 4))) & 0xffu) == 0) ? 1 : 0;
    const int inc = wave_incl_scan<int>(ex);
    if (lane == WAVE - 1) wsum[wave] = inc;
    __syncthreads();
    int before = inc - ex, tot = 0;
#pragma unroll
    for (int w = 0; w < VT / WAVE; ++w) {
      if (w < wave) before += wsum[w];
      tot += wsum[w];
    }
    int r = vrank + before;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = j0 + e;
      if (j < cnt) {
        const bool apx = ((fw[e / 4] >> (8 * (e % 4))) & 0xffu) != 0;
        const long long row = base + j;
        if (row < a.cap) a.vmap[row] = apx ? -1 : (int32_t)(vbase + r);
        r += apx ? 0 : 1;
      }
    }
    vrank += tot;
    aptr += inwin;
    __syncthreads();   // flags and wsum are reused by the next window
  }
}

__device__ __forceinline__ int find_head(const long long* off, int H, long long row) {
  int lo = 0, hi = H - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Grid-stride over the packed key rows: key row and position always, value
// row when vmap says the token keeps it (and it fits the value capacity).
__global__ __launch_bounds__(VT) void vector_copy_kernel(VCompactArgs a) {
  extern __shared__ long long dyn[];
  __shared__ long long wtot[2 * (VT / WAVE)];
  const int H = a.B * a.Hkv;
  long long* off = dyn;
  long long* voff = dyn + H + 1;
  scan_two(a, H, off, voff, wtot);
  const long long total = min(off[H], (long long)a.cap);
  const int tid = threadIdx.x;
  const int lpr = a.rowb / 16, sub = tid % lpr, rloc = tid / lpr, rpi = VT / lpr;
  for (long long row = (long long)blockIdx.x * rpi + rloc; row < total;
       row += (long long)gridDim.x * rpi) {
    const int head = find_head(off, H, row);
    const long long j = row - off[head];
    const int t = a.pool_idx[(size_t)head * a.N_max + j];
    if ((unsigned)t >= (unsigned)a.N_max) continue;
    const size_t src = ((size_t)head * a.N_max + t) * a.rowb + sub * 16;
    st16(a.kc + (size_t)row * a.rowb + sub * 16, ld16(a.k + src));
    const int vm = a.vmap[row];
    if (vm >= 0 && vm < a.vcap) st16(a.vc + (size_t)vm * a.rowb + sub * 16, ld16(a.v + src));
    if (sub == 0) a.pos[row] = t;
  }
}

}  // namespace
}  // namespace kvcc

using namespace kvcc;

extern "C" size_t kv_vector_route_workspace_size(int B, int Hkv) {
  if (B < 1 || Hkv < 1) return 0;
  return (size_t)2 * B * Hkv * sizeof(int32_t) + 256;
}

extern "C" int kv_vector_route(const float* scores, const int32_t* ctx_len, const void* k,
                               const void* v, const float* w, int B, int Hkv, int N_max, int d,
                               int dtype, float p_c, float p_a, float rope_base,
                               int32_t* pool_idx, int32_t* pool_count, float* neg_eps,
                               int32_t* apx_pos, int32_t* apx_count, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!scores || !k || !v || !w || !pool_idx || !pool_count || !neg_eps || !apx_pos ||
      !apx_count)
    return KV_ERR_NULL;
  if (!aligned16(scores) || !aligned16(ctx_len) || !aligned16(k) || !aligned16(v) ||
      !aligned16(w) || !aligned16(pool_idx) || !aligned16(pool_count) || !aligned16(neg_eps) ||
      !aligned16(apx_pos) || !aligned16(apx_count) || !aligned16(workspace))
    return KV_ERR_ALIGN;
  if (dtype != KV_F32 && dtype != KV_BF16) return KV_ERR_DTYPE;
  if (B < 1 || Hkv < 1 || N_max < 1 || (d != 64 && d != 128) ||
      (int64_t)B * Hkv * N_max >= (int64_t(1) << 31))
    return KV_ERR_SHAPE;
  if (!(p_c >= 0.f && p_c <= 1.f && p_a >= 0.f && p_a <= 1.f && rope_base >= 0.f))
    return KV_ERR_MODE;
  if (!workspace || workspace_bytes < kv_vector_route_workspace_size(B, Hkv))
    return KV_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* k_pool = static_cast<int32_t*>(workspace);
  int32_t* k_apx = k_pool + (size_t)B * Hkv;
  const int H = B * Hkv;
  launch("vector_counts", vector_counts_kernel, dim3(ceil_div(H, 256)), dim3(256), 0, st, ctx_len,
         B, Hkv, N_max, p_c, p_a, k_pool, k_apx);
  kv_budget pool{};
  pool.mode = KV_BUDGET_K;
  pool.k = k_pool;
  pool.max_ratio = 1.f;
  select_launch(scores, ctx_len, nullptr, B, Hkv, N_max, pool, false, pool_idx, pool_count, st,
                "vector_pool");
  ResidualArgs r;
  r.k = static_cast<const char*>(k); r.v = static_cast<const char*>(v); r.w = w;
  r.pool_idx = pool_idx; r.pool_count = pool_count; r.neg_eps = neg_eps;
  r.B = B; r.Hkv = Hkv; r.N_max = N_max; r.rope_base = rope_base;
  {
    // a few workgroups per head (W staged once each), walking 64-entry tiles
    const dim3 grid((unsigned)std::max(1, std::min(ceil_div(N_max, RPW), 8)), Hkv, B);
    const char* nm = "vector_residual";
    if (dtype == KV_BF16) {
      if (d == 128) launch(nm, vector_residual_kernel<__bf16, 128>, grid, dim3(VT), 0, st, r);
      else launch(nm, vector_residual_kernel<__bf16, 64>, grid, dim3(VT), 0, st, r);
    } else {
      if (d == 128) launch(nm, vector_residual_kernel<float, 128>, grid, dim3(VT), 0, st, r);
      else launch(nm, vector_residual_kernel<float, 64>, grid, dim3(VT), 0, st, r);
    }
  }
  kv_budget apx{};
  apx.mode = KV_BUDGET_K;
  apx.k = k_apx;
  apx.max_ratio = 1.f;
  select_launch(neg_eps, nullptr, pool_count, B, Hkv, N_max, apx, true, apx_pos, apx_count, st,
                "vector_apx");
  return launch_status();
}

extern "C" int kv_vector_compact(const void* k, const void* v, int B, int Hkv, int N_max, int d,
                                 int dtype, const int32_t* pool_idx, const int32_t* pool_count,
                                 const int32_t* apx_pos, const int32_t* apx_count, void* k_c,
                                 void* v_c, int32_t* pos, int32_t* vmap, int64_t* offsets,
                                 int64_t* voffsets, int64_t capacity_rows,
                                 int64_t v_capacity_rows, void* stream) {
  if (!k || !v || !pool_idx || !pool_count || !apx_pos || !apx_count || !offsets || !voffsets)
    return KV_ERR_NULL;
  if (capacity_rows > 0 && (!k_c || !pos || !vmap)) return KV_ERR_NULL;
  if (v_capacity_rows > 0 && !v_c) return KV_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(pool_idx) || !aligned16(pool_count) ||
      !aligned16(apx_pos) || !aligned16(apx_count) || !aligned16(k_c) || !aligned16(v_c) ||
      !aligned16(pos) || !aligned16(vmap) || !aligned16(offsets) || !aligned16(voffsets))
    return KV_ERR_ALIGN;
  if (dtype != KV_F32 && dtype != KV_BF16) return KV_ERR_DTYPE;
  if (B < 1 || Hkv < 1 || N_max < 1 || (d != 64 && d != 128) || capacity_rows < 0 ||
      v_capacity_rows < 0 || (int64_t)B * Hkv > MAX_HEADS ||
      (int64_t)B * Hkv * N_max >= (int64_t(1) << 31) || v_capacity_rows >= (int64_t(1) << 31))
    return KV_ERR_SHAPE;

  VCompactArgs a;
  a.k = static_cast<const char*>(k); a.v = static_cast<const char*>(v);
  a.B = B; a.Hkv = Hkv; a.N_max = N_max; a.rowb = d * (dtype == KV_BF16 ? 2 : 4);
  a.pool_idx = pool_idx; a.pool_count = pool_count; a.apx_pos = apx_pos; a.apx_count = apx_count;
  a.kc = static_cast<char*>(k_c); a.vc = static_cast<char*>(v_c);
  a.pos = pos; a.vmap = vmap; a.offsets = offsets; a.voffsets = voffsets;
  a.cap = capacity_rows; a.vcap = v_capacity_rows;
  const int H = B * Hkv;
  const size_t dyn = (size_t)2 * (H + 1) * sizeof(long long);
  hipStream_t st = static_cast<hipStream_t>(stream);
  launch("vector_vmap", vector_vmap_kernel, dim3(H), dim3(VT), (uint32_t)dyn, st, a);
  {
    const int rpi = VT / (a.rowb / 16);
    int64_t grid = ceil_div64(std::min<int64_t>(capacity_rows, (int64_t)H * N_max), rpi * 4);
    grid = std::max<int64_t>(1, std::min<int64_t>(grid, 2048));
    launch("vector_copy", vector_copy_kernel, dim3((unsigned)grid), dim3(VT), (uint32_t)dyn, st, a);
  }
  return launch_status();
}
