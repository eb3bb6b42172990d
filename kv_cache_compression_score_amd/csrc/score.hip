// Observation-window token scores on gfx950 MFMA.
//
// For KV head h of sequence b, the G*W window rows r = (query head j, window
// position w) give logits l[r,t] = scale*<q_r, k_t>; the score of token t is
// sum_r exp(l[r,t] - lse[r]) with lse[r] the row log-sum-exp ("KVSculpt: KV
// Cache Compression as Distillation", section 2.B, names this normaliser
// ell; the attention-based importance score is the one importance-based
// eviction uses, "A Simple Plug-in for Improving Eviction-Based KV Cache
// Compression", section "Enonce du Probleme").
//
// Both sweeps over K tile the logit matrix into 32x32 MFMA blocks with the
// K tile staged once per workgroup in LDS and each wave holding the Q
// fragments of two 32-row blocks in registers.  K tiles of 64 tokens go from
// HBM to LDS directly (no registers), NB - 1 tiles ahead of the MFMAs, into NB
// buffers (four for 16 KB tiles, else two) with XOR-swizzled 16-byte columns:
//   pass 1: C[token,row] = K * Q^T, so one lane owns one row and 16 tokens
//           per block and keeps a running (m, sum of 2^(x - m)) per row in
//           registers, m at or below the row maximum; the two half-waves are
//           merged by a lane swizzle and the chunk partials published.
//   fold:   16 lanes per row merge the row's chunk partials (lanes over
//           chunks, then a fixed butterfly) into a base-2 log-sum-exp.
//   pass 2: C[row,token] = Q * K^T, so one lane owns one token and 16 rows
//           per block; exp2(l*c - lse2[row]) is summed in-lane, then over
//           half-waves and waves through LDS in a fixed order.
// All logits are kept in base-2 units: c = scale*log2(e) is applied to the
// fp32 dot product after the MFMA (bf16 inputs are never rescaled).  The
// per-logit epilogue is kept to one FMA, one exp2 and one add (plus, in pass
// 1, a maximum over three of each lane's sixteen logits per block); masks only
// exist in tail tiles.
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "common.hpp"

namespace kvcc {
namespace {

constexpr int TOK = 64;          // tokens per LDS tile
constexpr int RBW = 2;           // 32-row blocks per wave
constexpr int SLOTS_1 = 256 * 2; // pass-1 chunking target: resident workgroups on 256 CUs
constexpr int RANGE_HEADS = 256;  // most heads (B * Hkv) the balanced pass-2 ranges take
constexpr int TAB_MAX = 2048;     // most pass-2 workgroups in that mode
constexpr int SELF_MERGE = 16;    // pass 2 merges pass 1's partials itself up to this many chunks

template <typename T> struct FragT;
template <> struct FragT<__bf16> { using vec = bf16x8; };   // 8 elements = 16 B
template <> struct FragT<float> { using vec = f32x8; };     // 8 elements = 32 B

// One 16-wide k-step.  bf16: a single 32x32x16 MFMA.  fp32: eight 32x32x2
// MFMAs; MFMA e pairs element e of both half-waves (dims e and 8+e), which
// covers the same 16 dims since A and B fragments use the same layout.
__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

template <typename T>
__device__ __forceinline__ typename FragT<T>::vec load_frag(const void* p);
template <>
__device__ __forceinline__ bf16x8 load_frag<__bf16>(const void* p) {
  return __builtin_bit_cast(bf16x8, ld16(p));
}
template <>
__device__ __forceinline__ f32x8 load_frag<float>(const void* p) {
  const uint4 a = ld16(p), b = ld16(static_cast<const char*>(p) + 16);
  f32x8 v;
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
  v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
  v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  return v;
}

// A K fragment from a swizzled LDS row: logical 16-byte piece c of the row
// sits at piece c ^ sw.  bf16: one piece; fp32: pieces c and c + 1.
template <typename T>
__device__ __forceinline__ typename FragT<T>::vec load_frag_sw(const unsigned char* row, int c, int sw);
template <>
__device__ __forceinline__ bf16x8 load_frag_sw<__bf16>(const unsigned char* row, int c, int sw) {
  return __builtin_bit_cast(bf16x8, ld16(row + 16 * (c ^ sw)));
}
template <>
__device__ __forceinline__ f32x8 load_frag_sw<float>(const unsigned char* row, int c, int sw) {
  const uint4 a = ld16(row + 16 * (c ^ sw)), b = ld16(row + 16 * ((c + 1) ^ sw));
  f32x8 v;
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
  v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
  v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  return v;
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at lds + 16 i (the LDS base goes in M0, which the block restores).  Issued
// from asm so that the compiler does not answer the pending LDS write with a
// full vector-memory wait before every later LDS read; the kernel orders them
// itself (vm_wait, then a barrier).  The load writes no register; its
// address operands are read at issue.
__device__ __forceinline__ void lds_dma16(const void* g, unsigned char* lds) {
  const uint32_t l = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(l)
      : "memory");
  (void)saved;
}

// As lds_dma16, from a wave-uniform base (SGPRs) plus a 32-bit per-lane
// byte offset: no per-load address arithmetic on the VALU.
__device__ __forceinline__ void lds_dma16_sv(const void* base, uint32_t off, unsigned char* lds) {
  const uint32_t l = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(l)
      : "memory");
  (void)saved;
}

// s_waitcnt on the vector-memory counter only (at most N outstanding).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

struct ScoreArgs {
  const void* q;
  const void* k;
  const int32_t* ctx;
  float* scores;
  float2* part;     // [B*Hkv][n_chunks][R_pad] per-chunk (max, sum of exp2) per row
  float* lse2;      // [B*Hkv][R_pad] base-2 row log-sum-exp (+inf: row adds nothing)
  float* row_lse;   // [B][Hq][W] natural log, optional
  const float* lse_in;  // [B][Hq][W] natural-log row LSE given by the caller (one-pass), or null
  int B, Hq, Hkv, N_max, W, G, R, R_pad, causal;
  int TC, n_chunks;    // pass-1 token chunks (fixed by the sizes: sets the merge order)
  int TC2, n_chunks2;  // pass-2 token chunks (free: no cross-chunk arithmetic)
  int ranges;          // pass 2: balanced tile ranges over G2 workgroups (see score_pass)
  int G2;              // pass-2 workgroups in that mode
  int4* tab;           // [TAB_MAX] the ranges, written by pass 1: {head, t0, t1, n}
  int self_merge;      // pass 2 merges the pass-1 partials (n_chunks <= SELF_MERGE); else the fold's lse2
  float c;             // scale * log2(e)
};

// Pass-2 work ranges, built by one workgroup of pass 1 so that pass 2 reads
// its range with one load.  Each head's 64-token tiles are cut into ranges
// of L tiles, L = ceil(T / G) if that leaves at most G ranges, else
// ceil(T / (G - H)) (T tiles in all, G = a.G2 workgroups, H heads), and range
// i goes to workgroup i in (sequence, head, range) order: with ragged lengths
// no workgroup gets more than about T / (G - H) tiles, where chunks sized for
// N_max leave some CUs whole heads and others nothing; with equal lengths the
// ranges are those chunks.  Unused entries get head -1.  `scr` is LDS for
// 2 B + 3 ints (B <= RANGE_HEADS).
__device__ void build_ranges(const ScoreArgs& a, int* scr) {
  const int tid = threadIdx.x, nt_thr = blockDim.x;
  const int B = a.B, Hkv = a.Hkv, H = B * Hkv, G = a.G2;
  int* seqr = scr;              // ranges per head of sequence b
  int* seqpre = scr + B;        // ranges before sequence b (B + 1 entries)
  int* tot = scr + 2 * B + 1;   // tiles, ranges
  auto len = [&](int bb) { return a.ctx ? min(max(a.ctx[bb], 0), a.N_max) : a.N_max; };
  if (tid == 0) { tot[0] = 0; tot[1] = 0; }
  __syncthreads();
  for (int bb = tid; bb < B; bb += nt_thr) atomicAdd(&tot[0], Hkv * ((len(bb) + TOK - 1) / TOK));
  __syncthreads();
  const int total = tot[0];
  int L = max(1, (total + G - 1) / G);
  for (int bb = tid; bb < B; bb += nt_thr)
    atomicAdd(&tot[1], Hkv * (((len(bb) + TOK - 1) / TOK + L - 1) / L));
  __syncthreads();
  if (tot[1] > G) L = max(1, (total + (G - H) - 1) / (G - H));
  for (int bb = tid; bb < B; bb += nt_thr) seqr[bb] = ((len(bb) + TOK - 1) / TOK + L - 1) / L;
  __syncthreads();
  if (tid == 0) {
    seqpre[0] = 0;
    for (int bb = 0; bb < B; ++bb) seqpre[bb + 1] = seqpre[bb] + Hkv * seqr[bb];
  }
  __syncthreads();
  const int R = seqpre[B];
  for (int i = tid; i < G; i += nt_thr) {
    int4 e = make_int4(-1, 0, 0, 0);
    if (i < R) {
      int lo = 0, hi = B - 1;   // largest b with seqpre[b] <= i (empty sequences are passed over)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seqpre[mid] <= i) lo = mid; else hi = mid - 1;
      }
      const int q = i - seqpre[lo], rb = seqr[lo];
      const int nb = len(lo);
      const int t0 = (q % rb) * L * TOK;
      e = make_int4(lo * Hkv + q / rb, t0, min(t0 + L * TOK, nb), nb);
    }
    a.tab[i] = e;
  }
}

template <typename T, int D, int NW, int PASS>
__global__ __launch_bounds__(NW * WAVE) void score_pass(ScoreArgs a) {
  using V = typename FragT<T>::vec;
  constexpr int KS = D / 16;
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int VPR = ROWB / 16;                 // 16-byte pieces per K row
  constexpr int TILE_VECS = TOK * VPR;
  // K tiles travel HBM -> LDS directly (no registers): NB buffers, tile t in
  // buffer t % NB, requested NB - 1 tiles ahead.
  constexpr int NB = TOK * ROWB <= 16384 ? 4 : 2;
  constexpr int NT = NW * WAVE;
  constexpr int LPT = (TILE_VECS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) unsigned char ktile[NB][TOK * ROWB];
  __shared__ float red[3][PASS == 2 ? NW : 1][TOK];
  __shared__ __attribute__((aligned(8))) int rowpos[PASS == 2 ? NW * RBW * 32 : 2];

  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int hf = lane >> 5, l32 = lane & 31;

  // The workgroup's tokens [t0, t1) of head (b, h).  Chunk mode: chunk
  // blockIdx.x of head (blockIdx.z, blockIdx.y).  Balanced mode (pass 2,
  // a.ranges): range blockIdx.x of the table that one workgroup of pass 1
  // built (build_ranges), read with one scalar load.
  int b, h, c, t0, t1, n;
  if (PASS == 1 && a.ranges && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) {
    build_ranges(a, reinterpret_cast<int*>(&ktile[0][0]));   // LDS not in use yet
    __syncthreads();
  }
  if (PASS == 2 && a.ranges) {
    const int4 e = a.tab[blockIdx.x];
    const int hd = __builtin_amdgcn_readfirstlane(e.x);
    if (hd < 0) return;   // fewer ranges than workgroups
    // the division runs on the VALU: bring the quotient back to SGPRs
    b = __builtin_amdgcn_readfirstlane(hd / a.Hkv); h = hd - b * a.Hkv; c = 0;
    t0 = __builtin_amdgcn_readfirstlane(e.y);
    t1 = __builtin_amdgcn_readfirstlane(e.z);
    n = __builtin_amdgcn_readfirstlane(e.w);
  } else {
    c = blockIdx.x; h = blockIdx.y; b = blockIdx.z;
    n = a.ctx ? min(max(a.ctx[b], 0), a.N_max) : a.N_max;
    const int TC = PASS == 1 ? a.TC : a.TC2;
    t0 = c * TC;
    if (t0 >= n) {
      if (PASS == 1)
        for (int r = tid; r < a.R_pad; r += NT)
          a.part[((size_t)(b * a.Hkv + h) * a.n_chunks + c) * a.R_pad + r] = make_float2(-INFINITY, 0.f);
      return;
    }
    t1 = min(t0 + TC, n);
  }
  const int head = b * a.Hkv + h;
  const int ntiles = (t1 - t0 + TOK - 1) / TOK;
  const char* kh = static_cast<const char*>(a.k) + (size_t)head * a.N_max * ROWB;
  const int last_w0 = n - a.W;   // position of window row 0; row w sits at last_w0 + w
  // Leading tiles whose every token exists and is visible to every row.
  int clean_tiles = (t1 - t0) / TOK;
  if (a.causal) clean_tiles = min(clean_tiles, max(0, (last_w0 + 1 - t0) / TOK));
  const float cc = a.c;

  // Q fragments of this wave's row blocks (zero for padding rows).
  // Loads are branch-free (clamped row, then a select) so they all issue at once.
  V qf[RBW][KS];
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int r = (wave * RBW + i) * 32 + l32;
    const int rc = min(r, a.R - 1);
    const int j = h * a.G + rc / a.W, w = rc % a.W;
    const char* qp = static_cast<const char*>(a.q) +
                     ((((size_t)b * a.Hq + j) * a.W + w) * D + 8 * hf) * sizeof(T);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const V v = load_frag<T>(qp + ks * 16 * sizeof(T));
      qf[i][ks] = r < a.R ? v : V{};
    }
  }

  // Causal limits: p_row[i] = position of the lane's pass-1 row (row block i);
  // rowpos[r] = window position (r mod W) of every row, for the pass-2 masks.
  int p_row[RBW];
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int r = (wave * RBW + i) * 32 + l32;
    p_row[i] = a.causal ? last_w0 + (r % a.W) : 0x7fffffff;
  }
  if (PASS == 2 && a.causal)
    for (int r = tid; r < NW * RBW * 32; r += NT) rowpos[r] = r % a.W;

  // Pass-1 running state (per row owned by the lane) / pass-2 negated row lse2.
  float m_run[RBW], s_run[RBW];
  float nl2[RBW][16];
  const float inv_w = 1.0f / (float)a.W;
  if (PASS == 1) {
#pragma unroll
    for (int i = 0; i < RBW; ++i) { m_run[i] = -INFINITY; s_run[i] = 0.f; }
  } else if (a.lse_in) {
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = (wave * RBW + i) * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
        // caller's natural-log LSE of row (j, w), to base 2;
        // rc / W by a float reciprocal: exact for rc < 1024 (error < 0.5/W)
        const int rc = min(r, a.R - 1);
        const int jw = (int)(((float)rc + 0.5f) * inv_w);
        const int j = h * a.G + jw, w = rc - jw * a.W;
        const float v = a.lse_in[((size_t)b * a.Hq + j) * a.W + w] * (float)LOG2E_D;
        nl2[i][e] = r < a.R ? -v : -INFINITY;
      }
    }
  } else if (!a.self_merge) {   // the fold's row LSEs
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = (wave * RBW + i) * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
        nl2[i][e] = r < a.R ? -a.lse2[(size_t)head * a.R_pad + min(r, a.R_pad - 1)] : -INFINITY;
      }
    }
  } else {
    // Base-2 LSE of each row from pass 1's per-chunk (m, sum) partials of
    // this head (at most 16, loads all issued at once): M = max of the m's,
    // then the sum of sum * 2^(m - M).  Staged in `red` (not in use before
    // tile 0).
    float* lse_s = &red[0][0][0];
    for (int r = tid; r < NW * RBW * 32; r += NT) {
      float v = INFINITY;
      if (r < a.R) {
        const float2* src = a.part + (size_t)head * a.n_chunks * a.R_pad + r;
        float2 pk[SELF_MERGE];
#pragma unroll
        for (int u = 0; u < SELF_MERGE; ++u)   // chunk u of the row: lanes read consecutive rows
          pk[u] = u < a.n_chunks ? src[(size_t)u * a.R_pad] : make_float2(-INFINITY, 0.f);
        float M = -INFINITY;
#pragma unroll
        for (int u = 0; u < SELF_MERGE; ++u) M = fmaxf(M, pk[u].x);
        if (M != -INFINITY) {
          float S = 0.f;
#pragma unroll
          for (int u = 0; u < SELF_MERGE; ++u) S = fmaf(pk[u].y, fast_exp2(pk[u].x - M), S);
          if (S > 0.f) v = M + log2f(S);
        }
      }
      lse_s[r] = v;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = (wave * RBW + i) * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
        nl2[i][e] = r < a.R ? -lse_s[r] : -INFINITY;
      }
    }
  }

  // K tile staging.  Piece v of a tile (16 bytes) sits at LDS slot v: row
  // v / VPR, column v % VPR, and holds the row's global column
  // (v % VPR) ^ (row % VPR), so the 32 rows a fragment read touches spread
  // over the banks without padding.  A wave's load instruction fills 64
  // consecutive slots (lane i -> slot base + i).
  // (a wave either loads all 64 of its pieces in a round or none of them)
  static_assert(TILE_VECS % WAVE == 0 && (TILE_VECS % NT == 0 || TILE_VECS < NT), "load rounds");
  // A whole tile's loads take the byte offsets computed here once, from the
  // tile's base address in SGPRs; a partial (last) tile clamps its rows.
  uint32_t poff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int v = tid + i * NT;
    poff[i] = (uint32_t)(((v / VPR) * VPR + ((v % VPR) ^ ((v / VPR) & (VPR - 1)))) * 16);
  }
  const int wslot = __builtin_amdgcn_readfirstlane(tid - lane);   // the wave's first slot
  auto gload_lds = [&](int buf, int tile) __attribute__((always_inline)) {
    const int tt0 = t0 + tile * TOK;
    const int rows = min(TOK, t1 - tt0);
    const char* base = kh + (size_t)tt0 * ROWB;
    if (rows == TOK) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        if (tid + i * NT >= TILE_VECS) break;   // uniform over the wave
        lds_dma16_sv(base, poff[i], &ktile[buf][(wslot + i * NT) * 16]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int v = tid + i * NT;
        if (v >= TILE_VECS) break;   // uniform over the wave
        // rows past the chunk end re-read its last row: their tokens are
        // masked (pass 1) or never written (pass 2)
        const int row = min(v / VPR, rows - 1);
        const int col = (v % VPR) ^ ((v / VPR) & (VPR - 1));
        lds_dma16(base + ((size_t)row * VPR + col) * 16, &ktile[buf][(wslot + i * NT) * 16]);
      }
    }
  };
  // Wait for this thread's pieces of tile t; the NB - 2 tiles requested
  // after it (fewer near the end) may stay in flight.
  auto wait_tile = [&](int tile) __attribute__((always_inline)) {
    static_assert(NB == 2 || NB == 4, "buffers");
    if constexpr (NB == 4) {
      const int later = min(NB - 2, ntiles - 1 - tile);
      if (later >= 2) vm_wait<2 * LPT>();
      else if (later == 1) vm_wait<LPT>();
      else vm_wait<0>();
    } else {
      vm_wait<0>();
    }
  };

  // ---- software pipeline over 32-token blocks j (two per 64-token tile) ----
  // The two 32-row blocks of the wave alternate between the matrix core and
  // the VALU: while the MFMAs of (block j, rows 0..31) run, the epilogue of
  // (block j-1, rows 32..63) executes, and while (block j, rows 32..63)
  // multiplies, (block j, rows 0..31) is finished.  Each MFMA is paired with
  // an eighth of the other row block's epilogue; sched_barrier keeps the
  // pairing, so the exp2 work hides under the MFMA pipe of the same wave.
  static_assert(RBW == 2, "the pipeline alternates two row blocks");
  V kf[KS];
  f32x16 acc[RBW];
  float col_cur = 0.f;                 // pass 2: column sum of the block in flight
  // per-epilogue scratch (pass 1)
  float e_nm = 0.f, e_sum = 0.f, e_mn = 0.f;

  auto load_k = [&](int buf, int sub) __attribute__((always_inline)) {
    const int r = sub * 32 + l32, sw = r & (VPR - 1);
    const unsigned char* krow = &ktile[buf][r * ROWB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = (8 * hf + 16 * ks) * (int)sizeof(T) / 16;   // first 16-byte piece
      kf[ks] = load_frag_sw<T>(krow, c, sw);
    }
  };
  auto mma_step = [&](int i, int q) __attribute__((always_inline)) {
    // q-th of 8 MFMA slots of row block i: k-steps [q*KS/8, (q+1)*KS/8)
#pragma unroll
    for (int ks = q * KS / 8; ks < (q + 1) * KS / 8; ++ks) {
      if (ks == 0)
        acc[i] = PASS == 1 ? mma(kf[0], qf[i][0], f32x16{}) : mma(qf[i][0], kf[0], f32x16{});
      else
        acc[i] = PASS == 1 ? mma(kf[ks], qf[i][ks], acc[i]) : mma(qf[i][ks], kf[ks], acc[i]);
    }
  };
  // q-th eighth of the epilogue of row block i for the block starting at token ts.
  auto epi_step = [&](int i, int q, int ts, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    if (PASS == 1) {
      // acc[i][e] = dot(row (wave*RBW+i)*32 + l32, token ts + 8*(e/4) + 4*hf + e%4)
      if (q == 0) {
        if (MASKED) {
          // token ts + off_e + 4*hf is kept iff off_e <= lim (off_e = 8*(e/4) + e%4)
          const int lim = min(t1 - 1, p_row[i]) - ts - 4 * hf;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            acc[i][e] = (8 * (e >> 2) + (e & 3)) > lim ? -INFINITY : acc[i][e];
        }
        if (MASKED) {
          // three-input maxima (v_max3): 16 values in 8 instructions
          const float a0 = fmaxf(acc[i][0], fmaxf(acc[i][1], acc[i][2]));
          const float a1 = fmaxf(acc[i][3], fmaxf(acc[i][4], acc[i][5]));
          const float a2 = fmaxf(acc[i][6], fmaxf(acc[i][7], acc[i][8]));
          e_mn = fmaxf(a0, fmaxf(a1, a2));
        } else {
          // The reference m of a running (m, sum of 2^(x - m)) pair need not
          // be the maximum: any m at or below it gives the same m + log2(sum)
          // while no term overflows.  Whole tiles take it from three of the
          // lane's sixteen logits; a block whose sum comes out above 2^64 is
          // redone from its exact maximum below.
          e_mn = fmaxf(acc[i][0], fmaxf(acc[i][7], acc[i][13]));
        }
      } else if (q == 1) {
        if (MASKED) {
          const float a3 = fmaxf(acc[i][9], fmaxf(acc[i][10], acc[i][11]));
          const float a4 = fmaxf(acc[i][12], fmaxf(acc[i][13], acc[i][14]));
          e_mn = fmaxf(acc[i][15], fmaxf(a3, fmaxf(a4, e_mn)));
        }
        e_mn = fmaxf(m_run[i], e_mn * cc);
        // a fully masked row keeps (-inf, 0): exp2(-inf - 0) = 0 everywhere
        e_nm = MASKED && e_mn == -INFINITY ? 0.f : -e_mn;
      } else {
        // slots 2..7 take 3,3,3,3,2,2 of the 16 exponentials
        constexpr int lo_tab[9] = {0, 0, 0, 3, 6, 9, 12, 14, 16};
        const int lo = lo_tab[q], hi = lo_tab[q + 1];
#pragma unroll
        for (int e = lo; e < hi; ++e) {
          const float x = fast_exp2(fmaf(acc[i][e], cc, e_nm));
          e_sum = e == 0 ? x : e_sum + x;
        }
        if (q == 7) {
          if (!MASKED && !(e_sum <= 0x1p64f)) {   // a logit far above the sampled ones
            float mx = acc[i][0];
#pragma unroll
            for (int e = 1; e < 16; ++e) mx = fmaxf(mx, acc[i][e]);
            e_mn = fmaxf(m_run[i], mx * cc);
            e_nm = -e_mn;
            e_sum = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) e_sum += fast_exp2(fmaf(acc[i][e], cc, e_nm));
          }
          s_run[i] = fmaf(s_run[i], fast_exp2(m_run[i] + e_nm), e_sum);
          m_run[i] = e_mn;
        }
      }
    } else {
      // acc[i][e] = dot(row (wave*RBW+i)*32 + 8*(e/4) + 4*hf + e%4, token ts + l32)
      // causal: the lane's token t sees row r iff t - last_w0 <= (r mod W), read from LDS
      int2 wpos = make_int2(0, 0);
      if (MASKED && a.causal)
        wpos = *reinterpret_cast<const int2*>(
            &rowpos[(wave * RBW + i) * 32 + 8 * (q >> 1) + 4 * hf + ((2 * q) & 3)]);
#pragma unroll
      for (int e = 2 * q; e < 2 * q + 2; ++e) {
        const float x = fast_exp2(fmaf(acc[i][e], cc, nl2[i][e]));
        if (MASKED && a.causal)
          col_cur += ts + l32 - last_w0 <= (e == 2 * q ? wpos.x : wpos.y) ? x : 0.f;
        else
          col_cur += x;
      }
    }
  };
  // One pipeline step: MFMAs of row block im (if any) paired with the
  // epilogue of row block ie of the block at token ts (if any).
  // (do_mma, im, do_epi, ie) are compile-time tags so acc[] stays in registers.
  auto step = [&](auto do_mma, auto im, auto do_epi, auto ie, int ts, auto masked_tag)
      __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if constexpr (decltype(do_mma)::value) mma_step(decltype(im)::value, q);
      if constexpr (decltype(do_epi)::value) epi_step(decltype(ie)::value, q, ts, masked_tag);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto step_m = [&](auto do_mma, auto im, auto do_epi, auto ie, int ts, bool masked)
      __attribute__((always_inline)) {
    if (masked) step(do_mma, im, do_epi, ie, ts, T_{});
    else step(do_mma, im, do_epi, ie, ts, F_{});
  };
  auto emit_col = [&](int tile, int sub) __attribute__((always_inline)) {   // pass 2: block column sums -> LDS
    if (PASS == 2) {
      // other half-wave's rows: v_permlane32_swap hands each lane the value
      // of lane l^32 (both halves of the result sum to col(l) + col(l^32))
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(col_cur),
                                                       __float_as_uint(col_cur), false, false);
      const float c2 = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      if (hf == 0) red[tile % 3][wave][sub * 32 + l32] = c2;
      col_cur = 0.f;
    }
  };
  auto reduce_tile = [&](int tile) {
    if (PASS == 2 && tid < TOK) {
      const int t = t0 + tile * TOK + tid;
      if (t < t1) {
        float s = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) s += red[tile % 3][w2][tid];
        a.scores[(size_t)head * a.N_max + t] = s;
      }
    }
  };
  auto masked_tile = [&](int tile) { return tile >= clean_tiles; };

  // Tiles 0 .. NB-2 requested up front; at tile t (after its barrier, which
  // also tells that every wave is done with tile t-1) tile t + NB - 1 goes
  // into the buffer tile t-1 used.
  for (int p = 0; p < NB - 1; ++p)
    if (p < ntiles) gload_lds(p, p);
  // tile 0
  wait_tile(0);
  __syncthreads();
  if (NB - 1 < ntiles) gload_lds(NB - 1, NB - 1);
  load_k(0, 0);
  step_m(T_{}, I0{}, F_{}, I1{}, 0, false);                     // MMA(0, r0)
  step_m(T_{}, I1{}, T_{}, I0{}, t0, masked_tile(0));           // MMA(0, r1) | epi(0, r0)
  load_k(0, 1);
  step_m(T_{}, I0{}, T_{}, I1{}, t0, masked_tile(0));           // MMA(1, r0) | epi(0, r1)
  emit_col(0, 0);
  step_m(T_{}, I1{}, T_{}, I0{}, t0 + 32, masked_tile(0));      // MMA(1, r1) | epi(1, r0)
  for (int tile = 1; tile < ntiles; ++tile) {
    const int tt0 = t0 + tile * TOK, buf = tile % NB;
    wait_tile(tile);
    __syncthreads();
    if (tile >= 2) reduce_tile(tile - 2);
    if (tile + NB - 1 < ntiles) gload_lds((tile + NB - 1) % NB, tile + NB - 1);
    load_k(buf, 0);
    step_m(T_{}, I0{}, T_{}, I1{}, tt0 - 32, masked_tile(tile - 1));  // MMA(2t, r0) | epi(2t-1, r1)
    emit_col(tile - 1, 1);
    step_m(T_{}, I1{}, T_{}, I0{}, tt0, masked_tile(tile));           // MMA(2t, r1) | epi(2t, r0)
    load_k(buf, 1);
    step_m(T_{}, I0{}, T_{}, I1{}, tt0, masked_tile(tile));           // MMA(2t+1, r0) | epi(2t, r1)
    emit_col(tile, 0);
    step_m(T_{}, I1{}, T_{}, I0{}, tt0 + 32, masked_tile(tile));      // MMA(2t+1, r1) | epi(2t+1, r0)
  }
  // drain: the last block's second row block
  step_m(F_{}, I0{}, T_{}, I1{}, t0 + (ntiles - 1) * TOK + 32, masked_tile(ntiles - 1));
  emit_col(ntiles - 1, 1);
  if (PASS == 2) {
    __syncthreads();
    if (ntiles >= 2) reduce_tile(ntiles - 2);
    reduce_tile(ntiles - 1);
  }

  if (PASS == 1) {
    // Merge the two half-waves (same row, disjoint tokens), then publish.
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      const float mo = __shfl_xor(m_run[i], 32, WAVE);
      const float so = __shfl_xor(s_run[i], 32, WAVE);
      const float mn = fmaxf(m_run[i], mo);
      float s = 0.f;
      if (mn != -INFINITY) s = s_run[i] * fast_exp2(m_run[i] - mn) + so * fast_exp2(mo - mn);
      const int r = (wave * RBW + i) * 32 + l32;
      if (hf == 0 && r < a.R_pad)
        a.part[((size_t)head * a.n_chunks + c) * a.R_pad + r] = make_float2(mn, s);
    }
  }
}

__device__ __forceinline__ void merge(float& m, float& s, float pm, float ps) {
  const float mn = fmaxf(m, pm);
  if (mn == -INFINITY) return;
  s = s * exp2f(m - mn) + ps * exp2f(pm - mn);
  m = mn;
}

// FOLD_LANES lanes per row (four rows per wave): the lanes merge chunks
// c = l, l + FOLD_LANES, ... in order, then a fixed butterfly merges the
// lanes; deterministic for fixed sizes.
constexpr int FOLD_LANES = 16;

__global__ __launch_bounds__(256) void score_fold(ScoreArgs a) {
  const int l = threadIdx.x & (FOLD_LANES - 1);
  const int row_id = blockIdx.x * (256 / FOLD_LANES) + threadIdx.x / FOLD_LANES;
  const bool live = row_id < a.B * a.Hkv * a.R_pad;   // the butterfly needs every lane
  const int head = row_id / a.R_pad, r = row_id % a.R_pad;
  float m = -INFINITY, s = 0.f;
  if (live && r < a.R) {
    const float2* src = a.part + (size_t)head * a.n_chunks * a.R_pad + r;
    for (int c = l; c < a.n_chunks; c += FOLD_LANES) {
      const float2 p = src[(size_t)c * a.R_pad];
      merge(m, s, p.x, p.y);
    }
  }
#pragma unroll
  for (int o = 1; o < FOLD_LANES; o <<= 1) {
    const float pm = __shfl_xor(m, o, WAVE), ps = __shfl_xor(s, o, WAVE);
    // both partners compute the same merge in the same operand order
    const bool lower = (l & o) == 0;
    float m1 = lower ? m : pm, s1 = lower ? s : ps;
    merge(m1, s1, lower ? pm : m, lower ? ps : s);
    m = m1; s = s1;
  }
  if (!live || l != 0) return;
  if (r >= a.R) {
    a.lse2[row_id] = INFINITY;
    return;
  }
  const bool seen = s > 0.f;
  const float l2v = seen ? m + log2f(s) : INFINITY;
  a.lse2[row_id] = l2v;
  if (a.row_lse) {
    const int b = head / a.Hkv, h = head % a.Hkv;
    const int j = h * a.G + r / a.W, w = r % a.W;
    a.row_lse[((size_t)b * a.Hq + j) * a.W + w] = seen ? l2v * LN2_F : -INFINITY;
  }
}

struct ScorePlan {
  int G, R, R_pad, NW, TC, n_chunks;
  size_t off_lse, off_tab, bytes;
};

// Tokens per workgroup: the tile count per chunk (at least `min_tiles`) that
// minimises rounds * tiles-per-chunk when `slots` workgroups are resident,
// i.e. the fewest tile-times for the whole grid; ties go to bigger chunks.
int chunk_tokens(int64_t heads, int N_max, int64_t slots, int min_tiles) {
  const int64_t tiles = ceil_div64(N_max, TOK);
  int64_t best = tiles, best_cost = INT64_MAX;
  for (int64_t tpc = std::min<int64_t>(min_tiles, tiles); tpc <= tiles; ++tpc) {
    const int64_t wgs = heads * ceil_div64(tiles, tpc);
    const int64_t cost = ceil_div64(wgs, slots) * tpc;
    if (cost <= best_cost) { best_cost = cost; best = tpc; }
  }
  return (int)(best * TOK);
}

bool plan_score(int B, int Hq, int Hkv, int N_max, int W, int d, ScorePlan* p) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || N_max < 1 || W < 1 || W > N_max) return false;
  if (d != 64 && d != 128) return false;
  if ((int64_t)B * Hkv * N_max >= (int64_t(1) << 31)) return false;
  const int64_t R64 = (int64_t)(Hq / Hkv) * W;
  if (R64 > 1024) return false;
  p->G = Hq / Hkv;
  p->R = (int)R64;
  const int RB = ceil_div(p->R, 32);
  p->R_pad = RB * 32;
  const int nw = ceil_div(RB, RBW);
  p->NW = nw <= 1 ? 1 : nw <= 2 ? 2 : nw <= 4 ? 4 : nw <= 8 ? 8 : 16;
  // Pass-1 chunking depends on the sizes only, so the merge order (and the
  // result, bit for bit) does not depend on the device.
  p->TC = chunk_tokens((int64_t)B * Hkv, N_max, SLOTS_1, 4);
  p->n_chunks = ceil_div(N_max, p->TC);
  const size_t part = (size_t)B * Hkv * p->n_chunks * p->R_pad * sizeof(float2);
  p->off_lse = (part + 255) & ~size_t(255);
  const size_t lse_end = p->off_lse + (size_t)B * Hkv * p->R_pad * sizeof(float);
  p->off_tab = (lse_end + 255) & ~size_t(255);
  p->bytes = p->off_tab + (size_t)TAB_MAX * sizeof(int4);
  return true;
}

// Resident workgroups of a kernel on the current device (cached per kernel).
template <typename K>
int64_t resident_slots(K kernel, int threads, int* cache) {
  if (*cache > 0) return *cache;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      cus < 1 || per_cu < 1)
    return SLOTS_1;
  *cache = cus * per_cu;
  return *cache;
}

template <typename T, int D, int NW>
void launch_score(ScoreArgs a, hipStream_t st) {
  static int slots2 = 0;
  a.TC2 = chunk_tokens((int64_t)a.B * a.Hkv, a.N_max,
                       resident_slots(score_pass<T, D, NW, 2>, NW * WAVE, &slots2), 4);
  a.n_chunks2 = ceil_div(a.N_max, a.TC2);
  const dim3 grid1(a.n_chunks, a.Hkv, a.B);
  dim3 grid2(a.n_chunks2, a.Hkv, a.B);
  // Balanced pass-2 ranges (two-pass path): one workgroup per resident slot,
  // at least two per head; pass 1 writes the table
  const int H = a.B * a.Hkv;
  a.G2 = std::min(slots2 > 0 ? slots2 : SLOTS_1, TAB_MAX);
  a.ranges = a.tab && !a.lse_in && H <= RANGE_HEADS && 2 * H <= a.G2 ? 1 : 0;
  if (a.ranges) grid2 = dim3((unsigned)a.G2, 1, 1);
  a.self_merge = a.n_chunks <= SELF_MERGE ? 1 : 0;
  if (a.lse_in) {   // row LSEs given: the column-sum pass alone
    launch("score_colsum", score_pass<T, D, NW, 2>, grid2, dim3(NW * WAVE), 0, st, a);
    return;
  }
  launch("score_rowstats", score_pass<T, D, NW, 1>, grid1, dim3(NW * WAVE), 0, st, a);
  // with few chunks pass 2 merges the partials of its own head, and the fold
  // runs only to hand the caller the row LSEs
  if (a.row_lse || !a.self_merge) {
    const int rows = a.B * a.Hkv * a.R_pad;
    launch("score_fold", score_fold, dim3(ceil_div(rows, 256 / FOLD_LANES)), dim3(256), 0, st, a);
  }
  launch("score_colsum", score_pass<T, D, NW, 2>, grid2, dim3(NW * WAVE), 0, st, a);
}

template <typename T, int D>
void launch_score_nw(const ScoreArgs& a, int NW, hipStream_t st) {
  switch (NW) {
    case 1: launch_score<T, D, 1>(a, st); break;
    case 2: launch_score<T, D, 2>(a, st); break;
    case 4: launch_score<T, D, 4>(a, st); break;
    case 8: launch_score<T, D, 8>(a, st); break;
    default: launch_score<T, D, 16>(a, st); break;
  }
}

}  // namespace
}  // namespace kvcc

using namespace kvcc;

extern "C" size_t kv_score_workspace_size(int B, int Hq, int Hkv, int N_max, int W, int d) {
  ScorePlan p;
  return plan_score(B, Hq, Hkv, N_max, W, d, &p) ? p.bytes : 0;
}

extern "C" int kv_score(const void* q_win, const void* k, const int32_t* ctx_len,
                        float* scores, float* row_lse,
                        int B, int Hq, int Hkv, int N_max, int W, int d, int dtype,
                        int causal, float scale,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_win || !k || !scores) return KV_ERR_NULL;
  if (!aligned16(q_win) || !aligned16(k) || !aligned16(scores) || !aligned16(ctx_len) ||
      !aligned16(row_lse) || !aligned16(workspace))
    return KV_ERR_ALIGN;
  if (dtype != KV_F32 && dtype != KV_BF16) return KV_ERR_DTYPE;
  ScorePlan p;
  if (!plan_score(B, Hq, Hkv, N_max, W, d, &p)) return KV_ERR_SHAPE;
  if (!workspace || workspace_bytes < p.bytes) return KV_ERR_WORKSPACE;

  ScoreArgs a;
  a.q = q_win; a.k = k; a.ctx = ctx_len; a.scores = scores; a.row_lse = row_lse;
  a.lse_in = nullptr;
  a.part = static_cast<float2*>(workspace);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.off_lse);
  a.tab = reinterpret_cast<int4*>(static_cast<char*>(workspace) + p.off_tab);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N_max = N_max; a.W = W; a.G = p.G;
  a.R = p.R; a.R_pad = p.R_pad; a.TC = p.TC; a.n_chunks = p.n_chunks;
  a.TC2 = p.TC; a.n_chunks2 = p.n_chunks;
  a.causal = causal ? 1 : 0;
  a.c = (float)((scale > 0.f ? (double)scale : 1.0 / sqrt((double)d)) * LOG2E_D);

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == KV_BF16) {
    if (d == 128) launch_score_nw<__bf16, 128>(a, p.NW, st);
    else launch_score_nw<__bf16, 64>(a, p.NW, st);
  } else {
    if (d == 128) launch_score_nw<float, 128>(a, p.NW, st);
    else launch_score_nw<float, 64>(a, p.NW, st);
  }
  return launch_status();
}

extern "C" int kv_score_from_lse(const void* q_win, const void* k, const int32_t* ctx_len,
                                 const float* row_lse_in, float* scores,
                                 int B, int Hq, int Hkv, int N_max, int W, int d, int dtype,
                                 int causal, float scale, void* stream) {
  if (!q_win || !k || !scores || !row_lse_in) return KV_ERR_NULL;
  if (!aligned16(q_win) || !aligned16(k) || !aligned16(scores) || !aligned16(ctx_len) ||
      !aligned16(row_lse_in))
    return KV_ERR_ALIGN;
  if (dtype != KV_F32 && dtype != KV_BF16) return KV_ERR_DTYPE;
  ScorePlan p;
  if (!plan_score(B, Hq, Hkv, N_max, W, d, &p)) return KV_ERR_SHAPE;

  ScoreArgs a;
  a.q = q_win; a.k = k; a.ctx = ctx_len; a.scores = scores; a.row_lse = nullptr;
  a.lse_in = row_lse_in; a.part = nullptr; a.lse2 = nullptr; a.tab = nullptr;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N_max = N_max; a.W = W; a.G = p.G;
  a.R = p.R; a.R_pad = p.R_pad; a.TC = p.TC; a.n_chunks = p.n_chunks;
  a.TC2 = p.TC; a.n_chunks2 = p.n_chunks;
  a.causal = causal ? 1 : 0;
  a.c = (float)((scale > 0.f ? (double)scale : 1.0 / sqrt((double)d)) * LOG2E_D);

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == KV_BF16) {
    if (d == 128) launch_score_nw<__bf16, 128>(a, p.NW, st);
    else launch_score_nw<__bf16, 64>(a, p.NW, st);
  } else {
    if (d == 128) launch_score_nw<float, 128>(a, p.NW, st);
    else launch_score_nw<float, 64>(a, p.NW, st);
  }
  return launch_status();
}
