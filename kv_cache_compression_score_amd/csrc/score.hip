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
// fragments of two 32-row blocks in registers:
//   pass 1: C[token,row] = K * Q^T, so one lane owns one row and 16 tokens
//           per block and keeps a running (max, sum of exp2) per row in
//           registers; the two half-waves and then the token chunks are
//           merged into a base-2 log-sum-exp per row.
//   pass 2: C[row,token] = Q * K^T, so one lane owns one token and 16 rows
//           per block; exp2(l*c - lse2[row]) is summed in-lane, then over
//           half-waves and waves through LDS in a fixed order.
// All logits are kept in base-2 units: c = scale*log2(e) is applied to the
// fp32 dot product after the MFMA (bf16 inputs are never rescaled).
#include <math.h>

#include "common.hpp"

namespace kvcc {
namespace {

constexpr int TOK = 64;          // tokens per LDS tile
constexpr int TSUB = TOK / 32;   // 32-token MFMA blocks per tile
constexpr int RBW = 2;           // 32-row blocks per wave

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

struct ScoreArgs {
  const void* q;
  const void* k;
  const int32_t* ctx;
  float* scores;
  float2* part;     // [B*Hkv][n_chunks][R_pad] running (max, sum) per row, base 2
  float* lse2;      // [B*Hkv][R_pad] base-2 row log-sum-exp (+inf: row adds nothing)
  float* row_lse;   // [B][Hq][W] natural log, optional
  int B, Hq, Hkv, N_max, W, G, R, R_pad, TC, n_chunks, causal;
  float c;          // scale * log2(e)
};

template <typename T, int D, int NW, int PASS>
__global__ __launch_bounds__(NW * WAVE) void score_pass(ScoreArgs a) {
  using V = typename FragT<T>::vec;
  constexpr int KS = D / 16;
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int LDS_STRIDE = ROWB + 16;          // pad rows against bank conflicts
  constexpr int VPR = ROWB / 16;
  constexpr int TILE_VECS = TOK * VPR;
  constexpr int NT = NW * WAVE;
  constexpr int LPT = (TILE_VECS + NT - 1) / NT;
  constexpr int NRED = PASS == 2 ? 2 * NW : 1;

  __shared__ __attribute__((aligned(16))) unsigned char ktile[2][TOK * LDS_STRIDE];
  __shared__ float red[2][NRED][TOK];

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int hf = lane >> 5, l32 = lane & 31;
  const int n = a.ctx ? min(max(a.ctx[b], 0), a.N_max) : a.N_max;
  const int head = b * a.Hkv + h;
  const int t0 = c * a.TC;

  if (t0 >= n) {
    if (PASS == 1) {
      float2* dst = a.part + ((size_t)head * a.n_chunks + c) * a.R_pad;
      for (int r = tid; r < a.R_pad; r += NT) dst[r] = make_float2(-INFINITY, 0.f);
    }
    return;
  }
  const int t1 = min(t0 + a.TC, n);
  const int ntiles = (t1 - t0 + TOK - 1) / TOK;
  const char* kh = static_cast<const char*>(a.k) + (size_t)head * a.N_max * ROWB;
  const int last_w0 = n - a.W;   // position of window row 0; row w sits at last_w0 + w

  // Q fragments of this wave's row blocks (zero for padding rows).
  V qf[RBW][KS];
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int r = (wave * RBW + i) * 32 + l32;
    if (r < a.R) {
      const int j = h * a.G + r / a.W, w = r % a.W;
      const char* qp = static_cast<const char*>(a.q) +
                       ((((size_t)b * a.Hq + j) * a.W + w) * D + 8 * hf) * sizeof(T);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[i][ks] = load_frag<T>(qp + ks * 16 * sizeof(T));
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[i][ks] = V{};
    }
  }

  // Pass-1 running state (per row owned by the lane) / pass-2 row lse2.
  float m_run[RBW], s_run[RBW];
  float l2[RBW][16];
  if (PASS == 1) {
#pragma unroll
    for (int i = 0; i < RBW; ++i) { m_run[i] = -INFINITY; s_run[i] = 0.f; }
  } else {
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = (wave * RBW + i) * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
        l2[i][e] = r < a.R ? a.lse2[(size_t)head * a.R_pad + r] : INFINITY;
      }
    }
  }

  uint4 pre[LPT];
  auto gload = [&](int tile) {
    const int tt0 = t0 + tile * TOK;
    const int rows = min(TOK, t1 - tt0);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int v = tid + i * NT;
      const int row = v / VPR, col = v % VPR;
      if (v < TILE_VECS && row < rows)
        pre[i] = ld16(kh + (size_t)(tt0 + row) * ROWB + col * 16);
      else
        pre[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int v = tid + i * NT;
      if (v < TILE_VECS) {
        const int row = v / VPR, col = v % VPR;
        *reinterpret_cast<uint4*>(&ktile[buf][row * LDS_STRIDE + col * 16]) = pre[i];
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    const int tt0 = t0 + tile * TOK;
    if (tile + 1 < ntiles) gload(tile + 1);

#pragma unroll
    for (int sub = 0; sub < TSUB; ++sub) {
      const int ts = tt0 + sub * 32;   // first token of this 32-token block
      f32x16 acc[RBW];
#pragma unroll
      for (int i = 0; i < RBW; ++i) acc[i] = f32x16{};
      const unsigned char* krow = &ktile[buf][(sub * 32 + l32) * LDS_STRIDE + 8 * hf * sizeof(T)];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const V kf = load_frag<T>(krow + ks * 16 * sizeof(T));
#pragma unroll
        for (int i = 0; i < RBW; ++i)
          acc[i] = PASS == 1 ? mma(kf, qf[i][ks], acc[i]) : mma(qf[i][ks], kf, acc[i]);
      }

      const bool clean = (ts + 32 <= t1) && (!a.causal || ts + 31 <= last_w0);
      if (PASS == 1) {
        // acc[i][e] = dot(row (wave*RBW+i)*32 + l32, token ts + 8*(e/4) + 4*hf + e%4)
#pragma unroll
        for (int i = 0; i < RBW; ++i) {
          const int r = (wave * RBW + i) * 32 + l32;
          float v[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) v[e] = acc[i][e];
          if (!clean) {
            const int p = a.causal ? last_w0 + (r % a.W) : 0x7fffffff;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int t = ts + 8 * (e >> 2) + 4 * hf + (e & 3);
              if (t >= t1 || t > p) v[e] = -INFINITY;
            }
          }
          float vmax = v[0];
#pragma unroll
          for (int e = 1; e < 16; ++e) vmax = fmaxf(vmax, v[e]);
          const float mn = fmaxf(m_run[i], vmax * a.c);
          if (mn != -INFINITY) {
            float sum = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) sum += fast_exp2(fmaf(v[e], a.c, -mn));
            s_run[i] = s_run[i] * fast_exp2(m_run[i] - mn) + sum;
            m_run[i] = mn;
          }
        }
      } else {
        // acc[i][e] = dot(row (wave*RBW+i)*32 + 8*(e/4) + 4*hf + e%4, token ts + l32)
        float col = 0.f;
        if (!a.causal || ts + 31 <= last_w0) {
#pragma unroll
          for (int i = 0; i < RBW; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) col += fast_exp2(fmaf(acc[i][e], a.c, -l2[i][e]));
        } else {
          const int t = ts + l32;
#pragma unroll
          for (int i = 0; i < RBW; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int r = (wave * RBW + i) * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
              const float x = fast_exp2(fmaf(acc[i][e], a.c, -l2[i][e]));
              if (t <= last_w0 + (r % a.W)) col += x;
            }
        }
        red[buf][wave * 2 + hf][sub * 32 + l32] = col;
      }
    }

    if (tile + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();

    if (PASS == 2 && tid < TOK) {
      const int t = tt0 + tid;
      if (t < t1) {
        float s = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NRED; ++w2) s += red[buf][w2][tid];
        a.scores[(size_t)head * a.N_max + t] = s;
      }
    }
  }

  if (PASS == 1) {
    // Merge the two half-waves (same row, disjoint tokens), then publish.
    float2* dst = a.part + ((size_t)head * a.n_chunks + c) * a.R_pad;
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      const float mo = __shfl_xor(m_run[i], 32, WAVE);
      const float so = __shfl_xor(s_run[i], 32, WAVE);
      const float mn = fmaxf(m_run[i], mo);
      float s = 0.f;
      if (mn != -INFINITY) s = s_run[i] * fast_exp2(m_run[i] - mn) + so * fast_exp2(mo - mn);
      const int r = (wave * RBW + i) * 32 + l32;
      if (hf == 0 && r < a.R_pad) dst[r] = make_float2(mn, s);
    }
  }
}

// Fold the per-chunk (max, sum) of every row, in chunk order, into lse2.
__global__ __launch_bounds__(256) void score_lse(ScoreArgs a) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int total = a.B * a.Hkv * a.R_pad;
  if (idx >= total) return;
  const int head = idx / a.R_pad, r = idx % a.R_pad;
  if (r >= a.R) { a.lse2[idx] = INFINITY; return; }
  float m = -INFINITY, s = 0.f;
  const float2* src = a.part + (size_t)head * a.n_chunks * a.R_pad + r;
  for (int c = 0; c < a.n_chunks; ++c) {
    const float2 p = src[(size_t)c * a.R_pad];
    if (p.x == -INFINITY) continue;
    const float mn = fmaxf(m, p.x);
    s = s * exp2f(m - mn) + p.y * exp2f(p.x - mn);
    m = mn;
  }
  const bool seen = s > 0.f;
  const float l2v = seen ? m + log2f(s) : INFINITY;
  a.lse2[idx] = l2v;
  if (a.row_lse) {
    const int b = head / a.Hkv, h = head % a.Hkv;
    const int j = h * a.G + r / a.W, w = r % a.W;
    a.row_lse[((size_t)b * a.Hq + j) * a.W + w] = seen ? l2v * LN2_F : -INFINITY;
  }
}

struct ScorePlan {
  int G, R, R_pad, NW, TC, n_chunks;
  size_t off_lse, bytes;
};

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
  // Aim at ~2048 workgroups over the whole call; chunks are whole tiles.
  const int64_t total = (int64_t)B * Hkv * N_max;
  int64_t tc = ceil_div64(total, 2048);
  tc = ceil_div64(tc, TOK) * TOK;
  if (tc < 256) tc = 256;
  if (tc > 8192) tc = 8192;
  const int64_t nmax_r = ceil_div64(N_max, TOK) * TOK;
  if (tc > nmax_r) tc = nmax_r;
  p->TC = (int)tc;
  p->n_chunks = ceil_div(N_max, p->TC);
  const size_t part = (size_t)B * Hkv * p->n_chunks * p->R_pad * sizeof(float2);
  p->off_lse = (part + 255) & ~size_t(255);
  p->bytes = p->off_lse + (size_t)B * Hkv * p->R_pad * sizeof(float);
  return true;
}

template <typename T, int D, int NW>
void launch_score(const ScoreArgs& a, hipStream_t st) {
  const dim3 grid(a.n_chunks, a.Hkv, a.B);
  {
    TimedLaunch t("score_rowstats", st);
    score_pass<T, D, NW, 1><<<grid, NW * WAVE, 0, st>>>(a);
  }
  {
    TimedLaunch t("score_lse", st);
    const int rows = a.B * a.Hkv * a.R_pad;
    score_lse<<<ceil_div(rows, 256), 256, 0, st>>>(a);
  }
  {
    TimedLaunch t("score_colsum", st);
    score_pass<T, D, NW, 2><<<grid, NW * WAVE, 0, st>>>(a);
  }
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
  a.part = static_cast<float2*>(workspace);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.off_lse);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N_max = N_max; a.W = W; a.G = p.G;
  a.R = p.R; a.R_pad = p.R_pad; a.TC = p.TC; a.n_chunks = p.n_chunks;
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
