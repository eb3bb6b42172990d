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
// lane, RPG rows in flight), forms the G dot products with a DPP reduction
// inside the group, and keeps a base-2 (max, sum, o) per query
// head.  Groups merge through LDS in a fixed order into one partial per item;
// a second kernel merges each head's items in item order, so the result is
// deterministic.
#include <math.h>

#include "common.hpp"

namespace kvcc {
namespace {

constexpr int DT = 256;
constexpr int CH = 256;          // rows per work item (two passes of NG*RPG rows)
constexpr int RPG = 8;           // rows per lane group per pass over an item
constexpr bool PERSISTENT = false;   // grid = resident workgroups, items walked grid-stride
constexpr int MAX_HEADS = 4096;

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
};

// Row offsets clipped to the capacity, and the first item of every head.
__device__ void build_items(const DecodeArgs& a, long long* off, int* ist, int* wtot) {
  const int H = a.B * a.Hkv;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  constexpr int NWV = DT / WAVE;
  for (int i = tid; i <= H; i += DT) {
    const long long o = a.offsets[i];
    off[i] = o < 0 ? 0 : (o > a.cap ? a.cap : o);
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

template <typename T, int D, int GT, bool VEC>
__global__ __launch_bounds__(DT) void decode_split(DecodeArgs a) {
  constexpr int EPL = 16 / (int)sizeof(T);     // elements per lane
  constexpr int LPR = D / EPL;                 // lanes per row (power of two, <= 32)
  constexpr int NG = DT / LPR;                 // row groups per workgroup
  constexpr int PASS = NG * RPG;               // rows per pass over an item
  constexpr int ROWB = D * (int)sizeof(T);

  __shared__ int wtot[DT / WAVE];
  __shared__ float sm_m[NG][GT], sm_l[NG][GT];
  __shared__ float sm_o[NG][GT][D];
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
  // revolutions per position of this lane's rotary pairs (routed cache only)
  double rope_g[VEC ? EPL / 2 : 1];
  if constexpr (VEC) {
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

    // query slices (this lane's EPL elements) of the GT query heads, in base 2
    float qv[GT][EPL];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const int jg = qsub * GT + g;
      if (jg < a.G) {
        const int j = h * a.G + jg;
        const char* qp = static_cast<const char*>(a.q) +
                         (((size_t)b * a.Hq + j) * D + sub * EPL) * sizeof(T);
        unpack16<T>(ld16(qp), qv[g]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[g][e] *= a.c;
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[g][e] = 0.f;
      }
    }

    float mg[GT], lg[GT], og[GT][EPL];
    float ou[VEC ? GT : 1][EPL];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      mg[g] = -INFINITY;
      lg[g] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) og[g][e] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < (VEC ? GT : 1); ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) ou[g][e] = 0.f;
    for (long long base = r0; base < r1; base += PASS) {
      uint4 kr[RPG], vr[RPG];
      int vm[VEC ? RPG : 1], pp[VEC ? RPG : 1];
#pragma unroll
      for (int u = 0; u < RPG; ++u) {
        const long long row = base + grp + (long long)u * NG;
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
        if constexpr (VEC) { vm[u] = -1; pp[u] = 0; }
        if (row < r1) {
          kr[u] = ld16(a.kc + (size_t)row * ROWB + sub * 16);
          if constexpr (VEC) {
            vm[u] = a.vmap[row];
            pp[u] = a.pos[row];
            if (vm[u] >= 0 && vm[u] < a.vcap) vr[u] = ld16(a.vc + (size_t)vm[u] * ROWB + sub * 16);
          } else {
            vr[u] = ld16(a.vc + (size_t)row * ROWB + sub * 16);
          }
        }
      }
      float sc[RPG][GT];
#pragma unroll
      for (int u = 0; u < RPG; ++u) {
        float kx[EPL];
        unpack16<T>(kr[u], kx);
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) s = fmaf(qv[g][e], kx[e], s);
          sc[u][g] = group_sum<LPR>(s);
        }
      }
      // online merge of this pass into the group's running (max, sum, o)
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float m = mg[g];
#pragma unroll
        for (int u = 0; u < RPG; ++u)
          if (base + grp + (long long)u * NG < r1) m = fmaxf(m, sc[u][g]);
        if (m != -INFINITY && m != mg[g]) {
          const float w = fast_exp2(mg[g] - m);   // 0 when mg was -inf
          lg[g] *= w;
#pragma unroll
          for (int e = 0; e < EPL; ++e) og[g][e] *= w;
          if constexpr (VEC) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) ou[g][e] *= w;
          }
          mg[g] = m;
        }
      }
#pragma unroll
      for (int u = 0; u < RPG; ++u) {
        if (base + grp + (long long)u * NG < r1) {
          float vx[EPL];
          bool rebuilt = false;
          if constexpr (VEC) rebuilt = vm[u] < 0;
          if (rebuilt) {
            // de-rotated key: pairs (2i, 2i+1) of this lane's elements turn back
            unpack16<T>(kr[u], vx);
            if (a.rope_base > 0.f) {
#pragma unroll
              for (int m2 = 0; m2 < EPL / 2; ++m2) {
                double r = (double)pp[u] * rope_g[m2];
                r -= floor(r);
                const float rv = (float)r;
                const float s = __builtin_amdgcn_sinf(rv), c = __builtin_amdgcn_cosf(rv);
                const float x = vx[2 * m2], y = vx[2 * m2 + 1];
                vx[2 * m2] = x * c + y * s;
                vx[2 * m2 + 1] = y * c - x * s;
              }
            }
          } else {
            unpack16<T>(vr[u], vx);
          }
#pragma unroll
          for (int g = 0; g < GT; ++g) {
            const float p = fast_exp2(sc[u][g] - mg[g]);
            lg[g] += p;
            if constexpr (VEC) {
              if (rebuilt) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) ou[g][e] = fmaf(p, vx[e], ou[g][e]);
                continue;
              }
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) og[g][e] = fmaf(p, vx[e], og[g][e]);
          }
        }
      }
    }

    // merge the row groups (fixed order) into this item's partial
    const size_t pbase = ((size_t)qsub * a.items_max + it) * GT;
#pragma unroll
    for (int half = 0; half < (VEC ? 2 : 1); ++half) {
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        if (half == 0 && sub == 0) { sm_m[grp][g] = mg[g]; sm_l[grp][g] = lg[g]; }
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          sm_o[grp][g][sub * EPL + e] = half == 0 ? og[g][e] : ou[VEC ? g : 0][e];
      }
      __syncthreads();
      for (int x = tid; x < GT * D; x += DT) {
        const int g = x / D, e = x % D;
        float M = -INFINITY;
        for (int r = 0; r < NG; ++r) M = fmaxf(M, sm_m[r][g]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
          for (int r = 0; r < NG; ++r) {
            const float w = fast_exp2(sm_m[r][g] - M);
            L = fmaf(sm_l[r][g], w, L);
            O = fmaf(sm_o[r][g][e], w, O);
          }
        }
        (half == 0 ? a.part_o : a.part_u)[(pbase + g) * D + e] = O;
        if (half == 0 && e == 0) a.part_ml[pbase + g] = make_float2(M, L);
      }
      __syncthreads();
    }
  }
}

// Per (head, query sub-group): merge the head's items in item order.  Loads
// are batched so a head's items are fetched a few at a time, not one by one.
// Per (head, query sub-group): merge the head's items in item order, loads
// batched 32 items at a time (the batch maximum first, then the weights).  A routed cache also merges the rebuilt-row
// sums U and adds W U (one d x d product per query head) before dividing.
template <int D, int GT, bool VEC>
__global__ __launch_bounds__(GT * D) void decode_merge(DecodeArgs a) {
  constexpr int U = 32;
  __shared__ float su[VEC ? GT : 1][VEC ? D : 1];
  const int head = blockIdx.x, qsub = blockIdx.y;
  const int b = head / a.Hkv, h = head % a.Hkv;
  const int i0 = a.item_start[head], i1 = a.item_start[head + 1];
  const size_t base = (size_t)qsub * a.items_max;
  const int x = threadIdx.x;
  const int g = x / D, e = x % D, jg = qsub * GT + g;
  const bool live = jg < a.G;
  float M = -INFINITY, L = 0.f, O = 0.f, Uv = 0.f;
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
    if (live) {   // O += (W U)[e]: row e of W_h against this query head's U
      const float4* wr = reinterpret_cast<const float4*>(a.w + ((size_t)h * D + e) * D);
      float acc = 0.f;
#pragma unroll 8
      for (int i = 0; i < D / 4; ++i) {
        const float4 wv = wr[i];
        acc = fmaf(wv.x, su[g][4 * i], acc);
        acc = fmaf(wv.y, su[g][4 * i + 1], acc);
        acc = fmaf(wv.z, su[g][4 * i + 2], acc);
        acc = fmaf(wv.w, su[g][4 * i + 3], acc);
      }
      O += acc;
    }
  }
  if (!live) return;
  const size_t bj = (size_t)b * a.Hq + h * a.G + jg;
  const bool any = L > 0.f;
  a.out[bj * D + e] = any ? O / L : 0.f;
  if (a.lse && e == 0) a.lse[bj] = any ? (M + log2f(L)) * LN2_F : -INFINITY;
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

// Resident workgroups of a kernel on the current device.
template <typename K>
int resident_slots(K kernel, int threads, size_t dyn) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, dyn) != hipSuccess ||
      cus < 1 || per_cu < 1)
    return 8192;
  return cus * per_cu;
}

template <typename T, int D, int GT, bool VEC>
void launch_decode(const DecodeArgs& a, hipStream_t st) {
  const size_t dyn = (size_t)(a.B * a.Hkv + 1) * (sizeof(long long) + sizeof(int));
  const int gx = PERSISTENT ? resident_slots(decode_split<T, D, GT, VEC>, DT, dyn) : 8192;
  const dim3 grid((unsigned)std::min(a.items_max, gx), a.n_sub);
  {
    TimedLaunch t(VEC ? "vector_decode_split" : "decode_split", st);
    decode_split<T, D, GT, VEC><<<grid, DT, dyn, st>>>(a);
  }
  {
    TimedLaunch t(VEC ? "vector_decode_merge" : "decode_merge", st);
    decode_merge<D, GT, VEC><<<dim3(a.B * a.Hkv, a.n_sub), GT * D, 0, st>>>(a);
  }
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

  launch_decode_any<false>(a, dtype, d, p.GT, static_cast<hipStream_t>(stream));
  return launch_status();
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

  launch_decode_any<true>(a, dtype, d, p.GT, static_cast<hipStream_t>(stream));
  return launch_status();
}
