// Ordered stream compaction of the kept K/V rows into one packed cache.
//
// The edited cache keeps the plain row layout an ordinary attention kernel
// reads ("KV Cache Transform Coding for Compact Storage in LLM Inference",
// section 3; "KVzap: Fast, Adaptive, and Faithful KV Cache Pruning",
// section 1): heads are packed (sequence, KV head) row-major, each head's
// rows in ascending original position, with the position kept beside it.
//
// Every workgroup scans the per-head counts into int64 offsets in LDS, then
// walks the flat space of output rows grid-stride; a row finds its head by
// binary search over the offsets.  A group of d*sizeof(T)/16 lanes copies
// one row with 16-byte loads and stores, so a wave moves whole rows and the
// copy is bit-exact.  Output rows at or past the capacity are skipped; a
// kept index outside [0, N_max) packs a zero K/V row (its pos holds the index).
#include "common.hpp"

namespace kvcc {
namespace {

constexpr int CT = 256;
constexpr int MAX_HEADS = 4096;
constexpr int RU = 4;   // rows in flight per thread

struct CompactArgs {
  const char* k;
  const char* v;
  int B, Hkv, N_max, rowb;
  const int32_t* idx;
  const int32_t* cnt;
  char* kc;
  char* vc;
  int32_t* pos;
  int64_t* offsets;
  int64_t cap;
};

// Exclusive scan of the B*Hkv counts into off[0..H] (LDS), block-wide.
__device__ void scan_counts(const int32_t* cnt, int H, long long* off, long long* wtot) {
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  constexpr int NWV = CT / WAVE;
  long long carry = 0;
  for (int base = 0; base < H; base += CT) {
    const int i = base + tid;
    const long long c = i < H ? (long long)max(cnt[i], 0) : 0ll;
    const long long inc = wave_incl_scan<long long>(c);
    if (lane == WAVE - 1) wtot[wave] = inc;
    __syncthreads();
    long long before = 0, chunk = 0;
    for (int w = 0; w < NWV; ++w) {
      if (w < wave) before += wtot[w];
      chunk += wtot[w];
    }
    if (i < H) off[i] = carry + before + inc - c;
    carry += chunk;
    __syncthreads();
  }
  if (tid == 0) off[H] = carry;
  __syncthreads();
}

__device__ __forceinline__ int find_head(const long long* off, int H, long long row) {
  int lo = 0, hi = H - 1;   // largest i with off[i] <= row (row < off[H])
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(CT) void compact_kernel(CompactArgs a) {
  extern __shared__ long long off[];   // [B*Hkv + 1]
  __shared__ long long wtot[CT / WAVE];
  const int H = a.B * a.Hkv;
  const int tid = threadIdx.x;
  scan_counts(a.cnt, H, off, wtot);
  if (blockIdx.x == 0)
    for (int i = tid; i <= H; i += CT) a.offsets[i] = off[i];
  const long long total = min(off[H], (long long)a.cap);

  const int lpr = a.rowb / 16;            // lanes per row
  const int sub = tid % lpr, rloc = tid / lpr, rpi = CT / lpr;
  const long long step = (long long)gridDim.x * rpi * RU;
  for (long long r0 = (long long)blockIdx.x * rpi * RU + rloc; r0 < total; r0 += step) {
    uint4 kb[RU], vb[RU];
    int tt[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const long long row = r0 + (long long)u * rpi;
      tt[u] = -1;
      if (row < total) {
        const int head = find_head(off, H, row);
        const long long r = row - off[head];
        const int t = r < a.N_max ? a.idx[(size_t)head * a.N_max + r] : -1;
        kb[u] = make_uint4(0, 0, 0, 0);   // an index outside [0, N_max): zero row
        vb[u] = make_uint4(0, 0, 0, 0);
        if ((unsigned)t < (unsigned)a.N_max) {
          const size_t src = ((size_t)head * a.N_max + t) * a.rowb + sub * 16;
          kb[u] = ld16(a.k + src);
          vb[u] = ld16(a.v + src);
        }
        tt[u] = t;
      }
    }
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const long long row = r0 + (long long)u * rpi;
      if (row < total) {
        const size_t dst = (size_t)row * a.rowb + sub * 16;
        st16(a.kc + dst, kb[u]);
        st16(a.vc + dst, vb[u]);
        if (sub == 0) a.pos[row] = tt[u];
      }
    }
  }
}

}  // namespace
}  // namespace kvcc

using namespace kvcc;

extern "C" int kv_compact(const void* k, const void* v, int B, int Hkv, int N_max, int d,
                          int dtype, const int32_t* kept_idx, const int32_t* kept_count,
                          void* k_c, void* v_c, int32_t* pos, int64_t* offsets,
                          int64_t capacity_rows, void* stream) {
  if (!k || !v || !kept_idx || !kept_count || !offsets) return KV_ERR_NULL;
  if (capacity_rows > 0 && (!k_c || !v_c || !pos)) return KV_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(kept_idx) || !aligned16(kept_count) ||
      !aligned16(k_c) || !aligned16(v_c) || !aligned16(pos) || !aligned16(offsets))
    return KV_ERR_ALIGN;
  if (dtype != KV_F32 && dtype != KV_BF16) return KV_ERR_DTYPE;
  if (B < 1 || Hkv < 1 || N_max < 1 || (d != 64 && d != 128) || capacity_rows < 0 ||
      (int64_t)B * Hkv > MAX_HEADS || (int64_t)B * Hkv * N_max >= (int64_t(1) << 31))
    return KV_ERR_SHAPE;

  CompactArgs a;
  a.k = static_cast<const char*>(k); a.v = static_cast<const char*>(v);
  a.B = B; a.Hkv = Hkv; a.N_max = N_max;
  a.rowb = d * (dtype == KV_BF16 ? 2 : 4);
  a.idx = kept_idx; a.cnt = kept_count;
  a.kc = static_cast<char*>(k_c); a.vc = static_cast<char*>(v_c);
  a.pos = pos; a.offsets = offsets; a.cap = capacity_rows;

  const int64_t rows_ub = std::min<int64_t>(capacity_rows, (int64_t)B * Hkv * N_max);
  const int rpi = CT / (a.rowb / 16);
  int64_t grid = ceil_div64(rows_ub, (int64_t)rpi * RU);
  grid = std::max<int64_t>(1, std::min<int64_t>(grid, 2048));
  const size_t dyn = ((size_t)B * Hkv + 1) * sizeof(long long);
  hipStream_t st = static_cast<hipStream_t>(stream);
  launch("compact", compact_kernel, dim3((unsigned)grid), dim3(CT), (uint32_t)dyn, st, a);
  return launch_status();
}
