/*
 * kvcc.h - C ABI of the MI355X (gfx950) KV-cache scoring / selection /
 * compaction / decode library (libkvcc.so).
 *
 * The four calls are the steps of importance-based eviction as the pages
 * describe it: score every cached token, keep a budgeted subset per KV head,
 * and leave a plain dense cache that an ordinary attention kernel reads.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *   never allocates, frees or retains a pointer beyond the call.  Scratch
 *   memory comes only from the caller's `workspace`, sized by the matching
 *   *_workspace_size() function (a pure host function).  Calls that share
 *   one workspace must not overlap in time (e.g. on two streams).
 * - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *   enqueue work on it and never synchronise; buffers must stay alive until
 *   the stream has passed the call.
 * - Host-side validation runs before any launch.  On failure the call returns
 *   a non-zero kv_status and launches nothing.  A launch failure returns
 *   KV_ERR_LAUNCH.  Faults during execution surface at the caller's next
 *   synchronisation.
 * - Tensor pointers must be 16-byte aligned.  Head dimension d is 64 or 128.
 *   dtype is KV_F32 (fp32) or KV_BF16 (bfloat16) and applies to every
 *   q / k / v / k_c / v_c tensor of the call; scores, outputs and statistics
 *   are fp32.
 * - Query head j belongs to KV head j / G with G = Hq / Hkv (contiguous
 *   groups); Hq must be a multiple of Hkv.
 * - ctx_len (device int32 [B]) gives each sequence's length n_b
 *   (0 <= n_b <= N_max); NULL means n_b = N_max for all b.  Rows t >= n_b
 *   are never read and never selected.
 * - Results are deterministic bit for bit for fixed inputs and sizes.
 */
#ifndef KVCC_H
#define KVCC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kv_status {
  KV_OK = 0,
  KV_ERR_NULL = 1,       /* a required pointer is NULL */
  KV_ERR_ALIGN = 2,      /* a tensor pointer is not 16-byte aligned */
  KV_ERR_SHAPE = 3,      /* a size is out of range or inconsistent */
  KV_ERR_DTYPE = 4,      /* dtype is not KV_F32 / KV_BF16 */
  KV_ERR_MODE = 5,       /* unknown budget mode or out-of-range budget value */
  KV_ERR_WORKSPACE = 6,  /* workspace missing or smaller than required */
  KV_ERR_LAUNCH = 7      /* the HIP runtime rejected a kernel launch */
} kv_status;

typedef enum kv_dtype { KV_F32 = 0, KV_BF16 = 1 } kv_dtype;

typedef enum kv_budget_mode {
  KV_BUDGET_K = 0,          /* keep k tokens per head */
  KV_BUDGET_RATIO = 1,      /* keep a fraction r of each head's n tokens */
  KV_BUDGET_THRESHOLD = 2,  /* keep tokens whose score is >= tau */
  KV_BUDGET_MASS = 3        /* keep the fewest top tokens holding a fraction f of the score mass */
} kv_budget_mode;

/*
 * Per-head budget (host struct; the arrays it points to are device memory).
 *   mode == KV_BUDGET_K:     k_h = clamp(k ? k[head] : k_scalar, 1, n)
 *   mode == KV_BUDGET_RATIO: k_h = clamp(floor(r*n + 1/2), 1, n) with
 *                            r = ratio ? ratio[head] : ratio_scalar, evaluated
 *                            in double from the fp32 value.
 *   mode == KV_BUDGET_THRESHOLD: k_h = #{t : s_t >= tau} (fp32 compare),
 *                            clamped to [lo, hi].
 *   mode == KV_BUDGET_MASS:  k_h = min{k >= 1 : C(k) >= mass * C(n)}, C(k) the
 *                            sum of the k largest scores, clamped to [lo, hi].
 *   lo = max(1, floor(min_ratio*n + 1/2)), hi = min(n, max(1, floor(max_ratio*n + 1/2))).
 * A head with n = 0 keeps nothing.  `head` is b*Hkv + h.
 * Protected tokens: the first n_sink and the last n_recent tokens of every
 * head (P, |P| = min(n, n_sink + n_recent) after clamping each to [0, n])
 * come first in the order, ahead of every other token, and are always kept:
 * the threshold count is #{t in P or s_t >= tau}, C(k) sums the real scores
 * of P first, and k_h = min(n, max(k_h, |P|)) after the mode's clamps.  The
 * recent window follows KVzap's sliding window (same section 2.3); sinks and
 * window are the tokens "KV Cache Transform Coding for Compact Storage in LLM
 * Inference", section 3, leaves uncompressed.  0 / 0 protects nothing.
 * Threshold pruning with a fixed tau follows "KVzap: Fast, Adaptive, and
 * Faithful KV Cache Pruning", section 2.3; per-head budgets (any allocation
 * across heads) follow "KVSculpt: KV Cache Compression as Distillation",
 * section 2.D.
 */
typedef struct kv_budget {
  int32_t mode;
  const int32_t* k;        /* device [B*Hkv] or NULL */
  const float* ratio;      /* device [B*Hkv] or NULL */
  int32_t k_scalar;
  float ratio_scalar;      /* 0 <= r <= 1 */
  float tau;
  float mass;              /* 0 <= f <= 1 */
  float min_ratio;         /* 0 <= min_ratio <= 1 */
  float max_ratio;         /* 0 <= max_ratio <= 1 */
  int32_t n_sink;          /* >= 0: first tokens always kept */
  int32_t n_recent;        /* >= 0: last tokens always kept */
} kv_budget;

/* ----------------------------------------------------------------------
 * kv_score - observation-window attention score of every cached token.
 *
 * Importance-based eviction scores tokens by the attention they receive
 * ("A Simple Plug-in for Improving Eviction-Based KV Cache Compression",
 * section "Enonce du Probleme", which names SnapKV); the row normaliser is
 * the log-sum-exp ell of "KVSculpt: KV Cache Compression as Distillation",
 * section 2.B.  For KV head h of sequence b and window row r = (query head
 * j in h's group, window position w):
 *   l[r,t]   = scale * <q_win[b,j,w,:], k[b,h,t,:]>        for t < n_b
 *   lse[r]   = log sum_t exp(l[r,t])
 *   s[b,h,t] = sum_r exp(l[r,t] - lse[r])     (so sum_t s[b,h,t] = W*G)
 * With causal != 0, window row w sits at position n_b - W + w and does not
 * see tokens after it (requires W <= n_b; a row that sees nothing adds 0).
 *
 * q_win   [B][Hq][W][d] dtype, window queries (already position-encoded)
 * k       [B][Hkv][N_max][d] dtype
 * ctx_len [B] int32 or NULL
 * scores  [B][Hkv][N_max] fp32 out; entries t >= n_b are not written
 * row_lse [B][Hq][W] fp32 out (natural log) or NULL
 * scale   softmax scale; <= 0 selects 1/sqrt(d)
 * Limits: 1 <= W <= N_max, G*W <= 1024, B*Hkv*N_max < 2^31.
 * ---------------------------------------------------------------------- */
size_t kv_score_workspace_size(int B, int Hq, int Hkv, int N_max, int W, int d);
int kv_score(const void* q_win, const void* k, const int32_t* ctx_len,
             float* scores, float* row_lse,
             int B, int Hq, int Hkv, int N_max, int W, int d, int dtype,
             int causal, float scale,
             void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * kv_score_from_lse - the same scores in one sweep over K, given the row
 * log-sum-exps.
 *
 * Pruning runs after the attention op ("KVzap: Fast, Adaptive, and Faithful
 * KV Cache Pruning", section 2.3), and a prefill attention pass already
 * yields each window row's log-sum-exp ell ("KVSculpt: KV Cache Compression
 * as Distillation", section 2.B).  Given it, the first sweep of kv_score is
 * skipped:
 *   s[b,h,t] = sum_r exp(l[r,t] - row_lse_in[r])
 * with l, r, the GQA group and the causal rule as in kv_score.  The scores
 * are the normalised ones only if row_lse_in is the LSE over the same keys
 * (same ctx_len, scale and causal flag); the call trusts it.  A row whose
 * row_lse_in is +inf adds nothing; -inf and NaN are outside the contract.
 *
 * row_lse_in [B][Hq][W] fp32 (natural log), device memory, read only
 * other arguments as kv_score; no workspace.
 * ---------------------------------------------------------------------- */
int kv_score_from_lse(const void* q_win, const void* k, const int32_t* ctx_len,
                      const float* row_lse_in, float* scores,
                      int B, int Hq, int Hkv, int N_max, int W, int d, int dtype,
                      int causal, float scale, void* stream);

/* ----------------------------------------------------------------------
 * kv_select - per-head budgeted top-k over the scores.
 *
 * Keeps, per KV head, the k_h first tokens of the order "protected tokens
 * first, then higher score first, equal scores by lower token index" (-0.0
 * equals +0.0; NaN and +inf scores are outside the contract), k_h and the
 * protected tokens given by `budget`.  Low scorers are
 * evicted as in importance-based eviction ("A Simple Plug-in for Improving
 * Eviction-Based KV Cache Compression", section "Enonce du Probleme").
 *
 * scores     [B][Hkv][N_max] fp32 (entries t >= n_b are ignored)
 * budget     host pointer, see kv_budget
 * kept_idx   [B][Hkv][N_max] int32 out: the first kept_count[head] entries
 *            of each head are its kept token indices in ascending order; the
 *            rest are not written
 * kept_count [B*Hkv] int32 out
 * workspace  kv_select_workspace_size() bytes: 0 (NULL allowed) for
 *            N_max <= 32768.  Above, heads under a count budget (k, ratio,
 *            threshold) are split over several workgroups that exchange radix
 *            histograms through it; given less, every head takes one
 *            workgroup (same result, slower).
 * ---------------------------------------------------------------------- */
size_t kv_select_workspace_size(int B, int Hkv, int N_max);
int kv_select(const float* scores, const int32_t* ctx_len,
              int B, int Hkv, int N_max, const kv_budget* budget,
              int32_t* kept_idx, int32_t* kept_count,
              void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * kv_score_select - kv_score followed by kv_select in one call.
 *
 * The same scores (and row LSEs) as kv_score and the same kept indices and
 * counts as kv_select on them, bit for bit: the score of every cached token
 * ("KVSculpt: KV Cache Compression as Distillation", section 2.B; the
 * attention-based importance of "A Simple Plug-in for Improving
 * Eviction-Based KV Cache Compression", section "Enonce du Probleme"), then
 * the budgeted per-head selection that evicts the low scorers.  Under a k or
 * kept-fraction budget with no protected tokens the second score sweep also
 * counts each head's scores by their top 11 key bits, so the selection
 * starts from that histogram: for N_max <= 32768 one workgroup per head
 * resolves the lower key bits from the scores it holds in registers; longer
 * heads skip the first of the part path's launches.  The scores of finite
 * inputs are sums of exponentials (never negative), on which both orders
 * agree; NaN inputs are outside the contract, as for kv_select.
 *
 * Arguments as kv_score (q_win ... scale) and kv_select (budget, kept_idx,
 * kept_count); workspace: kv_score_select_workspace_size() bytes (one
 * buffer for both steps).
 * ---------------------------------------------------------------------- */
size_t kv_score_select_workspace_size(int B, int Hq, int Hkv, int N_max, int W, int d);
int kv_score_select(const void* q_win, const void* k, const int32_t* ctx_len,
                    const kv_budget* budget, float* scores, float* row_lse,
                    int32_t* kept_idx, int32_t* kept_count,
                    int B, int Hq, int Hkv, int N_max, int W, int d, int dtype,
                    int causal, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * kv_compact - gather the kept rows into one packed, ordered cache.
 *
 * The result keeps the plain K/V row layout so an ordinary attention kernel
 * reads it ("KV Cache Transform Coding for Compact Storage in LLM
 * Inference", section 3; "KVzap: Fast, Adaptive, and Faithful KV Cache
 * Pruning", section 1).  Heads are packed (b, h) row-major:
 *   offsets[0] = 0, offsets[i+1] = offsets[i] + kept_count[i]
 *   k_c[offsets[i] + r] = k[b,h,kept_idx[b,h,r]]   (bit-exact), same for v_c
 *   pos[offsets[i] + r] = kept_idx[b,h,r]          (original token index)
 *
 * k, v          [B][Hkv][N_max][d] dtype
 * kept_idx, kept_count as produced by kv_select.  A kept index outside
 *               [0, N_max) (or a count above N_max) packs a zero K row and
 *               a zero V row; its pos entry holds the index as given (-1
 *               past N_max entries).
 * k_c, v_c      [capacity_rows][d] dtype out
 * pos           [capacity_rows] int32 out
 * offsets       [B*Hkv + 1] int64 out; always the true prefix sums
 * capacity_rows rows available in k_c / v_c / pos.  Rows at or beyond it are
 *               not written; the caller detects truncation after
 *               synchronising as offsets[B*Hkv] > capacity_rows.
 * Limits: B*Hkv <= 4096.
 * ---------------------------------------------------------------------- */
int kv_compact(const void* k, const void* v, int B, int Hkv, int N_max, int d, int dtype,
               const int32_t* kept_idx, const int32_t* kept_count,
               void* k_c, void* v_c, int32_t* pos, int64_t* offsets,
               int64_t capacity_rows, void* stream);

/* ----------------------------------------------------------------------
 * kv_decode_attn - one decode query per query head over the packed cache.
 *
 * Decode reads the compacted cache as ordinary softmax attention; it is
 * bandwidth-bound ("KVzap: Fast, Adaptive, and Faithful KV Cache Pruning",
 * section 4).  For query head j of KV head h (rows o..o+k-1 of head
 * b*Hkv+h, clipped to capacity_rows):
 *   u_i = scale * <q[b,j,:], k_c[o+i,:]>
 *   out[b,j,:] = sum_i softmax(u)_i v_c[o+i,:],  lse[b,j] = log sum_i exp(u_i)
 * A head with no rows gives out = 0 and lse = -inf.
 *
 * q             [B][Hq][d] dtype
 * k_c, v_c      [capacity_rows][d] dtype;  offsets [B*Hkv+1] int64
 * out           [B][Hq][d] fp32 out;  lse [B][Hq] fp32 out (natural log) or NULL
 * scale         <= 0 selects 1/sqrt(d)
 * workspace     kv_decode_workspace_size() bytes
 * Limits: B*Hkv <= 4096, capacity_rows < 2^31.
 * ---------------------------------------------------------------------- */
size_t kv_decode_workspace_size(int B, int Hq, int Hkv, int d, int64_t capacity_rows);
int kv_decode_attn(const void* q, const void* k_c, const void* v_c, const int64_t* offsets,
                   int B, int Hq, int Hkv, int d, int dtype, float scale,
                   int64_t capacity_rows, float* out, float* lse,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * kv_decode_attn_noalloc - kv_decode_attn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument and no
 * allocation of any kind; the split partials go to a scratch array the
 * library holds per GPU (16 MiB, kept until the process ends).
 *
 * Arguments, results and errors as kv_decode_attn.  KV_ERR_WORKSPACE: the
 * call needs more than the scratch holds, i.e.
 * kv_decode_workspace_size(B, Hq, Hkv, d, capacity_rows) > 16 MiB (about
 * 2 million capacity rows at B*Hkv = 128, G = 4, d = 128).  KV_ERR_LAUNCH:
 * the scratch address could not be looked up on the current device.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (nothing in it needs clearing): calls that overlap in
 * time on one GPU (e.g. on two streams) race and give wrong results.
 * ---------------------------------------------------------------------- */
int kv_decode_attn_noalloc(const void* q, const void* k_c, const void* v_c,
                           const int64_t* offsets, int B, int Hq, int Hkv, int d, int dtype,
                           float scale, int64_t capacity_rows, float* out, float* lse,
                           void* stream);

/* ----------------------------------------------------------------------
 * kv_compact_decode - kv_compact and kv_decode_attn in one pass over the
 * kept rows.
 *
 * Decode over the packed cache is bandwidth-bound ("KVzap: Fast, Adaptive,
 * and Faithful KV Cache Pruning", section 4), and the compaction has just
 * moved the same rows, so the split kernel gathers each kept row from k / v
 * through kept_idx, writes it to k_c / v_c (and its token to pos) and feeds
 * it to the attention in the same visit.  Outputs equal kv_compact followed
 * by kv_decode_attn over k_c / v_c with capacity_rows (bit for bit): the same
 * packed cache, offsets, pos, out and lse, also for a kept index outside
 * [0, N_max), which packs a zero K/V row (as kv_compact) that the attention
 * reads like any other row.
 *
 * Arguments as in kv_compact (k, v, kept_idx, kept_count, k_c, v_c, pos,
 * offsets, capacity_rows) and kv_decode_attn (q [B][Hq][d] dtype, scale,
 * out, lse); workspace: kv_decode_workspace_size(B, Hq, Hkv, d,
 * capacity_rows) bytes.  Limits: B*Hkv <= 4096.
 * ---------------------------------------------------------------------- */
int kv_compact_decode(const void* k, const void* v, const int32_t* kept_idx,
                      const int32_t* kept_count, int B, int Hq, int Hkv, int N_max,
                      int d, int dtype, int64_t capacity_rows, const void* q,
                      float scale, void* k_c, void* v_c, int32_t* pos,
                      int64_t* offsets, float* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * VECTOR three-way routing: retain, approximate or evict.
 *
 * "A Simple Plug-in for Improving Eviction-Based KV Cache Compression"
 * (VECTOR), section "Methodologie: VECTOR": for a removed fraction p_c and
 * an approximated fraction p_a, the scores pick an enlarged pool of
 *   k_pool = clamp(floor((1 - p_c + p_a) n + 1/2), 1, n)
 * tokens per head (first k_pool of the kv_select order); each pool token t
 * gets eps_t = ||V_t - W_h RoPE^-1(K_t)||^2, with W_h an offline linear map
 * (out = W_h in) and RoPE^-1 turning each adjacent pair (2i, 2i+1) back by
 * t * rope_base^(-2i/d) (rope_base 0: no rotation); the
 *   k_apx = min(k_pool, floor(2 p_a n + 1/2))
 * pool tokens of lowest eps (ties: lower token index) keep their key but
 * drop their value, rebuilt as W_h RoPE^-1(K_t) when decode reads it; the
 * other pool tokens keep K and V.  Count arithmetic is float64 on the fp32
 * fractions.
 * ---------------------------------------------------------------------- */

/* kv_vector_route: pool, residuals and the approximated subset.
 * scores, ctx_len   as kv_select; k, v [B][Hkv][N_max][d] dtype;
 * w                 [Hkv][d][d] fp32 device, row-major (out index first)
 * pool_idx, pool_count  out, as kv_select's kept_idx / kept_count
 * neg_eps           [B][Hkv][N_max] fp32 out: -eps of pool entry j at j,
 *                   -inf for j >= pool_count
 * apx_pos, apx_count    out: per head the ascending pool-entry positions j
 *                   (indices into that head's pool list) whose value is
 *                   dropped, and how many (may be 0)
 * workspace         kv_vector_route_workspace_size(B, Hkv) bytes
 * Errors: KV_ERR_MODE if p_c, p_a are outside [0, 1] or rope_base < 0. */
size_t kv_vector_route_workspace_size(int B, int Hkv);
int kv_vector_route(const float* scores, const int32_t* ctx_len, const void* k, const void* v,
                    const float* w, int B, int Hkv, int N_max, int d, int dtype, float p_c,
                    float p_a, float rope_base, int32_t* pool_idx, int32_t* pool_count,
                    float* neg_eps, int32_t* apx_pos, int32_t* apx_count, void* workspace,
                    size_t workspace_bytes, void* stream);

/* kv_vector_compact: the routed cache.  Key rows for every pool token, packed
 * (b, h) row-major as kv_compact (offsets, pos, k_c), value rows only for
 * the tokens that keep them, packed the same way (voffsets, v_c), and
 *   vmap[r] = the v_c row of key row r, or -1 when its value is rebuilt.
 * Key rows past capacity_rows and value rows past v_capacity_rows are not
 * written; offsets and voffsets always hold the true prefix sums, so the
 * caller detects overflow after the stream reaches this point. */
int kv_vector_compact(const void* k, const void* v, int B, int Hkv, int N_max, int d, int dtype,
                      const int32_t* pool_idx, const int32_t* pool_count, const int32_t* apx_pos,
                      const int32_t* apx_count, void* k_c, void* v_c, int32_t* pos,
                      int32_t* vmap, int64_t* offsets, int64_t* voffsets,
                      int64_t capacity_rows, int64_t v_capacity_rows, void* stream);

/* kv_vector_decode: decode attention over the routed cache, as
 * kv_decode_attn with each row's value taken from v_c[vmap[r]] or, for
 * vmap[r] < 0, rebuilt as W_h RoPE^-1(k_c[r]) at position pos[r].  The
 * rebuilt rows enter as W_h (sum_r p_r RoPE^-1(k_c[r])), one d x d product
 * per query head.  A vmap entry at or beyond v_capacity_rows reads as a zero
 * value row.  A head with no rows gives out = 0 and lse = -inf.
 * workspace: kv_vector_decode_workspace_size() bytes. */
size_t kv_vector_decode_workspace_size(int B, int Hq, int Hkv, int d, int64_t capacity_rows);
int kv_vector_decode(const void* q, const void* k_c, const void* v_c, const int32_t* vmap,
                     const int32_t* pos, const int64_t* offsets, const float* w, float rope_base,
                     int B, int Hq, int Hkv, int d, int dtype, float scale,
                     int64_t capacity_rows, int64_t v_capacity_rows, float* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------
 * Measurement hook (not part of the method): per-kernel GPU time.
 *
 * kv_timing_enable(1) clears earlier records and makes every kernel the
 * library launches afterwards carry a start/stop hipEvent pair that its
 * dispatch stamps at kernel start and end, on that launch's own stream;
 * kv_timing_enable(0) stops recording.  kv_timing_read waits for the
 * recorded events and writes up to max_entries per-kernel totals, each
 * with its last launch's shape (host array, caller-owned), returning the
 * number of distinct kernels (or a negative kv_status).  kv_timing_only(name) restricts the
 * recording to launches of that kernel name (one of "score_rowstats",
 * "score_fold" (launched only when row LSEs are requested or heads are so
 * long, and so few, that pass 1 cuts a head into more than 32 pieces),
 * "score_colsum", "select", "compact",
 * "compact_decode", "decode_split",
 * "decode_merge", "vector_counts", "vector_pool", "vector_residual",
 * "vector_apx", "vector_vmap", "vector_copy", "vector_decode_split",
 * "vector_decode_merge"); NULL or "" records every launch.  The name is copied.
 * Timed dispatches run a little slower (about 4 us per timed launch
 * within a step of back-to-back launches), so timing is meant for
 * measurement runs, not production.
 * ---------------------------------------------------------------------- */
typedef struct kv_kernel_time {
  char name[40];
  int64_t launches;
  double total_ms;
  int32_t grid;    /* workgroups of the kernel's last recorded launch */
  int32_t block;   /* threads per workgroup of that launch */
} kv_kernel_time;
int kv_timing_enable(int on);
int kv_timing_only(const char* name);
int kv_timing_read(kv_kernel_time* out, int max_entries);

/* Human-readable name of a kv_status value (static string). */
const char* kv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVCC_H */
