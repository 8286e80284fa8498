/*
 * gqa_decode.h — exact grouped-query decode attention over a KV cache,
 * hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * One decode step appends the new token's K/V rows to each sequence's cache
 * and then lets every query head attend over all cached keys of its KV group:
 *
 *   s_j  = scale * <q[b,h,:], K[b,j,g,:]>          j < n_b,  g = h / (Hq/Hkv)
 *   out  = sum_j exp(s_j - m) V[b,j,g,:] / sum_j exp(s_j - m),  m = max_j s_j
 *
 * (needle-core attn.rs, self_attn_incremental: push_kv then attend over the
 * cache; query head hi reads KV head hi / kv_repeat; each score is the q.k
 * dot product times head_dim^-0.5, and the softmax weights sum the value
 * rows.)
 * The result can also be handed out as a mergeable online-softmax carry
 * (m, l, acc) so that two branches over the same queries — for example a long
 * main cache and a recent window — fold into one (usearch
 * "linear-algebra", section Attention and struct DenseSoftmaxState).
 *
 * Conventions for every entry point:
 *  - Every data pointer is a DEVICE pointer, owned by the caller.  The library
 *    never allocates, frees or synchronises; every call only enqueues kernels
 *    on `stream` (NULL = the default stream) and returns.
 *  - Arguments are checked on the host before anything is enqueued; a failed
 *    check returns an error code and enqueues nothing.  No HIP call is made
 *    before the checks pass.  GQA_ERR_DEVICE reports a failed launch.
 *  - All sizes are element counts unless named *_bytes.
 *  - q, cache->k, cache->v and the workspace must be 16-byte aligned.
 *  - Shapes with a kernel: bf16, fp8 and fp32 caches with (dk, dv) in
 *    {(64, 64), (128, 128), (192, 128), (256, 256)} and 1..16 query heads per
 *    KV head run on the matrix cores (MFMA 16x16x32 bf16, or the exact-fp32
 *    MFMA 16x16x4 for fp32 caches); fp32 caches with other head widths —
 *    multiples of 4 up to 256, 1..16 query heads per KV head and a 64-token
 *    tile that fits 64 KiB of LDS — run on the vector ALUs (every entry point
 *    but gqa_attend_branches, gqa_decode_step_branches and
 *    gqa_attend_gathered, which need a matrix-core shape).
 *  - fp8 caches (GQA_DTYPE_FP8_E4M3): queries and new K/V rows are bf16.
 *  - Errors: GQA_ERR_INVALID_ARGUMENT (a required pointer is NULL, a size is
 *    non-positive, a scale is not finite), GQA_ERR_SHAPE_MISMATCH (the query
 *    heads are not a multiple of the KV heads — usearch requires the head
 *    count to split the rows evenly — or the sizes of two arguments disagree),
 *    GQA_ERR_UNSUPPORTED (no kernel for this dtype / head widths / group
 *    size), GQA_ERR_WORKSPACE_TOO_SMALL, GQA_ERR_DEVICE.
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_ABI_VERSION 5

/* Only the entry points below are exported from the shared library. */
#define GQA_API __attribute__((visibility("default")))

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARGUMENT = 1,
  GQA_ERR_SHAPE_MISMATCH = 2,
  GQA_ERR_UNSUPPORTED = 3,
  GQA_ERR_WORKSPACE_TOO_SMALL = 4,
  GQA_ERR_DEVICE = 5
} gqa_status;

/*
 * Storage type of K and V (and of q and new rows, except for fp8 caches,
 * whose q and new rows are bf16).  Outputs and carries are always fp32.
 *
 * GQA_DTYPE_FP8_E4M3: one byte per element, an OCP 8-bit floating-point
 * E4M3 ("E4M3FN") code: sign, 4 exponent bits (bias 7), 3 mantissa bits,
 * subnormals at exponent 0, NaN at S.1111.111, no infinities, largest
 * finite value 448.  Code c of KV head g of sequence b stands for
 * decode(c) * k_scale[b * num_kv_heads + g] (V: v_scale).  The pages leave
 * the compressed storage format open (usearch "linear-algebra", section
 * Attention: a value row comes back in whatever quantised form the index
 * keeps it; qualiaDB KvDictionary: a compressed-cache read path); this is the
 * library's choice, and attention over such a cache is exact attention over
 * the decoded values.
 */
typedef enum gqa_dtype {
  GQA_DTYPE_F32 = 0,
  GQA_DTYPE_BF16 = 1,
  GQA_DTYPE_FP8_E4M3 = 2
} gqa_dtype;

/*
 * A batch of KV caches (needle-core struct KvCache: keys and values stored
 * [max_len, num_kv_heads, head_dim]; here with a leading batch dimension and
 * separate key and value widths):
 *   k: [batch][max_len][num_kv_heads][dk]   contiguous, `dtype` elements
 *   v: [batch][max_len][num_kv_heads][dv]   contiguous, `dtype` elements
 * The per-sequence fill level lives in a separate device int32 array `lens`.
 * Slots at or past lens[b] are never read by attend.
 * k_scale, v_scale: fp32 [batch][num_kv_heads] device arrays (4-byte
 * aligned, finite and positive) for fp8 caches, required there and ignored
 * (may be NULL) for the other dtypes.
 */
typedef struct gqa_cache {
  void *k;
  void *v;
  int32_t batch;
  int32_t max_len;
  int32_t num_kv_heads;
  int32_t dk;
  int32_t dv;
  int32_t dtype; /* gqa_dtype */
  const float *k_scale;
  const float *v_scale;
} gqa_cache;

/*
 * Online-softmax carry, one row per query row r = b * num_q_heads + h
 * (usearch DenseSoftmaxState, owned by the caller, extended with the
 * accumulator):
 *   m   [rows]      maximum scaled logit so far, natural-log units
 *   l   [rows]      sum of exp(s - m) over the keys seen
 *   acc [rows][dv]  sum of exp(s - m) * v, NOT divided by l
 * A row with l == 0 is empty whatever its m (a zero-initialised carry is the
 * empty state).  Empty rows are written as (-inf, 0, 0).
 */
typedef struct gqa_carry {
  float *m;
  float *l;
  float *acc;
} gqa_carry;

/*
 * Split-K plan of one attend call.  The key axis of every sequence is cut into
 * chunks of `chunk_tokens`; one partial carry per (query row, chunk) goes to
 * the workspace, laid out as three fp32 arrays at 256-byte aligned offsets:
 *   part_m   [rows][num_chunks]       at byte 0
 *   part_l   [rows][num_chunks]       at off_l
 *   part_acc [rows][num_chunks][dv]   at off_acc
 * Only chunks c < ceil(min(lens[b], max_len) / chunk_tokens) are written.
 * A plan with many (sequence, KV group, chunk) items (sched_entries > 0) also
 * holds the work schedule the library computes on the device before each
 * partition launch: sched_entries int32 at off_sched (a block -> item table
 * that gives the GPU's eight XCDs equal shares of the live chunks).
 *
 * Balanced plans (balanced_groups > 0; the library's choice for a bf16 /
 * fp8 cache whose chunked launch would run in several rounds of
 * work-groups, or asked for with GQA_CHUNK_BALANCED, which suits batches of
 * very unequal lengths, since chunks of one length then leave some
 * work-groups far longer than others): a work queue.  Every sequence's
 * 32-token tiles are cut into runs — of 128 tiles over its first 3/4, of 32
 * tiles up to 23/25 of it, of 8 tiles over the rest — listed phase by phase,
 * sequence by sequence; queue item i is run i / num_kv_heads for KV group
 * i % num_kv_heads.  balanced_groups persistent work-groups take items from
 * the queue until it is empty, so the work spreads by the work-groups'
 * actual speed and ends with short items.  Then chunk_tokens = 32,
 * num_chunks = the most items the shape can need (one piece slot each), and
 *   part_m / part_l [num_chunks][hpk], part_acc [num_chunks][hpk][dv]:
 *       item i's partial state (hpk rows), in slot i;
 *   sched_entries int32 at off_sched: the queue (its counter, item count,
 *       phase starts, per-sequence run offsets and the runs themselves).
 *
 * The workspace needs no initialisation and is only scratch between the
 * partition and combine of one call.
 */
typedef struct gqa_plan {
  int32_t chunk_tokens;
  int32_t num_chunks;
  size_t off_l;
  size_t off_acc;
  size_t off_sched;
  int32_t sched_entries;
  size_t workspace_bytes;
  int32_t balanced_groups;
} gqa_plan;

/* Version of this ABI (GQA_ABI_VERSION). */
GQA_API int32_t gqa_abi_version(void);

/* Static, NUL-terminated name of a status code. */
GQA_API const char *gqa_status_string(int32_t status);

/*
 * Profiling aid (not a step of the method): the next call made on the
 * calling host thread that enqueues a partition kernel — the kernel that
 * streams the cache, launched by gqa_attend_decode, gqa_attend_partition,
 * gqa_decode_step, gqa_attend_branches, gqa_decode_step_branches and
 * gqa_attend_gathered — records `start` on its stream immediately before
 * that kernel and `stop` immediately after it, so that
 * hipEventElapsedTime(start, stop) is that one kernel's time on the device,
 * without the calls' other kernels (schedule or balance, combine).
 *   start, stop  events owned by the caller, created with timing enabled;
 *                both NULL cancels a pending request.
 * The request is consumed by that one launch; a call whose argument checks
 * fail enqueues nothing and leaves it pending.  GQA_ERR_INVALID_ARGUMENT if
 * exactly one of the two is NULL.  No HIP call is made here.
 */
GQA_API gqa_status gqa_profile_next_launch(hipEvent_t start, hipEvent_t stop);

/*
 * kv_append — needle-core KvCache::push_kv, batched.
 * For every sequence b with n = lens_in[b]:
 *   0 <= n < max_len: K[b][n][:][:] = k_new[b][:][:], V[b][n][:][:] =
 *     v_new[b][:][:] (bit copies), lens_out[b] = n + 1;
 *   otherwise (a full cache, or a negative length): nothing is written,
 *     lens_out[b] = n, and *dropped is incremented (if dropped != NULL).
 *     The page warns and returns without writing; here the drop is counted.
 * k_new [batch][num_kv_heads][dk], v_new [batch][num_kv_heads][dv], in the
 * cache dtype.  lens_out may alias lens_in.  dropped is a device int32.
 * fp8 caches: k_new / v_new are bf16 (16-byte aligned) and are quantised on
 * the way in: each value x of KV head g becomes the E4M3 code nearest to
 * x * r rounded to fp32, where r is 1 / scale[b][g] rounded to fp32 (ties to
 * the even mantissa; magnitudes above 448 saturate; NaN gives an unspecified
 * code).
 */
GQA_API gqa_status gqa_kv_append(const gqa_cache *cache, const void *k_new,
                         const void *v_new, const int32_t *lens_in,
                         int32_t *lens_out, int32_t *dropped,
                         hipStream_t stream);

/*
 * stream_append — one token per sequence into a streaming decoder's layout
 * (cortiq-engine NystromState: permanent exact sink keys and an exact window
 * ring per KV group, shared by the group's query heads; here the key that a
 * full ring evicts moves, exactly, into a main cache instead of the page's
 * approximate far field).
 *   sink  NULL (no sinks) or a cache of S slots; ring: a cache of W slots;
 *   main_cache  NULL (evicted keys leave attention) or a cache of M slots.
 *   All three share batch, num_kv_heads, dk, dv and dtype; K/V rows of
 *   num_kv_heads * d elements must be a multiple of 4 bytes.  fp8 caches:
 *   the three parts must share the scale arrays (the same k_scale and
 *   v_scale pointers, else GQA_ERR_INVALID_ARGUMENT), since an evicted row
 *   moves to main as its codes; k_new / v_new are then bf16 rows, 16-byte
 *   aligned, quantised into the new slot as gqa_kv_append does; dk and dv
 *   must be multiples of 16 (GQA_ERR_UNSUPPORTED otherwise).
 *   count_in [batch]: tokens seen so far by each sequence.  With t =
 *   count_in[b]: t < S puts the token in sink slot t; otherwise it takes ring
 *   slot (t - S) % W, and if the ring was full (t - S >= W) the token it held
 *   (position t - W) first moves to main slot t - S - W.  A negative t, or a
 *   full main cache, changes nothing and increments *dropped (if not NULL).
 *   count_out[b] = t + 1 (t when dropped); may alias count_in.
 *   lens_sink / lens_ring / lens_main [batch] receive each part's live keys
 *   (min(t', S), min(max(t' - S, 0), W), min(max(t' - S - W, 0), M)), the
 *   lengths gqa_attend_branches takes; lens_sink / lens_main are ignored
 *   without a sink / main cache.  Attending the three parts then equals
 *   attending the whole history (or sinks + window without a main cache).
 */
GQA_API gqa_status gqa_stream_append(const gqa_cache *sink,
                                     const gqa_cache *ring,
                                     const gqa_cache *main_cache,
                                     const void *k_new, const void *v_new,
                                     const int32_t *count_in,
                                     int32_t *count_out, int32_t *lens_sink,
                                     int32_t *lens_ring, int32_t *lens_main,
                                     int32_t *dropped, hipStream_t stream);

/*
 * Plan the split-K decomposition for `cache` and `num_q_heads` query heads.
 * chunk_tokens = 0 picks the library's choice (a balanced plan for a bf16 /
 * fp8 cache whose chunked launch would run in several rounds of
 * work-groups; chunks otherwise); GQA_CHUNK_BALANCED asks for a balanced
 * plan (bf16 / fp8 caches; GQA_ERR_UNSUPPORTED for fp32 or when a whole
 * unit's rows span 2 GiB or more); otherwise it must be a positive multiple
 * of 64 (a chunked plan).  Pure host computation (no HIP calls).
 */
#define GQA_CHUNK_BALANCED (-1)
GQA_API gqa_status gqa_attend_plan(const gqa_cache *cache, int32_t num_q_heads,
                           int32_t chunk_tokens, gqa_plan *plan);

/* Workspace bytes gqa_attend_decode needs (its own plan); 0 if invalid. */
GQA_API size_t gqa_attend_workspace_bytes(const gqa_cache *cache, int32_t num_q_heads);

/*
 * attend_decode — one query token per sequence attends over its cache.
 *   q     [batch][num_q_heads][dk], cache dtype (bf16 for fp8 caches).
 *   lens  [batch] device int32; keys attended are [0, clamp(lens[b], 0,
 *         max_len)).
 *   scale logit scale; 0 means 1/sqrt(dk) (usearch score_scale: zero is
 *         replaced by the derived scale, by convention 1/sqrt of the key
 *         width).  Must be finite.
 *   bias  NULL, or additive logit terms (needle-core self_attn_incremental,
 *         attn_bias: one term per cached position, added to the scaled dot
 *         product of every head): fp32, bias[b * bias_stride + t] for key t of
 *         sequence b.  bias_stride >= max_len and a multiple of 4; bias 16-byte
 *         aligned.  A term of -inf removes the key; a row whose keys are all
 *         removed is empty (out 0, carry (-inf, 0, 0), or carry_in).  Terms
 *         must not be NaN or +inf.  Ignored (with bias_stride) when NULL.
 *   carry_in   NULL, or a carry over the same query rows folded into this
 *              branch (usearch carry: one call resumes another on the same
 *              query rows, e.g. a recent-window branch).
 *   carry_out  NULL, or receives the merged carry; may alias carry_in.
 *   out   NULL, or [batch][num_q_heads][dv] fp32: the merged value mix
 *         normalised by the partition; rows with no keys at all get 0.
 *   At least one of out / carry_out must be given.
 *   workspace  device buffer of at least gqa_attend_workspace_bytes().
 * Enqueues the split-K partition kernel (preceded by the schedule kernel for
 * a plan with sched_entries > 0) and the log-sum-exp combine kernel; a plan
 * with a single chunk writes out and carry_out from the partition launch.
 */
GQA_API gqa_status gqa_attend_decode(const void *q, int32_t num_q_heads,
                             const gqa_cache *cache, const int32_t *lens,
                             float scale, const float *bias,
                             int64_t bias_stride, const gqa_carry *carry_in,
                             const gqa_carry *carry_out, float *out,
                             void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * attend_decode_noalloc — gqa_attend_decode without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  It
 * allocates nothing: its scratch is a 32 MiB array of the library's own that
 * every GPU the library runs on holds from the library's load until the
 * process ends.  Arguments as in gqa_attend_decode; the same kernels run.
 *   A call whose plan needs more than 32 MiB of workspace (more than
 *   gqa_attend_workspace_bytes reports would fit) returns
 *   GQA_ERR_WORKSPACE_TOO_SMALL; every argument check is made before any
 *   HIP call.  The first call on a device resolves the array's address on
 *   that device (the current device; `stream`, if not NULL, must belong to
 *   it, else GQA_ERR_INVALID_ARGUMENT).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (concurrent streams or host threads) race; calls in stream order do
 *   not.
 */
GQA_API gqa_status gqa_attend_decode_noalloc(const void *q, int32_t num_q_heads,
                                             const gqa_cache *cache,
                                             const int32_t *lens, float scale,
                                             const float *bias,
                                             int64_t bias_stride,
                                             const gqa_carry *carry_in,
                                             const gqa_carry *carry_out,
                                             float *out, hipStream_t stream);

/*
 * First half of attend_decode with an explicit plan: writes the partial
 * carries of every live (query row, chunk) into the workspace (layout in
 * gqa_plan).  Arguments as in gqa_attend_decode.
 */
GQA_API gqa_status gqa_attend_partition(const void *q, int32_t num_q_heads,
                                const gqa_cache *cache, const int32_t *lens,
                                float scale, const float *bias,
                                int64_t bias_stride, const gqa_plan *plan,
                                void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Second half of attend_decode: folds the live partials of each query row
 * (and carry_in) by log-sum-exp merge, writes out and/or carry_out.  `cache`
 * supplies the sizes only (its k/v pointers are not read).
 */
GQA_API gqa_status gqa_attend_combine(int32_t num_q_heads, const gqa_cache *cache,
                              const int32_t *lens, const gqa_plan *plan,
                              const void *workspace, size_t workspace_bytes,
                              const gqa_carry *carry_in,
                              const gqa_carry *carry_out, float *out,
                              hipStream_t stream);

/*
 * decode_step — kv_append then attend_decode, as one decode step (needle-core
 * self_attn_incremental: push_kv, then attend over the cache including the new
 * token), in one partition launch for the matrix-core shapes (preceded, for a
 * plan with a work schedule or queue, by the kernel that builds it, and
 * followed by the combine unless the plan is small enough to fold in the
 * launch).
 *   For every sequence b with n = lens_in[b]: if 0 <= n < max_len the token's
 *   K/V rows (k_new [batch][num_kv_heads][dk], v_new [...][dv]) are written to
 *   slot n and the query attends over [0, n + 1); otherwise nothing is written,
 *   *dropped (if not NULL) is incremented and the query attends over
 *   [0, clamp(n, 0, max_len)).  lens_out[b] receives n + 1, or n when nothing
 *   was written.
 *   lens_out must NOT alias lens_in (every work-group reads lens_in during the
 *   call); alternate two length arrays between steps.
 *   q, scale, bias, carry_in, carry_out, out: as in gqa_attend_decode (the
 *   bias row covers the new token's position too).  fp8 caches: k_new and
 *   v_new are bf16, quantised as in gqa_kv_append, and the step attends the
 *   new token's decoded codes.
 *   workspace: at least gqa_decode_step_workspace_bytes() bytes, ZERO-FILLED
 *   before its first use.  Its tail holds per-(sequence, KV group) arrival
 *   counters that every completed call leaves at zero again; calls that
 *   overlap on one workspace race.
 */
GQA_API size_t gqa_decode_step_workspace_bytes(const gqa_cache *cache,
                                               int32_t num_q_heads);

GQA_API gqa_status gqa_decode_step(const void *q, int32_t num_q_heads,
                                   const gqa_cache *cache, const void *k_new,
                                   const void *v_new, const int32_t *lens_in,
                                   int32_t *lens_out, int32_t *dropped,
                                   float scale, const float *bias,
                                   int64_t bias_stride,
                                   const gqa_carry *carry_in,
                                   const gqa_carry *carry_out, float *out,
                                   void *workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * One cache of a multi-branch attend: its own K/V (and max_len), lengths and
 * optional bias (as in gqa_attend_decode).  Every branch of a call has the
 * same batch, num_kv_heads, dk, dv and dtype (fp8 branches each carry their
 * own scales).
 */
typedef struct gqa_branch {
  gqa_cache cache;
  const int32_t *lens;   /* [batch] device int32 */
  const float *bias;     /* NULL or [batch][bias_stride] fp32 */
  int64_t bias_stride;
} gqa_branch;

#define GQA_MAX_BRANCHES 4

/* Workspace bytes gqa_attend_branches needs; 0 if the branches are invalid. */
GQA_API size_t gqa_attend_branches_workspace_bytes(const gqa_branch *branches,
                                                   int32_t num_branches,
                                                   int32_t num_q_heads);

/*
 * attend_branches — the queries attend over the union of several caches'
 * live keys (branch i: keys [0, clamp(lens_i[b], 0, max_len_i)) of its own
 * cache), folded with carry_in, in one partition launch and one combine.
 * The branches' partial softmax states merge exactly as carries do (usearch
 * carry: one branch resumes another on the same query rows), so the result
 * is one pass over the concatenated keys: e.g. permanent sink keys, a recent
 * window and a main cache (cortiq-engine NystromState: exact window ring and
 * sink buffer, kept once per KV group).
 *   1 <= num_branches <= GQA_MAX_BRANCHES; matrix-core head shapes only
 *   (GQA_ERR_UNSUPPORTED otherwise).  Other arguments as in
 *   gqa_attend_decode; workspace: gqa_attend_branches_workspace_bytes().
 */
GQA_API gqa_status gqa_attend_branches(const void *q, int32_t num_q_heads,
                                       const gqa_branch *branches,
                                       int32_t num_branches, float scale,
                                       const gqa_carry *carry_in,
                                       const gqa_carry *carry_out, float *out,
                                       void *workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * decode_step_branches — decode_step over several caches: the new token
 * (k_new, v_new) is appended to branch `append_branch` at slot lens[b] of
 * that branch (its `lens` field is the lens_in of gqa_decode_step; a full
 * cache or negative length drops the token and counts it in *dropped), and
 * the queries attend over every branch's keys including the new token, in
 * one partition launch and one combine.  lens_out [batch] receives the
 * append branch's new lengths and must not alias its lens.  The workspace
 * is that of gqa_attend_branches (no initialisation needed).  E.g. a long
 * cache attended as is plus the recent window taking the new token.
 */
GQA_API gqa_status gqa_decode_step_branches(
    const void *q, int32_t num_q_heads, const gqa_branch *branches,
    int32_t num_branches, int32_t append_branch, const void *k_new,
    const void *v_new, int32_t *lens_out, int32_t *dropped, float scale,
    const gqa_carry *carry_in, const gqa_carry *carry_out, float *out,
    void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attend_gathered — index-gathered decode (the sparse attention the metrale
 * DSA reference feeds from its selection): sequence b's query attends only
 * the cache slots its index row names.  idx [batch][width] device int32;
 * as in topk_to_mask, duplicates collapse (a repeated slot is attended
 * once), and negative (INVALID) entries and slots at or past
 * clamp(lens[b], 0, max_len) are dropped.  The selected rows are gathered
 * in ascending slot order.  Matrix-core head shapes, max_len <= 2^20, and a
 * sequence's K or V rows spanning less than 2 GiB; other arguments as in
 * gqa_attend_decode (no bias).  Workspace:
 * gqa_attend_gathered_workspace_bytes(); it needs no initialisation.
 */
GQA_API size_t gqa_attend_gathered_workspace_bytes(const gqa_cache *cache,
                                                   int32_t num_q_heads,
                                                   int32_t width);

GQA_API gqa_status gqa_attend_gathered(const void *q, int32_t num_q_heads,
                                       const gqa_cache *cache,
                                       const int32_t *lens, const int32_t *idx,
                                       int32_t width, float scale,
                                       const gqa_carry *carry_in,
                                       const gqa_carry *carry_out, float *out,
                                       void *workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * softmax_state_merge — dst = merge(a, b) row by row (usearch carry,
 * partial softmaxes rescaled to a common maximum): m = max(m_a, m_b),
 * l = e^(m_a-m) l_a +
 * e^(m_b-m) l_b, acc = e^(m_a-m) acc_a + e^(m_b-m) acc_b; an empty row
 * (l == 0) is the identity.  dst may alias a or b.  out, if not NULL,
 * receives acc / l ([rows][dv] fp32, 0 for empty rows).
 */
GQA_API gqa_status gqa_softmax_state_merge(const gqa_carry *a, const gqa_carry *b,
                                   const gqa_carry *dst, int64_t rows,
                                   int32_t dv, float *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H */
