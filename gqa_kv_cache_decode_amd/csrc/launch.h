// Internal interface between the host ABI (abi.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gqa_decode.h"

namespace gqa {

// Every argument check of gqa_attend_decode except those of the workspace
// (pure host computation, no HIP call); on success *workspace_bytes is the
// workspace its plan needs.
gqa_status attend_decode_check(const void *q, int32_t hq, const gqa_cache *c,
                               const int32_t *lens, float scale,
                               const float *bias, int64_t bias_stride,
                               const gqa_carry *carry_in,
                               const gqa_carry *carry_out, const float *out,
                               size_t *workspace_bytes);

// Wavefronts per work-group of the fp32 matrix-core partition kernel.  The
// fp32 caches that matter are short and latency-bound: with four, a 64-token
// chunk is one 16-token tile per wavefront (tiny decode step launch measured
// 7.53 -> 6.95 us, partition 5.14 -> 4.69 us, against two).
constexpr int kPartitionWaves = 4;

// Work-group width of the bf16 / fp8 partition kernel, measured on MI355X
// over the workload shapes.  With one work-group per CU, each wavefront keeps
// one tile of loads in flight, and the HBM read stream of this access pattern
// ran fastest at about 32 KB in flight per CU (a load-only probe of the
// batched shape: 38 us at 32 KB, 42 us at 64 KB for the same bytes): bf16
// takes two wavefronts (16 KB tiles at d = 128), fp8 four (8 KB tiles), or
// eight for the narrowest fp8 heads (dk + dv <= 128, 4 KB tiles).
constexpr int partition_waves(int dk, int dv, bool fp8 = false) {
  return fp8 ? (dk + dv <= 128 ? 8 : 4) : 2;
}

// Group split: a plain chunked launch over an fp8 cache with 64-wide heads
// gives each wavefront of a work-group its own KV group over the whole chunk,
// the work-group holding split_waves consecutive groups of one sequence
// (partition_mfma16.h, partition_split_kernel).  Returns the groups per
// work-group, or 1 where it does not apply.  Measured on the batched fp8 shape
// (B 16, 8 KV heads, 4096 tokens), same box: 64-wide heads 22.2-22.6 ->
// 21.7-22.0 us per step (kernel 21.5 -> 20.2-20.8 us); 128-wide heads slower,
// 32.1-32.8 -> 33.3-34.3 us (the kernel the same, 29.8 us, and eight partials
// per query row to combine instead of two), and slower still with eight
// wavefronts per work-group (34.3) or two work-groups per CU (35.3-35.6), so
// the other widths keep the shared-group launch.  It is taken where its
// work-groups are one round of one per CU, at least kSplitMinGroups and fewer
// than kSplitMaxGroups (more take a scheduled or balanced plan): the planner
// sizes chunks for it, a wavefront streaming a whole chunk of its group.
constexpr int split_waves(int dk, int dv) { return partition_waves(dk, dv, true); }
constexpr int group_split(int dk, int dv, bool fp8, int num_kv_heads) {
  return fp8 && dk + dv <= 128 && num_kv_heads % split_waves(dk, dv) == 0
             ? split_waves(dk, dv)
             : 1;
}
constexpr int kSplitMinGroups = 256;
constexpr int kSplitMaxGroups = 512;

// A further cache attended by the same launch (multi-branch attention: the
// branches' partials share one partial row per query row and one combine).
// Every branch has the launch's batch, heads and head widths.
struct ExtraBranch {
  const void *k, *v;
  const float *k_scale, *v_scale;  // fp8 launches: [B][Hkv] each
  const int32_t *lens;
  const float *bias;
  long long bias_stride;
  int max_len, chunk_tokens, num_chunks;
  int col_base;   // first partial column of the branch
  int item_base;  // first block of the branch (a multiple of 8)
};

constexpr int kMaxExtraBranches = 3;

struct PartitionArgs {
  const void *q;        // [B][Hkv*hpk][dk]
  const void *k;        // [B][max_len][Hkv][dk]
  const void *v;        // [B][max_len][Hkv][dv]
  // fp8 (E4M3) storage: code c of (b, g) stands for decode(c) * scale[b][g];
  // fp8 = 0 (bf16 / fp32 storage) leaves the scales unused.
  int fp8;
  const float *k_scale, *v_scale;  // [B][Hkv] each
  const int32_t *lens;  // [B]
  int batch, max_len, num_kv_heads, hpk, dk, dv;
  int chunk_tokens, num_chunks;
  // Partial layout and work items over all branches of the launch: a single
  // branch has total_cols = num_chunks, col_base = 0 and total_items =
  // batch * num_kv_heads * num_chunks.
  int total_cols, col_base, total_items;
  int num_extra;        // branches after the first, 0..kMaxExtraBranches
  int append_branch;    // decode step: the branch receiving the new token
  ExtraBranch extra[kMaxExtraBranches];
  float scale_log2;     // logit scale times log2(e)
  const float *bias;    // [B][bias_stride] additive logit terms, or NULL
  long long bias_stride;
  int has_bias;         // any branch of the launch has a bias
  // Index-gathered launch: sequence b attends the distinct slots below
  // clamp(lens[b], 0, cache_len) that its index row idx[b * width ..
  // + width) names, in ascending order, as a cache of that many keys
  // (max_len is then the selection's capacity, min(width, cache_len)); the
  // launch writes each sequence's selection size to sel_count[b].  NULL
  // otherwise, with cache_len = max_len.
  const int32_t *idx;
  int width;
  int32_t *sel_count;
  int cache_len;
  float *part_m;        // [rows][num_chunks]  (natural-log units)
  float *part_l;        // [rows][num_chunks]
  float *part_acc;      // [rows][num_chunks][dv]
  // Block -> item table of a scheduled launch (schedule.hip), or NULL for the
  // fixed map; sched_len entries, one per block.
  const int32_t *sched;
  int sched_len;
  // Balanced launch (balanced > 0 persistent work-groups,
  // partition_balanced_kernel): the work queue the balance kernel built (see
  // the kQueue* layout below); part_* then hold one piece slot of hpk rows
  // per queue item.
  int32_t *queue = nullptr;
  int balanced = 0;
  // fp32 launches of a few work-groups: 8 blocks per item, block 8i doing
  // item i (all on one XCD); set by the fp32 launcher
  int one_xcd = 0;
};

// Work queue of a balanced plan (int32 words, built by the balance kernel):
//   [kQueueCounter]   next item to take (0 before the partition launch)
//   [kQueueItems]     items: runs * num_kv_heads
//   [kQueueBase + k]  first run of phase k, k = 0..3 (the last: all runs)
//   [kQueuePre + k * (batch + 1) + b]  sequence b's first run within phase k
//   then 3 words per run: sequence, first tile, end tile (32-token tiles).
// Phase k cuts each sequence's tiles into runs of kQueueRun<k> tiles: phase
// 0 takes the whole runs of its first 3/4, phase 1 those of the next part
// up to 23/25, phase 2 the rest (its last run may be short).
constexpr int kQueueCounter = 0;
constexpr int kQueueItems = 1;
constexpr int kQueueBase = 2;
constexpr int kQueuePre = 6;
constexpr int kQueueRun0 = 128, kQueueRun1 = 32, kQueueRun2 = 8;
constexpr int kQueuePhases = 3;

__host__ __device__ constexpr int queue_runs_offset(int batch) {
  return kQueuePre + kQueuePhases * (batch + 1);
}

// Inputs of the schedule kernel and of the balance kernel (one work-group
// each; the balance kernel writes the work queue into `table`).
struct ScheduleArgs {
  const int32_t *lens;  // [B]
  int step;             // lengths are decode-step inputs (the new token counts)
  // decode step: the per-sequence bookkeeping, done here for every sequence
  // (a sequence with nothing to attend has no work item to do it)
  int32_t *lens_out;    // [B]
  int32_t *dropped;     // [1] or NULL
  int batch, max_len, num_kv_heads, chunk_tokens, num_chunks;
  int32_t *table;       // [table_len]
  int table_len;
};

// Extra inputs of a partition launch that runs a whole decode step (k_new ..
// counters), or that writes final results itself (the carry and out fields):
// with `direct` (a single chunk per sequence) each work-group folds carry_in
// into its group's state and writes out/carry_out; with `fuse` (decode step
// only) the last work-group of a group to finish folds the group's partials.
struct StepParams {
  const void *k_new;        // [B][Hkv][dk]
  const void *v_new;        // [B][Hkv][dv]
  const int32_t *lens_in;   // [B]
  int32_t *lens_out;        // [B], never aliasing lens_in
  int32_t *dropped;         // [1] or NULL
  int *counters;            // [B][Hkv], zero on entry and on exit
  const float *in_m, *in_l, *in_acc;  // carry_in, all NULL if absent
  float *out_m, *out_l, *out_acc;     // carry_out, all NULL if absent
  float *out;               // [rows][dv] or NULL
  int fuse;                 // the last work-group of a group folds partials
  int direct;               // num_chunks == 1: write final results directly
};

// One branch's partial columns for the combine kernel.
struct CombineBranch {
  const int32_t *lens;
  int max_len, chunk_tokens, col_base;
};

struct CombineArgs {
  int batch, num_q_heads, dv;
  int total_cols;  // partial columns per query row
  int num_branches;
  CombineBranch br[1 + kMaxExtraBranches];
  const float *part_m, *part_l, *part_acc;
  // Balanced plan (balanced > 0): each query row's pieces (one per queue
  // item of its sequence and KV group) are folded; queue: the work queue.
  int balanced = 0, hpk = 0;
  const int32_t *queue = nullptr;
  const float *in_m, *in_l, *in_acc;   // carry_in, all NULL if absent
  float *out_m, *out_l, *out_acc;      // carry_out, all NULL if absent
  float *out;                          // [rows][dv] or NULL
};

struct MergeArgs {
  const float *a_m, *a_l, *a_acc;
  const float *b_m, *b_l, *b_acc;
  float *d_m, *d_l, *d_acc;
  float *out;  // or NULL
  int64_t rows;
  int dv;
};

struct AppendArgs {
  void *k, *v;
  const void *k_new, *v_new;
  const int32_t *lens_in;
  int32_t *lens_out;
  int32_t *dropped;
  int batch, max_len, row_bytes_k, row_bytes_v;  // bytes of one token's K/V row
  // fp8 caches: k_new / v_new are bf16 rows [Hkv][d], quantised with the
  // sequence's scales (row_bytes_* are then the code rows' bytes, Hkv * d)
  int fp8, num_kv_heads;
  const float *k_scale, *v_scale;  // [B][Hkv] each
};

// One token per sequence into a streaming layout: permanent sink slots, a
// window ring, and a main cache receiving the keys the full ring evicts.
struct StreamAppendArgs {
  void *sink_k, *sink_v;  // [B][S][Hkv][d] or NULL (S = 0)
  void *ring_k, *ring_v;  // [B][W][Hkv][d]
  void *main_k, *main_v;  // [B][M][Hkv][d] or NULL (evicted keys dropped)
  const void *k_new, *v_new;
  const int32_t *count_in;
  int32_t *count_out;
  int32_t *lens_sink, *lens_ring, *lens_main;  // live keys after the append
  int32_t *dropped;
  int batch, sink, window, main_len;
  int row_bytes_k, row_bytes_v;  // bytes of one token's K/V row (multiple of 4)
  // fp8 caches: the three parts share the scales; k_new / v_new are bf16
  // rows [Hkv][d] quantised into the new slot (row_bytes_* are the code rows'
  // bytes, Hkv * d), and an evicted row moves to main as its codes
  int fp8, num_kv_heads;
  const float *k_scale, *v_scale;  // [B][Hkv] each
};

// Longest chunk of an index-gathered launch (its slots are staged in LDS).
constexpr int kGatherChunk = 2048;

// Kernel families compiled into the library.
bool partition_bf16_supported(int dk, int dv, int hpk);
bool partition_f32_supported(int dk, int dv, int hpk);
bool partition_f32_uses_mfma(int dk, int dv);
size_t partition_f32_lds_bytes(int dk, int dv, int hpk);

// `ep` carries the final-result epilogue (ep.direct) or is zero (partials
// only); the fp32 vector-ALU family always writes partials.
hipError_t launch_partition_bf16(const PartitionArgs &a, const StepParams &ep,
                                 hipStream_t s);
hipError_t launch_partition_f32(const PartitionArgs &a, const StepParams &ep,
                                hipStream_t s);
// One launch for append + partition (+ fold, when sp.fuse); matrix-core
// shapes only.  `a.lens` is unused (lengths come from sp.lens_in).
hipError_t launch_step_bf16(const PartitionArgs &a, const StepParams &sp,
                            hipStream_t s);
// fp8 (E4M3) caches: the bf16 family's shapes, a.fp8 set, q and new rows bf16.
hipError_t launch_partition_fp8(const PartitionArgs &a, const StepParams &ep,
                                hipStream_t s);
hipError_t launch_step_fp8(const PartitionArgs &a, const StepParams &sp,
                           hipStream_t s);
hipError_t launch_step_f32(const PartitionArgs &a, const StepParams &sp,
                           hipStream_t s);
hipError_t launch_combine(const CombineArgs &a, hipStream_t s);
size_t schedule_lds_bytes(int batch, int num_chunks);
hipError_t launch_schedule(const ScheduleArgs &a, hipStream_t s);
// The work queue of a balanced plan (and a decode step's bookkeeping).
hipError_t launch_balance(const ScheduleArgs &a, hipStream_t s);
constexpr int kBalanceTile = 32;  // tokens per tile of a balanced plan
hipError_t launch_merge(const MergeArgs &a, hipStream_t s);
hipError_t launch_append(const AppendArgs &a, hipStream_t s);
hipError_t launch_stream_append(const StreamAppendArgs &a, hipStream_t s);

}  // namespace gqa
