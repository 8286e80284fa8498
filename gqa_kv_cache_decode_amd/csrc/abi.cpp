// Host side of the C ABI declared in include/gqa_decode.h: argument checks,
// the split-K plan and kernel dispatch.  Nothing here allocates, frees or
// synchronises, and no HIP call happens before the checks pass.
#include "gqa_decode.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>

#include "launch.h"

namespace {

using gqa::AppendArgs;
using gqa::CombineArgs;
using gqa::MergeArgs;
using gqa::PartitionArgs;

constexpr size_t kAlign = 256;
constexpr int kChunkQuantum = 64;
constexpr int kMaxCombineDv = 256;
// A decode step folds a KV group's partials inside the step launch (in the
// group's last work-group to finish) only when the launch is small: there the
// saved launch outweighs the arrival count every work-group then performs.
// Larger launches, or partial sets above kFuseBytes per group, use the combine
// kernel, which spreads the fold over one work-group per query row.
constexpr size_t kFuseBytes = 64 * 1024;
constexpr int64_t kFuseMaxGroups = 64;
// Split-K chunking (measured on MI355X over the workload shapes): every CU
// gets at least one work-group, and a wavefront streams at most this many
// tokens of a chunk, in long uninterrupted runs.
constexpr int64_t kMinGroups = 256;
constexpr int64_t kMaxTokensPerWave = 2048;
constexpr int32_t kMaxChunk = 4096;  // longer chunks unbalance ragged batches
// A launch of at least kScheduleMinItems (sequence, KV group, chunk) items runs
// in several rounds of work-groups; it is scheduled (schedule.hip) so that the
// eight XCDs get equal shares of live chunks whatever the lengths.  The
// schedule kernel holds per-sequence state in LDS: up to kScheduleMaxSeqs
// sequences and kScheduleMaxChunks chunks.
constexpr int64_t kScheduleMinItems = 1024;
constexpr int32_t kScheduledMaxChunk = 2048;
constexpr int64_t kScheduleMaxSeqs = 8192;
constexpr int64_t kScheduleMaxChunks = 4096;
// Such a launch over a bf16 / fp8 cache with the library's own chunking is
// balanced instead: kBalancedGroups persistent work-groups (two per CU of
// the MI355X's 256) take items from a work queue of runs that shrink
// towards its end, so no ragged last round is left and faster work-groups
// take more of the work.
constexpr int kNumCUs = 256;
constexpr int kBalancedGroups = 2 * kNumCUs;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) {
  return (reinterpret_cast<uintptr_t>(p) & 15) == 0;
}

int esize(int32_t dtype) {
  return dtype == GQA_DTYPE_F32 ? 4 : dtype == GQA_DTYPE_BF16 ? 2 : 1;
}

gqa_status check_cache_dims(const gqa_cache *c) {
  if (!c) return GQA_ERR_INVALID_ARGUMENT;
  if (c->batch <= 0 || c->max_len <= 0 || c->num_kv_heads <= 0 || c->dk <= 0 ||
      c->dv <= 0)
    return GQA_ERR_INVALID_ARGUMENT;
  if (c->dtype != GQA_DTYPE_F32 && c->dtype != GQA_DTYPE_BF16 &&
      c->dtype != GQA_DTYPE_FP8_E4M3)
    return GQA_ERR_INVALID_ARGUMENT;
  return GQA_OK;
}

gqa_status check_cache_data(const gqa_cache *c) {
  if (!c->k || !c->v) return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned16(c->k) || !aligned16(c->v)) return GQA_ERR_INVALID_ARGUMENT;
  if (c->dtype == GQA_DTYPE_FP8_E4M3) {
    if (!c->k_scale || !c->v_scale) return GQA_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(c->k_scale) |
         reinterpret_cast<uintptr_t>(c->v_scale)) & 3)
      return GQA_ERR_INVALID_ARGUMENT;
  }
  return GQA_OK;
}

gqa_status check_heads(const gqa_cache *c, int32_t hq) {
  if (hq <= 0) return GQA_ERR_INVALID_ARGUMENT;
  if (hq % c->num_kv_heads != 0) return GQA_ERR_SHAPE_MISMATCH;
  const int hpk = hq / c->num_kv_heads;
  if (c->dv > kMaxCombineDv) return GQA_ERR_UNSUPPORTED;
  // fp8 caches run the bf16 kernel family (codes decoded to bf16)
  const bool ok = c->dtype == GQA_DTYPE_F32
                      ? gqa::partition_f32_supported(c->dk, c->dv, hpk)
                      : gqa::partition_bf16_supported(c->dk, c->dv, hpk);
  return ok ? GQA_OK : GQA_ERR_UNSUPPORTED;
}

gqa_status check_carry(const gqa_carry *x) {
  if (!x) return GQA_OK;
  return (x->m && x->l && x->acc) ? GQA_OK : GQA_ERR_INVALID_ARGUMENT;
}

bool uses_mfma(const gqa_cache *c) {
  return c->dtype != GQA_DTYPE_F32 || gqa::partition_f32_uses_mfma(c->dk, c->dv);
}

// Wavefronts per partition work-group of the bf16 / fp8 kernel (the rule
// and its measurements are in launch.h).
int partition_waves(const gqa_cache *c) {
  if (c->dtype == GQA_DTYPE_F32) return gqa::kPartitionWaves;
  return gqa::partition_waves(c->dk, c->dv, c->dtype == GQA_DTYPE_FP8_E4M3);
}

// KV groups per work-group of a plain chunked launch (group split, launch.h):
// 1 except for fp8 caches whose KV heads divide into sets of partition_waves.
int64_t group_split(const gqa_cache *c) {
  return uses_mfma(c) ? gqa::group_split(c->dk, c->dv,
                                         c->dtype == GQA_DTYPE_FP8_E4M3,
                                         c->num_kv_heads)
                      : 1;
}

// Whether a plan of nchunk chunks over this cache launches the group split:
// split-K, and its work-groups one round of one per CU (launch.h).
bool split_plan(const gqa_cache *c, int64_t nchunk) {
  const int64_t split = group_split(c);
  const int64_t wgs = (int64_t)c->batch * c->num_kv_heads / split * nchunk;
  return split > 1 && nchunk > 1 && wgs >= gqa::kSplitMinGroups &&
         wgs < gqa::kSplitMaxGroups;
}

// Chunk length for `sets` work-groups per chunk index and `wave_share`
// wavefronts per (KV group, chunk): the largest power of two up to kMaxChunk
// that still gives at least `min_groups` work-groups, one per CU (short caches
// go down to kChunkQuantum tokens, so a small branch spreads over more
// work-groups), with at most kMaxTokensPerWave tokens per wavefront, and no
// longer than the cache needs.
int32_t chunk_length(const gqa_cache *c, int64_t sets, int64_t wave_share,
                     int64_t min_groups) {
  int32_t chunk = kMaxChunk;
  while (chunk > kChunkQuantum &&
         (chunk / wave_share > kMaxTokensPerWave ||
          sets * ((c->max_len + chunk - 1) / chunk) < min_groups))
    chunk /= 2;
  while (chunk > kChunkQuantum && chunk / 2 >= c->max_len) chunk /= 2;
  // A launch big enough to be scheduled runs in several rounds; there the
  // last round's chunks set the tail, and shorter ones measured faster.
  const int64_t nchunk = (c->max_len + chunk - 1) / chunk;
  if (uses_mfma(c) && chunk > kScheduledMaxChunk && nchunk > 1 &&
      sets * nchunk >= kScheduleMinItems)
    chunk = kScheduledMaxChunk;
  return chunk;
}

// The library's chunk length.  A batch with enough (sequence, KV group) units
// and short caches gets a single chunk: its partition launch then writes the
// final results itself.  A split-K plan over a cache that allows the group
// split (launch.h) is sized for it (a work-group holds `split` KV groups, a
// wavefront a whole chunk of its group) when that launch is one round of one
// work-group per CU.
int32_t auto_chunk(const gqa_cache *c) {
  const int64_t units = (int64_t)c->batch * c->num_kv_heads;
  const int64_t waves = uses_mfma(c) ? partition_waves(c) : 1;
  // A cache of at most two tiles per wavefront is one chunk: its launch is
  // latency-bound, and a single chunk writes the results directly instead of
  // passing partials through a second kernel or an arrival count.
  const int64_t tile = c->dtype == GQA_DTYPE_F32 ? 16 : 32;
  if (uses_mfma(c) && c->max_len <= 2 * waves * tile)
    return (c->max_len + kChunkQuantum - 1) / kChunkQuantum * kChunkQuantum;
  const int32_t chunk = chunk_length(c, units, waves, kMinGroups);
  const int64_t split = group_split(c);
  if (split > 1 && (c->max_len + chunk - 1) / chunk > 1) {
    const int32_t sc = chunk_length(c, units / split,
                                    waves > split ? waves / split : 1,
                                    gqa::kSplitMinGroups);
    if (split_plan(c, (c->max_len + sc - 1) / sc)) return sc;
  }
  return chunk;
}

// Runs the balance kernel may cut a sequence of at most `tiles` 32-token
// tiles into (its three phases, launch.h): at most tiles * 0.0212 + 12.
int64_t queue_runs_per_seq(int64_t tiles) { return tiles * 212 / 10000 + 12; }

// The layout of a balanced plan (false when the shape does not allow one):
// one piece slot of hpk rows per queue item (part_m / part_l / part_acc),
// then the work queue (int32 words at off_sched).
bool balanced_plan(const gqa_cache *c, int32_t hq, gqa_plan *p) {
  const int64_t tiles = ((int64_t)c->max_len + gqa::kBalanceTile - 1) /
                        gqa::kBalanceTile;
  const int64_t runs = (int64_t)c->batch * queue_runs_per_seq(tiles);
  const int64_t items = runs * c->num_kv_heads;
  const int64_t words = gqa::queue_runs_offset(c->batch) + 3 * runs;
  // a run's rows are addressed with 32-bit offsets from the sequence start
  const int64_t span = (int64_t)c->max_len * c->num_kv_heads *
                       (c->dk > c->dv ? c->dk : c->dv) * esize(c->dtype);
  const int64_t hpk = hq / c->num_kv_heads;
  if (items * hpk > std::numeric_limits<int32_t>::max() ||
      words > std::numeric_limits<int32_t>::max() ||
      (int64_t)c->batch * tiles > std::numeric_limits<int32_t>::max() ||
      span >= ((int64_t)1 << 31))
    return false;
  const size_t ml = (size_t)items * hpk * sizeof(float);
  p->chunk_tokens = gqa::kBalanceTile;
  p->num_chunks = (int32_t)items;
  p->off_l = align_up(ml);
  p->off_acc = p->off_l + align_up(ml);
  p->off_sched = p->off_acc + align_up(ml * c->dv);
  p->sched_entries = (int32_t)words;
  p->workspace_bytes = p->off_sched + align_up((size_t)words * sizeof(int32_t));
  p->balanced_groups = kBalancedGroups;
  return true;
}

gqa_status make_plan(const gqa_cache *c, int32_t hq, int32_t chunk_tokens,
                     gqa_plan *p) {
  gqa_status st = check_cache_dims(c);
  if (st != GQA_OK) return st;
  if ((st = check_heads(c, hq)) != GQA_OK) return st;
  if (chunk_tokens == GQA_CHUNK_BALANCED) {  // requested explicitly
    if (c->dtype == GQA_DTYPE_F32 || !uses_mfma(c)) return GQA_ERR_UNSUPPORTED;
    return balanced_plan(c, hq, p) ? GQA_OK : GQA_ERR_UNSUPPORTED;
  }
  if (chunk_tokens < 0 || chunk_tokens % kChunkQuantum != 0)
    return GQA_ERR_INVALID_ARGUMENT;
  const int32_t chunk = chunk_tokens ? chunk_tokens : auto_chunk(c);
  // a chunk's rows of one KV group are addressed with 32-bit byte offsets
  const int64_t span = (int64_t)chunk * c->num_kv_heads *
                       (c->dk > c->dv ? c->dk : c->dv) * esize(c->dtype);
  if (span >= ((int64_t)1 << 31)) return GQA_ERR_UNSUPPORTED;
  const int64_t nchunk = ((int64_t)c->max_len + chunk - 1) / chunk;
  const int64_t groups = (int64_t)c->batch * c->num_kv_heads * nchunk;
  const int64_t rows = (int64_t)c->batch * hq;
  if (groups > std::numeric_limits<int32_t>::max() ||
      rows > std::numeric_limits<int32_t>::max())
    return GQA_ERR_UNSUPPORTED;
  const size_t ml = (size_t)rows * nchunk * sizeof(float);
  p->chunk_tokens = chunk;
  p->num_chunks = (int32_t)nchunk;
  p->off_l = align_up(ml);
  p->off_acc = p->off_l + align_up(ml);
  p->workspace_bytes = p->off_acc + align_up(ml * c->dv);
  // Schedule table: 8 entries per round of XCDs; the snake order keeps every
  // XCD's list within one sequence's items (num_kv_heads * nchunk) of the
  // mean, so 8 * (ceil(groups / 8) + num_kv_heads * nchunk) entries suffice.
  p->off_sched = 0;
  p->sched_entries = 0;
  p->balanced_groups = 0;
  // (a group-split launch is one round of work-groups: never scheduled)
  const bool multi_round = nchunk > 1 && groups >= kScheduleMinItems &&
                           uses_mfma(c) && c->batch <= kScheduleMaxSeqs &&
                           !split_plan(c, nchunk);
  if (multi_round && chunk_tokens == 0 && c->dtype != GQA_DTYPE_F32 &&
      balanced_plan(c, hq, p))
    return GQA_OK;
  const int64_t entries = 8 * ((groups + 7) / 8 + c->num_kv_heads * nchunk);
  if (multi_round && nchunk <= kScheduleMaxChunks &&
      entries <= std::numeric_limits<int32_t>::max()) {
    p->off_sched = p->workspace_bytes;
    p->sched_entries = (int32_t)entries;
    p->workspace_bytes += align_up((size_t)entries * sizeof(int32_t));
  }
  return GQA_OK;
}

// A caller's plan must be the one make_plan gives for its chunk length.
gqa_status check_plan(const gqa_cache *c, int32_t hq, const gqa_plan *plan,
                      size_t ws_bytes, const void *ws) {
  if (!plan) return GQA_ERR_INVALID_ARGUMENT;
  gqa_plan want;
  gqa_status st = make_plan(
      c, hq, plan->balanced_groups ? GQA_CHUNK_BALANCED : plan->chunk_tokens,
      &want);
  if (st != GQA_OK) return st;
  if (plan->chunk_tokens == 0 || want.chunk_tokens != plan->chunk_tokens ||
      want.num_chunks != plan->num_chunks ||
      want.off_l != plan->off_l || want.off_acc != plan->off_acc ||
      want.off_sched != plan->off_sched ||
      want.sched_entries != plan->sched_entries ||
      want.balanced_groups != plan->balanced_groups ||
      want.workspace_bytes != plan->workspace_bytes)
    return GQA_ERR_SHAPE_MISMATCH;
  if (!ws) return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned16(ws)) return GQA_ERR_INVALID_ARGUMENT;
  if (ws_bytes < plan->workspace_bytes) return GQA_ERR_WORKSPACE_TOO_SMALL;
  return GQA_OK;
}

gqa_status device_status(hipError_t e) {
  return e == hipSuccess ? GQA_OK : GQA_ERR_DEVICE;
}

// The storage fields of a partition launch (fp8 flag and scales).
void set_storage(PartitionArgs *a, const gqa_cache *c) {
  const bool fp8 = c->dtype == GQA_DTYPE_FP8_E4M3;
  a->fp8 = fp8 ? 1 : 0;
  a->k_scale = fp8 ? c->k_scale : nullptr;
  a->v_scale = fp8 ? c->v_scale : nullptr;
}

// The calling host thread's pending profiling request
// (gqa_profile_next_launch): events to record around its next partition
// launch.
thread_local hipEvent_t t_prof_start = nullptr;
thread_local hipEvent_t t_prof_stop = nullptr;

// Enqueues one partition (or decode-step) kernel, bracketed by the pending
// profiling events if there are any (the request is consumed here).
template <class Launch>
hipError_t profiled(hipStream_t s, Launch launch) {
  hipEvent_t e0 = t_prof_start, e1 = t_prof_stop;
  if (!e0) return launch();
  t_prof_start = t_prof_stop = nullptr;
  hipError_t e = hipEventRecord(e0, s);
  if (e != hipSuccess) return e;
  if ((e = launch()) != hipSuccess) return e;
  return hipEventRecord(e1, s);
}

// The partition (or whole decode step) kernel family of the cache's dtype.
hipError_t launch_partition(const gqa_cache *c, const PartitionArgs &a,
                            const gqa::StepParams &ep, hipStream_t s) {
  return profiled(s, [&] {
    switch (c->dtype) {
      case GQA_DTYPE_BF16: return gqa::launch_partition_bf16(a, ep, s);
      case GQA_DTYPE_FP8_E4M3: return gqa::launch_partition_fp8(a, ep, s);
      default: return gqa::launch_partition_f32(a, ep, s);
    }
  });
}

hipError_t launch_step(const gqa_cache *c, const PartitionArgs &a,
                       const gqa::StepParams &sp, hipStream_t s) {
  return profiled(s, [&] {
    switch (c->dtype) {
      case GQA_DTYPE_BF16: return gqa::launch_step_bf16(a, sp, s);
      case GQA_DTYPE_FP8_E4M3: return gqa::launch_step_fp8(a, sp, s);
      default: return gqa::launch_step_f32(a, sp, s);
    }
  });
}

// The partial layout and work items of a one-cache launch.
void single_branch(PartitionArgs *a) {
  a->total_cols = a->num_chunks;
  a->col_base = 0;
  // (make_plan keeps a chunked plan's items within int32; a balanced plan's
  // num_chunks counts piece slots, and its launch takes items from the queue
  // instead)
  const int64_t items = (int64_t)a->batch * a->num_kv_heads * a->num_chunks;
  a->total_items = items <= std::numeric_limits<int32_t>::max() ? (int)items : 0;
  a->num_extra = 0;
  a->append_branch = 0;
  a->idx = nullptr;
  a->width = 0;
  a->sel_count = nullptr;
  a->cache_len = a->max_len;
}

// Enqueues the schedule kernel of a scheduled plan and points the partition
// launch at its table (a no-op for an unscheduled plan).
gqa_status schedule_checked(const gqa_cache *c, const gqa_plan &plan,
                            const int32_t *lens, bool step, int32_t *lens_out,
                            int32_t *dropped, void *ws, PartitionArgs *a,
                            hipStream_t s) {
  a->sched = nullptr;
  a->sched_len = 0;
  a->queue = nullptr;
  a->balanced = 0;
  if (plan.sched_entries == 0) return GQA_OK;
  gqa::ScheduleArgs sa;
  sa.lens = lens;
  sa.step = step ? 1 : 0;
  sa.lens_out = lens_out;
  sa.dropped = dropped;
  sa.batch = c->batch;
  sa.max_len = c->max_len;
  sa.num_kv_heads = c->num_kv_heads;
  sa.chunk_tokens = plan.chunk_tokens;
  sa.num_chunks = plan.num_chunks;
  sa.table = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + plan.off_sched);
  sa.table_len = plan.sched_entries;
  if (plan.balanced_groups) {  // the work queue, then the persistent launch
    gqa_status st = device_status(gqa::launch_balance(sa, s));
    if (st != GQA_OK) return st;
    a->queue = sa.table;
    a->balanced = plan.balanced_groups;
    return GQA_OK;
  }
  gqa_status st = device_status(gqa::launch_schedule(sa, s));
  if (st != GQA_OK) return st;
  a->sched = sa.table;
  a->sched_len = sa.table_len;
  return GQA_OK;
}

// The epilogue of a partition launch that writes final results: carry_in,
// carry_out and out, with `direct` set when the plan has a single chunk.
gqa::StepParams final_epilogue(const gqa_cache *c, const gqa_plan &plan,
                               const gqa_carry *cin, const gqa_carry *cout,
                               float *out) {
  gqa::StepParams ep{};
  ep.in_m = cin ? cin->m : nullptr;
  ep.in_l = cin ? cin->l : nullptr;
  ep.in_acc = cin ? cin->acc : nullptr;
  ep.out_m = cout ? cout->m : nullptr;
  ep.out_l = cout ? cout->l : nullptr;
  ep.out_acc = cout ? cout->acc : nullptr;
  ep.out = out;
  ep.direct = plan.num_chunks == 1 && uses_mfma(c) ? 1 : 0;
  return ep;
}

// Whether the partition launch leaves no fold to a combine launch.
bool finished_in_partition(const gqa_plan &, const gqa::StepParams &ep) {
  return ep.direct != 0;
}

gqa_status partition_checked(const void *q, int32_t hq, const gqa_cache *c,
                             const int32_t *lens, float scale,
                             const float *bias, int64_t bias_stride,
                             const gqa_plan *plan, void *ws,
                             const gqa::StepParams &ep, hipStream_t s) {
  const int hpk = hq / c->num_kv_heads;
  const double sc = scale != 0.0f ? (double)scale : 1.0 / std::sqrt((double)c->dk);
  PartitionArgs a;
  a.q = q;
  a.k = c->k;
  a.v = c->v;
  a.lens = lens;
  a.batch = c->batch;
  a.max_len = c->max_len;
  a.num_kv_heads = c->num_kv_heads;
  a.hpk = hpk;
  a.dk = c->dk;
  a.dv = c->dv;
  a.chunk_tokens = plan->chunk_tokens;
  a.num_chunks = plan->num_chunks;
  single_branch(&a);
  set_storage(&a, c);
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  a.bias = bias;
  a.bias_stride = bias ? bias_stride : 0;
  a.has_bias = bias ? 1 : 0;
  char *base = static_cast<char *>(ws);
  a.part_m = reinterpret_cast<float *>(base);
  a.part_l = reinterpret_cast<float *>(base + plan->off_l);
  a.part_acc = reinterpret_cast<float *>(base + plan->off_acc);
  gqa_status st =
      schedule_checked(c, *plan, lens, false, nullptr, nullptr, ws, &a, s);
  if (st != GQA_OK) return st;
  return device_status(launch_partition(c, a, ep, s));
}

gqa_status combine_checked(int32_t hq, const gqa_cache *c, const int32_t *lens,
                           const gqa_plan *plan, const void *ws,
                           const gqa_carry *cin, const gqa_carry *cout,
                           float *out, hipStream_t s) {
  CombineArgs a;
  a.balanced = plan->balanced_groups;
  a.hpk = hq / c->num_kv_heads;
  a.queue = a.balanced ? reinterpret_cast<const int32_t *>(
                             static_cast<const char *>(ws) + plan->off_sched)
                       : nullptr;
  a.batch = c->batch;
  a.num_q_heads = hq;
  a.dv = c->dv;
  a.total_cols = plan->num_chunks;
  a.num_branches = 1;
  a.br[0] = gqa::CombineBranch{lens, c->max_len, plan->chunk_tokens, 0};
  const char *base = static_cast<const char *>(ws);
  a.part_m = reinterpret_cast<const float *>(base);
  a.part_l = reinterpret_cast<const float *>(base + plan->off_l);
  a.part_acc = reinterpret_cast<const float *>(base + plan->off_acc);
  a.in_m = cin ? cin->m : nullptr;
  a.in_l = cin ? cin->l : nullptr;
  a.in_acc = cin ? cin->acc : nullptr;
  a.out_m = cout ? cout->m : nullptr;
  a.out_l = cout ? cout->l : nullptr;
  a.out_acc = cout ? cout->acc : nullptr;
  a.out = out;
  return device_status(gqa::launch_combine(a, s));
}

gqa_status check_attend_args(const void *q, int32_t hq, const gqa_cache *c,
                             const int32_t *lens, float scale) {
  gqa_status st = check_cache_dims(c);
  if (st != GQA_OK) return st;
  if ((st = check_cache_data(c)) != GQA_OK) return st;
  if ((st = check_heads(c, hq)) != GQA_OK) return st;
  if (!q || !lens) return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q)) return GQA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARGUMENT;
  return GQA_OK;
}

// The additive bias: NULL, or fp32 rows of bias_stride >= max_len values per
// sequence, 16-byte aligned rows (the kernels read four positions at once).
gqa_status check_bias(const gqa_cache *c, const float *bias,
                      int64_t bias_stride) {
  if (!bias) return GQA_OK;
  if (bias_stride < c->max_len || bias_stride % 4 != 0 || !aligned16(bias))
    return GQA_ERR_INVALID_ARGUMENT;
  return GQA_OK;
}

gqa_status check_combine_args(int32_t hq, const gqa_cache *c,
                              const int32_t *lens, const gqa_carry *cin,
                              const gqa_carry *cout, const float *out) {
  gqa_status st = check_cache_dims(c);
  if (st != GQA_OK) return st;
  if ((st = check_heads(c, hq)) != GQA_OK) return st;
  if (!lens) return GQA_ERR_INVALID_ARGUMENT;
  if ((st = check_carry(cin)) != GQA_OK) return st;
  if ((st = check_carry(cout)) != GQA_OK) return st;
  if (!out && !cout) return GQA_ERR_INVALID_ARGUMENT;
  return GQA_OK;
}

size_t step_counter_bytes(const gqa_cache *c) {
  return align_up((size_t)c->batch * c->num_kv_heads * sizeof(int));
}

bool step_fuses(const gqa_cache *c, int32_t hq, const gqa_plan &plan) {
  const size_t hpk = hq / c->num_kv_heads;
  const int64_t groups = (int64_t)c->batch * c->num_kv_heads * plan.num_chunks;
  return groups <= kFuseMaxGroups &&
         hpk * plan.num_chunks * (c->dv + 2) * sizeof(float) <= kFuseBytes;
}

// Chunking and workspace layout of a multi-branch attend: per-branch chunk
// lengths (each branch's own plan rule), the partial columns of all
// branches, and the partial arrays' offsets.
struct BranchesPlan {
  int32_t chunk[GQA_MAX_BRANCHES];
  int32_t num_chunks[GQA_MAX_BRANCHES];
  int32_t col_base[GQA_MAX_BRANCHES];
  int64_t item_base[GQA_MAX_BRANCHES];
  int32_t total_cols;
  int64_t total_items;
  size_t off_l, off_acc, workspace_bytes;
};

gqa_status plan_branches(const gqa_branch *br, int32_t n, int32_t hq,
                         BranchesPlan *p) {
  if (!br || n < 1 || n > GQA_MAX_BRANCHES) return GQA_ERR_INVALID_ARGUMENT;
  int64_t cols = 0, items = 0;
  for (int32_t i = 0; i < n; ++i) {
    const gqa_cache *c = &br[i].cache;
    gqa_status st = check_cache_dims(c);
    if (st != GQA_OK) return st;
    const gqa_cache *c0 = &br[0].cache;
    if (c->batch != c0->batch || c->num_kv_heads != c0->num_kv_heads ||
        c->dk != c0->dk || c->dv != c0->dv || c->dtype != c0->dtype)
      return GQA_ERR_SHAPE_MISMATCH;
    if ((st = check_heads(c, hq)) != GQA_OK) return st;
    if (!uses_mfma(c)) return GQA_ERR_UNSUPPORTED;
    gqa_plan one;  // (the library's chunking, never a balanced plan)
    if ((st = make_plan(c, hq, auto_chunk(c), &one)) != GQA_OK) return st;
    p->chunk[i] = one.chunk_tokens;
    p->num_chunks[i] = one.num_chunks;
    p->col_base[i] = (int32_t)cols;
    // each branch's blocks start at a multiple of 8 so that its items spread
    // evenly over the eight XCDs (block i runs on XCD i % 8)
    items = (items + 7) / 8 * 8;
    p->item_base[i] = items;
    cols += one.num_chunks;
    items += (int64_t)c->batch * c->num_kv_heads * one.num_chunks;
  }
  const int64_t rows = (int64_t)br[0].cache.batch * hq;
  if (cols > std::numeric_limits<int32_t>::max() ||
      items > std::numeric_limits<int32_t>::max() ||
      rows * cols > std::numeric_limits<int32_t>::max())
    return GQA_ERR_UNSUPPORTED;
  p->total_cols = (int32_t)cols;
  p->total_items = items;
  const size_t ml = (size_t)rows * cols * sizeof(float);
  p->off_l = align_up(ml);
  p->off_acc = p->off_l + align_up(ml);
  p->workspace_bytes = p->off_acc + align_up(ml * br[0].cache.dv);
  return GQA_OK;
}

// Inputs of a multi-branch decode step: the new token goes to one branch.
struct BranchStep {
  int32_t append_branch;
  const void *k_new, *v_new;
  int32_t *lens_out, *dropped;
};

gqa_status branches_checked(const void *q, int32_t num_q_heads,
                            const gqa_branch *branches, int32_t num_branches,
                            float scale, const gqa_carry *carry_in,
                            const gqa_carry *carry_out, float *out,
                            void *workspace, size_t workspace_bytes,
                            const BranchStep *step, hipStream_t stream) {
  BranchesPlan p;
  gqa_status st = plan_branches(branches, num_branches, num_q_heads, &p);
  if (st != GQA_OK) return st;
  bool any_bias = false;
  for (int32_t i = 0; i < num_branches; ++i) {
    const gqa_branch &b = branches[i];
    if ((st = check_attend_args(q, num_q_heads, &b.cache, b.lens, scale)) !=
        GQA_OK)
      return st;
    if ((st = check_cache_data(&b.cache)) != GQA_OK) return st;
    if ((st = check_bias(&b.cache, b.bias, b.bias_stride)) != GQA_OK) return st;
    any_bias = any_bias || b.bias != nullptr;
  }
  const gqa_cache *c0 = &branches[0].cache;
  if ((st = check_combine_args(num_q_heads, c0, branches[0].lens, carry_in,
                               carry_out, out)) != GQA_OK)
    return st;
  if (step) {
    const int32_t ab = step->append_branch;
    if (ab < 0 || ab >= num_branches) return GQA_ERR_INVALID_ARGUMENT;
    if (!step->k_new || !step->v_new || !step->lens_out ||
        step->lens_out == branches[ab].lens)
      return GQA_ERR_INVALID_ARGUMENT;
    if (!aligned16(step->k_new) || !aligned16(step->v_new))
      return GQA_ERR_INVALID_ARGUMENT;
  }
  if (!workspace || !aligned16(workspace)) return GQA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < p.workspace_bytes) return GQA_ERR_WORKSPACE_TOO_SMALL;

  const double sc =
      scale != 0.0f ? (double)scale : 1.0 / std::sqrt((double)c0->dk);
  PartitionArgs a;
  a.q = q;
  a.k = c0->k;
  a.v = c0->v;
  a.lens = branches[0].lens;
  a.batch = c0->batch;
  a.max_len = c0->max_len;
  a.num_kv_heads = c0->num_kv_heads;
  a.hpk = num_q_heads / c0->num_kv_heads;
  a.dk = c0->dk;
  a.dv = c0->dv;
  a.chunk_tokens = p.chunk[0];
  a.num_chunks = p.num_chunks[0];
  a.total_cols = p.total_cols;
  a.col_base = 0;
  a.total_items = (int)p.total_items;
  a.num_extra = num_branches - 1;
  a.append_branch = step ? step->append_branch : -1;
  a.idx = nullptr;
  a.width = 0;
  a.sel_count = nullptr;
  a.cache_len = c0->max_len;
  set_storage(&a, c0);
  for (int32_t i = 1; i < num_branches; ++i) {
    const gqa_branch &b = branches[i];
    gqa::ExtraBranch &x = a.extra[i - 1];
    x.k = b.cache.k;
    x.v = b.cache.v;
    x.k_scale = a.fp8 ? b.cache.k_scale : nullptr;
    x.v_scale = a.fp8 ? b.cache.v_scale : nullptr;
    x.lens = b.lens;
    x.bias = b.bias;
    x.bias_stride = b.bias ? b.bias_stride : 0;
    x.max_len = b.cache.max_len;
    x.chunk_tokens = p.chunk[i];
    x.num_chunks = p.num_chunks[i];
    x.col_base = p.col_base[i];
    x.item_base = (int)p.item_base[i];
  }
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  a.bias = branches[0].bias;
  a.bias_stride = a.bias ? branches[0].bias_stride : 0;
  a.has_bias = any_bias ? 1 : 0;
  char *base = static_cast<char *>(workspace);
  a.part_m = reinterpret_cast<float *>(base);
  a.part_l = reinterpret_cast<float *>(base + p.off_l);
  a.part_acc = reinterpret_cast<float *>(base + p.off_acc);
  a.sched = nullptr;
  a.sched_len = 0;
  if (step) {
    gqa::StepParams sp{};
    sp.k_new = step->k_new;
    sp.v_new = step->v_new;
    sp.lens_in = branches[step->append_branch].lens;
    sp.lens_out = step->lens_out;
    sp.dropped = step->dropped;
    st = device_status(launch_step(c0, a, sp, stream));
  } else {
    st = device_status(launch_partition(c0, a, gqa::StepParams{}, stream));
  }
  if (st != GQA_OK) return st;

  CombineArgs cb;
  cb.batch = c0->batch;
  cb.num_q_heads = num_q_heads;
  cb.dv = c0->dv;
  cb.total_cols = p.total_cols;
  cb.num_branches = num_branches;
  for (int32_t i = 0; i < num_branches; ++i) {
    const int32_t *lens = branches[i].lens;
    if (step && i == step->append_branch) lens = step->lens_out;
    cb.br[i] = gqa::CombineBranch{lens, branches[i].cache.max_len, p.chunk[i],
                                  p.col_base[i]};
  }
  cb.part_m = a.part_m;
  cb.part_l = a.part_l;
  cb.part_acc = a.part_acc;
  cb.in_m = carry_in ? carry_in->m : nullptr;
  cb.in_l = carry_in ? carry_in->l : nullptr;
  cb.in_acc = carry_in ? carry_in->acc : nullptr;
  cb.out_m = carry_out ? carry_out->m : nullptr;
  cb.out_l = carry_out ? carry_out->l : nullptr;
  cb.out_acc = carry_out ? carry_out->acc : nullptr;
  cb.out = out;
  return device_status(gqa::launch_combine(cb, stream));
}

// Layout of an index-gathered attend: the split-K plan of the selection
// (a cache of min(width, max_len) slots per sequence, chunks of at most
// kGatherChunk), then the selection sizes [batch] the partition launch
// writes for the combine.
struct GatherPlan {
  gqa_cache vcache;
  gqa_plan plan;
  int32_t sel_cap;
  size_t off_count, workspace_bytes;
};

// Longest cache an index-gathered launch takes: each of its work-groups
// rebuilds the sequence's selection over the live length, one LDS bitmap
// window at a time.
constexpr int32_t kGatherMaxLen = 1 << 20;

gqa_status plan_gathered(const gqa_cache *c, int32_t hq, int32_t width,
                         GatherPlan *g) {
  gqa_status st = check_cache_dims(c);
  if (st != GQA_OK) return st;
  if ((st = check_heads(c, hq)) != GQA_OK) return st;
  if (width < 1) return GQA_ERR_INVALID_ARGUMENT;
  if (!uses_mfma(c) || c->max_len > kGatherMaxLen) return GQA_ERR_UNSUPPORTED;
  // gathered rows are addressed with 32-bit offsets from the sequence start
  const int64_t span = (int64_t)c->max_len * c->num_kv_heads *
                       (c->dk > c->dv ? c->dk : c->dv) * esize(c->dtype);
  if (span >= ((int64_t)1 << 31)) return GQA_ERR_UNSUPPORTED;
  g->sel_cap = width < c->max_len ? width : c->max_len;
  g->vcache = *c;
  g->vcache.max_len = g->sel_cap;
  // the library's chunking (never a balanced plan), chunks of at most
  // kGatherChunk slots
  const int32_t chunk = std::min(auto_chunk(&g->vcache), gqa::kGatherChunk);
  if ((st = make_plan(&g->vcache, hq, chunk, &g->plan)) != GQA_OK) return st;
  g->off_count = g->plan.workspace_bytes;
  g->workspace_bytes =
      g->off_count + align_up((size_t)c->batch * sizeof(int32_t));
  return GQA_OK;
}

}  // namespace

namespace gqa {

gqa_status attend_decode_check(const void *q, int32_t hq, const gqa_cache *c,
                               const int32_t *lens, float scale,
                               const float *bias, int64_t bias_stride,
                               const gqa_carry *carry_in,
                               const gqa_carry *carry_out, const float *out,
                               size_t *workspace_bytes) {
  gqa_status st = check_attend_args(q, hq, c, lens, scale);
  if (st != GQA_OK) return st;
  if ((st = check_bias(c, bias, bias_stride)) != GQA_OK) return st;
  if ((st = check_combine_args(hq, c, lens, carry_in, carry_out, out)) !=
      GQA_OK)
    return st;
  gqa_plan plan;
  if ((st = make_plan(c, hq, 0, &plan)) != GQA_OK) return st;
  *workspace_bytes = plan.workspace_bytes;
  return GQA_OK;
}

}  // namespace gqa

extern "C" {

int32_t gqa_abi_version(void) { return GQA_ABI_VERSION; }

gqa_status gqa_profile_next_launch(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr)) return GQA_ERR_INVALID_ARGUMENT;
  t_prof_start = start;
  t_prof_stop = stop;
  return GQA_OK;
}

const char *gqa_status_string(int32_t status) {
  switch (status) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_INVALID_ARGUMENT: return "GQA_ERR_INVALID_ARGUMENT";
    case GQA_ERR_SHAPE_MISMATCH: return "GQA_ERR_SHAPE_MISMATCH";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED";
    case GQA_ERR_WORKSPACE_TOO_SMALL: return "GQA_ERR_WORKSPACE_TOO_SMALL";
    case GQA_ERR_DEVICE: return "GQA_ERR_DEVICE";
    default: return "GQA_ERR_UNKNOWN";
  }
}

gqa_status gqa_kv_append(const gqa_cache *cache, const void *k_new,
                         const void *v_new, const int32_t *lens_in,
                         int32_t *lens_out, int32_t *dropped,
                         hipStream_t stream) {
  gqa_status st = check_cache_dims(cache);
  if (st != GQA_OK) return st;
  if ((st = check_cache_data(cache)) != GQA_OK) return st;
  if (!k_new || !v_new || !lens_in || !lens_out) return GQA_ERR_INVALID_ARGUMENT;
  const bool fp8 = cache->dtype == GQA_DTYPE_FP8_E4M3;
  const int64_t rk = (int64_t)cache->num_kv_heads * cache->dk * esize(cache->dtype);
  const int64_t rv = (int64_t)cache->num_kv_heads * cache->dv * esize(cache->dtype);
  // (bf16 rows of an fp8 cache are read twice as wide as the code rows)
  if (2 * rk > std::numeric_limits<int32_t>::max() ||
      2 * rv > std::numeric_limits<int32_t>::max())
    return GQA_ERR_UNSUPPORTED;
  if (fp8) {  // sixteen codes per 16-byte piece, from 16-byte bf16 pieces
    if (cache->dk % 16 || cache->dv % 16) return GQA_ERR_UNSUPPORTED;
    if (!aligned16(k_new) || !aligned16(v_new)) return GQA_ERR_INVALID_ARGUMENT;
  }
  AppendArgs a;
  a.k = cache->k;
  a.v = cache->v;
  a.k_new = k_new;
  a.v_new = v_new;
  a.lens_in = lens_in;
  a.lens_out = lens_out;
  a.dropped = dropped;
  a.batch = cache->batch;
  a.max_len = cache->max_len;
  a.row_bytes_k = (int)rk;
  a.row_bytes_v = (int)rv;
  a.fp8 = fp8 ? 1 : 0;
  a.num_kv_heads = cache->num_kv_heads;
  a.k_scale = fp8 ? cache->k_scale : nullptr;
  a.v_scale = fp8 ? cache->v_scale : nullptr;
  return device_status(gqa::launch_append(a, stream));
}

gqa_status gqa_stream_append(const gqa_cache *sink, const gqa_cache *ring,
                             const gqa_cache *main_cache, const void *k_new,
                             const void *v_new, const int32_t *count_in,
                             int32_t *count_out, int32_t *lens_sink,
                             int32_t *lens_ring, int32_t *lens_main,
                             int32_t *dropped, hipStream_t stream) {
  gqa_status st = check_cache_dims(ring);
  if (st != GQA_OK) return st;
  if ((st = check_cache_data(ring)) != GQA_OK) return st;
  const bool fp8 = ring->dtype == GQA_DTYPE_FP8_E4M3;
  for (const gqa_cache *c : {sink, main_cache}) {
    if (!c) continue;
    if ((st = check_cache_dims(c)) != GQA_OK) return st;
    if ((st = check_cache_data(c)) != GQA_OK) return st;
    if (c->batch != ring->batch || c->num_kv_heads != ring->num_kv_heads ||
        c->dk != ring->dk || c->dv != ring->dv || c->dtype != ring->dtype)
      return GQA_ERR_SHAPE_MISMATCH;
    // fp8: an evicted row moves to main as its codes, so the parts must
    // share the scales
    if (fp8 && (c->k_scale != ring->k_scale || c->v_scale != ring->v_scale))
      return GQA_ERR_INVALID_ARGUMENT;
  }
  if (fp8) {  // four codes of one KV head per word, from 16-byte bf16 rows
    if (ring->dk % 16 || ring->dv % 16) return GQA_ERR_UNSUPPORTED;
    if (!aligned16(k_new) || !aligned16(v_new)) return GQA_ERR_INVALID_ARGUMENT;
  }
  if (!k_new || !v_new || !count_in || !count_out || !lens_ring ||
      (sink && !lens_sink) || (main_cache && !lens_main))
    return GQA_ERR_INVALID_ARGUMENT;
  const int64_t rk = (int64_t)ring->num_kv_heads * ring->dk * esize(ring->dtype);
  const int64_t rv = (int64_t)ring->num_kv_heads * ring->dv * esize(ring->dtype);
  // (bf16 rows of an fp8 cache are read twice as wide as the code rows)
  if (rk % 4 || rv % 4 || 2 * rk > std::numeric_limits<int32_t>::max() ||
      2 * rv > std::numeric_limits<int32_t>::max())
    return GQA_ERR_UNSUPPORTED;
  const uintptr_t bits = reinterpret_cast<uintptr_t>(k_new) |
                         reinterpret_cast<uintptr_t>(v_new);
  if (bits & 3) return GQA_ERR_INVALID_ARGUMENT;
  gqa::StreamAppendArgs a;
  a.sink_k = sink ? sink->k : nullptr;
  a.sink_v = sink ? sink->v : nullptr;
  a.ring_k = ring->k;
  a.ring_v = ring->v;
  a.main_k = main_cache ? main_cache->k : nullptr;
  a.main_v = main_cache ? main_cache->v : nullptr;
  a.k_new = k_new;
  a.v_new = v_new;
  a.count_in = count_in;
  a.count_out = count_out;
  a.lens_sink = sink ? lens_sink : nullptr;
  a.lens_ring = lens_ring;
  a.lens_main = main_cache ? lens_main : nullptr;
  a.dropped = dropped;
  a.batch = ring->batch;
  a.sink = sink ? sink->max_len : 0;
  a.window = ring->max_len;
  a.main_len = main_cache ? main_cache->max_len : 0;
  a.row_bytes_k = (int)rk;
  a.row_bytes_v = (int)rv;
  a.fp8 = fp8 ? 1 : 0;
  a.num_kv_heads = ring->num_kv_heads;
  a.k_scale = fp8 ? ring->k_scale : nullptr;
  a.v_scale = fp8 ? ring->v_scale : nullptr;
  return device_status(gqa::launch_stream_append(a, stream));
}

gqa_status gqa_attend_plan(const gqa_cache *cache, int32_t num_q_heads,
                           int32_t chunk_tokens, gqa_plan *plan) {
  if (!plan) return GQA_ERR_INVALID_ARGUMENT;
  return make_plan(cache, num_q_heads, chunk_tokens, plan);
}

size_t gqa_attend_workspace_bytes(const gqa_cache *cache, int32_t num_q_heads) {
  gqa_plan p;
  return make_plan(cache, num_q_heads, 0, &p) == GQA_OK ? p.workspace_bytes : 0;
}

gqa_status gqa_attend_partition(const void *q, int32_t num_q_heads,
                                const gqa_cache *cache, const int32_t *lens,
                                float scale, const float *bias,
                                int64_t bias_stride, const gqa_plan *plan,
                                void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  gqa_status st = check_attend_args(q, num_q_heads, cache, lens, scale);
  if (st != GQA_OK) return st;
  if ((st = check_bias(cache, bias, bias_stride)) != GQA_OK) return st;
  if ((st = check_plan(cache, num_q_heads, plan, workspace_bytes, workspace)) !=
      GQA_OK)
    return st;
  return partition_checked(q, num_q_heads, cache, lens, scale, bias,
                           bias_stride, plan, workspace, gqa::StepParams{},
                           stream);
}

gqa_status gqa_attend_combine(int32_t num_q_heads, const gqa_cache *cache,
                              const int32_t *lens, const gqa_plan *plan,
                              const void *workspace, size_t workspace_bytes,
                              const gqa_carry *carry_in,
                              const gqa_carry *carry_out, float *out,
                              hipStream_t stream) {
  gqa_status st =
      check_combine_args(num_q_heads, cache, lens, carry_in, carry_out, out);
  if (st != GQA_OK) return st;
  if ((st = check_plan(cache, num_q_heads, plan, workspace_bytes, workspace)) !=
      GQA_OK)
    return st;
  return combine_checked(num_q_heads, cache, lens, plan, workspace, carry_in,
                         carry_out, out, stream);
}

gqa_status gqa_attend_decode(const void *q, int32_t num_q_heads,
                             const gqa_cache *cache, const int32_t *lens,
                             float scale, const float *bias,
                             int64_t bias_stride, const gqa_carry *carry_in,
                             const gqa_carry *carry_out, float *out,
                             void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  size_t need = 0;
  gqa_status st = gqa::attend_decode_check(q, num_q_heads, cache, lens, scale,
                                           bias, bias_stride, carry_in,
                                           carry_out, out, &need);
  if (st != GQA_OK) return st;
  gqa_plan plan;
  if ((st = make_plan(cache, num_q_heads, 0, &plan)) != GQA_OK) return st;
  if ((st = check_plan(cache, num_q_heads, &plan, workspace_bytes, workspace)) !=
      GQA_OK)
    return st;
  const gqa::StepParams ep =
      final_epilogue(cache, plan, carry_in, carry_out, out);
  st = partition_checked(q, num_q_heads, cache, lens, scale, bias, bias_stride,
                         &plan, workspace, ep, stream);
  if (st != GQA_OK || finished_in_partition(plan, ep)) return st;
  return combine_checked(num_q_heads, cache, lens, &plan, workspace, carry_in,
                         carry_out, out, stream);
}

gqa_status gqa_softmax_state_merge(const gqa_carry *a, const gqa_carry *b,
                                   const gqa_carry *dst, int64_t rows,
                                   int32_t dv, float *out, hipStream_t stream) {
  if (!a || !b || !dst) return GQA_ERR_INVALID_ARGUMENT;
  gqa_status st;
  if ((st = check_carry(a)) != GQA_OK || (st = check_carry(b)) != GQA_OK ||
      (st = check_carry(dst)) != GQA_OK)
    return st;
  if (rows <= 0 || dv <= 0) return GQA_ERR_INVALID_ARGUMENT;
  if (rows > std::numeric_limits<int32_t>::max()) return GQA_ERR_UNSUPPORTED;
  MergeArgs m;
  m.a_m = a->m;
  m.a_l = a->l;
  m.a_acc = a->acc;
  m.b_m = b->m;
  m.b_l = b->l;
  m.b_acc = b->acc;
  m.d_m = dst->m;
  m.d_l = dst->l;
  m.d_acc = dst->acc;
  m.out = out;
  m.rows = rows;
  m.dv = dv;
  return device_status(gqa::launch_merge(m, stream));
}

size_t gqa_attend_branches_workspace_bytes(const gqa_branch *branches,
                                           int32_t num_branches,
                                           int32_t num_q_heads) {
  BranchesPlan p;
  return plan_branches(branches, num_branches, num_q_heads, &p) == GQA_OK
             ? p.workspace_bytes
             : 0;
}

gqa_status gqa_attend_branches(const void *q, int32_t num_q_heads,
                               const gqa_branch *branches,
                               int32_t num_branches, float scale,
                               const gqa_carry *carry_in,
                               const gqa_carry *carry_out, float *out,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return branches_checked(q, num_q_heads, branches, num_branches, scale,
                          carry_in, carry_out, out, workspace,
                          workspace_bytes, nullptr, stream);
}

gqa_status gqa_decode_step_branches(
    const void *q, int32_t num_q_heads, const gqa_branch *branches,
    int32_t num_branches, int32_t append_branch, const void *k_new,
    const void *v_new, int32_t *lens_out, int32_t *dropped, float scale,
    const gqa_carry *carry_in, const gqa_carry *carry_out, float *out,
    void *workspace, size_t workspace_bytes, hipStream_t stream) {
  const BranchStep step{append_branch, k_new, v_new, lens_out, dropped};
  return branches_checked(q, num_q_heads, branches, num_branches, scale,
                          carry_in, carry_out, out, workspace,
                          workspace_bytes, &step, stream);
}

size_t gqa_attend_gathered_workspace_bytes(const gqa_cache *cache,
                                           int32_t num_q_heads,
                                           int32_t width) {
  GatherPlan g;
  return plan_gathered(cache, num_q_heads, width, &g) == GQA_OK
             ? g.workspace_bytes
             : 0;
}

gqa_status gqa_attend_gathered(const void *q, int32_t num_q_heads,
                               const gqa_cache *cache, const int32_t *lens,
                               const int32_t *idx, int32_t width, float scale,
                               const gqa_carry *carry_in,
                               const gqa_carry *carry_out, float *out,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  gqa_status st = check_attend_args(q, num_q_heads, cache, lens, scale);
  if (st != GQA_OK) return st;
  if ((st = check_combine_args(num_q_heads, cache, lens, carry_in, carry_out,
                               out)) != GQA_OK)
    return st;
  if (!idx) return GQA_ERR_INVALID_ARGUMENT;
  GatherPlan g;
  if ((st = plan_gathered(cache, num_q_heads, width, &g)) != GQA_OK) return st;
  if (!workspace || !aligned16(workspace)) return GQA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < g.workspace_bytes) return GQA_ERR_WORKSPACE_TOO_SMALL;
  char *base = static_cast<char *>(workspace);
  int32_t *count = reinterpret_cast<int32_t *>(base + g.off_count);

  // the selection attended as a cache of at most sel_cap keys: the partition
  // launch's work-groups select from the index rows themselves and write
  // each sequence's selection size for the combine
  const gqa::StepParams ep =
      final_epilogue(&g.vcache, g.plan, carry_in, carry_out, out);
  const double sc =
      scale != 0.0f ? (double)scale : 1.0 / std::sqrt((double)cache->dk);
  PartitionArgs a;
  a.q = q;
  a.k = cache->k;
  a.v = cache->v;
  a.lens = lens;
  a.batch = cache->batch;
  a.max_len = g.sel_cap;
  a.num_kv_heads = cache->num_kv_heads;
  a.hpk = num_q_heads / cache->num_kv_heads;
  a.dk = cache->dk;
  a.dv = cache->dv;
  a.chunk_tokens = g.plan.chunk_tokens;
  a.num_chunks = g.plan.num_chunks;
  single_branch(&a);
  set_storage(&a, cache);
  a.idx = idx;
  a.width = width;
  a.sel_count = count;
  a.cache_len = cache->max_len;
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  a.bias = nullptr;
  a.bias_stride = 0;
  a.has_bias = 0;
  a.part_m = reinterpret_cast<float *>(base);
  a.part_l = reinterpret_cast<float *>(base + g.plan.off_l);
  a.part_acc = reinterpret_cast<float *>(base + g.plan.off_acc);
  a.sched = nullptr;
  a.sched_len = 0;
  st = device_status(launch_partition(cache, a, ep, stream));
  if (st != GQA_OK || ep.direct) return st;
  return combine_checked(num_q_heads, &g.vcache, count, &g.plan, workspace,
                         carry_in, carry_out, out, stream);
}

size_t gqa_decode_step_workspace_bytes(const gqa_cache *cache,
                                       int32_t num_q_heads) {
  gqa_plan p;
  if (make_plan(cache, num_q_heads, 0, &p) != GQA_OK) return 0;
  return p.workspace_bytes + step_counter_bytes(cache);
}

gqa_status gqa_decode_step(const void *q, int32_t num_q_heads,
                           const gqa_cache *cache, const void *k_new,
                           const void *v_new, const int32_t *lens_in,
                           int32_t *lens_out, int32_t *dropped, float scale,
                           const float *bias, int64_t bias_stride,
                           const gqa_carry *carry_in,
                           const gqa_carry *carry_out, float *out,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  gqa_status st = check_attend_args(q, num_q_heads, cache, lens_in, scale);
  if (st != GQA_OK) return st;
  if ((st = check_combine_args(num_q_heads, cache, lens_in, carry_in,
                               carry_out, out)) != GQA_OK)
    return st;
  if ((st = check_bias(cache, bias, bias_stride)) != GQA_OK) return st;
  if (!k_new || !v_new || !lens_out || lens_out == lens_in)
    return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned16(k_new) || !aligned16(v_new)) return GQA_ERR_INVALID_ARGUMENT;
  gqa_plan plan;
  if ((st = make_plan(cache, num_q_heads, 0, &plan)) != GQA_OK) return st;
  if (!workspace || !aligned16(workspace)) return GQA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < plan.workspace_bytes + step_counter_bytes(cache))
    return GQA_ERR_WORKSPACE_TOO_SMALL;

  if (!uses_mfma(cache)) {  // vector-ALU shapes: the same step as three launches
    st = gqa_kv_append(cache, k_new, v_new, lens_in, lens_out, dropped, stream);
    if (st != GQA_OK) return st;
    st = partition_checked(q, num_q_heads, cache, lens_out, scale, bias,
                           bias_stride, &plan, workspace, gqa::StepParams{},
                           stream);
    if (st != GQA_OK) return st;
    return combine_checked(num_q_heads, cache, lens_out, &plan, workspace,
                           carry_in, carry_out, out, stream);
  }

  const double sc =
      scale != 0.0f ? (double)scale : 1.0 / std::sqrt((double)cache->dk);
  PartitionArgs a;
  a.q = q;
  a.k = cache->k;
  a.v = cache->v;
  a.lens = lens_in;
  a.batch = cache->batch;
  a.max_len = cache->max_len;
  a.num_kv_heads = cache->num_kv_heads;
  a.hpk = num_q_heads / cache->num_kv_heads;
  a.dk = cache->dk;
  a.dv = cache->dv;
  a.chunk_tokens = plan.chunk_tokens;
  a.num_chunks = plan.num_chunks;
  single_branch(&a);
  set_storage(&a, cache);
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  a.bias = bias;
  a.bias_stride = bias ? bias_stride : 0;
  a.has_bias = bias ? 1 : 0;
  char *base = static_cast<char *>(workspace);
  a.part_m = reinterpret_cast<float *>(base);
  a.part_l = reinterpret_cast<float *>(base + plan.off_l);
  a.part_acc = reinterpret_cast<float *>(base + plan.off_acc);

  if ((st = schedule_checked(cache, plan, lens_in, true, lens_out, dropped,
                             workspace, &a, stream)) != GQA_OK)
    return st;
  gqa::StepParams sp = final_epilogue(cache, plan, carry_in, carry_out, out);
  sp.k_new = k_new;
  sp.v_new = v_new;
  sp.lens_in = lens_in;
  sp.lens_out = lens_out;
  sp.dropped = dropped;
  sp.counters = reinterpret_cast<int *>(base + plan.workspace_bytes);
  sp.fuse = !sp.direct && step_fuses(cache, num_q_heads, plan) ? 1 : 0;
  st = device_status(launch_step(cache, a, sp, stream));
  if (st != GQA_OK || sp.fuse || finished_in_partition(plan, sp)) return st;
  return combine_checked(num_q_heads, cache, lens_out, &plan, workspace,
                         carry_in, carry_out, out, stream);
}

}  // extern "C"
