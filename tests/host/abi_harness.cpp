// Host-only harness for the library's C ABI (gqa_kv_cache_decode_amd/csrc/
// abi.cpp), built with the address and undefined-behaviour sanitizers and no
// device code.  The kernel launchers the ABI calls are replaced here by
// checks: every buffer a launch names must lie inside one of the caller's
// buffers at the extent its kernel reads or writes (inputs, outputs and the
// workspace), and the launch's plan must cover the keys.  Device pointers are
// addresses in a made-up address space (nothing is dereferenced on the host),
// so shapes of any size cost nothing.
//
// Usage:
//   abi_harness sweep SEED ITERATIONS < support_table
//   abi_harness plans SEED COUNT      < support_table
// The support table lists "dtype dk dv hpk" for every kernel shape the
// compiled library accepts (as its gqa_attend_plan reports them); the
// stand-in support functions below answer from it.  `sweep` calls every
// entry point on random shapes and prints "violations N" (exit status 1 when
// N > 0 or a valid call is refused); `plans` prints random plan queries and
// their results for comparison against the compiled library.
#include <algorithm>
#include <cinttypes>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "gqa_decode.h"
#include "launch.h"

namespace {

// ---- the made-up device address space ------------------------------------

struct Buffer {
  uintptr_t addr;
  size_t bytes;
  std::string name;
};

std::vector<Buffer> g_buffers;
uintptr_t g_next = (uintptr_t)1 << 40;
long g_violations = 0, g_launches = 0;
// partition launches seen, by kind
long g_balanced = 0, g_scheduled = 0, g_gathered = 0, g_branches = 0,
     g_steps = 0, g_fused = 0, g_direct = 0;
std::string g_case;  // the current call, for messages

void violation(const char *fmt, ...) {
  ++g_violations;
  if (g_violations > 20) return;
  va_list ap;
  va_start(ap, fmt);
  std::fprintf(stderr, "VIOLATION [%s]: ", g_case.c_str());
  std::vfprintf(stderr, fmt, ap);
  std::fprintf(stderr, "\n");
  va_end(ap);
}

void reset_buffers() {
  g_buffers.clear();
  g_next = (uintptr_t)1 << 40;
}

// A buffer of `bytes` at a 256-byte aligned address, with a gap after it.
void *fake(size_t bytes, const char *name) {
  const uintptr_t a = g_next;
  g_next += (bytes + 4096 + 255) / 256 * 256;
  g_buffers.push_back({a, bytes, name});
  return reinterpret_cast<void *>(a);
}

// The extent [p, p + bytes) must lie in one caller buffer (bytes = 0: any p).
void need(const void *p, size_t bytes, const char *what) {
  if (bytes == 0) return;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (!p) {
    violation("%s: NULL for %zu bytes", what, bytes);
    return;
  }
  for (const Buffer &b : g_buffers)
    if (a >= b.addr && a < b.addr + b.bytes + 1) {
      if (a + bytes > b.addr + b.bytes)
        violation("%s: %zu bytes at +%zu overrun %s (%zu bytes)", what, bytes,
                  (size_t)(a - b.addr), b.name.c_str(), b.bytes);
      return;
    }
  violation("%s: %zu bytes at %#" PRIxPTR " in no buffer", what, bytes, a);
}

// ---- the support table (the compiled library's shapes) --------------------

std::set<std::tuple<int, int, int, int>> g_support;  // dtype, dk, dv, hpk

bool supported(int dtype, int dk, int dv, int hpk) {
  return g_support.count({dtype, dk, dv, hpk}) != 0;
}

}  // namespace

// ---- stand-ins for the device translation units ----------------------------

namespace gqa {

bool partition_bf16_supported(int dk, int dv, int hpk) {
  return supported(GQA_DTYPE_BF16, dk, dv, hpk);
}
bool partition_f32_supported(int dk, int dv, int hpk) {
  return supported(GQA_DTYPE_F32, dk, dv, hpk);
}
// The fp32 matrix-core shapes are the bf16 kernel's shapes (partition_f32.hip)
bool partition_f32_uses_mfma(int dk, int dv) {
  return (dk == 64 && dv == 64) || (dk == 128 && dv == 128) ||
         (dk == 192 && dv == 128) || (dk == 256 && dv == 256);
}

namespace {

size_t esize(int fp8, bool f32) { return f32 ? 4 : fp8 ? 1 : 2; }

// What a partition (or decode-step) launch reads and writes.
void check_partition(const PartitionArgs &a, const StepParams *sp, bool f32,
                     bool step) {
  ++g_launches;
  g_balanced += a.balanced != 0;
  g_scheduled += a.sched != nullptr;
  g_gathered += a.idx != nullptr;
  g_branches += a.num_extra > 0;
  g_steps += step;
  g_fused += step && sp && sp->fuse;
  g_direct += sp && sp->direct;
  const size_t B = a.batch, Hkv = a.num_kv_heads, hpk = a.hpk;
  const size_t rows = B * Hkv * hpk, es = esize(a.fp8, f32);
  const size_t qes = f32 ? 4 : 2;
  if (a.batch <= 0 || a.num_kv_heads <= 0 || a.hpk <= 0 || a.chunk_tokens <= 0 ||
      a.num_chunks <= 0)
    violation("partition: empty shape");
  need(a.q, rows * a.dk * qes, "q");
  need(a.k, B * a.cache_len * Hkv * a.dk * es, "k");
  need(a.v, B * a.cache_len * Hkv * a.dv * es, "v");
  if (!step) need(a.lens, B * 4, "lens");
  if (a.fp8) {
    need(a.k_scale, B * Hkv * 4, "k_scale");
    need(a.v_scale, B * Hkv * 4, "v_scale");
  }
  if (a.bias) {
    if (a.bias_stride < a.max_len) violation("bias stride below max_len");
    need(a.bias, B * a.bias_stride * 4, "bias");
  }
  if (a.idx) {
    need(a.idx, B * a.width * 4, "idx");
    need(a.sel_count, B * 4, "sel_count");
    if (a.max_len > a.cache_len || a.max_len > a.width)
      violation("gathered capacity %d above cache %d / width %d", a.max_len,
                a.cache_len, a.width);
  } else if (a.cache_len != a.max_len) {
    violation("cache_len %d != max_len %d", a.cache_len, a.max_len);
  }
  if (a.balanced) {
    // piece slots: num_chunks items of hpk rows; the queue in the workspace
    const size_t pieces = (size_t)a.num_chunks * hpk;
    need(a.part_m, pieces * 4, "piece m");
    need(a.part_l, pieces * 4, "piece l");
    need(a.part_acc, pieces * a.dv * 4, "piece acc");
    need(a.queue, (size_t)queue_runs_offset(a.batch) * 4, "queue head");
    if (a.chunk_tokens != kBalanceTile) violation("balanced chunk_tokens");
    if (a.balanced % 8) violation("balanced work-groups not a multiple of 8");
  } else {
    if ((int64_t)a.chunk_tokens * a.num_chunks < a.max_len)
      violation("chunks %d x %d do not cover %d keys", a.num_chunks,
                a.chunk_tokens, a.max_len);
    if (a.col_base + a.num_chunks > a.total_cols) violation("partial columns");
    need(a.part_m, rows * a.total_cols * 4, "part_m");
    need(a.part_l, rows * a.total_cols * 4, "part_l");
    need(a.part_acc, rows * a.total_cols * a.dv * 4, "part_acc");
    size_t items = B * Hkv * a.num_chunks;
    for (int e = 0; e < a.num_extra; ++e) {
      const ExtraBranch &x = a.extra[e];
      need(x.k, B * x.max_len * Hkv * a.dk * es, "extra k");
      need(x.v, B * x.max_len * Hkv * a.dv * es, "extra v");
      need(x.lens, B * 4, "extra lens");
      if (x.bias) need(x.bias, B * x.bias_stride * 4, "extra bias");
      if (a.fp8) {
        need(x.k_scale, B * Hkv * 4, "extra k_scale");
        need(x.v_scale, B * Hkv * 4, "extra v_scale");
      }
      if ((int64_t)x.chunk_tokens * x.num_chunks < x.max_len)
        violation("extra branch chunks do not cover its keys");
      if (x.col_base + x.num_chunks > a.total_cols) violation("extra columns");
      if (x.item_base % 8 || (size_t)x.item_base < items)
        violation("extra item_base %d", x.item_base);
      items = x.item_base + B * Hkv * x.num_chunks;
    }
    if ((size_t)a.total_items < items) violation("total_items below the items");
    if (a.sched) need(a.sched, (size_t)a.sched_len * 4, "schedule table");
  }
  if (sp) {
    if (step) {
      const size_t nes = f32 ? 4 : 2;  // new rows: fp32, else bf16
      need(sp->k_new, B * Hkv * a.dk * nes, "k_new");
      need(sp->v_new, B * Hkv * a.dv * nes, "v_new");
      need(sp->lens_in, B * 4, "lens_in");
      need(sp->lens_out, B * 4, "lens_out");
      if (sp->lens_in == sp->lens_out) violation("lens_out aliases lens_in");
      if (sp->dropped) need(sp->dropped, 4, "dropped");
      if (sp->fuse) need(sp->counters, B * Hkv * 4, "counters");
    }
    if (sp->in_l) {
      need(sp->in_m, rows * 4, "carry_in m");
      need(sp->in_l, rows * 4, "carry_in l");
      need(sp->in_acc, rows * a.dv * 4, "carry_in acc");
    }
    if (sp->out_l) {
      need(sp->out_m, rows * 4, "carry_out m");
      need(sp->out_l, rows * 4, "carry_out l");
      need(sp->out_acc, rows * a.dv * 4, "carry_out acc");
    }
    if (sp->out) need(sp->out, rows * a.dv * 4, "out");
    if (sp->direct && a.num_chunks != 1) violation("direct with several chunks");
  }
}

}  // namespace

hipError_t launch_partition_bf16(const PartitionArgs &a, const StepParams &ep,
                                 hipStream_t) {
  check_partition(a, &ep, false, false);
  return hipSuccess;
}
hipError_t launch_partition_f32(const PartitionArgs &a, const StepParams &ep,
                                hipStream_t) {
  check_partition(a, &ep, true, false);
  return hipSuccess;
}
hipError_t launch_partition_fp8(const PartitionArgs &a, const StepParams &ep,
                                hipStream_t) {
  if (!a.fp8) violation("fp8 launch without the fp8 flag");
  check_partition(a, &ep, false, false);
  return hipSuccess;
}
hipError_t launch_step_bf16(const PartitionArgs &a, const StepParams &sp,
                            hipStream_t) {
  check_partition(a, &sp, false, true);
  return hipSuccess;
}
hipError_t launch_step_fp8(const PartitionArgs &a, const StepParams &sp,
                           hipStream_t) {
  check_partition(a, &sp, false, true);
  return hipSuccess;
}
hipError_t launch_step_f32(const PartitionArgs &a, const StepParams &sp,
                           hipStream_t) {
  check_partition(a, &sp, true, true);
  return hipSuccess;
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t) {
  ++g_launches;
  const size_t rows = (size_t)a.batch * a.num_q_heads;
  if (a.balanced) {
    // the pieces' extent is checked at the partition launch; here the queue
    need(a.queue, (size_t)queue_runs_offset(a.batch) * 4, "combine queue");
    if (a.hpk <= 0 || a.num_q_heads % a.hpk) violation("combine hpk");
    need(a.part_m, 4, "combine piece m");
  } else {
    need(a.part_m, rows * a.total_cols * 4, "combine part_m");
    need(a.part_l, rows * a.total_cols * 4, "combine part_l");
    need(a.part_acc, rows * a.total_cols * a.dv * 4, "combine part_acc");
    for (int i = 0; i < a.num_branches; ++i) {
      const CombineBranch &br = a.br[i];
      need(br.lens, (size_t)a.batch * 4, "combine lens");
      const int64_t cols = ((int64_t)br.max_len + br.chunk_tokens - 1) / br.chunk_tokens;
      if (br.col_base + cols > a.total_cols) violation("combine branch columns");
    }
  }
  if (a.in_l) {
    need(a.in_m, rows * 4, "combine carry_in m");
    need(a.in_l, rows * 4, "combine carry_in l");
    need(a.in_acc, rows * a.dv * 4, "combine carry_in acc");
  }
  if (a.out_l) {
    need(a.out_m, rows * 4, "combine carry_out m");
    need(a.out_l, rows * 4, "combine carry_out l");
    need(a.out_acc, rows * a.dv * 4, "combine carry_out acc");
  }
  if (a.out) need(a.out, rows * a.dv * 4, "combine out");
  if (!a.out && !a.out_l) violation("combine writes nothing");
  return hipSuccess;
}

namespace {
void check_schedule(const ScheduleArgs &a, const char *what) {
  ++g_launches;
  need(a.lens, (size_t)a.batch * 4, what);
  if (a.step) {
    need(a.lens_out, (size_t)a.batch * 4, "schedule lens_out");
    if (a.dropped) need(a.dropped, 4, "schedule dropped");
  }
  need(a.table, (size_t)a.table_len * 4, "schedule table");
}
}  // namespace

hipError_t launch_schedule(const ScheduleArgs &a, hipStream_t) {
  check_schedule(a, "schedule lens");
  return hipSuccess;
}
hipError_t launch_balance(const ScheduleArgs &a, hipStream_t) {
  check_schedule(a, "balance lens");
  if (a.table_len < queue_runs_offset(a.batch))
    violation("queue of %d words below its head", a.table_len);
  return hipSuccess;
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t) {
  ++g_launches;
  const size_t r = (size_t)a.rows, dv = a.dv;
  need(a.a_m, r * 4, "merge a.m");
  need(a.a_l, r * 4, "merge a.l");
  need(a.a_acc, r * dv * 4, "merge a.acc");
  need(a.b_m, r * 4, "merge b.m");
  need(a.b_l, r * 4, "merge b.l");
  need(a.b_acc, r * dv * 4, "merge b.acc");
  need(a.d_m, r * 4, "merge dst.m");
  need(a.d_l, r * 4, "merge dst.l");
  need(a.d_acc, r * dv * 4, "merge dst.acc");
  if (a.out) need(a.out, r * dv * 4, "merge out");
  return hipSuccess;
}

hipError_t launch_append(const AppendArgs &a, hipStream_t) {
  ++g_launches;
  const size_t B = a.batch;
  need(a.k, B * a.max_len * a.row_bytes_k, "append k");
  need(a.v, B * a.max_len * a.row_bytes_v, "append v");
  // fp8: new rows are bf16, two bytes per code of the row
  const size_t nk = a.fp8 ? (size_t)a.row_bytes_k * 2 : a.row_bytes_k;
  const size_t nv = a.fp8 ? (size_t)a.row_bytes_v * 2 : a.row_bytes_v;
  need(a.k_new, B * nk, "append k_new");
  need(a.v_new, B * nv, "append v_new");
  need(a.lens_in, B * 4, "append lens_in");
  need(a.lens_out, B * 4, "append lens_out");
  if (a.dropped) need(a.dropped, 4, "append dropped");
  if (a.fp8) {
    need(a.k_scale, B * a.num_kv_heads * 4, "append k_scale");
    need(a.v_scale, B * a.num_kv_heads * 4, "append v_scale");
  }
  return hipSuccess;
}

hipError_t launch_stream_append(const StreamAppendArgs &a, hipStream_t) {
  ++g_launches;
  const size_t B = a.batch, rk = a.row_bytes_k, rv = a.row_bytes_v;
  if (a.sink) {
    need(a.sink_k, B * a.sink * rk, "sink k");
    need(a.sink_v, B * a.sink * rv, "sink v");
  }
  need(a.ring_k, B * a.window * rk, "ring k");
  need(a.ring_v, B * a.window * rv, "ring v");
  if (a.main_k) {
    need(a.main_k, B * a.main_len * rk, "main k");
    need(a.main_v, B * a.main_len * rv, "main v");
  }
  const size_t nk = a.fp8 ? rk * 2 : rk, nv = a.fp8 ? rv * 2 : rv;
  need(a.k_new, B * nk, "stream k_new");
  need(a.v_new, B * nv, "stream v_new");
  need(a.count_in, B * 4, "count_in");
  need(a.count_out, B * 4, "count_out");
  need(a.lens_ring, B * 4, "lens_ring");
  if (a.lens_sink) need(a.lens_sink, B * 4, "lens_sink");
  if (a.lens_main) need(a.lens_main, B * 4, "lens_main");
  if (a.dropped) need(a.dropped, 4, "stream dropped");
  if (a.fp8) {
    need(a.k_scale, B * a.num_kv_heads * 4, "stream k_scale");
    need(a.v_scale, B * a.num_kv_heads * 4, "stream v_scale");
  }
  return hipSuccess;
}

}  // namespace gqa

// The profiling request's event records (abi.cpp's only HIP runtime call).
extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
  return hipSuccess;
}

// ---- random calls ------------------------------------------------------------

namespace {

std::mt19937_64 g_rng;

int pick(int lo, int hi) {  // inclusive
  return std::uniform_int_distribution<int>(lo, hi)(g_rng);
}
bool chance(double p) { return std::uniform_real_distribution<double>(0, 1)(g_rng) < p; }

// A length spread over several orders of magnitude.
int length(int hi) {
  const double e = std::uniform_real_distribution<double>(0, std::log2((double)hi))(g_rng);
  return std::max(1, std::min(hi, (int)std::exp2(e)));
}

struct Shape {
  int dtype, dk, dv, hpk, hkv, batch, max_len;
};

std::vector<std::tuple<int, int, int, int>> g_support_list;

Shape random_shape() {
  Shape s;
  const auto &t = g_support_list[pick(0, (int)g_support_list.size() - 1)];
  s.dtype = std::get<0>(t);
  s.dk = std::get<1>(t);
  s.dv = std::get<2>(t);
  s.hpk = std::get<3>(t);
  const int hkvs[] = {1, 2, 3, 4, 8, 16};
  s.hkv = hkvs[pick(0, 5)];
  s.batch = chance(0.1) ? pick(1, 9000) : pick(1, 96);
  s.max_len = chance(0.1) ? length(1 << 21) : length(70000);
  return s;
}

size_t esz(int dtype) { return dtype == GQA_DTYPE_F32 ? 4 : dtype == GQA_DTYPE_BF16 ? 2 : 1; }

gqa_cache make_cache(const Shape &s, int max_len, const char *tag) {
  gqa_cache c;
  std::memset(&c, 0, sizeof c);
  const size_t tok = (size_t)s.hkv * esz(s.dtype);
  c.k = fake((size_t)s.batch * max_len * tok * s.dk, tag);
  c.v = fake((size_t)s.batch * max_len * tok * s.dv, tag);
  c.batch = s.batch;
  c.max_len = max_len;
  c.num_kv_heads = s.hkv;
  c.dk = s.dk;
  c.dv = s.dv;
  c.dtype = s.dtype;
  if (s.dtype == GQA_DTYPE_FP8_E4M3) {
    c.k_scale = static_cast<const float *>(fake((size_t)s.batch * s.hkv * 4, "k_scale"));
    c.v_scale = static_cast<const float *>(fake((size_t)s.batch * s.hkv * 4, "v_scale"));
  }
  return c;
}

gqa_carry make_carry(size_t rows, int dv, const char *tag) {
  gqa_carry x;
  x.m = static_cast<float *>(fake(rows * 4, tag));
  x.l = static_cast<float *>(fake(rows * 4, tag));
  x.acc = static_cast<float *>(fake(rows * dv * 4, tag));
  return x;
}

long g_calls = 0, g_refused = 0;

// A call that must succeed (valid arguments, and every launch is a stand-in).
void expect_ok(gqa_status st, const char *what) {
  ++g_calls;
  if (st != GQA_OK) {
    ++g_refused;
    violation("%s refused a valid call: %s", what, gqa_status_string(st));
  }
}

void expect_status(gqa_status st, gqa_status want, const char *what) {
  ++g_calls;
  if (st != want)
    violation("%s: %s, expected %s", what, gqa_status_string(st),
              gqa_status_string(want));
}

void one_case() {
  reset_buffers();
  const Shape s = random_shape();
  const int hq = s.hpk * s.hkv;
  char buf[160];
  std::snprintf(buf, sizeof buf, "dtype %d dk %d dv %d hpk %d hkv %d B %d T %d",
                s.dtype, s.dk, s.dv, s.hpk, s.hkv, s.batch, s.max_len);
  g_case = buf;
  gqa_cache c = make_cache(s, s.max_len, "cache");
  const size_t rows = (size_t)s.batch * hq;
  const size_t qes = s.dtype == GQA_DTYPE_F32 ? 4 : 2;
  const void *q = fake(rows * s.dk * qes, "q");
  const int32_t *lens = static_cast<const int32_t *>(fake((size_t)s.batch * 4, "lens"));
  float *out = static_cast<float *>(fake(rows * s.dv * 4, "out"));
  const float *bias = nullptr;
  int64_t bias_stride = 0;
  if (chance(0.3)) {
    bias_stride = (s.max_len + 3) / 4 * 4 + 4 * pick(0, 2);
    bias = static_cast<const float *>(fake((size_t)s.batch * bias_stride * 4, "bias"));
  }
  gqa_carry cin = make_carry(rows, s.dv, "carry_in");
  gqa_carry cout = make_carry(rows, s.dv, "carry_out");
  const gqa_carry *pin = chance(0.4) ? &cin : nullptr;
  const gqa_carry *pout = chance(0.5) ? &cout : nullptr;

  // plan query (the library's plan, or a chosen chunk, or balanced)
  int32_t chunk = 0;
  if (chance(0.15)) chunk = GQA_CHUNK_BALANCED;
  else if (chance(0.2)) chunk = 64 * pick(1, 64);
  gqa_plan plan;
  const gqa_status pst = gqa_attend_plan(&c, hq, chunk, &plan);
  const bool balanced_ok = s.dtype != GQA_DTYPE_F32 ||
                           gqa::partition_f32_uses_mfma(s.dk, s.dv);
  if (pst != GQA_OK) {
    // refusals the ABI documents: a balanced plan the shape does not allow,
    // 32-bit overflow of a huge shape
    ++g_calls;
    if (!(pst == GQA_ERR_UNSUPPORTED)) violation("plan refused: %s", gqa_status_string(pst));
    (void)balanced_ok;
  } else {
    // partition + combine on the caller's plan
    void *ws = fake(plan.workspace_bytes, "workspace");
    expect_ok(gqa_attend_partition(q, hq, &c, lens, 0.0f, bias, bias_stride, &plan,
                                   ws, plan.workspace_bytes, nullptr),
              "attend_partition");
    expect_ok(gqa_attend_combine(hq, &c, lens, &plan, ws, plan.workspace_bytes, pin,
                                 pout, out, nullptr),
              "attend_combine");
    if (plan.workspace_bytes > 0)
      expect_status(gqa_attend_partition(q, hq, &c, lens, 0.0f, bias, bias_stride,
                                         &plan, ws, plan.workspace_bytes - 1, nullptr),
                    GQA_ERR_WORKSPACE_TOO_SMALL, "short workspace");
  }

  // whole attend with the library's own workspace size
  const size_t wsb = gqa_attend_workspace_bytes(&c, hq);
  if (wsb > 0) {
    void *ws = fake(wsb, "attend workspace");
    expect_ok(gqa_attend_decode(q, hq, &c, lens, 0.0f, bias, bias_stride, pin, pout,
                                out, ws, wsb, nullptr),
              "attend_decode");
    // a misaligned q is refused before any launch
    const long before = g_launches;
    expect_status(gqa_attend_decode(static_cast<const char *>(q) + 2, hq, &c, lens,
                                    0.0f, bias, bias_stride, pin, pout, out, ws, wsb,
                                    nullptr),
                  GQA_ERR_INVALID_ARGUMENT, "misaligned q");
    if (g_launches != before) violation("a refused call launched");
  }

  // decode step (matrix-core shapes, and the fp32 vector family)
  const size_t swb = gqa_decode_step_workspace_bytes(&c, hq);
  if (swb > 0) {
    void *ws = fake(swb, "step workspace");
    const size_t nes = s.dtype == GQA_DTYPE_F32 ? 4 : 2;
    const void *kn = fake((size_t)s.batch * s.hkv * s.dk * nes, "k_new");
    const void *vn = fake((size_t)s.batch * s.hkv * s.dv * nes, "v_new");
    int32_t *lo = static_cast<int32_t *>(fake((size_t)s.batch * 4, "lens_out"));
    int32_t *dropped = static_cast<int32_t *>(fake(4, "dropped"));
    const gqa_status st =
        gqa_decode_step(q, hq, &c, kn, vn, lens, lo, chance(0.5) ? dropped : nullptr,
                        0.0f, bias, bias_stride, pin, pout, out, ws, swb, nullptr);
    if (st != GQA_ERR_UNSUPPORTED) expect_ok(st, "decode_step");
  }

  // index-gathered attend
  if (s.dtype != GQA_DTYPE_F32 || gqa::partition_f32_uses_mfma(s.dk, s.dv)) {
    const int width = chance(0.5) ? pick(1, 4096) : pick(1, 64);
    const size_t gwb = gqa_attend_gathered_workspace_bytes(&c, hq, width);
    if (gwb > 0) {
      void *ws = fake(gwb, "gather workspace");
      const int32_t *idx =
          static_cast<const int32_t *>(fake((size_t)s.batch * width * 4, "idx"));
      const gqa_status st = gqa_attend_gathered(q, hq, &c, lens, idx, width, 0.0f, pin,
                                                pout, out, ws, gwb, nullptr);
      if (st != GQA_ERR_UNSUPPORTED) expect_ok(st, "attend_gathered");
    }
  }

  // several branches of different lengths (matrix-core shapes)
  if (s.dtype != GQA_DTYPE_F32 || gqa::partition_f32_uses_mfma(s.dk, s.dv)) {
    const int nb = pick(2, GQA_MAX_BRANCHES);
    std::vector<gqa_branch> br(nb);
    for (int i = 0; i < nb; ++i) {
      const int len = i == 0 ? s.max_len : length(i == 1 ? 64 : 20000);
      br[i].cache = make_cache(s, len, "branch cache");
      br[i].lens = static_cast<const int32_t *>(fake((size_t)s.batch * 4, "branch lens"));
      br[i].bias = nullptr;
      br[i].bias_stride = 0;
      if (chance(0.3)) {
        br[i].bias_stride = (len + 3) / 4 * 4;
        br[i].bias = static_cast<const float *>(
            fake((size_t)s.batch * br[i].bias_stride * 4, "branch bias"));
      }
    }
    const size_t bwb = gqa_attend_branches_workspace_bytes(br.data(), nb, hq);
    if (bwb > 0) {
      void *ws = fake(bwb, "branches workspace");
      gqa_status st = gqa_attend_branches(q, hq, br.data(), nb, 0.0f, pin, pout, out,
                                          ws, bwb, nullptr);
      if (st != GQA_ERR_UNSUPPORTED) expect_ok(st, "attend_branches");
      const size_t nes = s.dtype == GQA_DTYPE_F32 ? 4 : 2;
      const void *kn = fake((size_t)s.batch * s.hkv * s.dk * nes, "k_new");
      const void *vn = fake((size_t)s.batch * s.hkv * s.dv * nes, "v_new");
      int32_t *lo = static_cast<int32_t *>(fake((size_t)s.batch * 4, "lens_out"));
      st = gqa_decode_step_branches(q, hq, br.data(), nb, pick(0, nb - 1), kn, vn, lo,
                                    nullptr, 0.0f, pin, pout, out, ws, bwb, nullptr);
      if (st != GQA_ERR_UNSUPPORTED) expect_ok(st, "decode_step_branches");
    }
  }

  // append and carry merge
  {
    const size_t nes = s.dtype == GQA_DTYPE_F32 ? 4 : 2;
    const void *kn = fake((size_t)s.batch * s.hkv * s.dk * nes, "k_new");
    const void *vn = fake((size_t)s.batch * s.hkv * s.dv * nes, "v_new");
    int32_t *lo = static_cast<int32_t *>(fake((size_t)s.batch * 4, "lens_out"));
    expect_ok(gqa_kv_append(&c, kn, vn, lens, lo, nullptr, nullptr), "kv_append");
    gqa_carry a = make_carry(rows, s.dv, "merge a"), b = make_carry(rows, s.dv, "merge b");
    expect_ok(gqa_softmax_state_merge(&a, &b, &a, (int64_t)rows, s.dv,
                                      chance(0.5) ? out : nullptr, nullptr),
              "softmax_state_merge");
  }
}

void read_support() {
  int dt, dk, dv, hpk;
  while (std::scanf("%d %d %d %d", &dt, &dk, &dv, &hpk) == 4) {
    g_support.insert({dt, dk, dv, hpk});
    g_support_list.push_back({dt, dk, dv, hpk});
  }
  if (g_support_list.empty()) {
    std::fprintf(stderr, "empty support table\n");
    std::exit(2);
  }
}

}  // namespace

int main(int argc, char **argv) {
  if (argc != 4) {
    std::fprintf(stderr, "usage: %s sweep|plans SEED N < support_table\n", argv[0]);
    return 2;
  }
  const std::string mode = argv[1];
  g_rng.seed(std::strtoull(argv[2], nullptr, 10));
  const long n = std::strtol(argv[3], nullptr, 10);
  read_support();
  if (mode == "plans") {
    for (long i = 0; i < n; ++i) {
      reset_buffers();
      const Shape s = random_shape();
      int32_t chunk = 0;
      if (chance(0.15)) chunk = GQA_CHUNK_BALANCED;
      else if (chance(0.2)) chunk = 64 * pick(1, 64);
      gqa_cache c = make_cache(s, s.max_len, "cache");
      gqa_plan p;
      std::memset(&p, 0, sizeof p);
      const gqa_status st = gqa_attend_plan(&c, s.hpk * s.hkv, chunk, &p);
      std::printf("%d %d %d %d %d %d %d %d -> %d %d %d %zu %zu %zu %d %zu %d\n", s.dtype,
                  s.dk, s.dv, s.hpk, s.hkv, s.batch, s.max_len, chunk, (int)st,
                  p.chunk_tokens, p.num_chunks, p.off_l, p.off_acc, p.off_sched,
                  p.sched_entries, p.workspace_bytes, p.balanced_groups);
    }
    return 0;
  }
  if (mode != "sweep") return 2;
  for (long i = 0; i < n; ++i) one_case();
  std::printf("kinds balanced %ld scheduled %ld gathered %ld branches %ld steps %ld "
              "fused %ld direct %ld\n",
              g_balanced, g_scheduled, g_gathered, g_branches, g_steps, g_fused,
              g_direct);
  std::printf("calls %ld launches %ld refused %ld violations %ld\n", g_calls, g_launches,
              g_refused, g_violations);
  return g_violations ? 1 : 0;
}
