// Partition launches for fp8 (E4M3) caches with per-(sequence, KV head)
// scales; the kernel (partition_mfma16.h) decodes codes to bf16 and has the
// bf16 family's head widths.
#include "partition_mfma16.h"

namespace gqa {

hipError_t launch_partition_fp8(const PartitionArgs &a, const StepParams &ep,
                                hipStream_t s) {
  return dispatch<false, true>(a, ep, s);
}

hipError_t launch_step_fp8(const PartitionArgs &a, const StepParams &sp,
                           hipStream_t s) {
  return dispatch<true, true>(a, sp, s);
}

}  // namespace gqa
