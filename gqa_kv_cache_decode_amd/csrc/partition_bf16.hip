// Partition launches for bf16 caches (kernel in partition_mfma16.h).
#include "partition_mfma16.h"

namespace gqa {

bool partition_bf16_supported(int dk, int dv, int hpk) {
  if (hpk < 1 || hpk > 16) return false;
  return (dk == 64 && dv == 64) || (dk == 128 && dv == 128) ||
         (dk == 192 && dv == 128) || (dk == 256 && dv == 256);
}

hipError_t launch_partition_bf16(const PartitionArgs &a, const StepParams &ep,
                                 hipStream_t s) {
  return dispatch<false, false>(a, ep, s);
}

hipError_t launch_step_bf16(const PartitionArgs &a, const StepParams &sp,
                            hipStream_t s) {
  return dispatch<true, false>(a, sp, s);
}

}  // namespace gqa
