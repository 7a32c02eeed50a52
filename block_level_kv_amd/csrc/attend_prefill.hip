// bf16 MFMA attention tiles for query chunks (head_dim 128).
#include "common.h"
#include "kernels.h"

namespace infllm {

bool prefill_supported(const AttendArgs& a) { (void)a; return false; }
int prefill_num_splits(const AttendArgs& a) { (void)a; return 1; }
hipError_t launch_attend_prefill(const AttendArgs& a, int splits, hipStream_t st) {
  (void)a; (void)splits; (void)st;
  return hipErrorNotSupported;
}

}  // namespace infllm
