// Chunked-prefill attention (MFMA).  Placeholder until the matrix-core kernel
// lands: the entry point reports "unsupported".
#include "common.h"
#include "kernels.h"

namespace vp {

hipError_t launch_prefill(const PrefillParams&, int, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace vp
