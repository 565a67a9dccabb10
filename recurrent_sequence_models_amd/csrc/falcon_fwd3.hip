// Chunked forward pass of Falcon-3 / 3A (window of Bw pairs) on gfx950.
#include "falcon_kernels.h"

namespace falcon {

hipError_t launch_chunk_fwd_window(int variant, bool bf16, int dk, int dv, int chunk, int nsplit,
                                   const FwdArgs &a, hipStream_t s) {
  (void)variant; (void)bf16; (void)dk; (void)dv; (void)chunk; (void)nsplit; (void)a; (void)s;
  return hipErrorInvalidValue;
}

}  // namespace falcon
