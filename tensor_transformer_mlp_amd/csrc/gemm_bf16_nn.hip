// bf16 GEMM instantiations for the kNN operand layout (see gemm_bf16_impl.h).
#include "gemm_bf16_impl.h"

namespace tpmlp {

hipError_t launch_bf16_nn(int tile, const GemmParams& p, Epilogue epi, bool gsum, hipStream_t s) {
  return launch_bf16_layout_tile<kNN>(tile, p, epi, gsum, s);
}

}  // namespace tpmlp
