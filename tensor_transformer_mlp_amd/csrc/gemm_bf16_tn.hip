// bf16 GEMM instantiations for the kTN operand layout (see gemm_bf16_impl.h).
#include "gemm_bf16_impl.h"

namespace tpmlp {

hipError_t launch_bf16_tn(int tile, const GemmParams& p, Epilogue epi, bool gsum, hipStream_t s) {
  return launch_bf16_layout_tile<kTN>(tile, p, epi, gsum, s);
}

}  // namespace tpmlp
