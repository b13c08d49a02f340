// One 3-bit instantiation of the MFMA dequant-GEMM (GATED = true, SPLIT = true: 32-channel groups),
// in a file of its own so that the build compiles the GEMM variants in parallel.
#include "gemm_kernel.hpp"

namespace awq {

void launch_gemm3_gated_g32(dim3 grid, const uint16_t* X, int64_t M, const uint32_t* qweight,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t mt, int64_t nt, int64_t per_xcd, hipStream_t stream) {
  hipLaunchKernelGGL((k_gemm<true, true, 3>), grid, dim3(256), 0, stream, X, M, qweight, scales,
                     zeros, N, K, group, Y, mt, nt, per_xcd);
}

}  // namespace awq
