// MFMA dequant-GEMM launcher: picks the instantiation for the code width, the group size
// and the gated epilogue (the kernel is in gemm_kernel.hpp; each instantiation is compiled
// in its own gemm_i<bits>_*.hip, so the build compiles them in parallel).
#include "gemm_kernel.hpp"

namespace awq {

void launch_gemm4_plain(dim3 grid, const uint16_t* X, int64_t M, const uint32_t* qweight,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t mt, int64_t nt, int64_t per_xcd, hipStream_t stream);
void launch_gemm4_gated(dim3 grid, const uint16_t* X, int64_t M, const uint32_t* qweight,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t mt, int64_t nt, int64_t per_xcd, hipStream_t stream);
void launch_gemm4_plain_g32(dim3 grid, const uint16_t* X, int64_t M, const uint32_t* qweight,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t mt, int64_t nt, int64_t per_xcd, hipStream_t stream);
void launch_gemm4_gated_g32(dim3 grid, const uint16_t* X, int64_t M, const uint32_t* qweight,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t mt, int64_t nt, int64_t per_xcd, hipStream_t stream);
void launch_gemm8_plain(dim3 grid, const uint16_t* X, int64_t M, const uint32_t* qweight,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t mt, int64_t nt, int64_t per_xcd, hipStream_t stream);
void launch_gemm8_gated(dim3 grid, const uint16_t* X, int64_t M, const uint32_t* qweight,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t mt, int64_t nt, int64_t per_xcd, hipStream_t stream);
void launch_gemm3_plain(dim3 grid, const uint16_t* X, int64_t M, const uint32_t* qweight,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t mt, int64_t nt, int64_t per_xcd, hipStream_t stream);
void launch_gemm3_gated(dim3 grid, const uint16_t* X, int64_t M, const uint32_t* qweight,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t mt, int64_t nt, int64_t per_xcd, hipStream_t stream);
void launch_gemm3_plain_g32(dim3 grid, const uint16_t* X, int64_t M, const uint32_t* qweight,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t mt, int64_t nt, int64_t per_xcd, hipStream_t stream);
void launch_gemm3_gated_g32(dim3 grid, const uint16_t* X, int64_t M, const uint32_t* qweight,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t mt, int64_t nt, int64_t per_xcd, hipStream_t stream);

hipError_t launch_gemm(const uint16_t* X, int64_t M, const uint32_t* qweight,
                       const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                       int group, int w_bit, uint16_t* Y, bool gated, hipStream_t stream) {
  const int64_t mt = (M + kBM - 1) / kBM;
  const int64_t nt = gated ? (N / 2 + kBN / 2 - 1) / (kBN / 2) : (N + kBN - 1) / kBN;
  const int64_t per_xcd = (mt * nt + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(per_xcd * kXcds));
  // 8-bit: one form for every group size (both lane halves' scales are loaded); 4- and
  // 3-bit: 32-channel groups (two scales per lane half) take the SPLIT form
  auto* f = w_bit == 8   ? (gated ? launch_gemm8_gated : launch_gemm8_plain)
            : w_bit == 3 ? (group == 32 ? (gated ? launch_gemm3_gated_g32 : launch_gemm3_plain_g32)
                                        : (gated ? launch_gemm3_gated : launch_gemm3_plain))
                         : (group == 32 ? (gated ? launch_gemm4_gated_g32 : launch_gemm4_plain_g32)
                                        : (gated ? launch_gemm4_gated : launch_gemm4_plain));
  f(grid, X, M, qweight, scales, zeros, N, K, group, Y, mt, nt, per_xcd, stream);
  return hipGetLastError();
}

}  // namespace awq
