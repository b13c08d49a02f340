// Equivalent transform (f2): fold 1/s into the producer of a linear's input.
//
// "AWQ量化实战" §2.2: the salient input channels of W are multiplied by s before the
// matrix is quantized and the other side is divided by s; "什么是激活感知权重量化（AWQ）",
// "工作机制": an equivalent transformation, X W^T = (X diag(1/s)) (W diag(s))^T. The
// division is applied where X is made: the activations or a norm weight (axis 1,
// A[r][k] / s_k) or the rows of the previous linear's weight (axis 0, A[k][j] / s_k).
//
// Elementwise and HBM-bound: each thread moves 8 fp16 (16 bytes) per step of a
// grid-stride loop; s is read through the cache. The fp32 quotient is correctly rounded
// and then rounded to fp16: with 24 >= 2 * 11 + 2 significand bits that double rounding
// equals the correctly rounded fp16 quotient, so results are bit-exact.
#include "common.hpp"
#include "launch.hpp"

namespace awq {

__global__ void __launch_bounds__(256)
    k_inverse_scale(const uint16_t* A, int64_t rows, int64_t cols, const uint16_t* s, int axis,
                    uint16_t* out, uint32_t* flags) {
  const int64_t chunks = rows * (cols / 8);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  bool overflow = false, nonfinite = false;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks; i += stride) {
    const int64_t r = i / (cols / 8);
    const int64_t c0 = (i - r * (cols / 8)) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(A + r * cols + c0);
    uint16_t sv[8];
    if (axis == 1) {
      const uint4 sw = *reinterpret_cast<const uint4*>(s + c0);
      const uint32_t w[4] = {sw.x, sw.y, sw.z, sw.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) sv[j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
    } else {
      const uint16_t sr = s[r];
#pragma unroll
      for (int j = 0; j < 8; ++j) sv[j] = sr;
    }
    const uint32_t a[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t pair = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float x = h2f((uint16_t)(a[j] >> (16 * h)));
        const float d = h2f(sv[2 * j + h]);
        const uint16_t q = f2h_bits(x / d);
        const bool fin = __builtin_isfinite(x) && __builtin_isfinite(d);
        nonfinite |= !fin;
        overflow |= fin && (q & 0x7C00u) == 0x7C00u;
        pair |= (uint32_t)q << (16 * h);
      }
      o[j] = pair;
    }
    *reinterpret_cast<uint4*>(out + r * cols + c0) = uint4{o[0], o[1], o[2], o[3]};
  }
  if (flags) {
    if (overflow) atomicOr(flags, AWQ_FLAG_OVERFLOW);
    if (nonfinite) atomicOr(flags, AWQ_FLAG_NONFINITE_INPUT);
  }
}

hipError_t launch_inverse_scale(const uint16_t* A, int64_t rows, int64_t cols, const uint16_t* s,
                                int axis, uint16_t* out, uint32_t* flags, hipStream_t stream) {
  const int64_t chunks = rows * (cols / 8);
  int64_t blocks = (chunks + 255) / 256;
  const int64_t cap = (int64_t)256 * 16;  // 16 blocks per CU: enough loads in flight
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(k_inverse_scale, dim3((unsigned)blocks), dim3(256), 0, stream, A, rows, cols,
                     s, axis, out, flags);
  return hipGetLastError();
}

}  // namespace awq
