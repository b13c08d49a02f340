// Data conditions of the linear path: NaN or Inf in the activations or the group scales.
//
// "AWQ量化技术Skill", "如何使用该技能 / 步骤 2": the model runs in fp16 on the packed
// format (quant_config, group scales); a non-finite activation or scale makes every output
// it reaches unspecified, so the linear entry points report it in the caller's flags word.
// The scan runs only when the caller passes that word, as its own launch ahead of the
// linear kernel: the linear kernels themselves carry no check. HBM-bound: 2 bytes per
// scanned element, 16 bytes per thread per step of a grid-stride loop, one vector atomic
// per wave that met a non-finite value.
#include "common.hpp"
#include "launch.hpp"

namespace awq {

// 1 when either fp16 half of w has the all-ones exponent (Inf or NaN), else 0
__device__ __forceinline__ uint32_t nonfinite_pair(uint32_t w) {
  return (uint32_t)((w & 0x7C00u) == 0x7C00u) | (uint32_t)((w & 0x7C000000u) == 0x7C000000u);
}

// Scans a (n elements, n % 8 == 0, 16-byte aligned) and b (m elements, any m, 2-byte
// aligned) for fp16 Inf / NaN.
__global__ void __launch_bounds__(256)
    k_nonfinite_scan(const uint16_t* __restrict__ a, int64_t n, const uint16_t* __restrict__ b,
                     int64_t m, uint32_t* __restrict__ flags) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  bool bad = false;
  for (int64_t i = tid; i < n / 8; i += stride) {
    const uint4 v = *reinterpret_cast<const uint4*>(a + i * 8);
    bad |= (nonfinite_pair(v.x) | nonfinite_pair(v.y) | nonfinite_pair(v.z) | nonfinite_pair(v.w)) != 0;
  }
  for (int64_t i = tid; i < m; i += stride) bad |= (b[i] & 0x7C00u) == 0x7C00u;
  const uint64_t hit = __builtin_amdgcn_ballot_w64(bad);
  if (hit && (threadIdx.x & 63) == (int)__builtin_ctzll(hit)) atomicOr(flags, AWQ_FLAG_NONFINITE_INPUT);
}

hipError_t launch_nonfinite_scan(const uint16_t* a, int64_t n, const uint16_t* b, int64_t m,
                                 uint32_t* flags, hipStream_t stream) {
  const int64_t work = (n / 8 > m ? n / 8 : m);
  int64_t blocks = (work + 255) / 256;
  if (blocks > 2048) blocks = 2048;  // 8 blocks per CU: enough loads in flight
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_nonfinite_scan, dim3((unsigned)blocks), dim3(256), 0, stream, a, n, b, m,
                     flags);
  return hipGetLastError();
}

}  // namespace awq
