// Calibration probes for the rooflines: the chip's HBM read bandwidth and dense fp16
// matrix-core rate, measured on the box in the same process as the kernels they judge.
//
// Neither probe computes anything of the method. The read stream moves a buffer through
// the vector memory path the decode GEMV uses (16-byte loads, every CU busy) and folds it
// into one word, so the loads cannot be removed; the matrix loop issues independent
// v_mfma_f32_32x32x16_f16 chains from registers (the instruction of the GEMM and the
// searches) on every SIMD and stores one value per wave.
#include "awq_peaks.h"
#include "common.hpp"

namespace awq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// XOR of every 16-byte piece of buf (n16 pieces): block b covers pieces
// [b * 256 * U, (b + 1) * 256 * U), thread t pieces b * 256 * U + u * 256 + t (u < U), all U
// loads issued before any is used (each wave instruction moves 1 KiB of consecutive bytes).
template <int U>
__global__ void __launch_bounds__(256)
    k_read_stream(const uint4* __restrict__ buf, int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * 256;
    v[u] = i < n16 ? buf[i] : make_uint4(0, 0, 0, 0);
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  // one store per wave; the value depends on every load
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  if ((threadIdx.x & 63) == 0) sink[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = x;
}

// Each wave runs `iters` rounds of 8 independent 32x32x16 fp16 MFMAs (4 accumulators,
// two operand pairs) and stores one lane's sum, so nothing is dead code.
__global__ void __launch_bounds__(256) k_mfma_loop(int64_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  half8 a0, a1, b0, b1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a0[i] = (_Float16)(0.001f * (lane + i));
    a1[i] = (_Float16)(0.002f * (lane - i));
    b0[i] = (_Float16)(0.003f * (i + 1));
    b1[i] = (_Float16)(-0.001f * (i + 2));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b1, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b0, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b0, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b1, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (lane == 0) sink[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = s;
}

}  // namespace awq

extern "C" {

// bytes % 16 == 0; per_thread in {4, 8, 16}; sink: device uint32 [4 * blocks] with
// blocks = ceil(bytes / (4096 * per_thread))
int awq_peak_read_stream(const void* buf, size_t bytes, uint32_t* sink, int32_t per_thread,
                         void* stream) {
  if (!buf || !sink || bytes % 16 || (per_thread != 4 && per_thread != 8 && per_thread != 16))
    return 2;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t blocks = (n16 + 256 * per_thread - 1) / (256 * per_thread);
  if (blocks < 1 || blocks > 0x7FFFFFFF) return 2;
  hipStream_t st = (hipStream_t)stream;
  if (per_thread == 4)
    hipLaunchKernelGGL(awq::k_read_stream<4>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint4*)buf, n16, sink);
  else if (per_thread == 8)
    hipLaunchKernelGGL(awq::k_read_stream<8>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint4*)buf, n16, sink);
  else
    hipLaunchKernelGGL(awq::k_read_stream<16>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint4*)buf, n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// sink: device float [blocks * 4]; flops = blocks * 4 waves * iters * 8 * 32768
int awq_peak_mfma(int64_t iters, float* sink, int32_t blocks, void* stream) {
  if (!sink || iters < 1 || blocks < 1) return 2;
  hipLaunchKernelGGL(awq::k_mfma_loop, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
