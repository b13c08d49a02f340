// Activation statistic (a1) and candidate scales (a2).
//
// "AWQ量化实战" §2.1: accumulate the calibration activations of each input channel and
// take the mean absolute value. "什么是激活感知权重量化（AWQ）", "工作机制": the protecting
// scale is set from these offline statistics; "AWQ量化实战" §2.2: it is chosen by a grid
// search over a candidate interval.
//
// The column sums are exact: each |x| is converted to an integer count of 2^-24 and
// summed in int64 (integer atomics, so any order gives the same bits), and the mean
// is one fp64 division. The candidate scale is an fp64 pow followed by a single
// round-to-nearest-even conversion to fp16.
#include "common.hpp"
#include "launch.hpp"

namespace awq {

constexpr int kStatRows = 8;     // tokens summed per thread before the atomic add
constexpr int kStatThreads = 64;  // one wave per block: many waves even for small K

__global__ void k_zero_u64(unsigned long long* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

// Thread = 8 consecutive channels x one slice of kStatRows tokens, all of the slice's loads
// issued before the first is used (rows past T read row T - 1 and are not added).
__global__ void __launch_bounds__(kStatThreads)
    k_act_sums(const uint16_t* __restrict__ X, int64_t T, int64_t K,
               unsigned long long* __restrict__ u, uint32_t* __restrict__ flags) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 8-channel chunk
  if (c * 8 >= K) return;
  const int64_t t0 = (int64_t)blockIdx.y * kStatRows;
  uint4 vs[kStatRows];
#pragma unroll
  for (int r = 0; r < kStatRows; ++r) {
    const int64_t t = t0 + r < T ? t0 + r : T - 1;
    vs[r] = *reinterpret_cast<const uint4*>(X + t * K + c * 8);
  }
  int64_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  bool bad = false;
#pragma unroll
  for (int r = 0; r < kStatRows; ++r) {
    if (t0 + r >= T) break;
    const uint4 v = vs[r];
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t lo = f16_abs_units((uint16_t)(d[i] & 0xFFFF));
      const int64_t hi = f16_abs_units((uint16_t)(d[i] >> 16));
      bad |= (lo < 0) | (hi < 0);
      acc[2 * i] += lo < 0 ? 0 : lo;
      acc[2 * i + 1] += hi < 0 ? 0 : hi;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) atomicAdd(u + c * 8 + i, (unsigned long long)acc[i]);
  if (bad && flags) atomicOr(flags, AWQ_FLAG_NONFINITE_INPUT);
}

__global__ void k_act_finalize(const unsigned long long* __restrict__ u, int64_t T, int64_t K,
                               double* __restrict__ act) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  // u < 2^53, so the conversion and the power-of-two scaling are exact.
  act[k] = ((double)u[k] * 0x1p-24) / (double)T;
}

// One thread per (grid point i, channel k): the n_grid pows of a channel run in parallel.
__global__ void k_scalegen(const double* __restrict__ act, int64_t K, int n_grid,
                           uint16_t* __restrict__ s_grid) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= (int64_t)n_grid * K) return;
  const int i = (int)(u / K);
  const int64_t k = u % K;
  if (i == 0) {
    s_grid[k] = 0x3C00;  // alpha = 0: s = 1
    return;
  }
  const double a = fmax(act[k], 0x1p-14);
  const double alpha = (double)i / (double)n_grid;
  s_grid[u] = f64_to_f16_rne(pow(a, alpha));
}

hipError_t launch_zero_u64(unsigned long long* p, int64_t n, hipStream_t stream) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_zero_u64, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_act_sums(const uint16_t* X, int64_t T, int64_t K, unsigned long long* u,
                           uint32_t* flags, hipStream_t stream) {
  const int64_t chunks = K / 8;
  dim3 grid((unsigned)((chunks + kStatThreads - 1) / kStatThreads),
            (unsigned)((T + kStatRows - 1) / kStatRows));
  hipLaunchKernelGGL(k_act_sums, grid, dim3(kStatThreads), 0, stream, X, T, K, u, flags);
  return hipGetLastError();
}

hipError_t launch_act_finalize(const unsigned long long* u, int64_t T, int64_t K, double* act,
                               hipStream_t stream) {
  hipLaunchKernelGGL(k_act_finalize, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, stream, u,
                     T, K, act);
  return hipGetLastError();
}

hipError_t launch_scalegen(const double* act, int64_t K, int n_grid, uint16_t* s_grid,
                           hipStream_t stream) {
  const int64_t n = (int64_t)n_grid * K;
  hipLaunchKernelGGL(k_scalegen, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, act, K,
                     n_grid, s_grid);
  return hipGetLastError();
}

}  // namespace awq
