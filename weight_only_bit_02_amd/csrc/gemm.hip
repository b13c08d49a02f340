// MFMA dequant-GEMM (a8): Y[M][N] = X[M][K] deq(W)^T for batches (prefill, M > 8).
//
// "AWQ量化技术Skill", "主要功能和特点": a GEMM kernel serves batch sizes above one;
// "AWQ量化实战" §2.3 / §3.4: weights stay 4-bit in memory and are dequantized on the fly.
//
// Block tile 128 (tokens) x 128 (output channels), K step = one quantization group
// (128 channels), four waves each owning a 64 x 64 sub-tile (2 x 2 tiles of
// v_mfma_f32_32x32x16_f16). Per K step the block stages through LDS:
//   - A: X[128][128] fp16, re-paired per 8 channels as (k, k+4) to match the codes;
//   - B: the 128 x 128 codes, widened exactly to (q - z) in fp16 and multiplied by the
//     group scale in fp16 (one rounding), in the same paired order.
// Both operands then feed the MFMA in the same channel order, so the contraction is
// the plain sum over K. fp32 accumulation, one fp16 rounding of the result.
#include "common.hpp"
#include "launch.hpp"

namespace awq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kLdsK = 128 + 8;  // halves per LDS row (16-byte pad)

__global__ void __launch_bounds__(256)
    k_gemm(const uint16_t* __restrict__ X, int64_t M, const uint32_t* __restrict__ qweight,
           const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int64_t N,
           int64_t K, uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLdsK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLdsK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m32 = lane & 31, khalf = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  const int64_t G = K / kGroup;
  const int64_t zb = (G + 1) / 2;
  const int64_t words = K / 8;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  for (int64_t g = 0; g < G; ++g) {
    // ---------------------------------------------------------------- stage A
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = i * 256 + tid;
      const int row = id >> 4, kc = id & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m0 + row < M) v = *reinterpret_cast<const uint4*>(X + (m0 + row) * K + g * kGroup + kc * 8);
      uint4 p;
      p.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
      p.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
      p.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
      p.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
      *reinterpret_cast<uint4*>(&As[row * kLdsK + kc * 8]) = p;
    }
    // ---------------------------------------------------------------- stage B
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = i * 256 + tid;
      const int n = id >> 2, wc = id & 3;
      uint4 cw = make_uint4(0, 0, 0, 0);
      half2v zz = {}, s2 = {};
      if (n0 + n < N) {
        const int64_t nn = n0 + n;
        cw = *reinterpret_cast<const uint4*>(qweight + nn * words + g * 16 + wc * 4);
        const uint32_t zbyte = zeros[nn * zb + (g >> 1)];
        const uint32_t z = (g & 1) ? (zbyte >> 4) : (zbyte & 0xF);
        const uint32_t zbits = 0x6400u + z;
        zz = -__builtin_bit_cast(half2v, zbits | (zbits << 16));
        const uint32_t sb = scales[nn * G + g];
        s2 = __builtin_bit_cast(half2v, sb | (sb << 16));
      } else {
        cw = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        zz = -__builtin_bit_cast(half2v, 0x64086408u);  // q = z = 8 -> 0
      }
      const uint32_t wd[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t u = ((wd[w] >> (4 * p)) & 0x000F000Fu) | 0x64006400u;
          const half2v d = (__builtin_bit_cast(half2v, u) + zz) * s2;
          o[p] = __builtin_bit_cast(uint32_t, d);
        }
        *reinterpret_cast<uint4*>(&Bs[n * kLdsK + wc * 32 + w * 8]) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    __syncthreads();
    // ---------------------------------------------------------------- MFMA
#pragma unroll
    for (int st = 0; st < kGroup / 16; ++st) {
      const int koff = st * 16 + khalf * 8;
      half8 A[2], B[2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        A[a] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&As[(wm * 64 + a * 32 + m32) * kLdsK + koff]));
#pragma unroll
      for (int b = 0; b < 2; ++b)
        B[b] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&Bs[(wn * 64 + b * 32 + m32) * kLdsK + koff]));
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[a], B[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogue
  // 32x32 accumulator layout: element e of lane l is (row 8(e/4) + 4(l/32) + e%4, col l%32).
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 64 + a * 32 + 8 * (e >> 2) + 4 * khalf + (e & 3);
        const int64_t col = n0 + wn * 64 + b * 32 + m32;
        if (row < M && col < N) Y[row * N + col] = f2h_bits(acc[a][b][e]);
      }
}

hipError_t launch_gemm(const uint16_t* X, int64_t M, const uint32_t* qweight,
                       const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                       uint16_t* Y, hipStream_t stream) {
  dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  hipLaunchKernelGGL(k_gemm, grid, dim3(256), 0, stream, X, M, qweight, scales, zeros, N, K, Y);
  return hipGetLastError();
}

}  // namespace awq
