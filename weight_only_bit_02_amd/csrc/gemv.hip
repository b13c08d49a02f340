// Dequant-fused GEMV for decode (a7): Y[M][N] = X[M][K] deq(W)^T for M <= 8.
//
// "AWQ量化实战" §3.4: decode is memory-bound, so the packed weights are streamed once
// from HBM and never expanded in memory; "AWQ量化技术Skill", "主要功能和特点": a GEMV
// kernel serves single-token generation.
//
// Mapping: a wave owns R consecutive rows of W; its lanes stride along K in chunks
// of 32 input channels (one 16-byte load of 4 packed words per row), so each load
// instruction moves 1 KiB of consecutive codes. A chunk lies inside one group, so one
// scale and one zero point apply to it. Codes are widened to fp16 exactly with the
// 0x6400 exponent trick ((1024 + q) as fp16), the zero is removed with a packed fp16
// add (exact: q - z is a small integer), and v_dot2_f32_f16 multiplies two channels
// at a time into fp32. The group scale multiplies the 32-channel partial once. The
// word's nibbles come out paired (k, k + 4), so the activations are re-paired the
// same way with v_perm_b32 (once per chunk, shared by the R rows). Rows finish with
// a DPP / shuffle reduction across the wave.
#include "common.hpp"
#include "launch.hpp"

namespace awq {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

template <int M, int R>
__global__ void __launch_bounds__(256)
    k_gemv(const uint16_t* __restrict__ X, const uint32_t* __restrict__ qweight,
           const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int64_t N,
           int64_t K, uint16_t* __restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t row0 = wave * R;
  if (row0 >= N) return;  // whole wave leaves together
  const int64_t C = K / 32;  // chunks per row
  const int64_t G = K / kGroup;
  const int64_t zb = (G + 1) / 2;
  const int64_t words = K / 8;

  int64_t rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = (row0 + r < N) ? row0 + r : N - 1;

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  for (int64_t c = lane; c < C; c += 64) {
    const int64_t g = c >> 2;
    half2v qz[R][16];
    float sc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint4 cw = *reinterpret_cast<const uint4*>(qweight + rows[r] * words + c * 4);
      sc[r] = h2f(scales[rows[r] * G + g]);
      const uint32_t zbyte = zeros[rows[r] * zb + (g >> 1)];
      const uint32_t z = (g & 1) ? (zbyte >> 4) : (zbyte & 0xF);
      const uint32_t zbits = 0x6400u + z;  // fp16 of 1024 + z
      const half2v zz = -__builtin_bit_cast(half2v, zbits | (zbits << 16));
      const uint32_t wd[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t u = ((wd[w] >> (4 * p)) & 0x000F000Fu) | 0x64006400u;  // (1024+q_p, 1024+q_{p+4})
          qz[r][w * 4 + p] = __builtin_bit_cast(half2v, u) + zz;                // exact (q - z)
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4* xp = reinterpret_cast<const uint4*>(X + (int64_t)m * K + c * 32);
      half2v xq[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint4 v = xp[w];  // channels 8w .. 8w+7 as (0,1) (2,3) (4,5) (6,7)
        xq[w * 4 + 0] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(v.z, v.x, 0x05040100u));
        xq[w * 4 + 1] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(v.z, v.x, 0x07060302u));
        xq[w * 4 + 2] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(v.w, v.y, 0x05040100u));
        xq[w * 4 + 3] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) part = __builtin_amdgcn_fdot2(qz[r][i], xq[i], part, false);
        acc[r][m] += sc[r] * part;
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float v = wave_sum(acc[r][m]);
      if (lane == 0 && row0 + r < N) Y[(int64_t)m * N + row0 + r] = f2h_bits(v);
    }
}

template <int M>
static hipError_t launch_gemv_m(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                                const uint8_t* z, int64_t N, int64_t K, uint16_t* Y,
                                hipStream_t stream) {
  constexpr int R = 4;
  const int64_t waves = (N + R - 1) / R;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((k_gemv<M, R>), dim3((unsigned)blocks), dim3(256), 0, stream, X, qw, sc, z,
                     N, K, Y);
  return hipGetLastError();
}

hipError_t launch_gemv(const uint16_t* X, int64_t M, const uint32_t* qweight,
                       const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                       uint16_t* Y, hipStream_t stream) {
  switch (M) {
    case 1: return launch_gemv_m<1>(X, qweight, scales, zeros, N, K, Y, stream);
    case 2: return launch_gemv_m<2>(X, qweight, scales, zeros, N, K, Y, stream);
    case 3: return launch_gemv_m<3>(X, qweight, scales, zeros, N, K, Y, stream);
    case 4: return launch_gemv_m<4>(X, qweight, scales, zeros, N, K, Y, stream);
    case 5: return launch_gemv_m<5>(X, qweight, scales, zeros, N, K, Y, stream);
    case 6: return launch_gemv_m<6>(X, qweight, scales, zeros, N, K, Y, stream);
    case 7: return launch_gemv_m<7>(X, qweight, scales, zeros, N, K, Y, stream);
    case 8: return launch_gemv_m<8>(X, qweight, scales, zeros, N, K, Y, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace awq
