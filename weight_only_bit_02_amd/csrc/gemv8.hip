// Vector GEMV for 8-bit codes (a7 with w_bit = 8): Y[M][N] = X[M][K] deq(W)^T, M <= 8.
//
// "AWQ量化实战" §3.3 (w_bit = 8, near lossless) and §5.2 / §5.3 (raise w_bit when 4-bit
// accuracy falls short); the decode GEMV then streams one byte per weight instead of half
// a byte.
//
// Same mapping as the 4-bit batched GEMV: a wave owns R rows, lane l walks 32-channel
// chunks c = l, l + 64, ...; a chunk's 32 codes are 8 words (two 16-byte loads), word u
// holding channels 4u .. 4u + 3 in its bytes. Widening is exact: v_perm_b32 against
// 0x64646464 turns bytes (a, b) into the fp16 pair (1024 + a, 1024 + b), and one packed
// fp16 add of -(1024 + z) leaves (q - z) (|q - z| <= 255, exact); v_dot2 with the
// activation pair accumulates in fp32, and the group scale multiplies each chunk's
// partial in fp32. The zero point is one byte per group.
#include "common.hpp"
#include "launch.hpp"

namespace awq {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

namespace {

constexpr uint32_t kPermLo = 0x04010400u;  // bytes (w.0, 0x64, w.1, 0x64)
constexpr uint32_t kPermHi = 0x04030402u;  // bytes (w.2, 0x64, w.3, 0x64)

__device__ __forceinline__ uint32_t magic_64x4() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64646464" : "=v"(m));
  return m;
}

}  // namespace

template <int M, int R, bool GATED>
__global__ void __launch_bounds__(256)
    k_gemv8(const uint16_t* __restrict__ X, const uint32_t* __restrict__ qweight,
            const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int64_t N,
            int64_t K, int gsh, uint16_t* __restrict__ Y) {
  static_assert(!GATED || R == 2, "a gated wave owns one gate row and one up row");
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nh = N / 2;
  const int64_t row0 = GATED ? wave : wave * R;
  if (row0 >= (GATED ? nh : N)) return;  // whole wave leaves together
  const int64_t C = K / 32;              // chunks per row
  const int64_t G = K >> (gsh + 5);      // groups per row
  const int64_t words = K / 4;
  const uint32_t magic = magic_64x4();

  int64_t rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    rows[r] = GATED ? row0 + r * nh : ((row0 + r < N) ? row0 + r : N - 1);

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  for (int64_t c = lane; c < C; c += 64) {
    const int64_t g = c >> gsh;  // group of this 32-channel chunk
    half2v qz[R][16];            // pair i = channels (2i, 2i + 1) of the chunk, as q - z
    float sc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint4* cp = reinterpret_cast<const uint4*>(qweight + rows[r] * words + c * 8);
      const uint4 c0 = cp[0], c1 = cp[1];
      sc[r] = h2f(scales[rows[r] * G + g]);
      const uint32_t zbits = 0x6400u + zeros[rows[r] * G + g];  // fp16 of 1024 + z
      const half2v zz = -__builtin_bit_cast(half2v, zbits | (zbits << 16));
      const uint32_t wd[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        qz[r][2 * u] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(magic, wd[u], kPermLo)) + zz;
        qz[r][2 * u + 1] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(magic, wd[u], kPermHi)) + zz;
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4* xp = reinterpret_cast<const uint4*>(X + (int64_t)m * K + c * 32);
      half2v xq[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint4 v = xp[w];  // channels 8w .. 8w + 7 as the pairs (0,1) (2,3) (4,5) (6,7)
        xq[w * 4 + 0] = __builtin_bit_cast(half2v, v.x);
        xq[w * 4 + 1] = __builtin_bit_cast(half2v, v.y);
        xq[w * 4 + 2] = __builtin_bit_cast(half2v, v.z);
        xq[w * 4 + 3] = __builtin_bit_cast(half2v, v.w);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) part = __builtin_amdgcn_fdot2(qz[r][i], xq[i], part, false);
        acc[r][m] = __builtin_fmaf(sc[r], part, acc[r][m]);
      }
    }
  }

  if constexpr (GATED) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float g = wave_sum(acc[0][m]), u = wave_sum(acc[R - 1][m]);
      if (lane == 0) Y[(int64_t)m * nh + row0] = f2h_bits(silu_f32(g) * u);
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float v = wave_sum(acc[r][m]);
        if (lane == 0 && row0 + r < N) Y[(int64_t)m * N + row0 + r] = f2h_bits(v);
      }
  }
}

// ------------------------------------------------------------------ skinny MFMA, 8-bit
// The 4-bit skinny kernel's mapping (a wave owns 32 weight rows and a slice of the
// 128-channel steps; lane l: row l % 32, h = l / 32, channels [32 h, 32 h + 32) and
// [64 + 32 h, 96 + 32 h) of each step), with each 32-channel half now 8 words (two 16-byte
// loads); k16 slice s takes words 2 (s % 4) and 2 (s % 4) + 1 of half s / 4 as its 8
// channels. Scales as in the 4-bit kernel: a fresh partial tile per group (one per step
// for 128-channel groups, one per half for 64), and for 32-channel groups, where the two
// lane halves of a slice lie in different groups, the fp16 operand carries the scale.
// M = 33..64: two 32-token tiles share each widened operand (4 waves per block), with the
// scale carried by the operand for every group size, as in the 4-bit kernel.
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

template <int MT>
struct SkinnyStage8 {
  uint4 b[4];          // words 8h .. 8h + 7 and 16 + 8h .. 16 + 8h + 7 of the step, row l % 32
  uint4 a[MT][8];      // X[token][same channels] per token tile, one 16-byte piece per k16 step
  uint32_t sc[2], zb;  // scales and zero bytes of the lane's two halves
};

__device__ __forceinline__ half8 widen8(uint32_t w0, uint32_t w1, half2v zz, uint32_t magic) {
  const half2v d0 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(magic, w0, kPermLo)) + zz;
  const half2v d1 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(magic, w0, kPermHi)) + zz;
  const half2v d2 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(magic, w1, kPermLo)) + zz;
  const half2v d3 = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(magic, w1, kPermHi)) + zz;
  return half8{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
}

}  // namespace

template <int S, int E, int MT, bool GATED>
__global__ void __launch_bounds__(S * 64)
    k_gemv_mfma8(const uint16_t* X, int64_t M, const uint32_t* qweight, const uint16_t* scales,
                 const uint8_t* zeros, int64_t N, int64_t K, int group, uint16_t* Y) {
  __shared__ float red[S][MT * E][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  const int lg = group == 128 ? 7 : group == 64 ? 6 : 5;
  const bool g128 = group == 128, g32 = group == 32;
  const int64_t G = K / kGroup;                 // 128-channel steps
  const int64_t Gs = K / group, words = K / 4;  // groups, words per row
  const int64_t nh = N / 2;
  int64_t n;
  if constexpr (GATED) {
    const int64_t o = (int64_t)blockIdx.x * 16 + (j & 15);
    n = (o < nh ? o : nh - 1) + (j >> 4) * nh;
  } else {
    const int64_t o = (int64_t)blockIdx.x * 32 + j;
    n = o < N ? o : N - 1;
  }
  int64_t xrow[MT];  // token row of lane l in tile t: 32 t + l % 32 (past M: row M - 1, never stored)
#pragma unroll
  for (int t = 0; t < MT; ++t) xrow[t] = (32 * t + j < M ? 32 * t + j : M - 1) * K;
  const int64_t g0 = G * wave / S, g1 = G * (wave + 1) / S;
  const uint32_t magic = magic_64x4();

  auto load = [&](SkinnyStage8<MT>& st, int64_t g) {
    const int64_t q0 = (g * kGroup + 32 * h) >> lg, q1 = (g * kGroup + 64 + 32 * h) >> lg;
    st.zb = (uint32_t)zeros[n * Gs + q0] | ((uint32_t)zeros[n * Gs + q1] << 8);
    st.sc[0] = scales[n * Gs + q0];
    st.sc[1] = scales[n * Gs + q1];
    const uint4* cp = reinterpret_cast<const uint4*>(qweight + n * words + g * 32 + h * 8);
    st.b[0] = cp[0];
    st.b[1] = cp[1];
    st.b[2] = cp[4];
    st.b[3] = cp[5];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint16_t* xp = X + xrow[t] + g * kGroup + h * 32;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        st.a[t][s] = *reinterpret_cast<const uint4*>(xp + (s & 3) * 8 + (s >> 2) * 64);
    }
  };

  float acc[MT][E];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[t][e] = 0.0f;
  f32x16 acc2[MT];  // MT = 2: the two token tiles, accumulated by the MFMAs themselves
#pragma unroll
  for (int t = 0; t < MT; ++t) acc2[t] = f32x16{};

  auto body = [&](const SkinnyStage8<MT>& st) {
    const uint32_t wd[16] = {st.b[0].x, st.b[0].y, st.b[0].z, st.b[0].w, st.b[1].x, st.b[1].y,
                             st.b[1].z, st.b[1].w, st.b[2].x, st.b[2].y, st.b[2].z, st.b[2].w,
                             st.b[3].x, st.b[3].y, st.b[3].z, st.b[3].w};
    half2v zz[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t zbits = 0x6400u + ((st.zb >> (8 * half)) & 0xFF);
      zz[half] = -__builtin_bit_cast(half2v, zbits | (zbits << 16));
    }
    auto operand = [&](int s) {  // slice s: words 2 (s % 4), + 1 of half s / 4
      const int w = 8 * (s >> 2) + 2 * (s & 3);
      return widen8(wd[w], wd[w + 1], zz[s >> 2], magic);
    };
    if constexpr (MT == 2) {
      // two token tiles: the operand carries the scale of its 32-channel half for every
      // group size ((q - z) sc in fp16, one rounding), the MFMAs accumulate the tiles
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint32_t sb = st.sc[s >> 2];
        const half2v s2 = __builtin_bit_cast(half2v, sb | (sb << 16));
        const half8 b = operand(s) * half8{s2[0], s2[1], s2[0], s2[1], s2[0], s2[1], s2[0], s2[1]};
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc2[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, st.a[t][s]), b,
                                                            acc2[t], 0, 0, 0);
      }
    } else if (g32) {
      f32x16 d = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint32_t sb = st.sc[s >> 2];
        const half2v s2 = __builtin_bit_cast(half2v, sb | (sb << 16));
        d = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(half8, st.a[0][s]),
            operand(s) * half8{s2[0], s2[1], s2[0], s2[1], s2[0], s2[1], s2[0], s2[1]}, d, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) acc[0][e] += d[e];
    } else if (g128) {
      f32x16 d = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s)
        d = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, st.a[0][s]), operand(s), d,
                                                   0, 0, 0);
      const float scf = h2f((uint16_t)st.sc[0]);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[0][e] = __builtin_fmaf(scf, d[e], acc[0][e]);
    } else {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x16 d = f32x16{};
#pragma unroll
        for (int s = 4 * half; s < 4 * half + 4; ++s)
          d = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, st.a[0][s]), operand(s),
                                                     d, 0, 0, 0);
        const float scf = h2f((uint16_t)st.sc[half]);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[0][e] = __builtin_fmaf(scf, d[e], acc[0][e]);
      }
    }
  };

  if (g1 > g0) {
    SkinnyStage8<MT> s0, s1;
    load(s0, g0);
    int64_t g = g0;
    for (; g + 2 <= g1; g += 2) {
      load(s1, g + 1);
      body(s0);
      load(s0, g + 2 < g1 ? g + 2 : g1 - 1);  // always issued: exact waits on every path
      body(s1);
    }
    if (g < g1) body(s0);
  }

  if constexpr (MT == 2) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[t][e] = acc2[t][e];
  }
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int e = 0; e < E; ++e) red[wave][t * E + e][lane] = acc[t][e];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float v = red[0][t * E + e][lane];
#pragma unroll
      for (int w = 1; w < S; ++w) v += red[w][t * E + e][lane];
      acc[t][e] = v;
    }
  // 32x32 accumulator layout: element e of lane l is (row 8(e/4) + 4(l/32) + e%4, col l%32)
  if constexpr (GATED) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float u = __shfl_down(acc[t][e], 16, 32);
        const int64_t o = (int64_t)blockIdx.x * 16 + j;
        const int64_t i = 32 * t + 8 * (e >> 2) + 4 * h + (e & 3);
        if (j < 16 && o < nh && i < M) Y[i * nh + o] = f2h_bits(silu_f32(acc[t][e]) * u);
      }
  } else {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int64_t o = (int64_t)blockIdx.x * 32 + j;
        const int64_t i = 32 * t + 8 * (e >> 2) + 4 * h + (e & 3);
        if (o < N && i < M) Y[i * N + o] = f2h_bits(acc[t][e]);
      }
  }
}

template <int S, int E, int MT, bool GATED>
static hipError_t launch_skinny8_x(const uint16_t* X, int64_t M, const uint32_t* qw,
                                   const uint16_t* sc, const uint8_t* z, int64_t N, int64_t K,
                                   int group, uint16_t* Y, hipStream_t stream) {
  const int64_t outs = GATED ? N / 2 : N;
  const int64_t per = GATED ? 16 : 32;
  const int64_t blocks = (outs + per - 1) / per;
  hipLaunchKernelGGL((k_gemv_mfma8<S, E, MT, GATED>), dim3((unsigned)blocks), dim3(S * 64), 0, stream,
                     X, M, qw, sc, z, N, K, group, Y);
  return hipGetLastError();
}

template <bool GATED>
static hipError_t launch_skinny8_t(const uint16_t* X, int64_t M, const uint32_t* qw,
                                   const uint16_t* sc, const uint8_t* z, int64_t N, int64_t K,
                                   int group, uint16_t* Y, hipStream_t stream) {
  if (M <= 8) return launch_skinny8_x<8, 4, 1, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
  if (M <= 16) return launch_skinny8_x<8, 8, 1, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
  if (M <= 32) return launch_skinny8_x<8, 16, 1, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
  // two token tiles: 4 waves per block, so a wave may also use the accumulation registers
  return launch_skinny8_x<4, 16, 2, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
}

hipError_t launch_gemv_mfma8(const uint16_t* X, int64_t M, const uint32_t* qweight,
                             const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                             int group, uint16_t* Y, bool gated, hipStream_t stream) {
  if (M < 1 || M > kSkinnyMaxM) return hipErrorInvalidValue;
  return gated ? launch_skinny8_t<true>(X, M, qweight, scales, zeros, N, K, group, Y, stream)
               : launch_skinny8_t<false>(X, M, qweight, scales, zeros, N, K, group, Y, stream);
}

template <int M, bool GATED>
static hipError_t launch_gemv8_m(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                                 const uint8_t* z, int64_t N, int64_t K, int gsh, uint16_t* Y,
                                 hipStream_t stream) {
  constexpr int R = GATED ? 2 : (M <= 2 ? 2 : 4);
  const int64_t waves = GATED ? N / 2 : (N + R - 1) / R;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((k_gemv8<M, R, GATED>), dim3((unsigned)blocks), dim3(256), 0, stream, X, qw,
                     sc, z, N, K, gsh, Y);
  return hipGetLastError();
}

template <bool GATED>
static hipError_t launch_gemv8_t(const uint16_t* X, int64_t M, const uint32_t* qw,
                                 const uint16_t* sc, const uint8_t* z, int64_t N, int64_t K,
                                 int gsh, uint16_t* Y, hipStream_t stream) {
  switch (M) {
    case 1: return launch_gemv8_m<1, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 2: return launch_gemv8_m<2, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 3: return launch_gemv8_m<3, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 4: return launch_gemv8_m<4, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 5: return launch_gemv8_m<5, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 6: return launch_gemv8_m<6, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 7: return launch_gemv8_m<7, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 8: return launch_gemv8_m<8, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv8(const uint16_t* X, int64_t M, const uint32_t* qweight,
                        const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                        int group, uint16_t* Y, bool gated, hipStream_t stream) {
  const int gsh = group == 128 ? 2 : group == 64 ? 1 : 0;  // chunk c (32 channels) is in group c >> gsh
  return gated ? launch_gemv8_t<true>(X, M, qweight, scales, zeros, N, K, gsh, Y, stream)
               : launch_gemv8_t<false>(X, M, qweight, scales, zeros, N, K, gsh, Y, stream);
}

}  // namespace awq
