// Skinny MFMA GEMV for small batches (a7 / a9): Y[M][N] = X[M][K] deq(W)^T for M <= 64.
//
// "AWQ量化实战" §3.4: decode is memory-bound, so the packed weights are streamed once and
// dequantized on the fly; "AWQ量化技术Skill", "主要功能和特点": a GEMV kernel serves the
// small batches of token generation.
//
// With more than one token, dot products on the vector ALU cost one v_dot2 per channel
// pair per token; here they go to the matrix cores instead, so the vector work per byte
// of codes (the exact widening to q - z) does not grow with M:
//   - a wave owns R tiles of 32 weight rows (each the 32 columns of a
//     v_mfma_f32_32x32x16_f16 tile; R = 2 on launches with enough rows, so each X piece
//     feeds both tiles) and a slice of the K groups; lane l works on row l % 32 and, h = l / 32, on channels
//     [32 h, 32 h + 32) and [64 + 32 h, 96 + 32 h) of each group (two 16-byte code loads
//     per group; lanes l and l + 32 read 32 contiguous bytes of the row together);
//   - word s of those 64 channels is the lane's B operand of k16 step s, widened exactly
//     to (q - z) in fp16 (0x6400 trick, packed fp16 add); the A operand is the 16 bytes
//     of X at the same channels for token l % 32 (rows past M repeat row M - 1 and are
//     never stored), read straight from global memory (X is tiny and stays in cache);
//   - the 8 MFMAs of a group start from zero, and the group scale multiplies that partial
//     tile in fp32 (one FMA per element), as in the M = 1 kernel; with 64-channel groups
//     the lane's first four words are one group and the last four the next, so the 8
//     MFMAs form two partial tiles of four, each with its own scale; with 32-channel
//     groups the two lane halves of one k16 slice lie in different groups, so there the
//     operand itself carries the scale ((q - z) sc in fp16, one rounding, as in the GEMM);
//   - M up to 32 is one token tile; 33..64 two (MT = 2): each widened B operand then feeds
//     one MFMA per token tile, so the vector work per byte of codes stays that of one tile.
//     To fit the registers of two tiles, the operand carries the group scale there for
//     every group size ((q - z) sc in fp16, one rounding, as in the GEMM) and the MFMAs
//     accumulate straight into the two tiles;
//   - the S waves of a block split K and meet in LDS at the end, where wave 0 adds the S
//     partial tiles in a fixed order: results do not depend on scheduling.
// Loads of group g + 1 are in flight while group g is multiplied (two register stages
// used alternately in a loop unrolled by two, so no register copy waits for them).
#include "common.hpp"
#include "launch.hpp"

namespace awq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

// dispatch: two row tiles per wave from this many blocks (see launch_skinny_t)
constexpr int64_t kSkinnyR2MinBlocks = 160, kSkinnyR2MinBlocksGated = 512;

template <int MT, int R>
struct SkinnyStage {
  uint4 b[R][2];     // per row tile: 8 packed words, channels 32 h + [0, 32) and 64 + 32 h + [0, 32), row l % 32
  uint4 a[MT][8];    // X[token][same channels] per token tile, one 16-byte piece per k16 step
  uint32_t sc[R][2], zb[R];  // per row tile: the lane's scales of words 0-3 and 4-7; the step's zero byte(s)
};

__device__ __forceinline__ uint32_t skinny_magic() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

// One packed word -> its 8 channels as exact fp16 (q - z), in channel order.
__device__ __forceinline__ half8 widen_word(uint32_t w, half2v zz, uint32_t magic) {
  half2v d[4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
    d[p] = __builtin_bit_cast(half2v, ((w >> (4 * p)) & 0x000F000Fu) | magic) + zz;
  return half8{d[0][0], d[0][1], d[1][0], d[1][1], d[2][0], d[2][1], d[3][0], d[3][1]};
}

}  // namespace

// E = accumulator elements kept per lane: rows 8 (e / 4) + 4 h + e % 4 of the 32 x 32 tile;
// E = 4 serves M <= 8, 8 serves M <= 16, 16 serves M <= 32; MT = 2 token tiles of 32 (rows
// 32 t + ...) serve M <= 64. R = row tiles of 32 per wave, all multiplied by the same X
// pieces: R = 2 halves the activation bytes a wave loads per weight byte.
template <int S, int E, int MT, int R, bool GATED>
__global__ void __launch_bounds__(S * 64)
    k_gemv_mfma(const uint16_t* X, int64_t M, const uint32_t* qweight, const uint16_t* scales,
                const uint8_t* zeros, int64_t N, int64_t K, int group, uint16_t* Y) {
  __shared__ float red[S][R * MT * E][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  const bool g64 = group == 64, g32 = group == 32;
  const int64_t G = K / kGroup;                 // 128-channel steps
  const int64_t Gs = K / group, zbytes = (Gs + 1) / 2, words = K / 8;  // scale groups
  // rows of this tile: plain, 32 consecutive rows; gated, 16 gate rows then their 16 up
  // rows (tile columns j and j + 16 hold g and u of output n0 + j)
  const int64_t nh = N / 2;
  int64_t n[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if constexpr (GATED) {
      const int64_t o = ((int64_t)blockIdx.x * R + r) * 16 + (j & 15);
      n[r] = (o < nh ? o : nh - 1) + (j >> 4) * nh;
    } else {
      const int64_t o = ((int64_t)blockIdx.x * R + r) * 32 + j;
      n[r] = o < N ? o : N - 1;
    }
  }
  int64_t xrow[MT];  // token row of lane l in tile t: 32 t + l % 32 (past M: row M - 1, never stored)
#pragma unroll
  for (int t = 0; t < MT; ++t) xrow[t] = (32 * t + j < M ? 32 * t + j : M - 1) * K;
  // this wave's groups: an even split of the G groups over the S waves
  const int64_t g0 = G * wave / S, g1 = G * (wave + 1) / S;
  const uint32_t magic = skinny_magic();

  auto load = [&](SkinnyStage<MT, R>& st, int64_t g) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t nr = n[r];
      if (g32) {
        // words 0-3 of lane half h: group 4g + h; words 4-7: group 4g + 2 + h
        st.zb[r] = (uint32_t)zeros[nr * zbytes + 2 * g] | ((uint32_t)zeros[nr * zbytes + 2 * g + 1] << 8);
        st.sc[r][0] = scales[nr * Gs + 4 * g + h];
        st.sc[r][1] = scales[nr * Gs + 4 * g + 2 + h];
      } else if (g64) {
        st.zb[r] = zeros[nr * zbytes + g];  // groups 2g (low nibble) and 2g + 1 (high)
        st.sc[r][0] = scales[nr * Gs + 2 * g];
        st.sc[r][1] = scales[nr * Gs + 2 * g + 1];
      } else {
        st.zb[r] = zeros[nr * zbytes + (g >> 1)];
        st.sc[r][0] = st.sc[r][1] = scales[nr * Gs + g];
      }
      const uint32_t* cp = qweight + nr * words + g * 16 + h * 4;
      st.b[r][0] = *reinterpret_cast<const uint4*>(cp);
      st.b[r][1] = *reinterpret_cast<const uint4*>(cp + 8);
    }
    // word s (k16 step s) covers channels 8 s' + 32 h + 64 (s / 4), s' = s % 4
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint16_t* xp = X + xrow[t] + g * kGroup + h * 32;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        st.a[t][s] = *reinterpret_cast<const uint4*>(xp + (s & 3) * 8 + (s >> 2) * 64);
    }
  };

  float acc[R][MT][E];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[r][t][e] = 0.0f;
  auto mfma = [&](const SkinnyStage<MT, R>& st, int s, half8 b, f32x16 (&d)[MT]) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
      d[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, st.a[t][s]), b, d[t], 0, 0, 0);
  };

  f32x16 acc2[R][MT];  // MT = 2: the two token tiles, accumulated by the MFMAs themselves
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc2[r][t] = f32x16{};

  auto body = [&](const SkinnyStage<MT, R>& st, int64_t g) {
#pragma unroll
   for (int r = 0; r < R; ++r) {
    const uint32_t wd[8] = {st.b[r][0].x, st.b[r][0].y, st.b[r][0].z, st.b[r][0].w,
                            st.b[r][1].x, st.b[r][1].y, st.b[r][1].z, st.b[r][1].w};
    auto zz_of = [](uint32_t z) {
      const uint32_t zbits = 0x6400u + z;
      return -__builtin_bit_cast(half2v, zbits | (zbits << 16));
    };
    if constexpr (MT == 2) {
      // words 0-3 / 4-7 of lane half h: zero nibble and scale of their group (128: the
      // step's group; 64: groups 2g, 2g + 1; 32: groups 4g + h, 4g + 2 + h)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint32_t z = g32 ? (st.zb[r] >> (8 * half + 4 * h)) & 0xF
                           : g64 ? (st.zb[r] >> (4 * half)) & 0xF
                                 : ((g & 1) ? (st.zb[r] >> 4) & 0xF : st.zb[r] & 0xF);
        const half2v zz = zz_of(z);
        const half2v s2 = __builtin_bit_cast(half2v, st.sc[r][half] | (st.sc[r][half] << 16));
#pragma unroll
        for (int s = 4 * half; s < 4 * half + 4; ++s)
          mfma(st, s, widen_word(wd[s], zz, magic) * half8{s2[0], s2[1], s2[0], s2[1], s2[0], s2[1], s2[0], s2[1]}, acc2[r]);
      }
    } else if (g32) {
      f32x16 d[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) d[t] = f32x16{};
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const half2v zz = zz_of((st.zb[r] >> (8 * half + 4 * h)) & 0xF);
        const half2v s2 = __builtin_bit_cast(half2v, st.sc[r][half] | (st.sc[r][half] << 16));
#pragma unroll
        for (int s = 4 * half; s < 4 * half + 4; ++s)
          mfma(st, s, widen_word(wd[s], zz, magic) * half8{s2[0], s2[1], s2[0], s2[1], s2[0], s2[1], s2[0], s2[1]}, d);
      }
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[r][t][e] += d[t][e];
    } else if (g64) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const half2v zz = zz_of((st.zb[r] >> (4 * half)) & 0xF);
        f32x16 d[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) d[t] = f32x16{};
#pragma unroll
        for (int s = 4 * half; s < 4 * half + 4; ++s) mfma(st, s, widen_word(wd[s], zz, magic), d);
        const float scf = h2f((uint16_t)st.sc[r][half]);
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[r][t][e] = __builtin_fmaf(scf, d[t][e], acc[r][t][e]);
      }
    } else {
      const half2v zz = zz_of((g & 1) ? (st.zb[r] >> 4) & 0xF : st.zb[r] & 0xF);
      f32x16 d[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) d[t] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) mfma(st, s, widen_word(wd[s], zz, magic), d);
      const float scf = h2f((uint16_t)st.sc[r][0]);
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[r][t][e] = __builtin_fmaf(scf, d[t][e], acc[r][t][e]);
    }
   }
  };

  if (g1 > g0) {
    SkinnyStage<MT, R> s0, s1;
    load(s0, g0);
    int64_t g = g0;
    for (; g + 2 <= g1; g += 2) {
      load(s1, g + 1);
      body(s0, g);
      load(s0, g + 2 < g1 ? g + 2 : g1 - 1);  // always issued: exact waits on every path
      body(s1, g + 1);
    }
    if (g < g1) body(s0, g);
  }

  if constexpr (MT == 2) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[r][t][e] = acc2[r][t][e];
  }
  // fixed-order reduction of the S partial tiles
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < E; ++e) red[wave][(r * MT + t) * E + e][lane] = acc[r][t][e];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float v = red[0][(r * MT + t) * E + e][lane];
#pragma unroll
        for (int w = 1; w < S; ++w) v += red[w][(r * MT + t) * E + e][lane];
        acc[r][t][e] = v;
      }
  // 32x32 accumulator layout: element e of lane l is (row 8(e/4) + 4(l/32) + e%4, col l%32)
  if constexpr (GATED) {
    // up partner of column j (< 16) is column j + 16, held by lane + 16 for the same rows
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float u = __shfl_down(acc[r][t][e], 16, 32);
          const int64_t o = ((int64_t)blockIdx.x * R + r) * 16 + j;
          const int64_t i = 32 * t + 8 * (e >> 2) + 4 * h + (e & 3);
          if (j < 16 && o < nh && i < M) Y[i * nh + o] = f2h_bits(silu_f32(acc[r][t][e]) * u);
        }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int64_t o = ((int64_t)blockIdx.x * R + r) * 32 + j;
          const int64_t i = 32 * t + 8 * (e >> 2) + 4 * h + (e & 3);
          if (o < N && i < M) Y[i * N + o] = f2h_bits(acc[r][t][e]);
        }
  }
}

template <int S, int E, int MT, int R, bool GATED>
static hipError_t launch_skinny_x(const uint16_t* X, int64_t M, const uint32_t* qw,
                                  const uint16_t* sc, const uint8_t* z, int64_t N, int64_t K,
                                  int group, uint16_t* Y, hipStream_t stream) {
  const int64_t outs = GATED ? N / 2 : N;
  const int64_t per = (GATED ? 16 : 32) * R;
  const int64_t blocks = (outs + per - 1) / per;
  hipLaunchKernelGGL((k_gemv_mfma<S, E, MT, R, GATED>), dim3((unsigned)blocks), dim3(S * 64), 0, stream,
                     X, M, qw, sc, z, N, K, group, Y);
  return hipGetLastError();
}

template <int R, bool GATED>
static hipError_t launch_skinny_r(const uint16_t* X, int64_t M, const uint32_t* qw,
                                  const uint16_t* sc, const uint8_t* z, int64_t N, int64_t K,
                                  int group, uint16_t* Y, hipStream_t stream) {
  if (M <= 8) return launch_skinny_x<8, 4, 1, R, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
  if (M <= 16) return launch_skinny_x<8, 8, 1, R, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
  if (M <= 32) return launch_skinny_x<8, 16, 1, R, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
  // two token tiles: 4 waves per block, so a wave may also use the accumulation registers
  return launch_skinny_x<4, 16, 2, R, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
}

// Two row tiles per wave halve the activation bytes loaded per weight byte but also halve
// the blocks; measured on the Llama-2 7B and 70B shapes it pays from 160 blocks of two
// tiles (7B q|k|v: +25% at M = 8..32; 70B gate|up: +14..20%), and loses below (7B o_proj
// and down_proj, 64 blocks: -30%); fused gate|up needs more (7B, 344 blocks: -4% at M = 64).
template <bool GATED>
static hipError_t launch_skinny_t(const uint16_t* X, int64_t M, const uint32_t* qw,
                                  const uint16_t* sc, const uint8_t* z, int64_t N, int64_t K,
                                  int group, uint16_t* Y, hipStream_t stream) {
  const int64_t outs = GATED ? N / 2 : N;
  const int64_t blocks2 = (outs + (GATED ? 32 : 64) - 1) / (GATED ? 32 : 64);
  if (blocks2 >= (GATED ? kSkinnyR2MinBlocksGated : kSkinnyR2MinBlocks))
    return launch_skinny_r<2, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
  return launch_skinny_r<1, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
}

hipError_t launch_gemv_mfma(const uint16_t* X, int64_t M, const uint32_t* qweight,
                            const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                            int group, uint16_t* Y, bool gated, hipStream_t stream) {
  if (M < 1 || M > kSkinnyMaxM) return hipErrorInvalidValue;
  return gated ? launch_skinny_t<true>(X, M, qweight, scales, zeros, N, K, group, Y, stream)
               : launch_skinny_t<false>(X, M, qweight, scales, zeros, N, K, group, Y, stream);
}

}  // namespace awq
