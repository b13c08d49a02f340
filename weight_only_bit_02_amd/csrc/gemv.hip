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
// packed layout puts the channel pair (2p, 2p+1) of a word in nibbles p and p+4, so
// one mask per pair yields two adjacent channels and the activations are used in
// their natural order (each 32-bit word of x is one pair). Rows finish with a DPP /
// shuffle reduction across the wave.
//
// Fused gate|up (GATED): the packed weight holds N/2 gate rows, then N/2 up rows
// ("AWQ量化技术Skill", "主要功能和特点": fused MLP modules). A wave computes gate row n
// and up row n + N/2 together and stores h_n = SiLU(g_n) * u_n (fp32, one fp16
// rounding) into Y[M][N/2].
#include "common.hpp"
#include "launch.hpp"

namespace awq {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

template <int M, int R, bool GATED>
__global__ void __launch_bounds__(256)
    k_gemv(const uint16_t* __restrict__ X, const uint32_t* __restrict__ qweight,
           const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int64_t N,
           int64_t K, int gsh, uint16_t* __restrict__ Y) {
  static_assert(!GATED || R == 2, "a gated wave owns one gate row and one up row");
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nh = N / 2;
  const int64_t row0 = GATED ? wave : wave * R;
  if (row0 >= (GATED ? nh : N)) return;  // whole wave leaves together
  const int64_t C = K / 32;  // chunks per row
  const int64_t G = (K >> (gsh + 5));
  const int64_t zb = (G + 1) / 2;
  const int64_t words = K / 8;

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
          const uint32_t u = ((wd[w] >> (4 * p)) & 0x000F000Fu) | 0x64006400u;  // (1024+q_2p, 1024+q_2p+1)
          qz[r][w * 4 + p] = __builtin_bit_cast(half2v, u) + zz;                // exact (q - z)
        }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4* xp = reinterpret_cast<const uint4*>(X + (int64_t)m * K + c * 32);
      half2v xq[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint4 v = xp[w];  // channels 8w .. 8w+7 as the pairs (0,1) (2,3) (4,5) (6,7)
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
        acc[r][m] += sc[r] * part;
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

// M = 1: the activation row is staged once per block in LDS, so the inner loop reads
// it with ds_read_b128 shared by the R rows of a wave. A lane's code loads for
// U chunks of each of its R rows are issued together, and the next batch is in flight
// while the current one is multiplied (two register buffers), so a wave keeps
// R * U * 16 bytes per lane of HBM reads outstanding.
template <int R, int U>
struct GemvBatch {
  uint4 cw[R][U];
  uint16_t sc[R][U];
  uint8_t zb[R][U];
};

template <int R, int U>
__device__ __forceinline__ void gemv1_load(GemvBatch<R, U>& bt, const uint32_t* qweight,
                                           const uint16_t* scales, const uint8_t* zeros,
                                           const int64_t (&rows)[R],
                                           int64_t C, int64_t words, int64_t G, int64_t zbytes,
                                           int64_t b, int lane, int gsh) {
  // Straight-line loads (chunk index clamped, results past the row end unused), so the
  // compiler can keep them all in flight and wait for each one only where it is used.
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int64_t c = (b * U + u) * 64 + lane;
    c = c < C ? c : C - 1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      bt.cw[r][u] = *reinterpret_cast<const uint4*>(qweight + rows[r] * words + c * 4);
      bt.sc[r][u] = scales[rows[r] * G + (c >> gsh)];
      bt.zb[r][u] = zeros[rows[r] * zbytes + (c >> (gsh + 1))];
    }
  }
}

// fp16 magic 1024.0 in both halves, held in a VGPR the optimizer cannot see through: the
// widening then compiles to one v_and_or_b32 per pair (mask from an SGPR, magic from
// this VGPR) instead of an AND and an OR with literal operands.
__device__ __forceinline__ uint32_t magic_1024x2() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

// Per chunk (4 words = 32 channels) and row: exact (q - z) in fp16, two channels per dot.
// Pairs p = 0, 2 of a word are masked at bits 0..3 of each half, pairs p = 1, 3 at bits
// 4..7 (one shift by 8 serves p = 2, 3): with the 0x6400 magic the latter read 1024 + 16 q,
// and subtracting 1024 + 16 z leaves 16 (q - z), still exact. They accumulate in part1,
// whose factor 16 is removed at the end; a power-of-two factor commutes with every fp32
// rounding, so the result is the same as with unscaled codes.
template <int R, int U>
__device__ __forceinline__ void gemv1_compute(const GemvBatch<R, U>& bt, const uint4* __restrict__ xs,
                                              float (&acc)[R], int64_t C, int64_t b, int lane,
                                              uint32_t magic, int gsh) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = (b * U + u) * 64 + lane;
    if (c < C) {
      half2v xq[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint4 v = xs[c * 4 + w];  // channels 8w .. 8w+7 as the pairs (0,1) (2,3) (4,5) (6,7)
        xq[w * 4 + 0] = __builtin_bit_cast(half2v, v.x);
        xq[w * 4 + 1] = __builtin_bit_cast(half2v, v.y);
        xq[w * 4 + 2] = __builtin_bit_cast(half2v, v.z);
        xq[w * 4 + 3] = __builtin_bit_cast(half2v, v.w);
      }
      const int nib = (int)((c >> gsh) & 1) * 4;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t z = (bt.zb[r][u] >> nib) & 0xF;
        const uint32_t z1 = 0x6400u + z, z16 = 0x6400u + 16 * z;  // fp16 1024 + z, 1024 + 16 z
        const half2v zz1 = -__builtin_bit_cast(half2v, z1 | (z1 << 16));
        const half2v zz16 = -__builtin_bit_cast(half2v, z16 | (z16 << 16));
        const uint32_t wd[4] = {bt.cw[r][u].x, bt.cw[r][u].y, bt.cw[r][u].z, bt.cw[r][u].w};
        float part0 = 0.0f, part1 = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t hi = wd[w] >> 8;
          const half2v d0 = __builtin_bit_cast(half2v, (wd[w] & 0x000F000Fu) | magic) + zz1;
          const half2v d1 = __builtin_bit_cast(half2v, (wd[w] & 0x00F000F0u) | magic) + zz16;
          const half2v d2 = __builtin_bit_cast(half2v, (hi & 0x000F000Fu) | magic) + zz1;
          const half2v d3 = __builtin_bit_cast(half2v, (hi & 0x00F000F0u) | magic) + zz16;
          part0 = __builtin_amdgcn_fdot2(d0, xq[w * 4 + 0], part0, false);
          part1 = __builtin_amdgcn_fdot2(d1, xq[w * 4 + 1], part1, false);
          part0 = __builtin_amdgcn_fdot2(d2, xq[w * 4 + 2], part0, false);
          part1 = __builtin_amdgcn_fdot2(d3, xq[w * 4 + 3], part1, false);
        }
        acc[r] = __builtin_fmaf(h2f(bt.sc[r][u]), part0 + part1 * 0.0625f, acc[r]);
      }
    }
  }
}

// Barrier for LDS data only: wait for this wave's LDS operations, then s_barrier. Unlike
// __syncthreads() it does not wait for outstanding global loads, so the HBM reads
// issued before it stay in flight. The memory clobber keeps the compiler from moving
// those loads past it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Each wave owns R rows. The activation loads go out first, then all of the wave's code
// loads for its rows (U chunks per lane per row, covering all of K when the batch count
// nb is 1); scheduler barriers keep that order, so the wait for the activations
// (in-order load counter) leaves the codes in flight, and the LDS-only barrier shares
// the activation row without waiting for them. For K above 64 * U * 32 the wave walks
// nb batches with the next batch's loads in flight (unconditional, clamped prefetch, so
// every path has the same loads outstanding and the waits stay exact).
template <int R, int U, int XR, int WPB, bool GATED>
__global__ void __launch_bounds__(WPB * 64)
    k_gemv1(const uint16_t* X, const uint32_t* qweight, const uint16_t* scales,
            const uint8_t* zeros, int64_t N, int64_t K, int gsh, uint16_t* Y) {
  static_assert(!GATED || R == 2, "a gated wave owns one gate row and one up row");
  // (no __restrict__: the code loads must stay ordered before the LDS barrier below)
  // XR * WPB * 64 entries (>= K / 8): entry i holds channels 8i..8i+7
  extern __shared__ uint4 xs[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t nh = N / 2;
  const int64_t wave_id = (int64_t)blockIdx.x * WPB + (tid >> 6);
  const int64_t row0 = GATED ? (wave_id < nh ? wave_id : nh - 1) : wave_id * R;
  const int64_t C = K / 32, G = (K >> (gsh + 5)), zbytes = (G + 1) / 2, words = K / 8;
  const int64_t nb = (C + 64 * U - 1) / (64 * U);
  __builtin_assume(nb >= 1);
  int64_t rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    rows[r] = GATED ? row0 + r * nh : ((row0 + r < N) ? row0 + r : N - 1);

  uint4 v[XR];
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int64_t i = j * WPB * 64 + tid;
    v[j] = *reinterpret_cast<const uint4*>(X + (i < words ? i : words - 1) * 8);
  }
  __builtin_amdgcn_sched_barrier(0);
  GemvBatch<R, U> b0, b1;
  gemv1_load(b0, qweight, scales, zeros, rows, C, words, G, zbytes, 0, lane, gsh);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int64_t i = j * WPB * 64 + tid;
    xs[i] = vgpr_copy(v[j]);  // the LDS row is padded to XR * WPB * 64 entries: no predicate
  }
  lds_barrier();

  const uint32_t magic = magic_1024x2();
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  if (nb == 1) {
    gemv1_compute(b0, xs, acc, C, 0, lane, magic, gsh);
  } else {
    for (int64_t b = 0; b < nb; b += 2) {
      const int64_t b1i = b + 1 < nb ? b + 1 : nb - 1;
      gemv1_load(b1, qweight, scales, zeros, rows, C, words, G, zbytes, b1i, lane, gsh);
      gemv1_compute(b0, xs, acc, C, b, lane, magic, gsh);
      const int64_t b2i = b + 2 < nb ? b + 2 : nb - 1;
      gemv1_load(b0, qweight, scales, zeros, rows, C, words, G, zbytes, b2i, lane, gsh);
      if (b + 1 < nb) gemv1_compute(b1, xs, acc, C, b + 1, lane, magic, gsh);
    }
  }
  if constexpr (GATED) {
    const float g = wave_sum(acc[0]), u = wave_sum(acc[R - 1]);
    if (lane == 0 && wave_id < nh) Y[wave_id] = f2h_bits(silu_f32(g) * u);
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float sum = wave_sum(acc[r]);
      if (lane == 0 && row0 + r < N) Y[row0 + r] = f2h_bits(sum);
    }
  }
}

template <int R, int U, int XR, int WPB, bool GATED>
static hipError_t launch_gemv1_x(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                                 const uint8_t* z, int64_t N, int64_t K, int gsh, uint16_t* Y,
                                 hipStream_t stream) {
  const int64_t waves = GATED ? N / 2 : (N + R - 1) / R;
  const int64_t blocks = (waves + WPB - 1) / WPB;
  hipLaunchKernelGGL((k_gemv1<R, U, XR, WPB, GATED>), dim3((unsigned)blocks), dim3(WPB * 64),
                     (size_t)XR * WPB * 64 * 16, stream, X, qw, sc, z, N, K, gsh, Y);
  return hipGetLastError();
}

// K <= 32768: the activation row (K / 8 16-byte entries) fits XR * WPB * 64 entries.
template <int R, int U, bool GATED, int WPB = 4>
static hipError_t launch_gemv1(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                               const uint8_t* z, int64_t N, int64_t K, int gsh, uint16_t* Y,
                               hipStream_t stream) {
  const int64_t per_thread = (K / 8 + WPB * 64 - 1) / (WPB * 64);
  if (per_thread <= 1) return launch_gemv1_x<R, U, 1, WPB, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
  if (per_thread <= 2) return launch_gemv1_x<R, U, 2, WPB, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
  if (per_thread <= 4) return launch_gemv1_x<R, U, 4, WPB, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
  if (per_thread <= 8) return launch_gemv1_x<R, U, 8, WPB, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
  return launch_gemv1_x<R, U, 16, WPB, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
}

// One batch covers K (at most 8 chunks per lane, K <= 16384), so only that path is
// compiled: half the registers of the batched kernel, eight waves per SIMD. Each wave
// owns RPW consecutive rows; with RPW = 2 the second row's codes are in flight while
// the first is multiplied (tall matrices, where waves otherwise load and then compute in
// lockstep). Stores are made by every lane with lane 0's sum (no branch); a row index
// past the matrix end is clamped to the wave's last row, whose value it rewrites.
template <int U, int XR, int WPB, int RPW, bool GATED>
__global__ void __launch_bounds__(WPB * 64)
    k_gemv1s(const uint16_t* X, const uint32_t* qweight, const uint16_t* scales,
             const uint8_t* zeros, int64_t N, int64_t K, int gsh, uint16_t* Y) {
  static_assert(!GATED || RPW == 2, "a gated wave owns one gate row and one up row");
  extern __shared__ uint4 xs[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * WPB + (tid >> 6);
  const int64_t C = K / 32, G = (K >> (gsh + 5)), zbytes = (G + 1) / 2, words = K / 8;
  // plain: rows wave_id * RPW + r, clamped to the wave's last row; gated: gate row n and
  // up row n + N/2, n clamped to the last output (its store rewrites the same value)
  const int64_t nh = N / 2;
  const int64_t n_out = wave_id < nh ? wave_id : nh - 1;
  const int64_t row0 = GATED ? n_out : wave_id * RPW;
  const int64_t lastrow = row0 + RPW - 1 < N ? row0 + RPW - 1 : N - 1;
  auto row_at = [&](int r) -> int64_t {
    if constexpr (GATED) return n_out + r * nh;
    const int64_t v = row0 + r;
    return v < lastrow ? v : lastrow;
  };

  uint4 v[XR];
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int64_t i = j * WPB * 64 + tid;
    v[j] = *reinterpret_cast<const uint4*>(X + (i < words ? i : words - 1) * 8);
  }
  __builtin_amdgcn_sched_barrier(0);
  GemvBatch<1, U> bt[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int64_t rows[1] = {row_at(r)};
    gemv1_load(bt[r], qweight, scales, zeros, rows, C, words, G, zbytes, 0, lane, gsh);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int64_t i = j * WPB * 64 + tid;
    xs[i] = vgpr_copy(v[j]);  // the LDS row is padded to XR * WPB * 64 entries: no predicate
  }
  lds_barrier();

  const uint32_t magic = magic_1024x2();
  float sums[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    float acc[1] = {0.0f};
    gemv1_compute(bt[r], xs, acc, C, 0, lane, magic, gsh);
    sums[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_sum(acc[0])), 0));
    if constexpr (!GATED) Y[row_at(r)] = f2h_bits(sums[r]);
  }
  if constexpr (GATED) Y[n_out] = f2h_bits(silu_f32(sums[0]) * sums[RPW - 1]);
}

template <int U, int XR, int WPB, int RPW, bool GATED>
static hipError_t launch_gemv1s_x(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                                  const uint8_t* z, int64_t N, int64_t K, int gsh, uint16_t* Y,
                                  hipStream_t stream) {
  const int64_t waves = GATED ? N / 2 : (N + RPW - 1) / RPW;
  const int64_t blocks = (waves + WPB - 1) / WPB;
  hipLaunchKernelGGL((k_gemv1s<U, XR, WPB, RPW, GATED>), dim3((unsigned)blocks), dim3(WPB * 64),
                     (size_t)XR * WPB * 64 * 16, stream, X, qw, sc, z, N, K, gsh, Y);
  return hipGetLastError();
}

// XR = U: the activation row (K / 8 entries) fits U * 256 entries, as U = ceil(K / 2048).
template <int U, int RPW, bool GATED>
static hipError_t launch_gemv1s(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                                const uint8_t* z, int64_t N, int64_t K, int gsh, uint16_t* Y,
                                hipStream_t stream) {
  return launch_gemv1s_x<U, U, 4, RPW, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
}

// M = 1 dispatch (K <= 32768, so the activation row fits 64 KiB of LDS). Up to eight
// chunks per lane (K <= 16384): the single-batch kernel, two rows per wave for tall
// matrices with at most two chunks per lane (measured on the Llama-2 7B shapes), else
// one; gated, always the gate row and the up row. Longer rows: plain, the single-batch
// kernel with one row per wave; gated, the batched kernel, four chunks per lane per batch.
template <bool GATED>
static hipError_t launch_gemv_m1(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                                 const uint8_t* z, int64_t N, int64_t K, int gsh, uint16_t* Y,
                                 hipStream_t stream) {
  const int64_t cpl = (K / 32 + 63) / 64;  // chunks per lane to cover K once
  const bool two = GATED || N >= 8192;
  switch (cpl) {
    case 1: return two ? launch_gemv1s<1, 2, GATED>(X, qw, sc, z, N, K, gsh, Y, stream)
                       : launch_gemv1s<1, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 2: return two ? launch_gemv1s<2, 2, GATED>(X, qw, sc, z, N, K, gsh, Y, stream)
                       : launch_gemv1s<2, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 3: return GATED ? launch_gemv1s<3, 2, GATED>(X, qw, sc, z, N, K, gsh, Y, stream)
                         : launch_gemv1s<3, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 4: return GATED ? launch_gemv1s<4, 2, GATED>(X, qw, sc, z, N, K, gsh, Y, stream)
                         : launch_gemv1s<4, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 5: return GATED ? launch_gemv1s<5, 2, GATED>(X, qw, sc, z, N, K, gsh, Y, stream)
                         : launch_gemv1s<5, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 6: return GATED ? launch_gemv1s<6, 2, GATED>(X, qw, sc, z, N, K, gsh, Y, stream)
                         : launch_gemv1s<6, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 7: return GATED ? launch_gemv1s<7, 2, GATED>(X, qw, sc, z, N, K, gsh, Y, stream)
                         : launch_gemv1s<7, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 8: return GATED ? launch_gemv1s<8, 2, GATED>(X, qw, sc, z, N, K, gsh, Y, stream)
                         : launch_gemv1s<8, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream);
    // longer rows (K up to 32768), plain: still one batch of all of a lane's loads (on the
    // Llama-2-70B down_proj, K = 28672, 25% faster than batches of four); gated: the
    // batched kernel (two rows per wave with all loads up front would take every register)
    case 9: if (!GATED) return launch_gemv1s<9, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream); break;
    case 10: if (!GATED) return launch_gemv1s<10, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream); break;
    case 11: if (!GATED) return launch_gemv1s<11, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream); break;
    case 12: if (!GATED) return launch_gemv1s<12, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream); break;
    case 13: if (!GATED) return launch_gemv1s<13, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream); break;
    case 14: if (!GATED) return launch_gemv1s<14, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream); break;
    case 15: if (!GATED) return launch_gemv1s<15, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream); break;
    case 16: if (!GATED) return launch_gemv1s<16, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream); break;
    default: break;
  }
  return GATED ? launch_gemv1<2, 4, GATED>(X, qw, sc, z, N, K, gsh, Y, stream)
               : launch_gemv1<1, 4, false>(X, qw, sc, z, N, K, gsh, Y, stream);
}

template <int M, bool GATED>
static hipError_t launch_gemv_m(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                                const uint8_t* z, int64_t N, int64_t K, int gsh, uint16_t* Y,
                                hipStream_t stream) {
  constexpr int R = GATED ? 2 : 4;
  const int64_t waves = GATED ? N / 2 : (N + R - 1) / R;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((k_gemv<M, R, GATED>), dim3((unsigned)blocks), dim3(256), 0, stream, X, qw,
                     sc, z, N, K, gsh, Y);
  return hipGetLastError();
}

template <bool GATED>
static hipError_t launch_gemv_t(const uint16_t* X, int64_t M, const uint32_t* qweight,
                                const uint16_t* scales, const uint8_t* zeros, int64_t N,
                                int64_t K, int gsh, uint16_t* Y, hipStream_t stream) {
  switch (M) {
    case 1:
      if (K <= 32768) return launch_gemv_m1<GATED>(X, qweight, scales, zeros, N, K, gsh, Y, stream);
      return launch_gemv_m<1, GATED>(X, qweight, scales, zeros, N, K, gsh, Y, stream);
    case 2: return launch_gemv_m<2, GATED>(X, qweight, scales, zeros, N, K, gsh, Y, stream);
    case 3: return launch_gemv_m<3, GATED>(X, qweight, scales, zeros, N, K, gsh, Y, stream);
    case 4: return launch_gemv_m<4, GATED>(X, qweight, scales, zeros, N, K, gsh, Y, stream);
    case 5: return launch_gemv_m<5, GATED>(X, qweight, scales, zeros, N, K, gsh, Y, stream);
    case 6: return launch_gemv_m<6, GATED>(X, qweight, scales, zeros, N, K, gsh, Y, stream);
    case 7: return launch_gemv_m<7, GATED>(X, qweight, scales, zeros, N, K, gsh, Y, stream);
    case 8: return launch_gemv_m<8, GATED>(X, qweight, scales, zeros, N, K, gsh, Y, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(const uint16_t* X, int64_t M, const uint32_t* qweight,
                       const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                       int group, uint16_t* Y, bool gated, hipStream_t stream) {
  const int gsh = group == 128 ? 2 : group == 64 ? 1 : 0;  // chunk c (32 channels) is in group c >> gsh
  return gated ? launch_gemv_t<true>(X, M, qweight, scales, zeros, N, K, gsh, Y, stream)
               : launch_gemv_t<false>(X, M, qweight, scales, zeros, N, K, gsh, Y, stream);
}

}  // namespace awq
