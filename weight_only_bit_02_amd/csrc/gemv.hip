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

// M = 1: the activation row is staged once per block in LDS, already re-paired, so
// the inner loop reads it with ds_read_b128 and no permutes. A lane's code loads for
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
                                           int64_t b, int lane) {
  // Straight-line loads (chunk index clamped, results past the row end unused), so the
  // compiler can keep them all in flight and wait for each one only where it is used.
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int64_t c = (b * U + u) * 64 + lane;
    c = c < C ? c : C - 1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      bt.cw[r][u] = *reinterpret_cast<const uint4*>(qweight + rows[r] * words + c * 4);
      bt.sc[r][u] = scales[rows[r] * G + (c >> 2)];
      bt.zb[r][u] = zeros[rows[r] * zbytes + (c >> 3)];
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

template <int R, int U>
__device__ __forceinline__ void gemv1_compute(const GemvBatch<R, U>& bt, const uint4* __restrict__ xs,
                                              float (&acc)[R], int64_t C, int64_t b, int lane,
                                              uint32_t magic) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = (b * U + u) * 64 + lane;
    if (c < C) {
      half2v xq[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint4 v = xs[c * 4 + w];
        xq[w * 4 + 0] = __builtin_bit_cast(half2v, v.x);
        xq[w * 4 + 1] = __builtin_bit_cast(half2v, v.y);
        xq[w * 4 + 2] = __builtin_bit_cast(half2v, v.z);
        xq[w * 4 + 3] = __builtin_bit_cast(half2v, v.w);
      }
      const int nib = (int)((c >> 2) & 1) * 4;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t z = (bt.zb[r][u] >> nib) & 0xF;
        const uint32_t zbits = 0x6400u + z;
        const half2v zz = -__builtin_bit_cast(half2v, zbits | (zbits << 16));
        const uint32_t wd[4] = {bt.cw[r][u].x, bt.cw[r][u].y, bt.cw[r][u].z, bt.cw[r][u].w};
        float part0 = 0.0f, part1 = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t q = ((wd[w] >> (4 * p)) & 0x000F000Fu) | magic;
            const half2v d = __builtin_bit_cast(half2v, q) + zz;  // exact (q - z)
            if (p & 1) part1 = __builtin_amdgcn_fdot2(d, xq[w * 4 + p], part1, false);
            else part0 = __builtin_amdgcn_fdot2(d, xq[w * 4 + p], part0, false);
          }
        acc[r] += h2f(bt.sc[r][u]) * (part0 + part1);
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
template <int R, int U, int XR>
__global__ void __launch_bounds__(256)
    k_gemv1(const uint16_t* X, const uint32_t* qweight, const uint16_t* scales,
            const uint8_t* zeros, int64_t N, int64_t K, uint16_t* Y) {
  // (no __restrict__: the code loads must stay ordered before the LDS barrier below)
  // XR * 256 entries (>= K / 8): channels 8i..8i+7 as (0,4) (1,5) (2,6) (3,7)
  extern __shared__ uint4 xs[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (tid >> 6)) * R;
  const int64_t C = K / 32, G = K / kGroup, zbytes = (G + 1) / 2, words = K / 8;
  const int64_t nb = (C + 64 * U - 1) / (64 * U);
  __builtin_assume(nb >= 1);
  int64_t rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = (row0 + r < N) ? row0 + r : N - 1;

  uint4 v[XR];
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int64_t i = j * 256 + tid;
    v[j] = *reinterpret_cast<const uint4*>(X + (i < words ? i : words - 1) * 8);
  }
  __builtin_amdgcn_sched_barrier(0);
  GemvBatch<R, U> b0, b1;
  gemv1_load(b0, qweight, scales, zeros, rows, C, words, G, zbytes, 0, lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int64_t i = j * 256 + tid;
    uint4 p;
    p.x = __builtin_amdgcn_perm(v[j].z, v[j].x, 0x05040100u);
    p.y = __builtin_amdgcn_perm(v[j].z, v[j].x, 0x07060302u);
    p.z = __builtin_amdgcn_perm(v[j].w, v[j].y, 0x05040100u);
    p.w = __builtin_amdgcn_perm(v[j].w, v[j].y, 0x07060302u);
    xs[i] = p;  // the LDS row is padded to XR * 256 entries, so no store is predicated
  }
  lds_barrier();

  const uint32_t magic = magic_1024x2();
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  if (nb == 1) {
    gemv1_compute(b0, xs, acc, C, 0, lane, magic);
  } else {
    for (int64_t b = 0; b < nb; b += 2) {
      const int64_t b1i = b + 1 < nb ? b + 1 : nb - 1;
      gemv1_load(b1, qweight, scales, zeros, rows, C, words, G, zbytes, b1i, lane);
      gemv1_compute(b0, xs, acc, C, b, lane, magic);
      const int64_t b2i = b + 2 < nb ? b + 2 : nb - 1;
      gemv1_load(b0, qweight, scales, zeros, rows, C, words, G, zbytes, b2i, lane);
      if (b + 1 < nb) gemv1_compute(b1, xs, acc, C, b + 1, lane, magic);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float sum = wave_sum(acc[r]);
    if (lane == 0 && row0 + r < N) Y[row0 + r] = f2h_bits(sum);
  }
}

template <int R, int U, int XR>
static hipError_t launch_gemv1_x(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                                 const uint8_t* z, int64_t N, int64_t K, uint16_t* Y,
                                 hipStream_t stream) {
  const int64_t blocks = (N + 4 * R - 1) / (4 * R);
  hipLaunchKernelGGL((k_gemv1<R, U, XR>), dim3((unsigned)blocks), dim3(256), (size_t)XR * 256 * 16,
                     stream, X, qw, sc, z, N, K, Y);
  return hipGetLastError();
}

template <int R, int U>
static hipError_t launch_gemv1(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                               const uint8_t* z, int64_t N, int64_t K, uint16_t* Y,
                               hipStream_t stream) {
  const int64_t per_thread = (K / 8 + 255) / 256;
  if (per_thread <= 2) return launch_gemv1_x<R, U, 2>(X, qw, sc, z, N, K, Y, stream);
  if (per_thread <= 4) return launch_gemv1_x<R, U, 4>(X, qw, sc, z, N, K, Y, stream);
  if (per_thread <= 8) return launch_gemv1_x<R, U, 8>(X, qw, sc, z, N, K, Y, stream);
  return launch_gemv1_x<R, U, 16>(X, qw, sc, z, N, K, Y, stream);
}

// M = 1 dispatch (K <= 32768, so the activation row fits 64 KiB of LDS): one batch of
// ceil(K / 2048) chunks per lane when that is at most 8, else batches of 4.
static hipError_t launch_gemv_m1(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                                 const uint8_t* z, int64_t N, int64_t K, uint16_t* Y,
                                 hipStream_t stream) {
  const int64_t cpl = (K / 32 + 63) / 64;  // chunks per lane to cover K once
  switch (cpl) {
    case 1: return launch_gemv1<2, 1>(X, qw, sc, z, N, K, Y, stream);
    case 2: return launch_gemv1<2, 2>(X, qw, sc, z, N, K, Y, stream);
    case 3: return launch_gemv1<2, 3>(X, qw, sc, z, N, K, Y, stream);
    case 4: return launch_gemv1<2, 4>(X, qw, sc, z, N, K, Y, stream);
    case 5: return launch_gemv1<2, 5>(X, qw, sc, z, N, K, Y, stream);
    case 6: return launch_gemv1<2, 6>(X, qw, sc, z, N, K, Y, stream);
    case 7: return launch_gemv1<1, 7>(X, qw, sc, z, N, K, Y, stream);
    case 8: return launch_gemv1<1, 8>(X, qw, sc, z, N, K, Y, stream);
    default: return launch_gemv1<1, 4>(X, qw, sc, z, N, K, Y, stream);
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
    case 1:
      if (K <= 32768) return launch_gemv_m1(X, qweight, scales, zeros, N, K, Y, stream);
      return launch_gemv_m<1>(X, qweight, scales, zeros, N, K, Y, stream);
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
