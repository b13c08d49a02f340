// Vector and skinny-MFMA GEMV for 3-bit codes (a7 with w_bit = 3): Y[M][N] = X[M][K] deq(W)^T.
//
// "AWQ量化实战" §4.3 names 3-bit weights as the extreme low width; the decode GEMV then
// streams 3/8 of a byte per weight.
//
// Packed layout: 12 words per 128-channel block, in two bit planes. Low-plane word i
// (i < 8) holds bits 0-1 of channel pair (16 i + 2 f, 16 i + 2 f + 1) at bits 2 f and
// 16 + 2 f; high-plane word 8 + j (j < 4) holds bit 2 of pair (32 j + 2 p, 32 j + 2 p + 1)
// at bits p and 16 + p. Masking both planes for one pair leaves the two 3-bit codes at bits
// 0-2 of each 16-bit half, below the 0x6400 exponent: the fp16 pair (1024 + a, 1024 + b),
// exactly, and a packed add of -(1024 + z) gives (q - z). Zeros are nibbles as for 4-bit.
#include "common.hpp"
#include "launch.hpp"

namespace awq {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

__device__ __forceinline__ uint32_t magic_6400() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

// Sum over the 16 pairs of a chunk of x * q (the zero point is taken out by the caller:
// sum x (q - z) = sum x q - z sum x). Pair p = 4 a + e (e = p % 4) keeps its 2 low bits in
// place, at bits 2e, 2e + 1 of low word a / 2 (shifted right by 8 for odd a: one shift per
// 4 pairs), and its high bit is moved to bit 2e + 2 (one shift) and inserted (v_bfi_b32).
// The pair is then the fp16 subnormal pair 4^e q 2^-24, exactly (4^3 * 7 < 1024), which
// v_dot2 multiplies by the activations exactly and accumulates in fp32; each e has its own
// partial, and the powers of two (4^-e 2^24) are removed at the end (they commute with the
// rounding). One shift, one AND, one insert and one dot per pair.
__device__ __forceinline__ float chunk_dot3(uint2 lo, uint32_t hi, const half2v (&xq)[16]) {
  const uint32_t lw[4] = {lo.x, lo.x >> 8, lo.y, lo.y >> 8};
  float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int e = p & 3, sh = p - 2 * e - 2;  // high bit p -> bit 2e + 2
    const uint32_t hm = 0x00040004u << (2 * e);
    const uint32_t hs = sh > 0 ? (hi >> sh) : sh < 0 ? (hi << -sh) : hi;
    uint32_t u;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(u) : "s"(hm), "v"(hs), "v"(lw[p >> 2] & (0x00030003u << (2 * e))));
    part[e] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, u), xq[p], part[e], false);
  }
  return (part[0] + part[1] * 0.25f + part[2] * 0.0625f + part[3] * 0.015625f) * 16777216.0f;
}

__device__ __forceinline__ uint32_t zero_nibble(const uint8_t* zrow, int64_t g) {
  return ((uint32_t)zrow[g >> 1] >> (4 * (g & 1))) & 0xFu;
}

}  // namespace

// ------------------------------------------------------------------ vector GEMV, M <= 8
// The 8-bit kernel's mapping: a wave owns R rows (gated: gate row n and up row n + N/2),
// lane l walks 32-channel chunks c = l, l + 64, ...; chunk c's codes are low-plane words
// 12 (c / 4) + 2 (c % 4) and + 1 (one 8-byte load) and high-plane word 12 (c / 4) + 8 + c % 4.
// v_dot2 with the activation pair accumulates in fp32; the group scale multiplies each
// chunk's partial in fp32.
template <int M, int R, bool GATED>
__global__ void __launch_bounds__(256)
    k_gemv3(const uint16_t* __restrict__ X, const uint32_t* __restrict__ qweight,
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
  const int64_t zb = (G + 1) / 2;        // zero bytes per row
  const int64_t words = K * 3 / 32;
  const uint32_t magic = magic_6400();

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
    half2v qz[R][16];            // pair p = channels (2p, 2p + 1) of the chunk, as q - z
    float sc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t* wp = qweight + rows[r] * words + (c >> 2) * 12;
      const uint2 lo = *reinterpret_cast<const uint2*>(wp + 2 * (c & 3));
      const uint32_t hi = wp[8 + (c & 3)];
      sc[r] = h2f(scales[rows[r] * G + g]);
      const uint32_t zbits = 0x6400u + zero_nibble(zeros + rows[r] * zb, g);  // fp16 of 1024 + z
      const half2v zz = -__builtin_bit_cast(half2v, zbits | (zbits << 16));
#pragma unroll
      for (int p = 0; p < 16; ++p)
        qz[r][p] = __builtin_bit_cast(half2v, widen3_pair(p < 8 ? lo.x : lo.y, hi, p & 7, p, magic)) + zz;
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

// ------------------------------------------------------------------ M = 1, K <= 16384
// The single-token structure of the 4-bit decode kernel: 4 waves per block share the
// activation row through LDS; each wave owns RPW rows (gated: gate row n and up row
// n + N/2) and issues every code load of its rows (U chunks per lane, covering K) before
// any arithmetic, so a lane keeps U * RPW * 12 bytes in flight. Scheduler barriers keep
// the activation loads first: the wait for them (in-order load counter) leaves the codes in
// flight, and the LDS-only barrier shares the row without waiting for the codes. Every lane
// stores lane 0's sum; a row index past the matrix end is clamped to the wave's last row,
// whose value it rewrites.
template <int U, int RPW, bool GATED>
__global__ void __launch_bounds__(256)
    k_gemv3_1(const uint16_t* X, const uint32_t* qweight, const uint16_t* scales,
              const uint8_t* zeros, int64_t N, int64_t K, int gsh, uint16_t* Y) {
  static_assert(!GATED || RPW == 2, "a gated wave owns one gate row and one up row");
  extern __shared__ uint4 xs[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t wave_id = (int64_t)blockIdx.x * 4 + (tid >> 6);
  const int64_t C = K / 32, G = K >> (gsh + 5), zbytes = (G + 1) / 2, words = K * 3 / 32;
  const int64_t xw = K / 8;  // 16-byte pieces of the activation row
  const int64_t nh = N / 2;
  const int64_t n_out = wave_id < nh ? wave_id : nh - 1;
  const int64_t row0 = GATED ? n_out : wave_id * RPW;
  const int64_t lastrow = row0 + RPW - 1 < N ? row0 + RPW - 1 : N - 1;
  auto row_at = [&](int r) -> int64_t {
    if constexpr (GATED) return n_out + r * nh;
    const int64_t v = row0 + r;
    return v < lastrow ? v : lastrow;
  };

  uint4 v[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t i = j * 256 + tid;
    v[j] = *reinterpret_cast<const uint4*>(X + (i < xw ? i : xw - 1) * 8);
  }
  __builtin_amdgcn_sched_barrier(0);
  uint2 lo[RPW][U];
  uint32_t hi[RPW][U];
  uint16_t sc[RPW][U];
  uint8_t zb[RPW][U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int64_t c = u * 64 + lane;
    c = c < C ? c : C - 1;  // results past the row end are loaded but unused
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int64_t row = row_at(r);
      const uint32_t* wp = qweight + row * words + (c >> 2) * 12;
      lo[r][u] = *reinterpret_cast<const uint2*>(wp + 2 * (c & 3));
      hi[r][u] = wp[8 + (c & 3)];
      sc[r][u] = scales[row * G + (c >> gsh)];
      zb[r][u] = zeros[row * zbytes + (c >> (gsh + 1))];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // U * 256 >= K / 8 entries, then the fp32 sum of each 32-channel chunk (four
  // consecutive lanes hold one chunk's activations)
  float* xsum = reinterpret_cast<float*>(xs + U * 256);
  const half2v one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int i = j * 256 + tid;
    xs[i] = vgpr_copy(v[j]);
    float t = 0.0f;
    t = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, v[j].x), one, t, false);
    t = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, v[j].y), one, t, false);
    t = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, v[j].z), one, t, false);
    t = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, v[j].w), one, t, false);
    t += __shfl_xor(t, 1);
    t += __shfl_xor(t, 2);
    if ((i & 3) == 0) xsum[i >> 2] = t;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // LDS only: codes stay in flight

  float sums[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = u * 64 + lane;
      if (c < C) {
        half2v xq[16];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint4 xv = xs[c * 4 + w];  // channels 8w .. 8w + 7 as pairs
          xq[w * 4 + 0] = __builtin_bit_cast(half2v, xv.x);
          xq[w * 4 + 1] = __builtin_bit_cast(half2v, xv.y);
          xq[w * 4 + 2] = __builtin_bit_cast(half2v, xv.z);
          xq[w * 4 + 3] = __builtin_bit_cast(half2v, xv.w);
        }
        const float z = (float)(((uint32_t)zb[r][u] >> (4 * ((c >> gsh) & 1))) & 0xFu);
        acc = __builtin_fmaf(h2f(sc[r][u]), __builtin_fmaf(-z, xsum[c], chunk_dot3(lo[r][u], hi[r][u], xq)), acc);
      }
    }
    sums[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_sum(acc)), 0));
    if constexpr (!GATED) Y[row_at(r)] = f2h_bits(sums[r]);
  }
  if constexpr (GATED) Y[n_out] = f2h_bits(silu_f32(sums[0]) * sums[RPW - 1]);
}

// ------------------------------------------------------------------ skinny MFMA, M <= 64
// The 4-bit skinny kernel's mapping: a wave owns 32 weight rows and a slice of the
// 128-channel steps; lane l takes row l % 32 and, with h = l / 32, the 32-channel chunks h
// and 2 + h of each step (channels [32 h, 32 h + 32) and [64 + 32 h, 96 + 32 h)). Chunk ch
// is low-plane words 2 ch, 2 ch + 1 and high-plane word 8 + ch of the step. k16 slice s
// takes 8 channels of chunk h + 2 (s / 4): pairs 4 (s % 4) .. 4 (s % 4) + 3. Scales as in
// the 4-bit kernel: a fresh partial tile per group (one per step for 128-channel groups, one
// per half for 64), and for 32-channel groups, where the two lane halves of a slice lie in
// different groups, the fp16 operand carries the scale.
// M = 33..64: two 32-token tiles share each widened operand (4 waves per block), with the
// scale carried by the operand for every group size, as in the 4-bit kernel.
namespace {

template <int MT>
struct SkinnyStage3 {
  uint2 lo[2];         // low-plane words of chunks h and 2 + h
  uint32_t hi[2];      // their high-plane words
  uint4 a[MT][8];      // X[token][same channels] per token tile, one 16-byte piece per k16 step
  uint32_t sc[2], zb;  // scales and zero nibbles of the lane's two chunks
};

// Slice s: pairs 4 (s % 4) .. 4 (s % 4) + 3 of chunk half = s / 4.
template <int MT>
__device__ __forceinline__ half8 operand3(const SkinnyStage3<MT>& st, int s, half2v zz, uint32_t magic) {
  const int half = s >> 2, p0 = 4 * (s & 3);
  const uint32_t lo = (p0 < 8) ? st.lo[half].x : st.lo[half].y;
  const half2v d0 = __builtin_bit_cast(half2v, widen3_pair(lo, st.hi[half], (p0 + 0) & 7, p0 + 0, magic)) + zz;
  const half2v d1 = __builtin_bit_cast(half2v, widen3_pair(lo, st.hi[half], (p0 + 1) & 7, p0 + 1, magic)) + zz;
  const half2v d2 = __builtin_bit_cast(half2v, widen3_pair(lo, st.hi[half], (p0 + 2) & 7, p0 + 2, magic)) + zz;
  const half2v d3 = __builtin_bit_cast(half2v, widen3_pair(lo, st.hi[half], (p0 + 3) & 7, p0 + 3, magic)) + zz;
  return half8{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
}

}  // namespace

template <int S, int E, int MT, bool GATED>
__global__ void __launch_bounds__(S * 64)
    k_gemv_mfma3(const uint16_t* X, int64_t M, const uint32_t* qweight, const uint16_t* scales,
                 const uint8_t* zeros, int64_t N, int64_t K, int group, uint16_t* Y) {
  __shared__ float red[S][MT * E][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  const int lg = group == 128 ? 7 : group == 64 ? 6 : 5;
  const bool g128 = group == 128, g32 = group == 32;
  const int64_t G = K / kGroup;                          // 128-channel steps
  const int64_t Gs = K / group, zbr = (Gs + 1) / 2;      // groups, zero bytes per row
  const int64_t words = K * 3 / 32;
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
  const uint32_t magic = magic_6400();
  const uint8_t* zrow = zeros + n * zbr;

  auto load = [&](SkinnyStage3<MT>& st, int64_t g) {
    const int64_t q0 = (g * kGroup + 32 * h) >> lg, q1 = (g * kGroup + 64 + 32 * h) >> lg;
    st.zb = zero_nibble(zrow, q0) | (zero_nibble(zrow, q1) << 8);
    st.sc[0] = scales[n * Gs + q0];
    st.sc[1] = scales[n * Gs + q1];
    const uint32_t* wp = qweight + n * words + g * 12;
    st.lo[0] = *reinterpret_cast<const uint2*>(wp + 2 * h);
    st.lo[1] = *reinterpret_cast<const uint2*>(wp + 4 + 2 * h);
    st.hi[0] = wp[8 + h];
    st.hi[1] = wp[10 + h];
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

  auto body = [&](const SkinnyStage3<MT>& st) {
    half2v zz[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t zbits = 0x6400u + ((st.zb >> (8 * half)) & 0xFF);
      zz[half] = -__builtin_bit_cast(half2v, zbits | (zbits << 16));
    }
    if constexpr (MT == 2) {
      // two token tiles: the operand carries the scale of its 32-channel half for every
      // group size ((q - z) sc in fp16, one rounding), the MFMAs accumulate the tiles
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint32_t sb = st.sc[s >> 2];
        const half2v s2 = __builtin_bit_cast(half2v, sb | (sb << 16));
        const half8 b = operand3(st, s, zz[s >> 2], magic) * half8{s2[0], s2[1], s2[0], s2[1], s2[0], s2[1], s2[0], s2[1]};
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
            operand3(st, s, zz[s >> 2], magic) * half8{s2[0], s2[1], s2[0], s2[1], s2[0], s2[1], s2[0], s2[1]},
            d, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) acc[0][e] += d[e];
    } else if (g128) {
      f32x16 d = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s)
        d = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, st.a[0][s]),
                                                   operand3(st, s, zz[s >> 2], magic), d, 0, 0, 0);
      const float scf = h2f((uint16_t)st.sc[0]);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[0][e] = __builtin_fmaf(scf, d[e], acc[0][e]);
    } else {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x16 d = f32x16{};
#pragma unroll
        for (int s = 4 * half; s < 4 * half + 4; ++s)
          d = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, st.a[0][s]),
                                                     operand3(st, s, zz[half], magic), d, 0, 0, 0);
        const float scf = h2f((uint16_t)st.sc[half]);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[0][e] = __builtin_fmaf(scf, d[e], acc[0][e]);
      }
    }
  };

  if (g1 > g0) {
    SkinnyStage3<MT> s0, s1;
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
static hipError_t launch_skinny3_x(const uint16_t* X, int64_t M, const uint32_t* qw,
                                   const uint16_t* sc, const uint8_t* z, int64_t N, int64_t K,
                                   int group, uint16_t* Y, hipStream_t stream) {
  const int64_t outs = GATED ? N / 2 : N;
  const int64_t per = GATED ? 16 : 32;
  const int64_t blocks = (outs + per - 1) / per;
  hipLaunchKernelGGL((k_gemv_mfma3<S, E, MT, GATED>), dim3((unsigned)blocks), dim3(S * 64), 0, stream,
                     X, M, qw, sc, z, N, K, group, Y);
  return hipGetLastError();
}

template <bool GATED>
static hipError_t launch_skinny3_t(const uint16_t* X, int64_t M, const uint32_t* qw,
                                   const uint16_t* sc, const uint8_t* z, int64_t N, int64_t K,
                                   int group, uint16_t* Y, hipStream_t stream) {
  if (M <= 8) return launch_skinny3_x<8, 4, 1, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
  if (M <= 16) return launch_skinny3_x<8, 8, 1, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
  if (M <= 32) return launch_skinny3_x<8, 16, 1, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
  // two token tiles: 4 waves per block, so a wave may also use the accumulation registers
  return launch_skinny3_x<4, 16, 2, GATED>(X, M, qw, sc, z, N, K, group, Y, stream);
}

hipError_t launch_gemv_mfma3(const uint16_t* X, int64_t M, const uint32_t* qweight,
                             const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                             int group, uint16_t* Y, bool gated, hipStream_t stream) {
  if (M < 1 || M > kSkinnyMaxM) return hipErrorInvalidValue;
  return gated ? launch_skinny3_t<true>(X, M, qweight, scales, zeros, N, K, group, Y, stream)
               : launch_skinny3_t<false>(X, M, qweight, scales, zeros, N, K, group, Y, stream);
}

template <int M, bool GATED>
static hipError_t launch_gemv3_m(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                                 const uint8_t* z, int64_t N, int64_t K, int gsh, uint16_t* Y,
                                 hipStream_t stream) {
  constexpr int R = GATED ? 2 : (M <= 2 ? 2 : 4);
  const int64_t waves = GATED ? N / 2 : (N + R - 1) / R;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((k_gemv3<M, R, GATED>), dim3((unsigned)blocks), dim3(256), 0, stream, X, qw,
                     sc, z, N, K, gsh, Y);
  return hipGetLastError();
}

template <bool GATED>
static hipError_t launch_gemv3_t(const uint16_t* X, int64_t M, const uint32_t* qw,
                                 const uint16_t* sc, const uint8_t* z, int64_t N, int64_t K,
                                 int gsh, uint16_t* Y, hipStream_t stream) {
  switch (M) {
    case 1: return launch_gemv3_m<1, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 2: return launch_gemv3_m<2, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 3: return launch_gemv3_m<3, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 4: return launch_gemv3_m<4, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 5: return launch_gemv3_m<5, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 6: return launch_gemv3_m<6, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 7: return launch_gemv3_m<7, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    case 8: return launch_gemv3_m<8, GATED>(X, qw, sc, z, N, K, gsh, Y, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int U, int RPW, bool GATED>
static hipError_t launch_gemv3_1x(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                                  const uint8_t* z, int64_t N, int64_t K, int gsh, uint16_t* Y,
                                  hipStream_t stream) {
  const int64_t waves = GATED ? N / 2 : (N + RPW - 1) / RPW;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((k_gemv3_1<U, RPW, GATED>), dim3((unsigned)blocks), dim3(256),
                     (size_t)U * 256 * 17, stream, X, qw, sc, z, N, K, gsh, Y);
  return hipGetLastError();
}

// M = 1 with U = ceil(K / 2048) <= 8 chunks per lane: two rows per wave for tall matrices
// (and always when gated), else one.
template <bool GATED>
static hipError_t launch_gemv3_1(const uint16_t* X, const uint32_t* qw, const uint16_t* sc,
                                 const uint8_t* z, int64_t N, int64_t K, int gsh, uint16_t* Y,
                                 hipStream_t stream) {
  const int64_t U = (K / 32 + 63) / 64;
  const bool two = GATED || N >= 8192;
#define AWQ_GEMV3_1(u)                                                                   \
  case u:                                                                                \
    return two ? launch_gemv3_1x<u, 2, GATED>(X, qw, sc, z, N, K, gsh, Y, stream)        \
               : launch_gemv3_1x<u, 1, false>(X, qw, sc, z, N, K, gsh, Y, stream);
  switch (U) {
    AWQ_GEMV3_1(1)
    AWQ_GEMV3_1(2)
    AWQ_GEMV3_1(3)
    AWQ_GEMV3_1(4)
    AWQ_GEMV3_1(5)
    AWQ_GEMV3_1(6)
    AWQ_GEMV3_1(7)
    AWQ_GEMV3_1(8)
    default: return hipErrorInvalidValue;
  }
#undef AWQ_GEMV3_1
}

hipError_t launch_gemv3(const uint16_t* X, int64_t M, const uint32_t* qweight,
                        const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                        int group, uint16_t* Y, bool gated, hipStream_t stream) {
  const int gsh = group == 128 ? 2 : group == 64 ? 1 : 0;  // chunk c (32 channels) is in group c >> gsh
  if (M == 1 && K <= 16384)
    return gated ? launch_gemv3_1<true>(X, qweight, scales, zeros, N, K, gsh, Y, stream)
                 : launch_gemv3_1<false>(X, qweight, scales, zeros, N, K, gsh, Y, stream);
  return gated ? launch_gemv3_t<true>(X, M, qweight, scales, zeros, N, K, gsh, Y, stream)
               : launch_gemv3_t<false>(X, M, qweight, scales, zeros, N, K, gsh, Y, stream);
}

}  // namespace awq
