// MFMA dequant-GEMM (a8): Y[M][N] = X[M][K] deq(W)^T for batches (prefill, M > 8).
// (The kernel template; each 4-bit instantiation is compiled in its own file, gemm_i*.hip,
// so the build compiles them in parallel.)
//
// "AWQ量化技术Skill", "主要功能和特点": a GEMM kernel serves batch sizes above one;
// "AWQ量化实战" §2.3 / §3.4: weights stay 4-bit in memory and are dequantized on the fly.
//
// Block tile 128 (tokens) x 256 (output channels), K step 128 (one group of 128, two of 64
// -- the lane half's 64 channels are then one group -- or four of 32, the lane half's
// words 0-3 one group and words 4-7 the next), four waves side by side
// along N, each owning 128 x 64 = 4 x 2 tiles of v_mfma_f32_32x32x16_f16.
//   - A (activations) is shared by the four waves: it goes global -> registers -> LDS,
//     double-buffered
//     with one barrier per K step; loads run two K steps ahead of the MFMAs.
//   - B (codes) is private to a wave: each lane loads two 16-byte chunks (8 packed words,
//     64 channels of one output column) straight into registers; word s is the lane's
//     B operand for the wave's k16 step s. The packed layout puts channel pairs (2p, 2p+1)
//     in nibbles p and p+4, so one mask per pair widens it, exactly, to (q - z) with the
//     0x6400 trick and a packed fp16 add, then multiplied by the group scale in fp16
//     (one rounding), so no LDS round trip and no barrier are needed for B.
// Within a K step the lane half h = lane / 32 covers channels [64 h, 64 h + 64) and k16
// step s covers 8 of them; A is read from LDS with the same channel map, so the contraction
// is the plain sum over K. fp32 accumulation, one fp16 rounding of the result.
// The 128-row A panels are handed to the XCDs in contiguous runs of tiles, so the
// blocks running together on one XCD share their A panel in that XCD's L2.
//
// Fused gate|up (GATED; "AWQ量化技术Skill", "主要功能和特点": fused MLP modules): the
// packed weight holds N/2 gate rows, then N/2 up rows. A block covers 128 outputs; a
// wave's first 32-column MFMA tile is gate column n, its second the up column n + N/2,
// so each lane holds g and u of the same output element and the epilogue stores
// SiLU(g) * u (fp32, one fp16 rounding) into Y[M][N/2] without any data exchange.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace awq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;
constexpr int kBN = 256;
constexpr int kBK = 128;              // channels per K step: one group of 128 or two of 64
constexpr int kAStride = kBK + 8;     // halves per LDS row of A (16-byte pad)
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t gemm_magic() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

// One packed word -> its 8 dequantized fp16 channels (q - z) * sc, in channel order.
__device__ __forceinline__ half8 dequant_word(uint32_t w, half2v zz, half2v s2, uint32_t magic) {
  half2v d[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t u = ((w >> (4 * p)) & 0x000F000Fu) | magic;
    d[p] = (__builtin_bit_cast(half2v, u) + zz) * s2;
  }
  return half8{d[0][0], d[0][1], d[1][0], d[1][1], d[2][0], d[2][1], d[3][0], d[3][1]};
}

// One packed 8-bit word pair -> 8 dequantized fp16 channels (q - z) * sc, in channel
// order: v_perm_b32 against 0x64646464 widens byte pairs exactly to (1024 + a, 1024 + b).
__device__ __forceinline__ half8 dequant_word8(uint32_t w0, uint32_t w1, half2v zz, half2v s2,
                                               uint32_t magic8) {
  half2v d[4];
  d[0] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(magic8, w0, 0x04010400u));
  d[1] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(magic8, w0, 0x04030402u));
  d[2] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(magic8, w1, 0x04010400u));
  d[3] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(magic8, w1, 0x04030402u));
#pragma unroll
  for (int p = 0; p < 4; ++p) d[p] = (d[p] + zz) * s2;
  return half8{d[0][0], d[0][1], d[1][0], d[1][1], d[2][0], d[2][1], d[3][0], d[3][1]};
}

// 4 channel pairs of 3-bit codes -> 8 dequantized fp16 channels (q - z) * sc, in channel
// order. Pair t (t = 0..3) has bits 0-1 in field F + t of the low-plane word `lo` (bits
// 2 (F + t) and 16 + 2 (F + t)) and bit 2 at bit P + t and 16 + P + t of the high-plane
// word `hi`; both land in place below the 0x6400 exponent, so the fp16 pair is exactly
// (1024 + q_even, 1024 + q_odd).
template <int F, int P>
__device__ __forceinline__ half8 dequant_word3(uint32_t lo, uint32_t hi, half2v zz, half2v s2,
                                               uint32_t magic) {
  half2v d[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    d[t] = (__builtin_bit_cast(half2v, widen3_pair(lo, hi, F + t, P + t, magic)) + zz) * s2;
  return half8{d[0][0], d[0][1], d[1][0], d[1][1], d[2][0], d[2][1], d[3][0], d[3][1]};
}

// Per-step operands that travel through registers: this thread's share of the A tile
// (8 x 16 bytes) and this lane's codes (2 columns x 32 bytes, or 64 with 8-bit codes)
// with their scales and zeros.
template <int BITS>
struct GemmStage {
  uint4 a[8];
  uint4 b[2][BITS / 2];       // 3-bit: the lane half's 4 low-plane words
  uint2 bh[2];                // 3-bit: the lane half's 2 high-plane words (unused otherwise)
  uint32_t zb[2], sc[2][2];  // per column: zero byte(s); scales of the lane's two 32-channel
                             // halves (the second only with 32-channel groups or 8-bit codes)
};

// SPLIT: 32-channel groups (two scales per lane half); otherwise 128 or 64, one scale.
// BITS = 8: 8-bit codes (16 words per lane half and step; both halves' scales and zero
// bytes always loaded). BITS = 3: 3-bit codes, 12 words per step (words 0-7 the low bit
// plane, 16 channels each; 8-11 the high plane, 32 channels each): lane half kh takes low
// words 4 kh .. 4 kh + 3 and high words 8 + 2 kh, 9 + 2 kh; zeros and scales as for 4-bit.
template <bool GATED, bool SPLIT, int BITS>
__global__ void __launch_bounds__(256)
    k_gemm(const uint16_t* X, int64_t M, const uint32_t* qweight, const uint16_t* scales,
           const uint8_t* zeros, int64_t N, int64_t K, int group, uint16_t* __restrict__ Y, int64_t mt,
           int64_t nt, int64_t per_xcd) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kAStride];

  // ---- XCD-aware tile order: XCD x (= blockIdx % 8) takes tiles [x * per_xcd, ...),
  // consecutive tiles share an A panel (m tile) and walk N.
  const int64_t t = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (t >= mt * nt) return;
  const int64_t m0 = (t / nt) * kBM;
  const int64_t n0 = (t % nt) * (GATED ? kBN / 2 : kBN);  // first output column of the tile
  const int64_t nh = N / 2;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m32 = lane & 31, kh = lane >> 5;
  // Lane half kh covers channels [64 kh, 64 kh + 64) of step `step`: group `step` with
  // zero nibble step & 1 (g = 128); group 2 step + kh, nibble kh (g = 64); groups
  // 4 step + 2 kh and 4 step + 2 kh + 1 for words 0-3 and 4-7, the low and high nibble of
  // byte 2 step + kh (g = 32)
  const int g64 = group == 64;
  const int64_t Gs = K / group, zb = BITS == 8 ? Gs : (Gs + 1) / 2, words = K * BITS / 32;
  const int lg = group == 128 ? 7 : group == 64 ? 6 : 5;
  const int64_t nsteps = K / kBK;
  const uint32_t magic = gemm_magic();
  uint32_t magic8 = 0;
  if constexpr (BITS == 8) asm volatile("v_mov_b32 %0, 0x64646464" : "=v"(magic8));

  // A staging map: 128 rows x 128 channels = 2048 16-byte pieces, 8 per thread.
  int64_t a_row[8];
  int a_kc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int id = i * 256 + tid;
    const int64_t r = m0 + (id >> 4);
    a_row[i] = (r < M ? r : M - 1) * K;
    a_kc[i] = id & 15;
  }
  // B map: this lane's two weight rows (gated: gate row n and up row n + N/2).
  int64_t b_col[2];
  if constexpr (GATED) {
    const int64_t n = n0 + wave * 32 + m32;
    b_col[0] = n < nh ? n : nh - 1;
    b_col[1] = b_col[0] + nh;
  } else {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t n = n0 + wave * 64 + b * 32 + m32;
      b_col[b] = n < N ? n : N - 1;
    }
  }

  // small loads first, then codes, then activations: waits for an older stage never
  // cover a younger one (in-order load counter)
  auto load = [&](GemmStage<BITS>& st, int64_t step) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if constexpr (BITS == 8) {
        const int64_t q0 = (step * kBK + 64 * kh) >> lg, q1 = (step * kBK + 64 * kh + 32) >> lg;
        st.zb[b] = (uint32_t)zeros[b_col[b] * zb + q0] | ((uint32_t)zeros[b_col[b] * zb + q1] << 8);
        st.sc[b][0] = scales[b_col[b] * Gs + q0];
        st.sc[b][1] = scales[b_col[b] * Gs + q1];
      } else if constexpr (SPLIT) {
        st.zb[b] = zeros[b_col[b] * zb + 2 * step + kh];
        st.sc[b][0] = scales[b_col[b] * Gs + 4 * step + 2 * kh];
        st.sc[b][1] = scales[b_col[b] * Gs + 4 * step + 2 * kh + 1];
      } else {
        st.zb[b] = zeros[b_col[b] * zb + (step >> (1 - g64))];
        st.sc[b][0] = scales[b_col[b] * Gs + (step << g64) + (g64 & kh)];
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if constexpr (BITS == 3) {
        const uint32_t* wp = qweight + b_col[b] * words + step * 12;
        st.b[b][0] = *reinterpret_cast<const uint4*>(wp + 4 * kh);
        st.bh[b] = *reinterpret_cast<const uint2*>(wp + 8 + 2 * kh);
      } else {
#pragma unroll
        for (int h = 0; h < BITS / 2; ++h)
          st.b[b][h] = *reinterpret_cast<const uint4*>(qweight + b_col[b] * words + step * (4 * BITS) +
                                                       kh * (2 * BITS) + h * 4);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      st.a[i] = *reinterpret_cast<const uint4*>(X + a_row[i] + step * kBK + a_kc[i] * 8);
  };
  auto store_a = [&](const GemmStage<BITS>& st, int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = i * 256 + tid;
      *reinterpret_cast<uint4*>(&As[buf][(id >> 4) * kAStride + a_kc[i] * 8]) = vgpr_copy(st.a[i]);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  // Prefetch distance 2: stage `cur` is being multiplied, `nxt` (one step ahead) has its A
  // in flight to LDS, `nn` (two steps ahead) is being loaded. The loop is unrolled by three
  // with the stages' roles rotated, so no register copy (which would wait for the loads
  // just issued) is ever needed. With 8- and 3-bit codes the three stages exceed the 256
  // architectural VGPRs and the compiler parks values in AGPRs; measured on the 7B shapes
  // at M = 2048 that still beats distance 1 (two stages, no spill): 530 -> 730 TFLOP/s
  // (8-bit), 725 -> 790 (3-bit).
  constexpr int PF = 2;
  GemmStage<BITS> S0, S1, S2;
  load(S0, 0);
  load(S1, nsteps > 1 ? 1 : 0);
  store_a(S0, 0);
  __syncthreads();

  auto body = [&](GemmStage<BITS>& cur, GemmStage<BITS>& nxt, GemmStage<BITS>& nn, int64_t step) {
    const int buf = (int)(step & 1);
    // always issued (clamped to the last step) so the load counter is the same on every
    // path and the waits below can be exact
    load(nn, step + PF < nsteps ? step + PF : nsteps - 1);
    constexpr bool kTwo = SPLIT || BITS == 8;  // a scale per 32-channel half
    half2v zz[2][2], s2[2][2];
#pragma unroll
    for (int i = 0; i < (kTwo ? 2 : 1); ++i) {
      const int hi = SPLIT ? i : g64 ? kh : (int)(step & 1);  // zero nibble (4-bit)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint32_t z = BITS == 8 ? (cur.zb[b] >> (8 * i)) & 0xFF
                           : hi      ? (cur.zb[b] >> 4)
                                     : (cur.zb[b] & 0xF);
        const uint32_t zbits = 0x6400u + z;
        zz[b][i] = -__builtin_bit_cast(half2v, zbits | (zbits << 16));
        s2[b][i] = __builtin_bit_cast(half2v, cur.sc[b][i] | (cur.sc[b][i] << 16));
      }
    }
    // lane half kh covers channels [64 kh, 64 kh + 64) of the step; k16 step s covers 8 of
    // them. Operands of step s + 1 (A from LDS, B dequantized) are produced while the
    // MFMAs of step s run.
    auto load_frags = [&](int s, half8 (&A)[4], half8 (&B)[2]) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        A[a] = __builtin_bit_cast(
            half8, *reinterpret_cast<const uint4*>(&As[buf][(a * 32 + m32) * kAStride + kh * 64 + s * 8]));
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int i = kTwo ? (s >> 2) : 0;
        if constexpr (BITS == 8) {
          // slice s: words 2 s, 2 s + 1 of the lane half's 16
          const uint4 q = cur.b[b][s >> 1];
          B[b] = (s & 1) ? dequant_word8(q.z, q.w, zz[b][i], s2[b][i], magic8)
                         : dequant_word8(q.x, q.y, zz[b][i], s2[b][i], magic8);
        } else if constexpr (BITS == 3) {
          // slice s = channels 8 s .. 8 s + 7 of the half: pairs 4 s .. 4 s + 3, i.e. low
          // word s / 2 (fields 4 (s % 2) ..) and high word s / 4 (bits 4 (s % 4) ..)
          const uint4 q = cur.b[b][0];
          const uint32_t lo = (s >> 1) == 0 ? q.x : (s >> 1) == 1 ? q.y : (s >> 1) == 2 ? q.z : q.w;
          const uint32_t hi = (s >> 2) ? cur.bh[b].y : cur.bh[b].x;
          B[b] = (s & 1) ? ((s & 2) ? dequant_word3<4, 12>(lo, hi, zz[b][i], s2[b][i], magic)
                                    : dequant_word3<4, 4>(lo, hi, zz[b][i], s2[b][i], magic))
                         : ((s & 2) ? dequant_word3<0, 8>(lo, hi, zz[b][i], s2[b][i], magic)
                                    : dequant_word3<0, 0>(lo, hi, zz[b][i], s2[b][i], magic));
        } else {
          const uint4 q = cur.b[b][s >> 2];
          const uint32_t w = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
          B[b] = dequant_word(w, zz[b][i], s2[b][i], magic);
        }
      }
    };
    half8 A0[4], B0[2], A1[4], B1[2];
    load_frags(0, A0, B0);
#pragma unroll
    for (int s = 0; s < kBK / 16; s += 2) {
      load_frags(s + 1, A1, B1);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0[a], B0[b], acc[a][b], 0, 0, 0);
      if (s + 2 < kBK / 16) load_frags(s + 2, A0, B0);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1[a], B1[b], acc[a][b], 0, 0, 0);
      // issue pattern for the 16 MFMAs above: each MFMA followed by a share of the next
      // step's LDS reads and dequant VALU work, so the matrix pipe never waits for them
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);  // 1 LDS read
        __builtin_amdgcn_sched_group_barrier(0x0002, 4, 0);  // 4 VALU
      }
    }
    if (step + 1 < nsteps) store_a(nxt, buf ^ 1);
    __syncthreads();
  };

  int64_t step = 0;
  for (; step + 3 <= nsteps; step += 3) {  // straight-line triples: one path through the loop
    body(S0, S1, S2, step);
    body(S1, S2, S0, step + 1);
    body(S2, S0, S1, step + 2);
  }
  if (step < nsteps) body(S0, S1, S2, step);
  if (step + 1 < nsteps) body(S1, S2, S0, step + 1);

  // ------------------------------------------------------------------ epilogue
  // 32x32 accumulator layout: element e of lane l is (row 8(e/4) + 4(l/32) + e%4, col l%32).
  // Tiles wholly inside the output store without per-element bounds checks: a lane's rows
  // are then uniform offsets from its own column pointer.
  const int64_t ldy = GATED ? nh : N;
  const bool full = m0 + kBM <= M && n0 + (GATED ? kBN / 2 : kBN) <= ldy;
  if (full) {
    uint16_t* yl = Y + (m0 + 4 * kh) * ldy + n0 + wave * (GATED ? 32 : 64) + m32;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t ro = (int64_t)(a * 32 + 8 * (e >> 2) + (e & 3)) * ldy;
        if constexpr (GATED) {
          yl[ro] = f2h_bits(silu_f32(acc[a][0][e]) * acc[a][1][e]);
        } else {
#pragma unroll
          for (int b = 0; b < 2; ++b) yl[ro + b * 32] = f2h_bits(acc[a][b][e]);
        }
      }
  } else if constexpr (GATED) {
    const int64_t col = n0 + wave * 32 + m32;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + a * 32 + 8 * (e >> 2) + 4 * kh + (e & 3);
        if (row < M && col < nh) Y[row * nh + col] = f2h_bits(silu_f32(acc[a][0][e]) * acc[a][1][e]);
      }
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int64_t col = n0 + wave * 64 + b * 32 + m32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t row = m0 + a * 32 + 8 * (e >> 2) + 4 * kh + (e & 3);
          if (row < M && col < N) Y[row * N + col] = f2h_bits(acc[a][b][e]);
        }
      }
  }
}

}  // namespace awq
