// MFMA dequant-GEMM with 256-row tiles and one wave per SIMD (a8; 4- and 3-bit codes, and
// 8-bit codes without the gated epilogue; 128-, 64- or 32-channel groups): Y[M][N] =
// X[M][K] deq(W)^T for batches of 128 rows and more.
//
// "AWQ量化技术Skill", "主要功能和特点": a GEMM kernel serves batch sizes above one;
// "AWQ量化实战" §2.3 / §3.4: weights stay 4-bit in memory and are dequantized on the fly.
//
// Block = 4 waves (one per SIMD), tile 256 (tokens) x WN (output channels, 256 or 128), K
// step 128 (one group of 128; two of 64: a lane half's 64 channels are then one group; four
// of 32: a lane half's words 0-3 one group, 4-7 the next).
// Wave w owns all 256 rows and columns [WN / 4 w, +WN / 4) of the tile: 8 x (WN / 128)
// accumulators of v_mfma_f32_32x32x16_f16 (256 or 128 registers, which the compiler keeps
// in AGPRs), so every B column is widened by exactly one wave. The launcher takes WN = 128
// when that fills more of the chip's 256 CUs (whole waves of tiles counted), else 256, whose
// tiles do twice the MFMA work per A fragment read and per barrier.
//   - Both operands travel global -> LDS by 16-byte LDS DMA (global_load_lds_dwordx4) into
//     the other of two buffers for the next step; every buffer is its own LDS object, so the
//     compiler waits only for the DMA of the buffer a step reads. A wave's transfers of a
//     step (16 of A, WN / 64 of B) are issued in four groups, one at the head of each pair
//     of k16 slices (all at the top of the step, the same kernel ran 7-10% slower: the wave
//     waited at its own transfers instead of feeding the matrix core).
//   - A (activations, 256 rows x 16 chunks of 16 bytes per step) is stored with chunk c of
//     row r in slot c ^ (r & 15), so the 32 rows a fragment read touches fall in distinct
//     banks; B (codes, WN columns x 64 bytes) quarter-major, so a lane's 16-byte read of 4
//     words for its column is conflict-free.
//   - Each wave widens its own B words from LDS to (q - z) sc in fp16: the packed layout puts
//     channels 2p, 2p + 1 in nibbles p and p + 4, so a mask and an exponent give a channel
//     pair as 1024 + q (nibbles at bits 0 / 16 under 0x6400) or 64 + q (nibbles at bits 4 /
//     20 under 0x5400, where one unit is 2^-4), one shift per word serving pairs 2 and 3;
//     a packed subtract of the same bias plus z gives q - z exactly and a packed multiply by
//     the scale rounds once. The 128-row GEMM computes the same fp16 values and the same
//     MFMA sequence per output (lane half kh covers channels [64 kh, 64 kh + 64) of a step,
//     k16 slice s covers 8 of them), so both GEMMs give bit-identical results.
// Tiles go to the XCDs in contiguous runs, ordered four row tiles at a time with the column
// index moving slowest, so the blocks of one XCD share A panels and B columns in its L2.
//
// Fused gate|up (GATED, WN = 256 only): a block covers 128 outputs; a wave's first 32-column
// MFMA tile is gate column n, its second the up column n + N/2, and the epilogue stores
// SiLU(g) * u.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace awq {

namespace {

typedef _Float16 half8w __attribute__((ext_vector_type(8)));
typedef _Float16 half2w __attribute__((ext_vector_type(2)));
typedef float f32x16w __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWM = 256, kWK = 128;
constexpr int kRT = 8;            // a wave's 32 x 32 MFMA tiles along rows
constexpr int64_t kGroupRows = 4;  // row tiles per group of the tile order

__device__ __forceinline__ uint32_t wide_magic() {
  uint32_t m;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
  return m;
}

// One packed word -> its 8 dequantized fp16 channels (q - z) sc, in channel order. zz holds
// -(1024 + z) and zz64 -(64 + z) in both halves, s2 the scale in both halves.
__device__ __forceinline__ half8w widen_word(uint32_t w, half2w zz, half2w zz64, half2w s2,
                                             uint32_t magic) {
  const uint32_t w8 = w >> 8;
  const uint32_t u0 = (w & 0x000F000Fu) | magic, u1 = (w & 0x00F000F0u) | 0x54005400u;
  const uint32_t u2 = (w8 & 0x000F000Fu) | magic, u3 = (w8 & 0x00F000F0u) | 0x54005400u;
  const half2w d0 = (__builtin_bit_cast(half2w, u0) + zz) * s2;
  const half2w d1 = (__builtin_bit_cast(half2w, u1) + zz64) * s2;
  const half2w d2 = (__builtin_bit_cast(half2w, u2) + zz) * s2;
  const half2w d3 = (__builtin_bit_cast(half2w, u3) + zz64) * s2;
  return half8w{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
}

// Two packed 8-bit words -> their 8 channels (q - z) sc, in channel order: v_perm_b32 against
// 0x64646464 puts byte pairs under the 0x64 exponent byte, (1024 + a, 1024 + b) exactly; zz holds
// -(1024 + z) in both halves.
__device__ __forceinline__ half8w widen_word8(uint32_t w0, uint32_t w1, half2w zz, half2w s2,
                                              uint32_t magic8) {
  const half2w d0 = (__builtin_bit_cast(half2w, __builtin_amdgcn_perm(magic8, w0, 0x04010400u)) + zz) * s2;
  const half2w d1 = (__builtin_bit_cast(half2w, __builtin_amdgcn_perm(magic8, w0, 0x04030402u)) + zz) * s2;
  const half2w d2 = (__builtin_bit_cast(half2w, __builtin_amdgcn_perm(magic8, w1, 0x04010400u)) + zz) * s2;
  const half2w d3 = (__builtin_bit_cast(half2w, __builtin_amdgcn_perm(magic8, w1, 0x04030402u)) + zz) * s2;
  return half8w{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
}

// Four channel pairs of 3-bit codes -> 8 channels (q - z) sc: pair t takes its low bits from
// field f + t of the low-plane word and bit 2 from bit p + t of the high-plane word (both in
// each 16-bit half), under the 0x6400 exponent: exactly (1024 + q, 1024 + q').
__device__ __forceinline__ half8w widen_word3(uint32_t lo, uint32_t hi, int f, int p, half2w zz,
                                              half2w s2, uint32_t magic) {
  half2w d[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    d[t] = (__builtin_bit_cast(half2w, widen3_pair(lo, hi, f + t, p + t, magic)) + zz) * s2;
  return half8w{d[0][0], d[0][1], d[1][0], d[1][1], d[2][0], d[2][1], d[3][0], d[3][1]};
}

template <bool GATED, int WN, int BITS, bool G32>
__global__ void __launch_bounds__(256)
    k_gemm_wide(const uint16_t* X, int64_t M, const uint32_t* qweight, const uint16_t* scales,
                const uint8_t* zeros, int64_t N, int64_t K, int group, uint16_t* __restrict__ Y,
                int64_t mt, int64_t nt, int64_t per_xcd) {
  __shared__ __attribute__((aligned(16))) uint4 a0s[kWM * 16];
  __shared__ __attribute__((aligned(16))) uint4 a1s[kWM * 16];
  static_assert((BITS == 4 && (WN == 256 || (WN == 128 && !GATED))) ||
                    (BITS == 8 && WN == 128 && !GATED) || (BITS == 3 && WN == 256),
                "tile widths: 8-bit codes fill LDS at 128 columns; 3-bit codes take 256");
  constexpr int kCT = WN / 128;         // a wave's 32 x 32 MFMA tiles along columns
  constexpr int kQ = BITS;              // 16-byte quarters of a column's 16 BITS code bytes per step
  constexpr int kBT = WN * kQ / 256;    // B transfers per wave and step
  __shared__ __attribute__((aligned(16))) uint4 b0s[WN * kQ];
  __shared__ __attribute__((aligned(16))) uint4 b1s[WN * kQ];
  // tile t: XCD blockIdx % 8 takes tiles [per_xcd (blockIdx % 8), +per_xcd); within a group
  // of kGroupRows row tiles the row index moves fastest
  const int64_t t = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (t >= mt * nt) return;
  const int64_t grp = t / (kGroupRows * nt), first_m = grp * kGroupRows;
  const int64_t gsz = mt - first_m < kGroupRows ? mt - first_m : kGroupRows;
  const int64_t within = t - grp * kGroupRows * nt;
  const int64_t m0 = (first_m + within % gsz) * kWM;
  const int64_t n0 = (within / gsz) * (GATED ? WN / 2 : WN);
  const int64_t nh = N / 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m32 = lane & 31, kh = lane >> 5;
  const int g64 = group == 64;
  // zeros: 4-bit, two nibbles per byte; 8-bit, one byte per group
  const int64_t Gs = K / group, zbw = BITS == 8 ? Gs : (Gs + 1) / 2, words = K * BITS / 32;
  const int64_t nsteps = K / kWK;
  const uint32_t magic = wide_magic();
  uint32_t magic8 = 0;
  if constexpr (BITS == 8) asm volatile("v_mov_b32 %0, 0x64646464" : "=v"(magic8));

  // A DMA map: wave transfer i (0..15) fills slots (wave * 16 + i) * 64 + lane of the buffer:
  // row r = (wave * 16 + i) * 4 + lane / 16, slot lane % 16 <- chunk (lane % 16) ^ (r % 16).
  // Rows past M read row M - 1 (their outputs are never stored). Offsets fit 32 bits: the
  // launcher takes this kernel only for 256 K < 2^32.
  const uint16_t* xblk = X + m0 * K;
  uint32_t aoff[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = (wave * 16 + i) * 4 + (lane >> 4);
    const int64_t gr = m0 + r < M ? r : M - 1 - m0;
    aoff[i] = (uint32_t)(gr * K + ((lane & 15) ^ (r & 15)) * 8);
  }
  // B DMA map, quarter-major: slot (wave * kBT + i) * 64 + lane = 16-byte quarter q (slot /
  // WN) of tile column c (slot % WN) of the columns' 16 kQ code bytes of a step, so a wave's
  // read of one quarter of 32 consecutive columns is 512 contiguous bytes (no bank
  // conflicts). Gated: tile columns [64 w, 64 w + 32) hold the gate rows and [64 w + 32,
  // 64 w + 64) the up rows of outputs n0 + 32 w .. n0 + 32 w + 31. Columns past the end
  // read the last one (never stored).
  const uint32_t* bptr[kBT];
#pragma unroll
  for (int i = 0; i < kBT; ++i) {
    const int slot = (wave * kBT + i) * 64 + lane;
    const int c = slot % WN, q = slot / WN;
    int64_t n;
    if constexpr (GATED) {
      int64_t o = n0 + (c >> 6) * 32 + (c & 31);
      o = o < nh ? o : nh - 1;
      n = (c & 63) >= 32 ? o + nh : o;
    } else {
      n = n0 + c < N ? n0 + c : N - 1;
    }
    bptr[i] = qweight + n * words + q * 4;
  }
  // this lane's weight rows (gated: gate row n and up row n + N/2): scales and zeros
  int64_t bcol[kCT];
  if constexpr (GATED) {
    const int64_t o = n0 + wave * 32 + m32;
    bcol[0] = o < nh ? o : nh - 1;
    bcol[1] = bcol[0] + nh;
  } else {
#pragma unroll
    for (int b = 0; b < kCT; ++b) {
      const int64_t n = n0 + wave * kCT * 32 + b * 32 + m32;
      bcol[b] = n < N ? n : N - 1;
    }
  }
  // per column, the zero(s) and scale(s) of the lane half's 64 channels of a step: one group
  // (128 channels: step; 64: 2 step + kh), or with 32-channel groups two (4 step + 2 kh for
  // words 0-3 of the half, the next for words 4-7)
  constexpr int kZ = G32 ? 2 : 1;
  struct ScaleZero {
    uint32_t zb[kCT], sc[kCT][kZ];
  };
  auto load_sz = [&](ScaleZero& st, int64_t step) {
#pragma unroll
    for (int b = 0; b < kCT; ++b) {
      if constexpr (G32) {
        const int64_t g0 = 4 * step + 2 * kh;
        if constexpr (BITS == 8)
          st.zb[b] = (uint32_t)zeros[bcol[b] * zbw + g0] | ((uint32_t)zeros[bcol[b] * zbw + g0 + 1] << 8);
        else
          st.zb[b] = zeros[bcol[b] * zbw + 2 * step + kh];  // nibbles: groups g0, g0 + 1
        st.sc[b][0] = scales[bcol[b] * Gs + g0];
        st.sc[b][1] = scales[bcol[b] * Gs + g0 + 1];
      } else {
        st.zb[b] = zeros[bcol[b] * zbw + (BITS == 8 ? (step << g64) + (g64 & kh) : step >> (1 - g64))];
        st.sc[b][0] = scales[bcol[b] * Gs + (step << g64) + (g64 & kh)];
      }
    }
  };

  f32x16w acc[kRT][kCT];
#pragma unroll
  for (int a = 0; a < kRT; ++a)
#pragma unroll
    for (int b = 0; b < kCT; ++b) acc[a][b] = f32x16w{};

  ScaleZero s0, s1;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(xblk + aoff[i]),
                                     (lds_void*)&a0s[(wave * 16 + i) * 64], 16, 0, 0);
#pragma unroll
  for (int i = 0; i < kBT; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(bptr[i]), (lds_void*)&b0s[(wave * kBT + i) * 64],
                                     16, 0, 0);
  load_sz(s0, 0);
  __syncthreads();

  // One K step on buffer BUF (a compile-time constant, so each LDS access names one object).
  auto body = [&](auto bufc, ScaleZero& cur, ScaleZero& nxt, int64_t step) {
    constexpr int BUF = decltype(bufc)::value;
    const uint4* ab = BUF ? a1s : a0s;
    const uint4* bb = BUF ? b1s : b0s;
    // the next step's operands (clamped: the last step reloads itself into the idle buffer)
    const int64_t sn = step + 1 < nsteps ? step + 1 : nsteps - 1;
    load_sz(nxt, sn);
    __builtin_amdgcn_sched_barrier(0);  // keep the scale loads at the top of the step
    uint4* const adn = BUF ? a0s : a1s;
    uint4* const bdn = BUF ? b0s : b1s;
    auto dma_a = [&](int i) {
      __builtin_amdgcn_global_load_lds((const void*)(xblk + sn * kWK + aoff[i]),
                                       (lds_void*)&adn[(wave * 16 + i) * 64], 16, 0, 0);
    };
    auto dma_b = [&](int i) {
      __builtin_amdgcn_global_load_lds((const void*)(bptr[i] + sn * (kQ * 4)),
                                       (lds_void*)&bdn[(wave * kBT + i) * 64], 16, 0, 0);
    };
    half2w zz[kCT][kZ], zz64[kCT][kZ], s2[kCT][kZ];
    const int hi = g64 ? kh : (int)(step & 1);  // zero nibble: group of 128 (step) or 64 (2 step + kh)
#pragma unroll
    for (int b = 0; b < kCT; ++b)
#pragma unroll
      for (int i = 0; i < kZ; ++i) {
        uint32_t z;
        if constexpr (G32)
          z = BITS == 8 ? (cur.zb[b] >> (8 * i)) & 0xFF : (cur.zb[b] >> (4 * i)) & 0xF;
        else
          z = BITS == 8 ? cur.zb[b] : hi ? (cur.zb[b] >> 4) : (cur.zb[b] & 0xF);
        const uint32_t z1024 = 0x6400u + z, z64 = 0x5400u + (z << 4);
        zz[b][i] = -__builtin_bit_cast(half2w, z1024 | (z1024 << 16));
        zz64[b][i] = -__builtin_bit_cast(half2w, z64 | (z64 << 16));
        s2[b][i] = __builtin_bit_cast(half2w, cur.sc[b][i] | (cur.sc[b][i] << 16));
      }
    // this lane's code words of the step, per column: 4- and 8-bit, words 2 kQ kh .., the
    // quarters kQ / 2 kh .. kQ / 2 kh + kQ / 2 - 1 (one 16-byte read each); 3-bit, low-plane
    // words 4 kh .. 4 kh + 3 (quarter kh) and high-plane words 8 + 2 kh, 9 + 2 kh (half of
    // quarter 2)
    constexpr int kQL = BITS == 3 ? 1 : kQ / 2;
    uint4 bq[kCT][kQL];
    uint2 bh[kCT];
#pragma unroll
    for (int b = 0; b < kCT; ++b) {
      const int col = wave * kCT * 32 + b * 32 + m32;
      if constexpr (BITS == 3) {
        bq[b][0] = bb[kh * WN + col];
        const uint4 h4 = bb[2 * WN + col];
        bh[b] = kh ? make_uint2(h4.z, h4.w) : make_uint2(h4.x, h4.y);
      } else {
#pragma unroll
        for (int h = 0; h < kQL; ++h) bq[b][h] = bb[(kQL * kh + h) * WN + col];
      }
    }
    auto frags = [&](int s, half8w (&A)[kRT], half8w (&B)[kCT]) {
      const int c = kh * 8 + s;
      const int zi = G32 ? (s >> 2) : 0;  // slices 0-3 lie in the half's first 32 channels
#pragma unroll
      for (int a = 0; a < kRT; ++a) {
        const int r = a * 32 + m32;
        A[a] = __builtin_bit_cast(half8w, ab[r * 16 + (c ^ (r & 15))]);
      }
#pragma unroll
      for (int b = 0; b < kCT; ++b) {
        if constexpr (BITS == 8) {
          // slice s: words 2 s, 2 s + 1 of the lane half's 16
          const uint4 q = bq[b][s >> 1];
          B[b] = (s & 1) ? widen_word8(q.z, q.w, zz[b][zi], s2[b][zi], magic8)
                         : widen_word8(q.x, q.y, zz[b][zi], s2[b][zi], magic8);
        } else if constexpr (BITS == 3) {
          // slice s = channel pairs 4 s .. 4 s + 3 of the half: low word s / 2 (fields
          // 4 (s % 2) ..), high word s / 4 (bits 4 (s % 4) ..)
          const uint4 q = bq[b][0];
          const uint32_t lo = (s >> 1) == 0 ? q.x : (s >> 1) == 1 ? q.y : (s >> 1) == 2 ? q.z : q.w;
          const uint32_t hiw = (s >> 2) ? bh[b].y : bh[b].x;
          B[b] = widen_word3(lo, hiw, 4 * (s & 1), 4 * (s & 3), zz[b][zi], s2[b][zi], magic);
        } else {
          const uint4 q = bq[b][s >> 2];
          const uint32_t w = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
          B[b] = widen_word(w, zz[b][zi], zz64[b][zi], s2[b][zi], magic);
        }
      }
    };
    half8w A0[kRT], B0[kCT], A1[kRT], B1[kCT];
    frags(0, A0, B0);
#pragma unroll
    for (int s = 0; s < kWK / 16; s += 2) {
      {  // a quarter of the next step's A transfers (4 s / 2 .. + 3) and B transfer s / 2
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma_a(2 * s + i);
        if ((s >> 1) < kBT) dma_b(s >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      frags(s + 1, A1, B1);
#pragma unroll
      for (int a = 0; a < kRT; ++a)
#pragma unroll
        for (int b = 0; b < kCT; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0[a], B0[b], acc[a][b], 0, 0, 0);
      if (s + 2 < kWK / 16) frags(s + 2, A0, B0);
#pragma unroll
      for (int a = 0; a < kRT; ++a)
#pragma unroll
        for (int b = 0; b < kCT; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1[a], B1[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();  // the next step's DMA has landed; this step's buffer is free
  };
  int64_t step = 0;
  for (; step + 2 <= nsteps; step += 2) {
    body(std::integral_constant<int, 0>{}, s0, s1, step);
    body(std::integral_constant<int, 1>{}, s1, s0, step + 1);
  }
  if (step < nsteps) body(std::integral_constant<int, 0>{}, s0, s1, step);

  // 32x32 accumulator layout: element e of lane l is (row 8(e/4) + 4(l/32) + e%4, col l%32).
  // Tiles wholly inside the output store without per-element bounds checks: a lane's rows
  // are then uniform offsets from its own column pointer.
  const int64_t ldy = GATED ? nh : N;
  const bool full = m0 + kWM <= M && n0 + (GATED ? WN / 2 : WN) <= ldy;
  if (full) {
    uint16_t* yl = Y + (m0 + 4 * kh) * ldy + n0 + wave * (GATED ? 32 : kCT * 32) + m32;
#pragma unroll
    for (int a = 0; a < kRT; ++a)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t ro = (int64_t)(a * 32 + 8 * (e >> 2) + (e & 3)) * ldy;
        if constexpr (GATED) {
          yl[ro] = f2h_bits(silu_f32(acc[a][0][e]) * acc[a][1][e]);
        } else {
#pragma unroll
          for (int b = 0; b < kCT; ++b) yl[ro + b * 32] = f2h_bits(acc[a][b][e]);
        }
      }
  } else if constexpr (GATED) {
    const int64_t col = n0 + wave * 32 + m32;
#pragma unroll
    for (int a = 0; a < kRT; ++a)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + a * 32 + 8 * (e >> 2) + 4 * kh + (e & 3);
        if (row < M && col < nh) Y[row * nh + col] = f2h_bits(silu_f32(acc[a][0][e]) * acc[a][1][e]);
      }
  } else {
#pragma unroll
    for (int a = 0; a < kRT; ++a)
#pragma unroll
      for (int b = 0; b < kCT; ++b) {
        const int64_t col = n0 + wave * kCT * 32 + b * 32 + m32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t row = m0 + a * 32 + 8 * (e >> 2) + 4 * kh + (e & 3);
          if (row < M && col < N) Y[row * N + col] = f2h_bits(acc[a][b][e]);
        }
      }
  }
}

}  // namespace

// Tile width for an M x N output: 128 columns when whole waves of those tiles keep more of
// the 256 CUs busy than 256-column tiles do (ties go to 256); gated outputs and 3-bit codes
// always 256, 8-bit codes always 128 (256 columns of them would not fit LDS with the A tile).
int gemm_wide_cols(int64_t M, int64_t N, bool gated, int w_bit) {
  if (gated || w_bit == 3) return 256;
  if (w_bit == 8) return 128;
  const int64_t mt = (M + kWM - 1) / kWM;
  const int64_t t256 = mt * ((N + 255) / 256), t128 = mt * ((N + 127) / 128);
  const int64_t w256 = (t256 + 255) / 256, w128 = (t128 + 255) / 256;  // waves of tiles
  // fill fraction t / (256 w): compare t128 / w128 against t256 / w256
  return t128 * w256 > t256 * w128 ? 128 : 256;
}

int64_t gemm_wide_tiles(int64_t M, int64_t N, bool gated, int w_bit) {
  const int64_t mt = (M + kWM - 1) / kWM;
  const int cols = gemm_wide_cols(M, N, gated, w_bit);
  const int64_t nt = gated ? (N / 2 + cols / 2 - 1) / (cols / 2) : (N + cols - 1) / cols;
  return mt * nt;
}

bool gemm_wide_supported(int64_t K, int group, int w_bit, bool gated) {
  return (w_bit == 4 || w_bit == 3 || (w_bit == 8 && !gated)) &&
         (group == 128 || group == 64 || group == 32) && (int64_t)kWM * K < ((int64_t)1 << 32);
}

namespace {

template <bool GATED, int WN, int BITS>
void launch_wide_t(dim3 grid, hipStream_t stream, const uint16_t* X, int64_t M, const uint32_t* qw,
                   const uint16_t* sc, const uint8_t* z, int64_t N, int64_t K, int group,
                   uint16_t* Y, int64_t mt, int64_t nt, int64_t per_xcd) {
  if (group == 32)
    hipLaunchKernelGGL((k_gemm_wide<GATED, WN, BITS, true>), grid, dim3(256), 0, stream, X, M, qw,
                       sc, z, N, K, group, Y, mt, nt, per_xcd);
  else
    hipLaunchKernelGGL((k_gemm_wide<GATED, WN, BITS, false>), grid, dim3(256), 0, stream, X, M, qw,
                       sc, z, N, K, group, Y, mt, nt, per_xcd);
}

}  // namespace

hipError_t launch_gemm_wide(const uint16_t* X, int64_t M, const uint32_t* qweight,
                            const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                            int group, int w_bit, uint16_t* Y, bool gated, hipStream_t stream) {
  if (!gemm_wide_supported(K, group, w_bit, gated)) return hipErrorInvalidValue;
  const int cols = gemm_wide_cols(M, N, gated, w_bit);
  const int64_t mt = (M + kWM - 1) / kWM;
  const int64_t nt = gated ? (N / 2 + cols / 2 - 1) / (cols / 2) : (N + cols - 1) / cols;
  const int64_t per_xcd = (mt * nt + 7) / 8;
  const dim3 grid((unsigned)(per_xcd * 8));
  if (w_bit == 8)
    launch_wide_t<false, 128, 8>(grid, stream, X, M, qweight, scales, zeros, N, K, group, Y, mt, nt, per_xcd);
  else if (w_bit == 3 && gated)
    launch_wide_t<true, 256, 3>(grid, stream, X, M, qweight, scales, zeros, N, K, group, Y, mt, nt, per_xcd);
  else if (w_bit == 3)
    launch_wide_t<false, 256, 3>(grid, stream, X, M, qweight, scales, zeros, N, K, group, Y, mt, nt, per_xcd);
  else if (gated)
    launch_wide_t<true, 256, 4>(grid, stream, X, M, qweight, scales, zeros, N, K, group, Y, mt, nt, per_xcd);
  else if (cols == 256)
    launch_wide_t<false, 256, 4>(grid, stream, X, M, qweight, scales, zeros, N, K, group, Y, mt, nt, per_xcd);
  else
    launch_wide_t<false, 128, 4>(grid, stream, X, M, qweight, scales, zeros, N, K, group, Y, mt, nt, per_xcd);
  return hipGetLastError();
}

}  // namespace awq
