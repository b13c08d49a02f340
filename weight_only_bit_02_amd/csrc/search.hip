// Activation-aware grid search (a5 + a6).
//
// "AWQ量化实战" §2.2 and §3.3 step 4: for every grid point, quantize W diag(s) and score
// how far the layer's calibration outputs move; "什么是激活感知权重量化（AWQ）", "工作机制":
// the scale is an equivalent transform W diag(s), X diag(1/s), found without
// backpropagation. For grid point i the score is
//   err_i = sum_t sum_n ( sum_k X_tk D_nk )^2,   D = W - Q(W diag(s_i)) diag(1/s_i).
//
// One block owns (grid point i, 64 rows of W, up to 64 * NW tokens) and walks K one
// quantization group at a time:
//   1. quantize: 16 lanes per (row, group), 8 weights each; the same group quantizer
//      as the pack kernel gives the codes; D is formed in fp32, scaled by a power of
//      two P chosen per (row, group) from a bound on |D| so that |D P| < 2^14, and
//      split into two fp16 halves hi + lo (22 significant bits). hi and lo go to LDS.
//   2. contract: each wave multiplies its 64 tokens of X (fp16, straight from global)
//      by the hi and lo tiles with v_mfma_f32_32x32x16_f16 into a per-group
//      accumulator, then folds it into the running E tile with the factor 1/P of its
//      column.
// After the last group the block squares and sums its E tile (fp64) and writes one
// partial; a second kernel adds the partials of each grid point in a fixed order and
// takes the first minimum. No floating-point atomics: results are bitwise
// reproducible.
//
// Weight clipping (f3; the nxmr.cn article "AWQ技术概述：重新定义大语言模型量化", §5.1
// "精度下降严重", names clip_steps, 200 suggested): with s fixed, every
// group tries the shrink ratios r_i = (steps - i) / steps of its range, scored by its own
// output contribution err[i][n][g] = sum_t (sum_{k in g} X_tk D_nk)^2. A block owns
// (ratio i, 128 rows, all T <= 512 tokens); the same tile quantizer (extremes times r)
// feeds the same MFMA contraction, but each group's accumulator starts from zero and is
// squared on its own, and the waves' per-row partials meet in LDS every group.
#include "common.hpp"
#include "launch.hpp"

namespace awq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRowTile = 128;        // rows of W per block
constexpr int kTokPerWave = 64;      // tokens per wave (2 MFMA row tiles)
constexpr int kLdsStride = 128 + 8;  // halves per LDS row (16-byte pad against bank conflicts)
constexpr int kXcds = 8;

// Per-row power-of-two scale of D. For every channel k of row n,
//   |D_nk| = |w'_nk - deq_nk| / s_k <= (max|w'| + 15 sc_h) / s_k
//          <= 3.01 * max_k |W_nk| * (max_k s_k / min_k s_k),
// so P_n = 2^(14 - e) with that bound in [2^(e-1), 2^e) keeps |D P| < 2^14 and the fp16
// hi part finite; hi + lo then carries 22 significant bits of D P.
__device__ __forceinline__ float row_scale(float rowmax, float srange) {
  const float bound = 3.01f * rowmax * srange;
  int ex = 0;
  (void)__builtin_frexpf(bound, &ex);
  if (!(bound > 0.0f) || !__builtin_isfinite(bound)) ex = 0;
  ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
  return __builtin_ldexpf(1.0f, 14 - ex);
}

// max |W| per row (fp16 magnitudes compared as integers: order-free, exact).
__global__ void __launch_bounds__(256) k_row_absmax(const uint16_t* __restrict__ W, int64_t N,
                                                    int64_t K, float* __restrict__ rowmax) {
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (row >= N) return;
  uint32_t m = 0;
  for (int64_t c = lane; c < K / 8; c += 64) {
    const uint4 v = *reinterpret_cast<const uint4*>(W + row * K + c * 8);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = max(m, d[i] & 0x7FFFu);
      m = max(m, (d[i] >> 16) & 0x7FFFu);
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if (lane == 0) rowmax[row] = m >= 0x7C00u ? __builtin_inff() : h2f((uint16_t)m);
}

// max s / min s of every grid point (one block per grid point; min/max are order-free).
__global__ void __launch_bounds__(256) k_scale_range(const uint16_t* __restrict__ s_grid, int64_t K,
                                                     float* __restrict__ srange,
                                                     uint32_t* __restrict__ flags) {
  __shared__ float lmin[256], lmax[256];
  const uint16_t* s = s_grid + (int64_t)blockIdx.x * K;
  float mn = __builtin_inff(), mx = 0.0f;
  for (int64_t k = threadIdx.x; k < K; k += 256) {
    const float v = h2f(s[k]);
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  lmin[threadIdx.x] = mn;
  lmax[threadIdx.x] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < 256; ++i) {
      mn = fminf(mn, lmin[i]);
      mx = fmaxf(mx, lmax[i]);
    }
    const float r = mx / mn;
    srange[blockIdx.x] = r;
    // beyond 2^10 the per-row scale leaves fewer than 12 of the 22 bits for small terms
    if (!(r <= 1024.0f) && flags) atomicOr(flags, AWQ_FLAG_SEARCH_RANGE);
  }
}

// X in the order the MFMA A operand reads it. For 64-token tile t (tokens 64 t .. 64 t + 63,
// zeros past T), 128-channel step j, k16 slice st and token half a, lane l's 16 bytes are
// X[64 t + 32 a + l % 32][128 j + 16 st + 8 (l / 32) .. + 8], so one wave's load of a slice
// is 1 KiB contiguous (X as stored puts each lane 8 KiB apart, and the lines a step needs
// do not stay in the L1 between the slices that share them).
__global__ void __launch_bounds__(256)
    k_pack_x(const uint16_t* __restrict__ X, int64_t T, int64_t K, int64_t tiles,
             uint4* __restrict__ xp) {
  const int64_t G = K / kGroup;
  const int64_t total = tiles * G * 8 * 2 * 64;  // 16-byte entries
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63);
    int64_t r = i >> 6;
    const int a = (int)(r & 1);
    r >>= 1;
    const int st = (int)(r & 7);
    r >>= 3;
    const int64_t j = r % G, t = r / G;
    const int64_t tok = t * 64 + a * 32 + (lane & 31);
    const int64_t ch = j * kGroup + st * 16 + (lane >> 5) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (tok < T) v = *reinterpret_cast<const uint4*>(X + tok * K + ch);
    xp[i] = v;
  }
}

// Entry (tile, j, st, a) of the packed X: the wave's 64 consecutive 16-byte pieces.
__device__ __forceinline__ const uint4* packed_x(const uint4* xp, int64_t G, int64_t tile,
                                                 int64_t j, int st, int a) {
  return xp + (((tile * G + j) * 8 + st) * 2 + a) * 64;
}

// Quantizes 128-channel step j of rows [row_base, row_base + NROWS) of the 128-row tile
// starting at row n0 into LDS as (D P) split into fp16 hi + lo,
// D = W - Q(W diag(s)) diag(1/s) (s == nullptr: s = 1), with NW waves (tid counts their
// threads from 0). With CLIP the group's extremes are shrunk by r before the quantizer
// sees them (weight clipping). 16 lanes per (row, 128 channels), 8 weights each; returns
// whether a non-finite value was met.
template <int NW, bool CLIP, int NROWS>
__device__ __forceinline__ bool quantize_tile_group(const uint16_t* W, int64_t N, int64_t K,
                                                    const uint16_t* s, float r, bool sym,
                                                    int group, float qmax, int64_t n0, int64_t j,
                                                    const float* lds_p, uint16_t* hi_buf,
                                                    uint16_t* lo_buf, int tid, int row_base,
                                                    float* pg_out) {
  constexpr int kRowsPerPass = NW * 4;
  constexpr int kPasses = NROWS / kRowsPerPass;
  static_assert(kPasses * kRowsPerPass == NROWS, "whole passes");
  const int q_row = row_base + (tid >> 4);
  const int li = tid & 15;
  const int64_t k0 = j * kGroup + li * 8;
  // the thread's 8 channels are the same in every pass: s and 1/s once
  uint4 sv = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);  // s = 1
  if (!CLIP || s) sv = *reinterpret_cast<const uint4*>(s + k0);
  float sf[8], rs[8];
  {
    const uint32_t sd[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sf[2 * i] = h2f((uint16_t)(sd[i] & 0xFFFF));
      sf[2 * i + 1] = h2f((uint16_t)(sd[i] >> 16));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) rs[i] = __builtin_amdgcn_rcpf(sf[i]);
  }
  bool bad = false;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int row = p * kRowsPerPass + q_row;
    const int64_t n = n0 + row;
    const int64_t nc = n < N ? n : N - 1;
    uint4 wv = *reinterpret_cast<const uint4*>(W + nc * K + k0);
    if (n >= N) wv = make_uint4(0, 0, 0, 0);
    const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
    float wf[8], wp[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wf[2 * i] = h2f((uint16_t)(wd[i] & 0xFFFF));
      wf[2 * i + 1] = h2f((uint16_t)(wd[i] >> 16));
      wp[2 * i] = wf[2 * i] * sf[2 * i];
      wp[2 * i + 1] = wf[2 * i + 1] * sf[2 * i + 1];
    }
    float mn = wp[0], mx = wp[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      mn = fminf(mn, wp[i]);
      mx = fmaxf(mx, wp[i]);
    }
    group_minmax(mn, mx, group);  // 16 lanes = one 128-channel group, two of 64, four of 32
    bad |= !__builtin_isfinite(mn) || !__builtin_isfinite(mx);
    if (CLIP) {
      mn = r * mn;
      mx = r * mx;
    }
    const GroupQ g = sym ? group_params_sym(mn, mx, qmax) : group_params(mn, mx, qmax);
    float qc[8];
    quant_codes(wp, g, qc);
    // D = (w' - deq) / s: w' = w s and deq = (q - z) sc_h are exact, and so is their
    // difference (both are multiples of the finer ulp and close in magnitude), so the
    // reciprocal's error (1 ulp) is relative to D itself; w - deq / s would carry it
    // relative to w, which is 30 (4-bit) to 500 (8-bit) times larger than D
    float dg[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float deq = (qc[c] - g.z) * g.scf;  // exact: small integer times an fp16
      dg[c] = (wp[c] - deq) * rs[c];
    }
    float P;
    if constexpr (CLIP) {
      // each group is scored on its own, so its scale comes from its own largest |D|:
      // P = 2^(14 - e) with that maximum in [2^(e-1), 2^e), so |D P| < 2^14 and hi + lo
      // keep 22 significant bits of every group, whatever the code width
      float dmx = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) dmx = fmaxf(dmx, __builtin_fabsf(dg[c]));
      float dmn = dmx;
      group_minmax(dmn, dmx, group);
      int ex = 0;
      (void)__builtin_frexpf(dmx, &ex);
      if (!(dmx > 0.0f) || !__builtin_isfinite(dmx)) ex = 0;
      ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
      P = __builtin_ldexpf(1.0f, 14 - ex);
      const int gl = group >> 3;  // lanes per group
      if ((li & (gl - 1)) == 0) pg_out[row * 4 + li / gl] = P;
    } else {
      P = lds_p[row];
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t h2[2], l2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = 2 * i + e;
        const float d = dg[c] * P;
        h2[e] = f2h_bits(d);
        l2[e] = f2h_bits(d - h2f(h2[e]));
      }
      hi[i] = (uint32_t)h2[0] | ((uint32_t)h2[1] << 16);
      lo[i] = (uint32_t)l2[0] | ((uint32_t)l2[1] << 16);
    }
    *reinterpret_cast<uint4*>(&hi_buf[row * kLdsStride + li * 8]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(&lo_buf[row * kLdsStride + li * 8]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  return bad;
}

template <int NW>
__global__ void __launch_bounds__(NW * 64)
    k_search_err(const uint4* xp, int64_t T, const uint16_t* W, int64_t N, int64_t K,
                 const uint16_t* s_grid, int n_grid, int sym, int group, int w_bit,
                 const float* rowmax,
                 const float* srange,
                 double* __restrict__ partials, uint32_t* __restrict__ flags, int64_t n_ntiles,
                 int64_t per_xcd) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_hi[2][kRowTile * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t lds_lo[2][kRowTile * kLdsStride];
  __shared__ float lds_p[kRowTile];
  __shared__ double lds_red[NW];

  // XCD-aware order: consecutive blocks of one XCD share a row tile (different grid
  // points), so the tile of W is read from HBM once per XCD.
  const int64_t t = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (t >= n_ntiles * n_grid) return;
  const int64_t ntile = t / n_grid;
  const int alpha = (int)(t % n_grid);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t n0 = ntile * kRowTile;
  const float qmax = (float)((1 << w_bit) - 1);
  const int64_t G = K / kGroup;
  const uint16_t* s = s_grid + (int64_t)alpha * K;
  const int64_t tchunk = (int64_t)NW * kTokPerWave;
  const int64_t n_tchunks = (T + tchunk - 1) / tchunk;

  const int m32 = lane & 31;
  const int khalf = lane >> 5;

  const float sr = srange[alpha];
  for (int r = tid; r < kRowTile; r += NW * 64)
    lds_p[r] = row_scale(n0 + r < N ? rowmax[n0 + r] : 0.0f, sr);
  __syncthreads();

  // The waves form two sets of NW / 2 (one wave of each per SIMD), each quantizing half
  // of the tile's rows. Per step, set A multiplies the current group and then quantizes
  // its half of the next one, set B does the same in the opposite order, so on each SIMD
  // one wave keeps the matrix core busy while the other runs the vector quantizer. The
  // one barrier per step still orders both buffers: a step reads the buffer written in
  // the step before and writes the one read there.
  constexpr int NH = NW / 2;
  const bool set_b = wave >= NH;
  const int tid_set = set_b ? tid - NH * 64 : tid;
  bool bad = false;
  auto quantize = [&](int64_t j, int buf) {
    bad |= quantize_tile_group<NH, false, kRowTile / 2>(W, N, K, s, 1.0f, sym, group, qmax, n0, j, lds_p,
                                                       lds_hi[buf], lds_lo[buf], tid_set,
                                                       set_b ? kRowTile / 2 : 0, nullptr);
  };

  for (int64_t tc = 0; tc < n_tchunks; ++tc) {
    const int64_t tw = tc * tchunk + (int64_t)wave * kTokPerWave;
    const bool active = tw < T;
    f32x16 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

    const int64_t tile = tw / kTokPerWave;  // the wave's 64-token tile of the packed X
    auto multiply = [&](int64_t j, int buf) {
      if (!active) return;
#pragma unroll 2
      for (int st = 0; st < kGroup / 16; ++st) {
        const int koff = st * 16 + khalf * 8;
        half8 A[2], Bh[4], Bl[4];
#pragma unroll
        for (int a = 0; a < 2; ++a)
          A[a] = __builtin_bit_cast(half8, packed_x(xp, G, tile, j, st, a)[lane]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = b * 32 + m32;
          Bh[b] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&lds_hi[buf][r * kLdsStride + koff]));
          Bl[b] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&lds_lo[buf][r * kLdsStride + koff]));
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[a], Bh[b], acc[a][b], 0, 0, 0);
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[a], Bl[b], acc[a][b], 0, 0, 0);
          }
      }
    };

    quantize(0, 0);
    __syncthreads();
    for (int64_t j = 0; j < G; ++j) {
      const int buf = (int)(j & 1);
      // next group's quantization (unconditional, clamped: the last one is redundant and
      // lands in the buffer nobody reads)
      const int64_t jn = j + 1 < G ? j + 1 : G - 1;
      if (!set_b) {
        multiply(j, buf);
        quantize(jn, buf ^ 1);
      } else {
        quantize(jn, buf ^ 1);
        multiply(j, buf);
      }
      __syncthreads();
    }

    // ------------------------------------------------------------------ sum of squares
    double ss = 0.0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const double pinv = 1.0 / (double)lds_p[b * 32 + m32];  // output column = lane % 32
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const double v = (double)acc[a][b][e] * pinv;
          ss += v * v;
        }
    }
    ss = wave_sum(ss);
    if (lane == 0) lds_red[wave] = ss;
    __syncthreads();
    if (tid == 0) {
      double tot = 0.0;
      for (int w = 0; w < NW; ++w) tot += lds_red[w];
      partials[((int64_t)alpha * n_ntiles + ntile) * n_tchunks + tc] = tot;
    }
    __syncthreads();
  }
  if (bad && flags && alpha == 0) atomicOr(flags, AWQ_FLAG_NONFINITE_INPUT);
}

template <int NW>
__global__ void __launch_bounds__(NW * 64)
    k_clip_err(const uint4* xp, int64_t T, const uint16_t* W, int64_t N, int64_t K,
               const uint16_t* s, int clip_steps, int n_shrink, int sym, int group, int w_bit,
               double* __restrict__ err, float* __restrict__ part, uint32_t* __restrict__ flags,
               int64_t n_ntiles, int64_t per_xcd) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_hi[2][kRowTile * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t lds_lo[2][kRowTile * kLdsStride];
  // power-of-two scale of each (row, group of the step), double-buffered with hi / lo
  __shared__ float lds_pg[2][kRowTile * 4];
  // 128-channel groups: per-row partial errors of each wave, slot = step parity, summed
  // over the waves after the end-of-step barrier (the one barrier per step). Smaller groups
  // (two or four per step) would need 2 x 4 slots, more than the LDS left: each wave stores
  // its partials of those groups to `part` instead, with no barrier, and the reduction
  // kernel sums the waves.
  __shared__ double lds_red[2][NW][kRowTile];

  const int64_t t = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (t >= n_ntiles * n_shrink) return;
  const int64_t ntile = t / n_shrink;
  const int ci = (int)(t % n_shrink);
  const float r = clip_ratio(ci, clip_steps);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t n0 = ntile * kRowTile;
  const float qmax = (float)((1 << w_bit) - 1);
  const int gps = kGroup / group;  // groups per 128-channel step: 1, 2 or 4
  const int per = 8 / gps;         // k16 slices per group: 8, 4 or 2
  const int64_t G = K / kGroup;    // 128-channel steps
  const int64_t Gs = K / group;    // groups
  const int m32 = lane & 31;
  const int khalf = lane >> 5;
  const int64_t tw = (int64_t)wave * kTokPerWave;
  const bool active = tw < T;

  // two sets of waves in opposite phase, as in the scale search: set A multiplies then
  // quantizes its half of the next step's rows, set B the reverse. Every wave runs the
  // same barriers in the same order (the pair stores of small groups included), so the
  // sets only drift apart between barriers.
  constexpr int NH = NW / 2;
  const bool set_b = wave >= NH;
  const int tid_set = set_b ? tid - NH * 64 : tid;
  bool bad = false;
  auto quantize = [&](int64_t jq, int qbuf) {
    bad |= quantize_tile_group<NH, true, kRowTile / 2>(W, N, K, s, r, sym, group, qmax, n0, jq,
                                                      nullptr, lds_hi[qbuf], lds_lo[qbuf], tid_set,
                                                      set_b ? kRowTile / 2 : 0, lds_pg[qbuf]);
  };
  quantize(0, 0);
  __syncthreads();
  for (int64_t j = 0; j < G; ++j) {
    const int buf = (int)(j & 1);
    const int64_t jn = j + 1 < G ? j + 1 : G - 1;
    if (set_b) quantize(jn, buf ^ 1);
    f32x16 acc[2][4];
    // the step's 8 k16 slices in quarters of two; a group spans per = 8, 4 or 2 slices and
    // its error is taken when its last slice is done
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if ((2 * c) % per == 0) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};
      }
      if (active) {
#pragma unroll
        for (int st = 2 * c; st < 2 * c + 2; ++st) {
          const int koff = st * 16 + khalf * 8;
          half8 A[2], Bh[4], Bl[4];
#pragma unroll
          for (int a = 0; a < 2; ++a)
            A[a] = __builtin_bit_cast(half8, packed_x(xp, G, wave, j, st, a)[lane]);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int row = b * 32 + m32;
            Bh[b] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&lds_hi[buf][row * kLdsStride + koff]));
            Bl[b] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&lds_lo[buf][row * kLdsStride + koff]));
          }
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[a], Bh[b], acc[a][b], 0, 0, 0);
              acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[a], Bl[b], acc[a][b], 0, 0, 0);
            }
        }
      }
      if ((2 * c + 2) % per == 0) {
        // the group's squares per row (output column = lane % 32; lanes l and l + 32 hold
        // the same column for different tokens). The lane's 32 squares are summed in fp32
        // (|acc| <= 65504 * 2^14 * 128, so no square overflows; the sum is within 32 * 2^-24
        // of exact), scaled by the exact power of two 1 / P^2 in fp64, and added across
        // the lane halves in fp64; across waves in fp64 too (LDS here, or the reduction
        // kernel from fp32 partials, each within 2^-24 of its fp64 value).
        const int gq = (2 * c + 2) / per - 1;  // group of the step
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          // P = 2^(pe - 1) exactly, so the scaling by 1 / P^2 is an exponent change
          int pe = 0;
          (void)__builtin_frexpf(lds_pg[buf][(b * 32 + m32) * 4 + gq], &pe);
          float s32 = 0.0f;
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int e = 0; e < 16; ++e) s32 = __builtin_fmaf(acc[a][b][e], acc[a][b][e], s32);
          double ss = __builtin_ldexp((double)s32, -2 * (pe - 1));
          ss += __shfl_xor(ss, 32);
          const int64_t row = n0 + b * 32 + m32;
          if (gps == 1) {
            if (khalf == 0) lds_red[buf][wave][b * 32 + m32] = ss;
          } else if (khalf == 0 && row < N) {
            // [ratio][group][wave][row]: a wave's 32 lanes store 128 consecutive bytes
            part[(((int64_t)ci * Gs + j * gps + gq) * NW + wave) * N + row] = (float)ss;
          }
        }
      }
    }
    if (!set_b) quantize(jn, buf ^ 1);
    // end of step: the next one reads the buffer just written (by both sets) and, with one
    // group per step, this step's errors are complete in their slot
    __syncthreads();
    if (gps == 1) {
      if (tid < kRowTile && n0 + tid < N) {
        double tot = lds_red[buf][0][tid];
        for (int w = 1; w < NW; ++w) tot += lds_red[buf][w][tid];
        err[((int64_t)ci * N + n0 + tid) * Gs + j] = tot;
      }
    }
  }
  if (bad && flags && ci == 0) atomicOr(flags, AWQ_FLAG_NONFINITE_INPUT);
}

// One thread per (row, group): the first ratio index with the smallest error. A
// non-finite error can only come from a NaN or Inf weight or activation (the tile's
// min / max drop a NaN), so it raises NONFINITE_INPUT.
__global__ void __launch_bounds__(256)
    k_clip_reduce(const double* __restrict__ err, int n_shrink, int64_t NG,
                  uint8_t* __restrict__ clip_idx, double* __restrict__ err_best,
                  uint32_t* __restrict__ flags) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= NG) return;
  double best = err[u];
  int bi = 0;
  bool bad = !__builtin_isfinite(best);
  for (int i = 1; i < n_shrink; ++i) {
    const double v = err[(int64_t)i * NG + u];
    bad |= !__builtin_isfinite(v);
    if (v < best) {
      best = v;
      bi = i;
    }
  }
  clip_idx[u] = (uint8_t)bi;
  if (err_best) err_best[u] = best;
  if (bad && flags) atomicOr(flags, AWQ_FLAG_NONFINITE_INPUT);
}

// Smaller groups: one thread per (group, row) (consecutive threads, consecutive rows: the
// partial reads coalesce). err_i = sum of the nw wave partials in wave order, in fp64; then
// the first minimum over the ratios, as above.
__global__ void __launch_bounds__(256)
    k_clip_reduce_waves(const float* __restrict__ part, int n_shrink, int64_t N, int64_t G,
                        int nw, uint8_t* __restrict__ clip_idx, double* __restrict__ err_best,
                        uint32_t* __restrict__ flags) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= N * G) return;
  const int64_t g = u / N, row = u - g * N;
  auto error = [&](int i) {
    const float* p = part + ((int64_t)i * G + g) * nw * N + row;
    double v = 0.0;
    for (int w = 0; w < nw; ++w) v += (double)p[(int64_t)w * N];
    return v;
  };
  double best = error(0);
  int bi = 0;
  bool bad = !__builtin_isfinite(best);
  for (int i = 1; i < n_shrink; ++i) {
    const double v = error(i);
    bad |= !__builtin_isfinite(v);
    if (v < best) {
      best = v;
      bi = i;
    }
  }
  clip_idx[row * G + g] = (uint8_t)bi;
  if (err_best) err_best[row * G + g] = best;
  if (bad && flags) atomicOr(flags, AWQ_FLAG_NONFINITE_INPUT);
}

static hipError_t launch_pack_x(const uint16_t* X, int64_t T, int64_t K, uint4* xp,
                                hipStream_t stream) {
  const int64_t tiles = (T + kTokPerWave - 1) / kTokPerWave;
  const int64_t total = tiles * (K / kGroup) * 8 * 2 * 64;
  const int64_t blocks = (total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192;
  hipLaunchKernelGGL(k_pack_x, dim3((unsigned)blocks), dim3(256), 0, stream, X, T, K, tiles, xp);
  return hipGetLastError();
}

size_t packed_x_bytes(int64_t T, int64_t K) {
  return (size_t)((T + kTokPerWave - 1) / kTokPerWave) * kTokPerWave * K * 2;
}

static int clip_waves(int64_t T) { return T <= 4 * kTokPerWave ? 4 : 8; }

size_t clip_err_bytes(int64_t T, int64_t N, int64_t K, int n_shrink, int group) {
  const size_t per = group == kGroup ? 8 : 4 * (size_t)clip_waves(T);  // fp64, or nw fp32 partials
  return (size_t)n_shrink * N * (K / group) * per;
}

hipError_t launch_clip_err(const uint16_t* X, int64_t T, const uint16_t* W, int64_t N,
                           int64_t K, const uint16_t* s, int clip_steps, int n_shrink, bool sym,
                           int group, int w_bit, uint4* xp, void* err, uint32_t* flags,
                           hipStream_t stream) {
  hipError_t e = launch_pack_x(X, T, K, xp, stream);
  if (e != hipSuccess) return e;
  const int64_t n_ntiles = (N + kRowTile - 1) / kRowTile;
  const int64_t per_xcd = (n_ntiles * n_shrink + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(per_xcd * kXcds));
  double* e64 = (double*)err;
  float* e32 = (float*)err;
  if (clip_waves(T) == 4)
    hipLaunchKernelGGL(k_clip_err<4>, grid, dim3(256), 0, stream, xp, T, W, N, K, s, clip_steps,
                       n_shrink, (int)sym, group, w_bit, e64, e32, flags, n_ntiles, per_xcd);
  else
    hipLaunchKernelGGL(k_clip_err<8>, grid, dim3(512), 0, stream, xp, T, W, N, K, s, clip_steps,
                       n_shrink, (int)sym, group, w_bit, e64, e32, flags, n_ntiles, per_xcd);
  return hipGetLastError();
}

hipError_t launch_clip_reduce(const void* err, int64_t T, int n_shrink, int64_t N, int64_t K,
                              int group, uint8_t* clip_idx, double* err_best, uint32_t* flags,
                              hipStream_t stream) {
  const int64_t G = K / group, NG = N * G;
  const dim3 grid((unsigned)((NG + 255) / 256));
  if (group == kGroup)
    hipLaunchKernelGGL(k_clip_reduce, grid, dim3(256), 0, stream, (const double*)err, n_shrink, NG,
                       clip_idx, err_best, flags);
  else
    hipLaunchKernelGGL(k_clip_reduce_waves, grid, dim3(256), 0, stream, (const float*)err, n_shrink,
                       N, G, clip_waves(T), clip_idx, err_best, flags);
  return hipGetLastError();
}

// One block: err_i = sum of partials of grid point i in index order; first minimum. A
// non-finite error can only come from a NaN or Inf weight or activation (the tile's
// min / max drop a NaN), so it raises NONFINITE_INPUT.
__global__ void __launch_bounds__(256)
    k_search_reduce(const double* __restrict__ partials, int n_grid, int64_t n_partials,
                    const uint16_t* __restrict__ s_grid, int64_t K, uint16_t* __restrict__ s_best,
                    int32_t* __restrict__ best_idx, double* __restrict__ err,
                    uint32_t* __restrict__ flags) {
  __shared__ double lds_err[64];
  __shared__ int lds_best;
  const int tid = threadIdx.x;
  if (tid < n_grid) {
    double tot = 0.0;
    const double* p = partials + (int64_t)tid * n_partials;
    for (int64_t i = 0; i < n_partials; ++i) tot += p[i];
    lds_err[tid] = tot;
    if (!__builtin_isfinite(tot) && flags) atomicOr(flags, AWQ_FLAG_NONFINITE_INPUT);
  }
  __syncthreads();
  if (tid == 0) {
    int best = 0;
    for (int i = 1; i < n_grid; ++i)
      if (lds_err[i] < lds_err[best]) best = i;
    lds_best = best;
    *best_idx = best;
  }
  __syncthreads();
  if (err && tid < n_grid) err[tid] = lds_err[tid];
  const uint16_t* src = s_grid + (int64_t)lds_best * K;
  for (int64_t k = tid; k < K; k += blockDim.x) s_best[k] = src[k];
}

int search_row_tile() { return kRowTile; }
int search_token_chunk(int64_t T) { return T <= 4 * kTokPerWave ? 4 * kTokPerWave : 8 * kTokPerWave; }

hipError_t launch_search_err(const uint16_t* X, int64_t T, const uint16_t* W, int64_t N,
                             int64_t K, const uint16_t* s_grid, int n_grid, bool sym, int group,
                             int w_bit, float* rowmax, float* srange, uint4* xp, double* partials,
                             uint32_t* flags, hipStream_t stream) {
  hipLaunchKernelGGL(k_row_absmax, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, stream, W, N, K, rowmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_pack_x(X, T, K, xp, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scale_range, dim3((unsigned)n_grid), dim3(256), 0, stream, s_grid, K, srange, flags);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_ntiles = (N + kRowTile - 1) / kRowTile;
  const int64_t per_xcd = (n_ntiles * n_grid + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(per_xcd * kXcds));
  if (T <= 4 * kTokPerWave)
    hipLaunchKernelGGL(k_search_err<4>, grid, dim3(256), 0, stream, xp, T, W, N, K, s_grid, n_grid,
                       (int)sym, group, w_bit, rowmax, srange, partials, flags, n_ntiles, per_xcd);
  else
    hipLaunchKernelGGL(k_search_err<8>, grid, dim3(512), 0, stream, xp, T, W, N, K, s_grid, n_grid,
                       (int)sym, group, w_bit, rowmax, srange, partials, flags, n_ntiles, per_xcd);
  return hipGetLastError();
}

hipError_t launch_search_reduce(const double* partials, int n_grid, int64_t n_partials,
                                const uint16_t* s_grid, int64_t K, uint16_t* s_best,
                                int32_t* best_idx, double* err, uint32_t* flags,
                                hipStream_t stream) {
  hipLaunchKernelGGL(k_search_reduce, dim3(1), dim3(256), 0, stream, partials, n_grid,
                     n_partials, s_grid, K, s_best, best_idx, err, flags);
  return hipGetLastError();
}

}  // namespace awq
