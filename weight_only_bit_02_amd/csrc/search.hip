// Activation-aware grid search (a5 + a6).
//
// "AWQ量化实战" §2.2 and §3.3 step 4: for every grid point, quantize W diag(s) and score
// how far the layer's calibration outputs move; "什么是激活感知权重量化（AWQ）", "工作机制":
// the scale is an equivalent transform W diag(s), X diag(1/s), found without
// backpropagation. For grid point i the score is
//   err_i = sum_t sum_n ( sum_k X_tk D_nk )^2,   D = W - Q(W diag(s_i)) diag(1/s_i).
//
// One block owns (grid point i, 128 rows of W, up to 64 * NW tokens) and walks K one
// 128-channel step at a time:
//   1. quantize: 16 lanes per (row, step), 8 weights each; the same group quantizer as
//      the pack kernel gives the codes; D is formed in fp32, scaled by a power of two P
//      of its (row, step) so that |D P| < 2^14, and split into two fp16 halves hi + lo
//      (22 significant bits). hi, lo and the exponent of P go to LDS.
//   2. contract: each wave multiplies its 64 tokens of X (fp16, from a copy of X in
//      operand order) by the hi and lo tiles with v_mfma_f32_32x32x16_f16 into its running
//      E tile, which is kept in the scale of the current step's P: when a row's P changes,
//      the row's accumulators are first multiplied by the ratio, an exact power of two.
// P follows each row's largest |D| with hysteresis: it is re-chosen (2 bits of headroom)
// only when the step's largest |D| would leave the fp16 range or falls 2^8 below it, so
// most steps keep it and skip the rescale; every term keeps 22 significant bits unless it
// is 2^8 below its step's largest, whatever the spread of s across the row.
// After the last step the block squares and sums its E tile (fp64) and writes one
// partial; a second kernel adds the partials of each grid point in a fixed order and
// takes the first minimum. No floating-point atomics: results are bitwise
// reproducible.
// Large searches (many weights and tokens) first score every grid point with hi alone:
// the rounding of D P to one fp16 term moves an error by a few 1e-6 relative at most once
// millions of terms are summed, and the pass does half the MFMA work and half the LDS
// operand reads. The grid points within a small relative gap of the smallest such error
// are then scored again with hi + lo (the other blocks of that launch leave at once), so
// the chosen index is always taken on two-term errors.
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
// Error terms as hi alone (then hi + lo for the near-minimal grid points) from this many
// weights and tokens: over that many terms the fp16 rounding of D P moves a grid point's
// error by ~2e-6 relative at most (CPU simulation of the rounding on 2048 x 2048 weights,
// 64 and 512 tokens, ordinary, wide-range and dead-channel activations, 3/4/8-bit codes),
// and kRefineGap re-scores with hi + lo every point within 2^-12 of the smallest error.
constexpr int64_t kOneTermMinWeights = (int64_t)1 << 22;
constexpr int64_t kOneTermMinTokens = 256;
constexpr double kRefineGap = 1.0 / 4096.0;

// Exponent state of the search's per-(row, step) scale P = 2^(14 - E): E is re-chosen as
// e + 2 (e: the exponent of the step's largest |D|, which lies in [2^(e-1), 2^e)) when
// unset, when e > E (|D P| would reach 2^14) or when e < E - 8; otherwise kept. Hence
// 2^5 <= max |D P| < 2^14 on every step. E stays within [-98, 102].
constexpr int kEUnset = -100000;
__device__ __forceinline__ int search_exponent(float dmx, int E) {
  int e = 0;
  (void)__builtin_frexpf(dmx, &e);
  if (!(dmx > 0.0f) || !__builtin_isfinite(dmx)) return E == kEUnset ? 0 : E;  // no constraint
  e = e < -100 ? -100 : (e > 100 ? 100 : e);
  if (E == kEUnset || e > E || e < E - 8) E = e + 2;
  return E;
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
template <int NW, int NROWS>
constexpr int quant_passes() {
  return NROWS / (NW * 4);
}

// The scales of a lane's 8 channels of one 128-channel step (fp32) and their hardware
// reciprocals (1 ulp); s == nullptr (clip search without s): s = 1.
struct StepScales {
  float sf[8], rs[8];
};

template <bool CLIP>
__device__ __forceinline__ StepScales step_scales(const uint16_t* s, int64_t k0) {
  uint4 sv = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);  // s = 1
  if (!CLIP || s) sv = *reinterpret_cast<const uint4*>(s + k0);
  StepScales sc;
  const uint32_t sd[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc.sf[2 * i] = h2f((uint16_t)(sd[i] & 0xFFFF));
    sc.sf[2 * i + 1] = h2f((uint16_t)(sd[i] >> 16));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) sc.rs[i] = __builtin_amdgcn_rcpf(sc.sf[i]);
  return sc;
}

// One row's 8 weights wv of a lane (16 lanes per (row, 128 channels)) -> (D P) split into
// fp16 hi + lo at hi_buf / lo_buf[row * kLdsStride + li * 8]; returns whether a non-finite
// value was met. Search (CLIP = false): the scale of each (row, step) comes from the row's
// exponent state e_state (search_exponent), and its exponent E is written to pe_out[row].
// Clip search: each group's own largest |D| sets its P, written to pg_out[row * 4 + group].
// LO = false keeps only hi (one fp16 term, 11 significant bits; lo_buf unused).
template <bool CLIP, bool LO = true>
__device__ __forceinline__ bool quantize_row(uint4 wv, const StepScales& sc, float r, bool sym,
                                             int group, float qmax, ScaleDiv sd, int& e_state,
                                             int* pe_out, uint16_t* hi_buf, uint16_t* lo_buf,
                                             int row, int li, float* pg_out) {
  const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
  float wp[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wp[2 * i] = h2f((uint16_t)(wd[i] & 0xFFFF)) * sc.sf[2 * i];
    wp[2 * i + 1] = h2f((uint16_t)(wd[i] >> 16)) * sc.sf[2 * i + 1];
  }
  float mn = wp[0], mx = wp[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = fminf(mn, wp[i]);
    mx = fmaxf(mx, wp[i]);
  }
  group_minmax(mn, mx, group);  // 16 lanes = one 128-channel group, two of 64, four of 32
  const bool bad = !__builtin_isfinite(mn) || !__builtin_isfinite(mx);
  if (CLIP) {
    mn = r * mn;
    mx = r * mx;
  }
  const GroupQ g = sym ? group_params_sym(mn, mx, qmax, sd) : group_params(mn, mx, qmax, sd);
  float qz[8];
  quant_centered(wp, g, qz);
  // D = (w' - deq) / s: w' = w s and deq = (q - z) sc_h are exact, and so is their
  // difference (both are multiples of the finer ulp and close in magnitude), so the
  // reciprocal's error (1 ulp) is relative to D itself; w - deq / s would carry it
  // relative to w, which is 30 (4-bit) to 500 (8-bit) times larger than D
  float dg[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float deq = qz[c] * g.scf;  // exact: small integer times an fp16
    dg[c] = (wp[c] - deq) * sc.rs[c];
  }
  float P;
  if constexpr (CLIP) {
    // each group is scored on its own, so its scale comes from its own largest |D|:
    // P = 2^(14 - e) with that maximum in [2^(e-1), 2^e), so |D P| < 2^14 and hi + lo
    // keep 22 significant bits of every group, whatever the code width
    float dmx = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) dmx = fmaxf(dmx, __builtin_fabsf(dg[c]));
    group_max(dmx, group);
    int ex = 0;
    (void)__builtin_frexpf(dmx, &ex);
    if (!(dmx > 0.0f) || !__builtin_isfinite(dmx)) ex = 0;
    ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
    P = __builtin_ldexpf(1.0f, 14 - ex);
    const int gl = group >> 3;  // lanes per group
    if ((li & (gl - 1)) == 0) pg_out[row * 4 + li / gl] = P;
  } else {
    // the (row, step) scale: the largest |D| over the step's 128 channels (16 lanes)
    float dmx = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) dmx = fmaxf(dmx, __builtin_fabsf(dg[c]));
    row16_max(dmx);
    const int E = search_exponent(dmx, e_state);
    e_state = E;
    P = __builtin_ldexpf(1.0f, 14 - E);
    if (li == 0) pe_out[row] = E;
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint16_t h2[2], l2[2] = {0, 0};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 2 * i + e;
      const float d = dg[c] * P;
      h2[e] = f2h_bits(d);
      if constexpr (LO) l2[e] = f2h_bits(d - h2f(h2[e]));
    }
    hi[i] = (uint32_t)h2[0] | ((uint32_t)h2[1] << 16);
    lo[i] = (uint32_t)l2[0] | ((uint32_t)l2[1] << 16);
  }
  *reinterpret_cast<uint4*>(&hi_buf[row * kLdsStride + li * 8]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  if constexpr (LO)
    *reinterpret_cast<uint4*>(&lo_buf[row * kLdsStride + li * 8]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  return bad;
}

// NR rows at once: the arithmetic of quantize_row value for value (so the same bits), with
// the rows' wave-uniform branches shared, one group-size branch and one close-call ballot
// per stage for all NR rows, so the compiler can interleave the rows' independent chains
// (DPP reductions, the group parameters, the codes) instead of running one row's latency
// after the other's.
template <int NR>
__device__ __forceinline__ void group_minmax_rows(float (&mn)[NR], float (&mx)[NR], int group) {
  if (group == 128) {
#pragma unroll
    for (int r = 0; r < NR; ++r) row16_minmax(mn[r], mx[r]);
  } else if (group == 64) {
#pragma unroll
    for (int r = 0; r < NR; ++r) row8_minmax(mn[r], mx[r]);
  } else {
#pragma unroll
    for (int r = 0; r < NR; ++r) quad_minmax(mn[r], mx[r]);
  }
}

template <int NR>
__device__ __forceinline__ void group_max_rows(float (&mx)[NR], int group) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    max_quad_xor1(mx[r]);
    max_quad_xor2(mx[r]);
  }
  if (group == 128) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      max_row_ror4(mx[r]);
      max_row_ror8(mx[r]);
    }
  } else if (group == 64) {
#pragma unroll
    for (int r = 0; r < NR; ++r) max_row_half_mirror(mx[r]);
  }
}

// group_params for NR rows: the zero points' close calls share one ballot.
template <int NR>
__device__ __forceinline__ void group_params_rows(const float (&mn)[NR], const float (&mx)[NR],
                                                  float qmax, ScaleDiv sd, bool sym,
                                                  GroupQ (&g)[NR]) {
#pragma clang fp contract(off)
  if (sym) {
#pragma unroll
    for (int r = 0; r < NR; ++r) g[r] = group_params_sym(mn[r], mx[r], qmax, sd);
    return;
  }
  float qa[NR];
  bool close[NR];
  bool any = false;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    g[r].qmax = qmax;
    float sc = div_small(mx[r] - mn[r], sd.d, sd.y);  // the correctly rounded (mx - mn) / qmax
    sc = fmaxf(sc, 0x1p-14f);
    g[r].clamped = sc > 65504.0f;
    sc = fminf(sc, 65504.0f);
    g[r].sch = f2h_bits(sc);
    g[r].scf = h2f(g[r].sch);
    g[r].rcp = __builtin_amdgcn_rcpf(g[r].scf);
    // z = rint(-mn / sc_h) as rint_quotients takes it
    qa[r] = -mn[r] * g[r].rcp;
    const float fl = __builtin_floorf(qa[r]);
    const float d = __builtin_fabsf((qa[r] - fl) - 0.5f);
    close[r] = !(d > __builtin_fabsf(qa[r]) * 0x1p-21f + 0x1p-60f);
    any |= close[r];
  }
  if (__builtin_amdgcn_ballot_w64(any)) {
    asm volatile("");  // keeps the division in this branch (not speculated into the common path)
#pragma unroll
    for (int r = 0; r < NR; ++r)
      if (close[r]) qa[r] = -mn[r] / g[r].scf;  // correctly rounded division
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) g[r].z = __builtin_amdgcn_fmed3f(__builtin_rintf(qa[r]), 0.0f, qmax);
}

// quant_centered for NR rows of 8 values, each row with its own group parameters.
template <int NR>
__device__ __forceinline__ void quant_centered_rows(const float (&w)[NR][8], const GroupQ (&g)[NR],
                                                    float (&qz)[NR][8]) {
#pragma clang fp contract(off)
  bool close[NR][8];
  bool any = false;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float half_sc = 0.5f * g[r].scf;  // exact
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qz[r][i] = __builtin_rintf(w[r][i] * g[r].rcp);
      const float e = __builtin_fmaf(-qz[r][i], g[r].scf, w[r][i]);
      close[r][i] = !(__builtin_fabsf(e) < half_sc);
      any |= close[r][i];
    }
  }
  if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (close[r][i]) qz[r][i] = __builtin_rintf(w[r][i] / g[r].scf);  // correctly rounded
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float lo = -g[r].z, hi = g[r].qmax - g[r].z;  // exact
#pragma unroll
    for (int i = 0; i < 8; ++i) qz[r][i] = __builtin_amdgcn_fmed3f(qz[r][i], lo, hi);
  }
}

// quantize_row for NR rows (rows[r], weights wv[r], exponent states e_state[r]).
template <bool CLIP, bool LO, int NR>
__device__ __forceinline__ bool quantize_rows(const uint4 (&wv)[NR], const StepScales& sc, float rr,
                                              bool sym, int group, float qmax, ScaleDiv sd,
                                              int* e_state, int* pe_out, uint16_t* hi_buf,
                                              uint16_t* lo_buf, const int (&row)[NR], int li,
                                              float* pg_out) {
#pragma clang fp contract(off)
  float wp[NR][8], mn[NR], mx[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const uint32_t wd[4] = {wv[r].x, wv[r].y, wv[r].z, wv[r].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wp[r][2 * i] = h2f((uint16_t)(wd[i] & 0xFFFF)) * sc.sf[2 * i];
      wp[r][2 * i + 1] = h2f((uint16_t)(wd[i] >> 16)) * sc.sf[2 * i + 1];
    }
    mn[r] = wp[r][0];
    mx[r] = wp[r][0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      mn[r] = fminf(mn[r], wp[r][i]);
      mx[r] = fmaxf(mx[r], wp[r][i]);
    }
  }
  group_minmax_rows<NR>(mn, mx, group);
  bool bad = false;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    bad |= !__builtin_isfinite(mn[r]) || !__builtin_isfinite(mx[r]);
    if (CLIP) {
      mn[r] = rr * mn[r];
      mx[r] = rr * mx[r];
    }
  }
  GroupQ g[NR];
  group_params_rows<NR>(mn, mx, qmax, sd, sym, g);
  float qz[NR][8];
  quant_centered_rows<NR>(wp, g, qz);
  float dg[NR][8], dmx[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    dmx[r] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float deq = qz[r][c] * g[r].scf;  // exact: small integer times an fp16
      dg[r][c] = (wp[r][c] - deq) * sc.rs[c];
      dmx[r] = fmaxf(dmx[r], __builtin_fabsf(dg[r][c]));
    }
  }
  float P[NR];
  if constexpr (CLIP) {
    group_max_rows<NR>(dmx, group);
    const int gl = group >> 3;  // lanes per group
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      int ex = 0;
      (void)__builtin_frexpf(dmx[r], &ex);
      if (!(dmx[r] > 0.0f) || !__builtin_isfinite(dmx[r])) ex = 0;
      ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
      P[r] = __builtin_ldexpf(1.0f, 14 - ex);
      if ((li & (gl - 1)) == 0) pg_out[row[r] * 4 + li / gl] = P[r];
    }
  } else {
#pragma unroll
    for (int r = 0; r < NR; ++r) row16_max(dmx[r]);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int E = search_exponent(dmx[r], e_state[r]);
      e_state[r] = E;
      P[r] = __builtin_ldexpf(1.0f, 14 - E);
      if (li == 0) pe_out[row[r]] = E;
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t h2[2], l2[2] = {0, 0};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float d = dg[r][2 * i + e] * P[r];
        h2[e] = f2h_bits(d);
        if constexpr (LO) l2[e] = f2h_bits(d - h2f(h2[e]));
      }
      hi[i] = (uint32_t)h2[0] | ((uint32_t)h2[1] << 16);
      lo[i] = (uint32_t)l2[0] | ((uint32_t)l2[1] << 16);
    }
    *reinterpret_cast<uint4*>(&hi_buf[row[r] * kLdsStride + li * 8]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    if constexpr (LO)
      *reinterpret_cast<uint4*>(&lo_buf[row[r] * kLdsStride + li * 8]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  return bad;
}

// Quantizes step j of rows [row_base, row_base + NROWS) of the tile with NW waves (tid
// counts their threads from 0), 4 rows per wave per pass.
template <int NW, bool CLIP, int NROWS, bool LO = true>
__device__ __forceinline__ bool quantize_tile_group(const uint16_t* W, int64_t N, int64_t K,
                                                    const uint16_t* s, float r, bool sym,
                                                    int group, float qmax, int64_t n0, int64_t j,
                                                    int (&e_state)[quant_passes<NW, NROWS>()],
                                                    int* pe_out, uint16_t* hi_buf,
                                                    uint16_t* lo_buf, int tid, int row_base,
                                                    float* pg_out, const float* cmul = nullptr) {
  constexpr int kRowsPerPass = NW * 4;
  constexpr int kPasses = quant_passes<NW, NROWS>();
  static_assert(kPasses * kRowsPerPass == NROWS, "whole passes");
  const int q_row = row_base + (tid >> 4);
  const int li = tid & 15;
  const int64_t k0 = j * kGroup + li * 8;
  // every pass's weights and the scales are loaded before any is used: the passes are
  // separated by the quantizer's wave-uniform branches, past which the compiler would not
  // hoist the loads, so each pass would otherwise wait out a full memory latency on its own
  uint4 wvs[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int64_t n = n0 + p * kRowsPerPass + q_row;
    wvs[p] = *reinterpret_cast<const uint4*>(W + (n < N ? n : N - 1) * K + k0);
  }
  // the thread's 8 channels are the same in every pass: s and 1/s once
  StepScales sc = step_scales<CLIP>(s, k0);
  if (cmul) {
    // D is wanted times a per-channel power of two: folded into 1/s (exact)
    const float4 c0 = *reinterpret_cast<const float4*>(cmul + k0);
    const float4 c1 = *reinterpret_cast<const float4*>(cmul + k0 + 4);
    const float cm[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) sc.rs[i] *= cm[i];
  }
  bool bad = false;
  // passes in pairs: two rows per lane through quantize_rows (kPasses is 1, 2 or 4)
  constexpr int NR = kPasses >= 2 ? 2 : 1;
#pragma unroll
  for (int p = 0; p < kPasses; p += NR) {
    uint4 wv[NR];
    int rows[NR];
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      rows[u] = (p + u) * kRowsPerPass + q_row;
      wv[u] = n0 + rows[u] < N ? wvs[p + u] : make_uint4(0, 0, 0, 0);
    }
    bad |= quantize_rows<CLIP, LO, NR>(wv, sc, r, sym, group, qmax, scale_divisor(qmax, sym),
                                       &e_state[p], pe_out, hi_buf, lo_buf, rows, li, pg_out);
  }
  return bad;
}

// LO: D P as two fp16 terms hi + lo (22 significant bits) or as hi alone (11 bits, half
// the MFMA work and LDS operand reads). cand (optional): only grid points with cand[i] != 0
// are scored; the other blocks leave at once (their partials are left as they were).
template <int NW, bool LO>
__global__ void __launch_bounds__(NW * 64)
    k_search_err(const uint4* xp, int64_t T, const uint16_t* W, int64_t N, int64_t K,
                 const uint16_t* s_grid, int n_grid, int sym, int group, int w_bit,
                 double* __restrict__ partials, uint32_t* __restrict__ flags, int64_t n_ntiles,
                 int64_t per_xcd, const uint8_t* __restrict__ cand) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_hi[2][kRowTile * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t lds_lo[LO ? 2 : 1][LO ? kRowTile * kLdsStride : 8];
  __shared__ int lds_pe[2][kRowTile];  // exponent E of each row's P = 2^(14 - E), per buffer
  __shared__ double lds_red[NW];

  // XCD-aware order: consecutive blocks of one XCD share a row tile (different grid
  // points), so the tile of W is read from HBM once per XCD.
  const int64_t t = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (t >= n_ntiles * n_grid) return;
  const int64_t ntile = t / n_grid;
  const int alpha = (int)(t % n_grid);
  if (cand && cand[alpha] == 0) return;  // block-uniform, before any barrier

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
  int e_state[quant_passes<NH, kRowTile / 2>()];
  auto quantize = [&](int64_t j, int buf) {
    bad |= quantize_tile_group<NH, false, kRowTile / 2, LO>(W, N, K, s, 1.0f, sym, group, qmax, n0,
                                                           j, e_state, lds_pe[buf], lds_hi[buf],
                                                           lds_lo[LO ? buf : 0], tid_set,
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
    int e_prev[4] = {0, 0, 0, 0};  // exponent of the P the accumulators of tile b are in
#pragma unroll
    for (int i = 0; i < quant_passes<NH, kRowTile / 2>(); ++i) e_state[i] = kEUnset;
    auto multiply = [&](int64_t j, int buf) {
      if (!active) return;
      // bring each row's running E into the scale of this step's P (exact powers of two;
      // the whole wave skips it when no row changed)
      int en[4];
      bool changed = false;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        en[b] = lds_pe[buf][b * 32 + m32];
        changed |= en[b] != e_prev[b];
      }
      if (__builtin_amdgcn_ballot_w64(changed)) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int d = e_prev[b] - en[b];  // P_new / P_old = 2^d
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = __builtin_ldexpf(acc[a][b][e], d);
        }
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) e_prev[b] = en[b];
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
          if constexpr (LO)
            Bl[b] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&lds_lo[buf][r * kLdsStride + koff]));
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[a], Bh[b], acc[a][b], 0, 0, 0);
            if constexpr (LO)
              acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[a], Bl[b], acc[a][b], 0, 0, 0);
          }
      }
    };

    quantize(0, 0);
    __syncthreads();
    for (int64_t j = 0; j < G; ++j) {
      const int buf = (int)(j & 1);
      // the next step's quantization (none after the last step: block-uniform)
      const bool more = j + 1 < G;
      if (!set_b) {
        multiply(j, buf);
        if (more) quantize(j + 1, buf ^ 1);
      } else {
        if (more) quantize(j + 1, buf ^ 1);
        multiply(j, buf);
      }
      __syncthreads();
    }

    // ------------------------------------------------------------------ sum of squares
    double ss = 0.0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const double pinv = __builtin_ldexp(1.0, e_prev[b] - 14);  // 1 / P; column = lane % 32
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
  int e_unused[quant_passes<NH, kRowTile / 2>()];
  auto quantize = [&](int64_t jq, int qbuf) {
    bad |= quantize_tile_group<NH, true, kRowTile / 2>(W, N, K, s, r, sym, group, qmax, n0, jq,
                                                      e_unused, nullptr, lds_hi[qbuf], lds_lo[qbuf],
                                                      tid_set, set_b ? kRowTile / 2 : 0,
                                                      lds_pg[qbuf]);
  };
  quantize(0, 0);
  __syncthreads();
  for (int64_t j = 0; j < G; ++j) {
    const int buf = (int)(j & 1);
    const bool more = j + 1 < G;  // the next step's quantization (none after the last step)
    if (set_b && more) quantize(j + 1, buf ^ 1);
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
    if (!set_b && more) quantize(j + 1, buf ^ 1);
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

// ------------------------------------------------------------------ Gram form (f3)
// With 128-channel groups, a group's error is a quadratic form in its weight errors:
//   err(n, g) = sum_t (sum_{k in g} X_tk D_nk)^2 = d^T G_g d,  G_g = X_g^T X_g (128 x 128),
// so once G_g is formed (2 T 128 flop per weight, shared by every ratio and row) a ratio
// costs 2 * 128 flop per weight instead of 2 T. Channels are balanced by powers of two:
// c_k = 2^-e_k with G_kk c_k^2 in (1/4, 1], G' = diag(c) G diag(c), D' = D diag(1/c), so
// d'^T G' d' is the same number, every |G'_kj| <= 1 (Cauchy-Schwarz) and D' carries each
// channel's weight error times its activation size. G' is kept as fp16 hi + lo and D' P
// (the group's own power of two, as in the direct form) as fp16 hi + lo; V = G' D'^T takes
// the products hi hi, lo hi and hi lo on the matrix cores (fp32), and err = sum_j D'_j V_j
// with D'_j = hi + lo (exact in fp32).

// The Gram kernels split the tokens over thread slices (contiguous token ranges) and add
// the slices' fp64 partials in slice order through LDS, so each sum is formed in a fixed
// order and enough waves are in flight to cover the load latency.
constexpr int kGramSlices = 8;

// e_k of every channel: G_kk = sum_t X_tk^2 (fp64) = m 2^E, m in [1/2, 1), e_k = ceil(E / 2),
// so G_kk 2^(-2 e_k) lies in [1/4, 1); cmul[k] = 2^e_k (multiplies D); a zero or non-finite
// G_kk takes e_k = 0. Block: 64 channels (8 threads of 8 channels, 16-byte loads) x 64 token
// slices, the slices' fp64 partials added in slice order through LDS.
constexpr int kScaleSlices = 64;
__global__ void __launch_bounds__(8 * kScaleSlices)
    k_gram_scale(const uint16_t* __restrict__ X, int64_t T, int64_t K, int* __restrict__ cexp,
                 float* __restrict__ cmul) {
  __shared__ double part[kScaleSlices][64];
  const int q = threadIdx.x & 7, sl = threadIdx.x >> 3;
  const int64_t k0 = (int64_t)blockIdx.x * 64 + q * 8;  // K is a multiple of 128
  const int64_t t0 = T * sl / kScaleSlices, t1 = T * (sl + 1) / kScaleSlices;
  double g[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t t = t0; t < t1; ++t) {
    const uint4 v = *reinterpret_cast<const uint4*>(X + t * K + k0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double a = (double)h2f((uint16_t)(w[i] & 0xFFFF));
      const double b = (double)h2f((uint16_t)(w[i] >> 16));
      g[2 * i] = __builtin_fma(a, a, g[2 * i]);
      g[2 * i + 1] = __builtin_fma(b, b, g[2 * i + 1]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[sl][q * 8 + i] = g[i];
  __syncthreads();
  if (threadIdx.x < 64) {
    const int c = threadIdx.x;
    double tot = 0.0;
    for (int u = 0; u < kScaleSlices; ++u) tot += part[u][c];
    int E = 0;
    if (tot > 0.0 && __builtin_isfinite(tot)) (void)__builtin_frexp(tot, &E);
    const int e = (E + 1) >> 1;  // ceil(E / 2), E may be negative
    const int64_t k = (int64_t)blockIdx.x * 64 + c;
    cexp[k] = e;
    cmul[k] = __builtin_ldexpf(1.0f, e);
  }
}

// G' in MFMA A-operand order: for group g, 32-row slice jt (0..3), k16 slice st (0..7) and
// part (hi, lo), lane l's 16 bytes are G'[32 jt + l % 32][16 st + 8 (l / 32) .. + 8], so a
// wave's load of one (jt, st, part) is 1 KiB contiguous. Block: one (g, jt, st) piece, 64
// lanes x kGramSlices token slices; lane l forms its 8 fp64 sums over the tokens, scaled by
// 2^-(e_j + e_k) (exact), hi = fp16(v), lo = fp16(v - hi).
__global__ void __launch_bounds__(64 * kGramSlices)
    k_gram_build(const uint16_t* __restrict__ X, int64_t T, int64_t K,
                 const int* __restrict__ cexp, uint4* __restrict__ gp,
                 uint32_t* __restrict__ flags) {
  __shared__ double part[kGramSlices - 1][8][64];
  const int lane = threadIdx.x & 63, sl = threadIdx.x >> 6;
  const int64_t piece = blockIdx.x;  // (g * 4 + jt) * 8 + st
  const int st = (int)(piece & 7);
  const int jt = (int)((piece >> 3) & 3);
  const int64_t g = piece >> 5;
  const int64_t kj = g * kGroup + jt * 32 + (lane & 31);
  const int64_t kk = g * kGroup + st * 16 + (lane >> 5) * 8;
  const int64_t t0 = T * sl / kGramSlices, t1 = T * (sl + 1) / kGramSlices;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto add = [&](uint16_t xh, uint4 v) {
    const double xj = (double)h2f(xh);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = __builtin_fma(xj, (double)h2f((uint16_t)(w[q] & 0xFFFF)), acc[2 * q]);
      acc[2 * q + 1] = __builtin_fma(xj, (double)h2f((uint16_t)(w[q] >> 16)), acc[2 * q + 1]);
    }
  };
  int64_t t = t0;
  for (; t + 4 <= t1; t += 4) {  // four tokens' loads in flight before the first is used
    uint16_t xh[4];
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xh[u] = X[(t + u) * K + kj];
      v[u] = *reinterpret_cast<const uint4*>(X + (t + u) * K + kk);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) add(xh[u], v[u]);
  }
  for (; t < t1; ++t) add(X[t * K + kj], *reinterpret_cast<const uint4*>(X + t * K + kk));
  if (sl > 0) {
#pragma unroll
    for (int c = 0; c < 8; ++c) part[sl - 1][c][lane] = acc[c];
  }
  __syncthreads();
  if (sl != 0) return;
  for (int u = 0; u < kGramSlices - 1; ++u)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += part[u][c][lane];
  uint32_t hi[4], lo[4];
  bool bad = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint16_t h2[2], l2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 2 * q + e;
      const double v = __builtin_ldexp(acc[c], -(cexp[kj] + cexp[kk + c]));
      bad |= !__builtin_isfinite(v);
      h2[e] = f2h_bits((float)v);
      l2[e] = f2h_bits((float)(v - (double)h2f(h2[e])));
    }
    hi[q] = (uint32_t)h2[0] | ((uint32_t)h2[1] << 16);
    lo[q] = (uint32_t)l2[0] | ((uint32_t)l2[1] << 16);
  }
  uint4* base = gp + piece * 2 * 64;
  base[lane] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  base[64 + lane] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  if (bad && flags) atomicOr(flags, AWQ_FLAG_NONFINITE_INPUT);
}

// Clip-search errors in the Gram form, 128-channel groups. A block owns (ratio i, 128 rows);
// per step (= group) the two wave sets quantize D' P into LDS as in k_clip_err (set A
// contracts then quantizes its half of the next group's rows, set B the reverse), and
// wave w computes the slice (j rows 32 (w % 4) .., W rows 32 NT (w / 4) ..; NT = 16 / NW
// tiles of 32 rows) of V^T = G' (D' P)^T: per k16 slice, G' hi / lo fragments from gp and D' P hi / lo
// fragments from LDS, three MFMAs per 32 x 32 tile. Then each lane forms
// sum_j V^T[j][n] (D' P)[n][j] over its 16 j of each tile (fp32), the lane halves and
// the four j slices add in fp64, scaled by 1 / P^2 (exact).
template <int NW>
__global__ void __launch_bounds__(NW * 64)
    k_clip_err_gram(const uint4* __restrict__ gp, const float* __restrict__ cmul,
                    const uint16_t* W, int64_t N, int64_t K, const uint16_t* s, int clip_steps,
                    int n_shrink, int sym, int w_bit, double* __restrict__ err,
                    uint32_t* __restrict__ flags, int64_t n_ntiles, int64_t per_xcd) {
  constexpr int NT = 16 / NW;  // 32 x 32 output tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t lds_hi[2][kRowTile * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t lds_lo[2][kRowTile * kLdsStride];
  __shared__ float lds_pg[2][kRowTile * 4];
  __shared__ double lds_red[2][4][kRowTile];  // [step parity][j slice][row]

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
  const int64_t G = K / kGroup;
  const int m32 = lane & 31;
  const int khalf = lane >> 5;
  const int jt = wave & 3;          // j slice of G' this wave multiplies
  const int nb = (wave >> 2) * NT;  // first of its 32-row tiles of the block's rows

  constexpr int NH = NW / 2;
  const bool set_b = wave >= NH;
  const int tid_set = set_b ? tid - NH * 64 : tid;
  bool bad = false;
  int e_unused[quant_passes<NH, kRowTile / 2>()];
  auto quantize = [&](int64_t jq, int qbuf) {
    bad |= quantize_tile_group<NH, true, kRowTile / 2>(W, N, K, s, r, sym, kGroup, qmax, n0, jq,
                                                      e_unused, nullptr, lds_hi[qbuf], lds_lo[qbuf],
                                                      tid_set, set_b ? kRowTile / 2 : 0,
                                                      lds_pg[qbuf], cmul);
  };
  auto contract = [&](int64_t j, int buf) {
    f32x16 acc[NT];
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[b] = f32x16{};
    const uint4* gbase = gp + (((j * 4 + jt) * 8) * 2) * 64;
#pragma unroll 2
    for (int st = 0; st < 8; ++st) {
      const half8 Ah = __builtin_bit_cast(half8, gbase[(st * 2) * 64 + lane]);
      const half8 Al = __builtin_bit_cast(half8, gbase[(st * 2 + 1) * 64 + lane]);
      const int koff = st * 16 + khalf * 8;
#pragma unroll
      for (int b = 0; b < NT; ++b) {
        const int row = (nb + b) * 32 + m32;
        const half8 Bh = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&lds_hi[buf][row * kLdsStride + koff]));
        const half8 Bl = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&lds_lo[buf][row * kLdsStride + koff]));
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ah, Bh, acc[b], 0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Al, Bh, acc[b], 0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ah, Bl, acc[b], 0, 0, 0);
      }
    }
    // acc[b][e] = V^T[j][n], n = 32 (nb + b) + lane % 32, j = 32 jt + 8 (e / 4) + 4 (lane / 32)
    // + e % 4: the lane's four runs of 4 consecutive j of row n
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const int row = (nb + b) * 32 + m32;
      float s32 = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int jj = jt * 32 + q * 8 + khalf * 4;
        const uint2 h = *reinterpret_cast<const uint2*>(&lds_hi[buf][row * kLdsStride + jj]);
        const uint2 l = *reinterpret_cast<const uint2*>(&lds_lo[buf][row * kLdsStride + jj]);
        const uint32_t hw[2] = {h.x, h.y}, lw[2] = {l.x, l.y};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint16_t hb = (uint16_t)(hw[u >> 1] >> (16 * (u & 1)));
          const uint16_t lb = (uint16_t)(lw[u >> 1] >> (16 * (u & 1)));
          const float d = h2f(hb) + h2f(lb);  // exact: 22 significant bits
          s32 = __builtin_fmaf(acc[b][q * 4 + u], d, s32);
        }
      }
      int pe = 0;
      (void)__builtin_frexpf(lds_pg[buf][row * 4], &pe);  // P = 2^(pe - 1)
      double ss = __builtin_ldexp((double)s32, -2 * (pe - 1));
      ss += __shfl_xor(ss, 32);
      if (khalf == 0) lds_red[buf][jt][row] = ss;
    }
  };

  quantize(0, 0);
  __syncthreads();
  for (int64_t j = 0; j < G; ++j) {
    const int buf = (int)(j & 1);
    const bool more = j + 1 < G;
    if (set_b && more) quantize(j + 1, buf ^ 1);
    contract(j, buf);
    if (!set_b && more) quantize(j + 1, buf ^ 1);
    __syncthreads();
    if (tid < kRowTile && n0 + tid < N) {
      const double tot = ((lds_red[buf][0][tid] + lds_red[buf][1][tid]) + lds_red[buf][2][tid]) +
                         lds_red[buf][3][tid];
      err[((int64_t)ci * N + n0 + tid) * G + j] = tot;
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

// The Gram form serves 128-channel groups from more than 256 calibration tokens (where it
// needs fewer matrix-core passes than the direct form: 3 x 128 against 2 x T per weight).
static bool clip_gram(int64_t T, int group) { return group == kGroup && T > 4 * kTokPerWave; }

static size_t gram_bytes(int64_t K) {
  return (size_t)K * kGroup * 2 * 2 + (size_t)K * 4 * 2;  // G' hi + lo, cexp, cmul
}

size_t clip_scratch_bytes(int64_t T, int64_t K, int group) {
  const size_t px = packed_x_bytes(T, K);
  return clip_gram(T, group) && gram_bytes(K) > px ? gram_bytes(K) : px;
}

hipError_t launch_clip_err(const uint16_t* X, int64_t T, const uint16_t* W, int64_t N,
                           int64_t K, const uint16_t* s, int clip_steps, int n_shrink, bool sym,
                           int group, int w_bit, uint4* xp, void* err, uint32_t* flags,
                           hipStream_t stream) {
  const int64_t n_ntiles = (N + kRowTile - 1) / kRowTile;
  const int64_t per_xcd = (n_ntiles * n_shrink + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(per_xcd * kXcds));
  if (clip_gram(T, group)) {
    // scratch: [G' in operand order: K * 512 B][cexp: int K][cmul: fp32 K]
    uint4* gp = xp;
    int* cexp = reinterpret_cast<int*>(reinterpret_cast<char*>(xp) + (size_t)K * kGroup * 4);
    float* cmul = reinterpret_cast<float*>(cexp + K);
    hipLaunchKernelGGL(k_gram_scale, dim3((unsigned)(K / 64)), dim3(8 * kScaleSlices), 0,
                       stream, X, T, K, cexp, cmul);
    hipLaunchKernelGGL(k_gram_build, dim3((unsigned)((K / kGroup) * 4 * 8)),
                       dim3(64 * kGramSlices), 0, stream, X, T, K, cexp, gp, flags);
    hipLaunchKernelGGL(k_clip_err_gram<16>, grid, dim3(1024), 0, stream, gp, cmul, W, N, K, s,
                       clip_steps, n_shrink, (int)sym, w_bit, (double*)err, flags, n_ntiles,
                       per_xcd);
    return hipGetLastError();
  }
  hipError_t e = launch_pack_x(X, T, K, xp, stream);
  if (e != hipSuccess) return e;
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

// Fixed-order fp64 sum of grid point i's partials.
__device__ __forceinline__ double sum_partials(const double* partials, int i, int64_t n_partials) {
  double tot = 0.0;
  const double* p = partials + (int64_t)i * n_partials;
  for (int64_t u = 0; u < n_partials; ++u) tot += p[u];
  return tot;
}

// After a one-term pass: errf_i from its partials, and cand_i = 1 for every grid point whose
// one-term error lies within a relative kRefineGap of the smallest one, when there are at
// least two such points (a lone minimum is already decided). One block, one thread per point.
__global__ void __launch_bounds__(64)
    k_search_candidates(const double* __restrict__ partials, int n_grid, int64_t n_partials,
                        double refine_gap, double* __restrict__ errf, uint8_t* __restrict__ cand) {
  __shared__ double lds_err[64];
  __shared__ int lds_n;
  const int tid = threadIdx.x;
  if (tid < n_grid) lds_err[tid] = sum_partials(partials, tid, n_partials);
  if (tid == 0) lds_n = 0;
  __syncthreads();
  double mn = lds_err[0];
  for (int i = 1; i < n_grid; ++i) mn = lds_err[i] < mn ? lds_err[i] : mn;
  const double lim = mn + refine_gap * __builtin_fabs(mn);
  const bool near = tid < n_grid && lds_err[tid] <= lim;  // false for NaN
  if (near) atomicAdd(&lds_n, 1);
  __syncthreads();
  if (tid < n_grid) {
    errf[tid] = lds_err[tid];
    cand[tid] = (uint8_t)(near && lds_n > 1 ? 1 : 0);
  }
}

// One block: err_i = sum of partials of grid point i in index order (with cand, only for
// the points marked in it; the others take errf_i), then the first minimum. A non-finite
// error can only come from a NaN or Inf weight or activation (the tile's min / max drop a
// NaN), so it raises NONFINITE_INPUT.
__global__ void __launch_bounds__(256)
    k_search_reduce(const double* __restrict__ partials, int n_grid, int64_t n_partials,
                    const uint8_t* __restrict__ cand, const double* __restrict__ errf,
                    const uint16_t* __restrict__ s_grid, int64_t K, uint16_t* __restrict__ s_best,
                    int32_t* __restrict__ best_idx, double* __restrict__ err,
                    uint32_t* __restrict__ flags) {
  __shared__ double lds_err[64];
  __shared__ int lds_best;
  const int tid = threadIdx.x;
  if (tid < n_grid) {
    const double tot =
        (!cand || cand[tid]) ? sum_partials(partials, tid, n_partials) : errf[tid];
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

bool search_one_term(int64_t T, int64_t N, int64_t K) {
  return T >= kOneTermMinTokens && N * K >= kOneTermMinWeights;
}

static void launch_search_pass(const uint4* xp, int64_t T, const uint16_t* W, int64_t N,
                               int64_t K, const uint16_t* s_grid, int n_grid, bool sym, int group,
                               int w_bit, double* partials, uint32_t* flags, bool lo,
                               const uint8_t* cand, hipStream_t stream) {
  const int64_t n_ntiles = (N + kRowTile - 1) / kRowTile;
  const int64_t per_xcd = (n_ntiles * n_grid + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(per_xcd * kXcds));
#define AWQ_SEARCH_LAUNCH(NW_, LO_)                                                              \
  hipLaunchKernelGGL((k_search_err<NW_, LO_>), grid, dim3(NW_ * 64), 0, stream, xp, T, W, N, K, \
                     s_grid, n_grid, (int)sym, group, w_bit, partials, flags, n_ntiles, per_xcd, \
                     cand)
  if (T <= 4 * kTokPerWave) {
    if (lo) AWQ_SEARCH_LAUNCH(4, true); else AWQ_SEARCH_LAUNCH(4, false);
  } else {
    if (lo) AWQ_SEARCH_LAUNCH(8, true); else AWQ_SEARCH_LAUNCH(8, false);
  }
#undef AWQ_SEARCH_LAUNCH
}

hipError_t launch_search_err(const uint16_t* X, int64_t T, const uint16_t* W, int64_t N,
                             int64_t K, const uint16_t* s_grid, int n_grid, bool sym, int group,
                             int w_bit, uint4* xp, double* partials, double* errf, uint8_t* cand,
                             bool one_term, uint32_t* flags, hipStream_t stream) {
  hipError_t e = launch_pack_x(X, T, K, xp, stream);
  if (e != hipSuccess) return e;
  if (!one_term) {
    launch_search_pass(xp, T, W, N, K, s_grid, n_grid, sym, group, w_bit, partials, flags, true,
                       nullptr, stream);
    return hipGetLastError();
  }
  // one-term pass over every grid point, then the two-term pass over the near-minimal ones
  launch_search_pass(xp, T, W, N, K, s_grid, n_grid, sym, group, w_bit, partials, flags, false,
                     nullptr, stream);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_search_candidates, dim3(1), dim3(64), 0, stream, partials, n_grid,
                     (int64_t)((N + kRowTile - 1) / kRowTile) *
                         ((T + search_token_chunk(T) - 1) / search_token_chunk(T)),
                     kRefineGap, errf, cand);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  launch_search_pass(xp, T, W, N, K, s_grid, n_grid, sym, group, w_bit, partials, flags, true,
                     cand, stream);
  return hipGetLastError();
}

hipError_t launch_search_reduce(const double* partials, int n_grid, int64_t n_partials,
                                const uint8_t* cand, const double* errf, const uint16_t* s_grid,
                                int64_t K, uint16_t* s_best, int32_t* best_idx, double* err,
                                uint32_t* flags, hipStream_t stream) {
  hipLaunchKernelGGL(k_search_reduce, dim3(1), dim3(256), 0, stream, partials, n_grid,
                     n_partials, cand, errf, s_grid, K, s_best, best_idx, err, flags);
  return hipGetLastError();
}

}  // namespace awq
