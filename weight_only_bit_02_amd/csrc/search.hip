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
#include "common.hpp"
#include "launch.hpp"

namespace awq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRowTile = 64;         // rows of W per block
constexpr int kTokPerWave = 64;      // tokens per wave (2 MFMA row tiles)
constexpr int kLdsStride = 128 + 8;  // halves per LDS row (16-byte pad against bank conflicts)

template <int NW>
__global__ void __launch_bounds__(NW * 64)
    k_search_err(const uint16_t* __restrict__ X, int64_t T, const uint16_t* __restrict__ W,
                 int64_t N, int64_t K, const uint16_t* __restrict__ s_grid,
                 double* __restrict__ partials, uint32_t* __restrict__ flags) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_hi[kRowTile * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t lds_lo[kRowTile * kLdsStride];
  __shared__ float lds_pinv[kRowTile];
  __shared__ double lds_red[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t ntile = blockIdx.x;
  const int alpha = blockIdx.y;
  const int64_t n0 = ntile * kRowTile;
  const int64_t G = K / kGroup;
  const uint16_t* s = s_grid + (int64_t)alpha * K;
  const int64_t tchunk = (int64_t)NW * kTokPerWave;
  const int64_t n_tchunks = (T + tchunk - 1) / tchunk;
  const int64_t n_ntiles = gridDim.x;

  // quantize-phase mapping
  constexpr int kRowsPerPass = NW * 4;
  constexpr int kPasses = kRowTile / kRowsPerPass;
  const int q_row = tid >> 4;
  const int li = tid & 15;

  // contract-phase mapping (32x32x16 operands: row/col = lane % 32, k-half = lane / 32)
  const int m32 = lane & 31;
  const int khalf = lane >> 5;

  bool bad = false;
  for (int64_t tc = 0; tc < n_tchunks; ++tc) {
    const int64_t tw = tc * tchunk + (int64_t)wave * kTokPerWave;
    const bool active = tw < T;
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

    for (int64_t j = 0; j < G; ++j) {
      // ---------------------------------------------------------------- quantize
#pragma unroll
      for (int p = 0; p < kPasses; ++p) {
        const int r = p * kRowsPerPass + q_row;
        const int64_t n = n0 + r;
        const int64_t k0 = j * kGroup + li * 8;
        uint4 wv = make_uint4(0, 0, 0, 0);
        if (n < N) wv = *reinterpret_cast<const uint4*>(W + n * K + k0);
        const uint4 sv = *reinterpret_cast<const uint4*>(s + k0);
        const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
        const uint32_t sd[4] = {sv.x, sv.y, sv.z, sv.w};
        float wf[8], sf[8], wp[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wf[2 * i] = h2f((uint16_t)(wd[i] & 0xFFFF));
          wf[2 * i + 1] = h2f((uint16_t)(wd[i] >> 16));
          sf[2 * i] = h2f((uint16_t)(sd[i] & 0xFFFF));
          sf[2 * i + 1] = h2f((uint16_t)(sd[i] >> 16));
        }
        float mn, mx, rsmax = 0.0f;
        float rs[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          wp[i] = wf[i] * sf[i];
          rs[i] = __builtin_amdgcn_rcpf(sf[i]);
          bad |= !__builtin_isfinite(wp[i]);
          mn = i ? fminf(mn, wp[i]) : wp[i];
          mx = i ? fmaxf(mx, wp[i]) : wp[i];
          rsmax = fmaxf(rsmax, rs[i]);
        }
        float dummy = -rsmax;
        row16_minmax(mn, mx);
        row16_minmax(dummy, rsmax);
        const GroupQ g = group_params(mn, mx);
        // |w' - deq| <= max|w'| + 15 sc_h, so |D| <= that / min s.
        const float bound = (fmaxf(__builtin_fabsf(mx), __builtin_fabsf(mn)) + 15.0f * g.scf) * rsmax;
        int ex = 0;
        (void)__builtin_frexpf(bound, &ex);
        ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
        const float P = __builtin_ldexpf(1.0f, 14 - ex);
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint16_t h2[2], l2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int c = 2 * i + e;
            const float q = quant_code(wp[c], g);
            const float deq = (q - g.z) * g.scf;  // exact: small integer times an fp16
            const float d = (wf[c] - deq * rs[c]) * P;
            h2[e] = f2h_bits(d);
            l2[e] = f2h_bits(d - h2f(h2[e]));
          }
          hi[i] = (uint32_t)h2[0] | ((uint32_t)h2[1] << 16);
          lo[i] = (uint32_t)l2[0] | ((uint32_t)l2[1] << 16);
        }
        *reinterpret_cast<uint4*>(&lds_hi[r * kLdsStride + li * 8]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *reinterpret_cast<uint4*>(&lds_lo[r * kLdsStride + li * 8]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        if (li == 0) lds_pinv[r] = __builtin_ldexpf(1.0f, ex - 14);
      }
      __syncthreads();

      // ---------------------------------------------------------------- contract
      if (active) {
        f32x16 tmp[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) tmp[a][b] = f32x16{};
#pragma unroll 2
        for (int st = 0; st < kGroup / 16; ++st) {
          const int koff = st * 16 + khalf * 8;
          half8 A[2], Bh[2], Bl[2];
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            const int64_t t = tw + a * 32 + m32;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (t < T) v = *reinterpret_cast<const uint4*>(X + t * K + j * kGroup + koff);
            A[a] = __builtin_bit_cast(half8, v);
          }
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const int r = b * 32 + m32;
            Bh[b] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&lds_hi[r * kLdsStride + koff]));
            Bl[b] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(&lds_lo[r * kLdsStride + koff]));
          }
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              tmp[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[a], Bh[b], tmp[a][b], 0, 0, 0);
              tmp[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[a], Bl[b], tmp[a][b], 0, 0, 0);
            }
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const float pv = lds_pinv[b * 32 + m32];  // output column = lane % 32
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] += tmp[a][b][e] * pv;
        }
      }
      __syncthreads();
    }

    // ------------------------------------------------------------------ sum of squares
    double ss = 0.0;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) ss += (double)acc[a][b][e] * (double)acc[a][b][e];
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

// One block: err_i = sum of partials of grid point i in index order; first minimum.
__global__ void __launch_bounds__(256)
    k_search_reduce(const double* __restrict__ partials, int n_grid, int64_t n_partials,
                    const uint16_t* __restrict__ s_grid, int64_t K, uint16_t* __restrict__ s_best,
                    int32_t* __restrict__ best_idx, double* __restrict__ err) {
  __shared__ double lds_err[64];
  __shared__ int lds_best;
  const int tid = threadIdx.x;
  if (tid < n_grid) {
    double tot = 0.0;
    const double* p = partials + (int64_t)tid * n_partials;
    for (int64_t i = 0; i < n_partials; ++i) tot += p[i];
    lds_err[tid] = tot;
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
                             int64_t K, const uint16_t* s_grid, int n_grid, double* partials,
                             uint32_t* flags, hipStream_t stream) {
  dim3 grid((unsigned)((N + kRowTile - 1) / kRowTile), (unsigned)n_grid);
  if (T <= 4 * kTokPerWave)
    hipLaunchKernelGGL(k_search_err<4>, grid, dim3(256), 0, stream, X, T, W, N, K, s_grid,
                       partials, flags);
  else
    hipLaunchKernelGGL(k_search_err<8>, grid, dim3(512), 0, stream, X, T, W, N, K, s_grid,
                       partials, flags);
  return hipGetLastError();
}

hipError_t launch_search_reduce(const double* partials, int n_grid, int64_t n_partials,
                                const uint16_t* s_grid, int64_t K, uint16_t* s_best,
                                int32_t* best_idx, double* err, hipStream_t stream) {
  hipLaunchKernelGGL(k_search_reduce, dim3(1), dim3(256), 0, stream, partials, n_grid,
                     n_partials, s_grid, K, s_best, best_idx, err);
  return hipGetLastError();
}

}  // namespace awq
