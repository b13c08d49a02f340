// Quantize + pack (a3 + a4): one pass over W, HBM-bound. 4-bit codes (the format measured),
// 8-bit ones (same quantizer with 255 levels, two natural-order words per lane) or 3-bit
// ones (7 levels; a lane pair ORs its shares into one low-plane word, a lane quad into one
// high-plane word).
//
// "AWQ量化实战" §2.3: 128 consecutive input channels share one quantization step;
// "大模型量化部署实战：GPTQ与AWQ算法", "大模型量化的核心原理与位宽选择": a 4-bit integer with a
// scale and a zero point. Layout of the packed result: see include/awq.h.
//
// Mapping: a wave owns one (row, 512 input channels) unit: 4 groups of 128, 8 of 64 or 16
// of 32 ("AWQ量化实战" §2.3 also names 64 and 32). Lane l
// reads 8 consecutive weights (one 16-byte load) and writes the 32-bit word that packs
// their 8 codes (channel i of the word in nibble kNibbleOf[i]), so loads and stores are
// fully coalesced; the 16 lanes of a DPP row (8 lanes for 64-channel groups, a quad for
// 32) form one group and find its min / max with row-local DPP (symmetric mode: the larger
// magnitude sets the scale, zero fixed at 8). With clip indices (the
// weight-clipping search), group (n, j) shrinks its extremes by r = clip_ratio(idx, steps)
// before the quantizer sees them.
#include "common.hpp"
#include "launch.hpp"

namespace awq {

__global__ void __launch_bounds__(256) k_quant_pack(const uint16_t* __restrict__ W, int64_t N,
                                                    int64_t K, const uint16_t* __restrict__ s,
                                                    uint32_t* __restrict__ qweight,
                                                    uint16_t* __restrict__ scales,
                                                    uint8_t* __restrict__ zeros,
                                                    const uint8_t* __restrict__ clip_idx,
                                                    int clip_steps, int sym, int group,
                                                    int w_bit, uint32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int lgl = group == 128 ? 4 : group == 64 ? 3 : 2;
  const int gl = 1 << lgl;            // lanes per group (8 channels per lane)
  const int gpu = 64 >> lgl;          // groups per unit
  const int gi = lane >> lgl;         // group within the unit
  const int li = lane & (gl - 1);     // lane within the group
  const int64_t G = K / group;
  const int64_t chunks = (G + gpu - 1) / gpu;
  const bool w8 = w_bit == 8, w3 = w_bit == 3;
  const float qmax = (float)((1 << w_bit) - 1);
  const ScaleDiv sdiv = scale_divisor(qmax, sym);
  const int64_t words = K * w_bit / 32;  // packed words per row
  const int64_t zbytes = w8 ? G : (G + 1) / 2;  // 8-bit: one zero byte per group
  // unit u = (row n, chunk ch) = n * chunks + ch; the wave walks u = wave0, wave0 + nwaves,
  // ... with (n, ch) stepped incrementally (wave-uniform, no division in the loop)
  const int64_t wave0 = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)));
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t dn = nwaves / chunks, dc = nwaves - dn * chunks;
  int64_t n = wave0 / chunks, ch = wave0 - n * chunks;

  for (; n < N; n += dn, ch += dc) {
    if (ch >= chunks) {
      ch -= chunks;
      ++n;
      if (n >= N) break;
    }
    const int64_t j = ch * gpu + gi;  // group index
    const bool valid = j < G;
    const int64_t k0 = j * group + li * 8;

    uint4 wv = make_uint4(0, 0, 0, 0);
    uint4 sv = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);  // s = 1
    if (valid) {
      wv = *reinterpret_cast<const uint4*>(W + n * K + k0);
      if (s) sv = *reinterpret_cast<const uint4*>(s + k0);
    }
    const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
    const uint32_t sd[4] = {sv.x, sv.y, sv.z, sv.w};
    float w[8];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = h2f((uint16_t)(wd[i] & 0xFFFF)) * h2f((uint16_t)(sd[i] & 0xFFFF));
      w[2 * i + 1] = h2f((uint16_t)(wd[i] >> 16)) * h2f((uint16_t)(sd[i] >> 16));
    }
    float mn = w[0], mx = w[0];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bad |= !__builtin_isfinite(w[i]);
      mn = fminf(mn, w[i]);
      mx = fmaxf(mx, w[i]);
    }
    group_minmax(mn, mx, group);
    if (clip_idx && valid) {
      const float r = clip_ratio(clip_idx[n * G + j], clip_steps);
      mn = r * mn;
      mx = r * mx;
    }
    const GroupQ g = sym ? group_params_sym(mn, mx, qmax, sdiv) : group_params(mn, mx, qmax, sdiv);
    float qc[8];
    quant_codes(w, g, qc);

    // 3-bit: this lane's 8 channels are half of a low-plane word (16 channels) and a
    // quarter of a high-plane word (32 channels); the OR across lanes completes both
    uint32_t lo3 = 0, hi3 = 0;
    if (w3) {
      planes3(qc, lo3, hi3);
      lo3 <<= 8 * (lane & 1);
      hi3 <<= 4 * (lane & 3);
      lo3 |= (uint32_t)__shfl_xor((int)lo3, 1);
      hi3 |= (uint32_t)__shfl_xor((int)hi3, 1);
      hi3 |= (uint32_t)__shfl_xor((int)hi3, 2);
    }
    const uint32_t zi = (uint32_t)g.z;
    const uint32_t z_next = (uint32_t)__shfl_down((int)zi, gl);  // zero of group j + 1
    if (valid) {
      if (w8) {
        // two words, byte i of word h = code of channel k0 + 4 h + i
        uint2 wd8;
        wd8.x = pack_bytes4(qc[0], qc[1], qc[2], qc[3]);
        wd8.y = pack_bytes4(qc[4], qc[5], qc[6], qc[7]);
        reinterpret_cast<uint2*>(qweight)[(n * K + k0) >> 3] = wd8;
      } else if (w3) {
        // block k0 / 128 holds words 12 b .. 12 b + 11: 8 low-plane words, then 4 high
        const int64_t wb = n * words + (k0 >> 7) * 12;
        const int c0 = (int)(k0 & 127);
        if ((lane & 1) == 0) qweight[wb + (c0 >> 4)] = lo3;
        if ((lane & 3) == 0) qweight[wb + 8 + (c0 >> 5)] = hi3;
      } else {
        qweight[(n * K + k0) >> 3] = pack_codes8(qc);
      }
      if (li == 0) {
        scales[n * G + j] = g.sch;
        if (w8) {
          zeros[n * zbytes + j] = (uint8_t)zi;
        } else if ((j & 1) == 0) {
          const uint32_t hi = (j + 1 < G) ? z_next : 0u;
          zeros[n * zbytes + (j >> 1)] = (uint8_t)(zi | (hi << 4));
        }
        if (g.clamped && flags) atomicOr(flags, AWQ_FLAG_SCALE_CLAMPED);
      }
      if (bad && flags) atomicOr(flags, AWQ_FLAG_NONFINITE_INPUT);
    }
  }
}

hipError_t launch_quant_pack(const uint16_t* W, int64_t N, int64_t K, const uint16_t* s,
                             uint32_t* qweight, uint16_t* scales, uint8_t* zeros,
                             const uint8_t* clip_idx, int clip_steps, bool sym, int group,
                             int w_bit, uint32_t* flags, hipStream_t stream) {
  const int64_t units = N * ((K / 512 + (K % 512 ? 1 : 0)));
  const int64_t blocks = units / 4 + 1 < 16384 ? units / 4 + 1 : 16384;
  hipLaunchKernelGGL(k_quant_pack, dim3((unsigned)blocks), dim3(256), 0, stream, W, N, K, s,
                     qweight, scales, zeros, clip_idx, clip_steps, (int)sym, group, w_bit, flags);
  return hipGetLastError();
}

}  // namespace awq
