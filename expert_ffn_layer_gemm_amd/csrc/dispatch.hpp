// Device-side building blocks of routing and dispatch, shared by the
// separate kernels (route.hip top-k, permute.hip scan, ffn.hip plan) and the
// single-workgroup routing + dispatch kernel for small batches (small.hip).
#pragma once

#include "ffn.hpp"

namespace moe {

// Order-preserving integer image of an fp32 value; -0 canonicalised to +0.
__device__ __forceinline__ uint32_t ordered_key(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) == 0) b = 0;                 // -0 ties with +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_to_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Top-k of token t by one wave (lane = lane index); NPL = logits per lane
// (E <= 64 NPL).  The logit of expert e is parts[0][t][e] + ... +
// parts[KS-1][t][e] (+ bias[e]), summed in that order; logits_out (may alias
// parts when KS == 1) receives it.  Each logit becomes a 64-bit key (ordered
// value << 32 | ~expert), so a wave max picks the largest logit and the lower
// expert among equal ones; k rounds of max + removal give the slots best
// first.  Lane j < k returns slot j's expert and its renormalised weight
// exp(l_j - l_0) / sum.
// One 64-bit key per lane through a DPP permutation (both halves).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)v, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(v >> 32), (int)(uint32_t)(v >> 32),
                                                            CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum of a 64-bit key over the 64 lanes of a wave, in every lane (all
// lanes active): DPP quad swaps and row mirrors within each row of 16, then
// gfx950's row swaps (v_permlane16_swap / v_permlane32_swap return both
// members of the lane ^ 16 and lane ^ 32 pairs).  Register moves instead of
// six LDS-crossbar round trips per reduction.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0xB1>(v));                 // quad_perm [1,0,3,2]: lane ^ 1
  v = max_u64(v, dpp_u64<0x4E>(v));                 // quad_perm [2,3,0,1]: lane ^ 2
  v = max_u64(v, dpp_u64<0x141>(v));                // row_half_mirror: the other quad of 8
  v = max_u64(v, dpp_u64<0x140>(v));                // row_mirror: the other half of 16
  {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    v = max_u64(((uint64_t)h[0] << 32) | l[0], ((uint64_t)h[1] << 32) | l[1]);
  }
  {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    v = max_u64(((uint64_t)h[0] << 32) | l[0], ((uint64_t)h[1] << 32) | l[1]);
  }
  return v;
}

template <int NPL>
__device__ __forceinline__ void topk_token(const float* parts, int KS, const float* bias,
                                           float* logits_out, int t, int T, int E, int k,
                                           int lane, int& out_e, float& out_w) {
  const size_t plane = (size_t)T * E;
  const size_t row = (size_t)t * E;
  // Every lane's sums first, the logit stores after them: logits_out may alias
  // parts, so a store between two lanes' worth of loads would hold the later
  // loads back until it is done.  The adds stay in plane order.
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = parts[row + min(lane + 64 * i, E - 1)];
#pragma unroll 4
  for (int s2 = 1; s2 < KS; ++s2) {
    float p[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) p[i] = parts[s2 * plane + row + min(lane + 64 * i, E - 1)];
#pragma unroll
    for (int i = 0; i < NPL; ++i) v[i] += p[i];
  }
  uint64_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    if (bias) v[i] += bias[min(e, E - 1)];
    key[i] = e < E ? ((uint64_t)ordered_key(v[i]) << 32) | (uint32_t)(~e) : 0ull;
  }
  if (logits_out) {
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + 64 * i < E) logits_out[row + lane + 64 * i] = v[i];
  }
  int my_e = 0;
  float my_v = 0.f, top_v = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < NPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    // Remove the winner (keys are unique: the expert index is part of them).
#pragma unroll
    for (int i = 0; i < NPL; ++i) key[i] = key[i] == best ? 0ull : key[i];
    const int e = (int)(~(uint32_t)best);
    const float v = key_to_value((uint32_t)(best >> 32));
    if (j == 0) top_v = v;
    if (lane == j) { my_e = e; my_v = v; }
  }
  float ex = lane < k ? expf(my_v - top_v) : 0.f;
  float sum = ex;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) sum += __shfl_xor(sum, m);
  out_e = my_e;
  out_w = ex / sum;
}

// Exclusive position of a + b among all threads of a 1024-thread workgroup
// (thread order, a before b) and the total.  wave_sum: 16 ints of LDS.
__device__ __forceinline__ void block_scan_pair(int a, int b, int* wave_sum, int& excl_a,
                                                int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = a + b;
  int incl = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) before += wave_sum[w];
    tot += wave_sum[w];
  }
  excl_a = before + incl - s;
  total = tot;
  __syncthreads();
}

// counts[g] = cnt[g] and offsets = their exclusive prefix sum, for G <= 2047
// groups; cnt is 2048 ints (zero past G); 1024-thread workgroup.  The offsets
// are also left in offs_lds (G + 1 ints) when it is non-null.
__device__ __forceinline__ void put_group(int g, int G, int c, int o, int32_t* counts,
                                          int32_t* offsets, int* offs_lds) {
  if (g < G) counts[g] = c;
  if (g <= G) {
    offsets[g] = o;
    if (offs_lds) offs_lds[g] = o;
  }
}

__device__ __forceinline__ void scan_groups(const int* cnt, int G, int32_t* counts,
                                            int32_t* offsets, int* offs_lds, int* wave_sum) {
  const int tid = threadIdx.x;
  const int a = cnt[2 * tid], b = cnt[2 * tid + 1];
  int excl, total;
  block_scan_pair(a, b, wave_sum, excl, total);
  (void)total;
  put_group(2 * tid, G, a, excl, counts, offsets, offs_lds);
  put_group(2 * tid + 1, G, b, excl + a, counts, offsets, offs_lds);
}

// Work lists of the grouped FFN from the group offsets (1024-thread
// workgroup, G <= 2048): groups of 1 .. sc.skinny_max rows as 16-row slices,
// larger groups as equal-height row tiles in bands of kTileBand.
__device__ __forceinline__ void plan_groups(const int32_t* offsets, const Sched& sc,
                                            int* wave_sum) {
  const int tid = threadIdx.x, G = sc.G;
  int m[2], sl[2], nt[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int g = 2 * tid + q;
    m[q] = g < G ? offsets[g + 1] - offsets[g] : 0;
    sl[q] = m[q] > 0 && m[q] <= sc.skinny_max ? ceil_div(m[q], kSliceRows) : 0;
    nt[q] = m[q] > sc.skinny_max ? ceil_div(m[q], group_tile_rows(m[q], sc.tile_rows)) : 0;
  }
  int sl_pos, sl_total;
  block_scan_pair(sl[0], sl[1], wave_sum, sl_pos, sl_total);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int first = sl_pos;
    for (int i = 0; i < sl[q]; ++i) {
      sc.skinny[4 * sl_pos] = 2 * tid + q;
      sc.skinny[4 * sl_pos + 1] = i * kSliceRows;
      sc.skinny[4 * sl_pos + 2] = first;
      sc.skinny[4 * sl_pos + 3] = sl[q];
      ++sl_pos;
    }
  }
  if (tid == 0) *sc.n_skinny = sl_total;
  int nt_pos, nt_total;
  block_scan_pair(nt[0], nt[1], wave_sum, nt_pos, nt_total);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int g = 2 * tid + q;
    const int first = nt_pos;
    for (int i = 0; i < nt[q]; ++i) {
      const int band = i / kTileBand;
      sc.tiles[4 * nt_pos] = g;
      sc.tiles[4 * nt_pos + 1] = i * group_tile_rows(m[q], sc.tile_rows);
      sc.tiles[4 * nt_pos + 2] = first + band * kTileBand;
      sc.tiles[4 * nt_pos + 3] = min(kTileBand, nt[q] - band * kTileBand);
      ++nt_pos;
    }
  }
  if (tid == 0) *sc.n_tiles = nt_total;
}

// Quantisation of one bf16 row of H channels (src) into e4m3 codes (dst) by
// the threads tid = 0 .. nthreads-1 (nthreads a multiple of 64, consecutive
// lanes of whole waves), 8 channels per thread and step.
//   fp8 (MX = false): per 128-channel group, scale = amax / 448 (1 for an
//     all-zero group); 16 lanes cover a group, the group maximum is a 16-lane
//     DPP reduction that leaves it in all 16;
//   MXFP8 (MX = true): per 32-channel block, E8M0 = max(biased exponent of
//     amax - 8, 0), codes of v * 2^-(E8M0 - 127); 4 lanes cover a block.
// Codes round to nearest even after clamping to +-448.  Every lane of a group
// calls put_scale(group, scale, its lane within the group) (fp8: float scale,
// lanes 0..15; MXFP8: E8M0 byte, lanes 0..3), so the caller decides where, and
// by how many lanes, the scale is stored.
template <bool MX, typename PutScale>
__device__ __forceinline__ void quantize_row(const uint16_t* __restrict__ src, uint8_t* __restrict__ dst,
                                             PutScale put_scale, int H, int tid, int nthreads) {
  const int chunks = H / 8;
  const u32x4_t* s8 = reinterpret_cast<const u32x4_t*>(src);
  for (int c = tid; c < chunks; c += nthreads) {
    float v[8];
    unpack_bf16x8(s8[c], v);
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
    uint32_t lo = 0, hi = 0;
    if constexpr (MX) {
      amax = wave_max_xor(amax, 4);
      const uint32_t e8 = mx_e8m0(amax);
      const float inv = mx_inv_scale(e8);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t code = f32_to_e4m3(fminf(fmaxf(v[q] * inv, -448.f), 448.f));
        if (q < 4) lo |= code << (8 * q); else hi |= code << (8 * (q - 4));
      }
      put_scale(c / 4, e8, c & 3);
    } else {
      amax = row16_max(amax);
      const float scale = amax == 0.f ? 1.f : amax / 448.f;
      float d[8];
      if (scale >= kDivFastMin) {         // eight quotients from one reciprocal (bit-identical)
        const float y = 1.f / scale;
#pragma unroll
        for (int q = 0; q < 8; ++q) d[q] = div_rn_by(v[q], scale, y);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) d[q] = v[q] / scale;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float qv = fminf(fmaxf(d[q], -448.f), 448.f);
        const uint32_t code = f32_to_e4m3(qv);
        if (q < 4) lo |= code << (8 * q); else hi |= code << (8 * (q - 4));
      }
      put_scale(c / 16, scale, c & 15);
    }
    *reinterpret_cast<uint2*>(dst + c * 8) = make_uint2(lo, hi);
  }
}

}  // namespace moe
