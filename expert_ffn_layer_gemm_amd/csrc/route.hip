// Router: logits = x W_r^T (+ bias) on MFMA, then per-token top-k with
// renormalised softmax weights ("Lower latency and higher throughput with
// multi-node DeepSeek deployment", MoE Router section).
//
// Router GEMM.  x is bf16 (exact in fp32) and W_r is fp32.  Each fp32 weight is
// split on load into three bf16 terms w = hi + mid + lo (each the
// round-to-nearest-even of the remaining residual, so the split is exact to
// about 2^-25 relative), and x W^T = x hi^T + x mid^T + x lo^T runs on the bf16
// MFMA with fp32 accumulation: three bf16 MFMAs per product, ~5x the fp32
// MFMA rate, with products that are exact in fp32.
//
// Top-k.  One wave per token.  Each logit becomes a 64-bit key
// (order-preserving integer image of the fp32 value << 32 | ~expert), with
// -0 canonicalised to +0 first, so a wave-wide max picks the largest logit and
// the lower expert index among equal ones; k rounds of max + removal give the
// slots best first.  The result does not depend on reduction order.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// ------------------------------------------------------------ router GEMM ----
// One wave computes a (16*MT tokens) x (16*NT experts) logits tile over its
// share of H; a workgroup of KSPLIT waves covers all of H and reduces the
// partial tiles through LDS in wave order (deterministic).
template <int MT, int NT, int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void k_router_gemm(
    const uint16_t* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ logits, int T, int H, int E) {
  constexpr int TM = 16 * MT, TN = 16 * NT;
  __shared__ float red[KSPLIT > 1 ? KSPLIT * TM * TN : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TM, e0 = blockIdx.y * TN;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;

  const int steps = H / 32;
  const int s_begin = (steps * wave) / KSPLIT, s_end = (steps * (wave + 1)) / KSPLIT;

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint16_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    int t = t0 + i * 16 + r16;
    xok[i] = t < T;
    xrow[i] = x + (size_t)(xok[i] ? t : 0) * H + kq;
  }
  const float* wrow[NT];
  bool wok[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int e = e0 + j * 16 + r16;
    wok[j] = e < E;
    wrow[j] = w + (size_t)(wok[j] ? e : 0) * H + kq;
  }

  for (int s = s_begin; s < s_end; ++s) {
    const int k = s * 32;
    u32x4_t a[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
      a[i] = xok[i] ? *reinterpret_cast<const u32x4_t*>(xrow[i] + k) : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      float wv[8];
      if (wok[j]) {
        const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(wrow[j] + k);
        const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(wrow[j] + k + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) { wv[q] = w0[q]; wv[4 + q] = w1[q]; }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) wv[q] = 0.f;
      }
      float hi[8], mid[8], lo[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        hi[q] = bf16_bits_to_f32(f32_to_bf16_bits(wv[q]));
        float r1 = wv[q] - hi[q];
        mid[q] = bf16_bits_to_f32(f32_to_bf16_bits(r1));
        lo[q] = r1 - mid[q];
      }
      const u32x4_t bh = pack_bf16x8(hi), bm = pack_bf16x8(mid), bl = pack_bf16x8(lo);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        acc[i][j] = mfma_bf16_16x16x32(a[i], bl, acc[i][j]);
        acc[i][j] = mfma_bf16_16x16x32(a[i], bm, acc[i][j]);
        acc[i][j] = mfma_bf16_16x16x32(a[i], bh, acc[i][j]);
      }
    }
  }

  // Lane holds D[4*(lane/16) + q][lane%16] of each 16x16 block.
  const int rbase = (lane >> 4) * 4;
  if constexpr (KSPLIT > 1) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          red[(wave * TM + i * 16 + rbase + q) * TN + j * 16 + r16] = acc[i][j][q];
    __syncthreads();
    for (int o = threadIdx.x; o < TM * TN; o += 64 * KSPLIT) {
      const int tt = o / TN, ee = o % TN;
      const int t = t0 + tt, e = e0 + ee;
      float v = red[tt * TN + ee];
      for (int w2 = 1; w2 < KSPLIT; ++w2) v += red[(w2 * TM + tt) * TN + ee];
      if (t < T && e < E) logits[(size_t)t * E + e] = bias ? v + bias[e] : v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = t0 + i * 16 + rbase + q, e = e0 + j * 16 + r16;
          if (t < T && e < E) {
            float v = acc[i][j][q];
            logits[(size_t)t * E + e] = bias ? v + bias[e] : v;
          }
        }
  }
}

// ------------------------------------------------------------------ top-k ----
__device__ __forceinline__ uint32_t ordered_key(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) == 0) b = 0;                 // -0 ties with +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_to_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

constexpr int kTopkMaxPerLane = 16;  // E <= 1024

__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits,
                                              int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w, int T, int E, int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  uint64_t key[kTopkMaxPerLane];
#pragma unroll
  for (int i = 0; i < kTopkMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? ((uint64_t)ordered_key(row[e]) << 32) | (uint32_t)(~e) : 0ull;
  }
  int my_e = 0;
  float my_v = 0.f, top_v = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < kTopkMaxPerLane; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      uint32_t lo = __shfl_xor((uint32_t)best, m), hi = __shfl_xor((uint32_t)(best >> 32), m);
      uint64_t o = ((uint64_t)hi << 32) | lo;
      best = o > best ? o : best;
    }
    // Remove the winner (keys are unique: the expert index is part of them).
#pragma unroll
    for (int i = 0; i < kTopkMaxPerLane; ++i)
      if (key[i] == best) key[i] = 0ull;
    const int e = (int)(~(uint32_t)best);
    const float v = key_to_value((uint32_t)(best >> 32));
    if (j == 0) top_v = v;
    if (lane == j) { my_e = e; my_v = v; }
  }
  float ex = lane < k ? expf(my_v - top_v) : 0.f;
  float sum = ex;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) sum += __shfl_xor(sum, m);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = my_e;
    topk_w[(size_t)t * k + lane] = ex / sum;
  }
}

// ---------------------------------------------------------------- launchers ----
hipError_t launch_router_gemm(const uint16_t* x, const float* w, const float* bias, float* logits,
                              int T, int H, int E, hipStream_t s) {
  if (T <= 256) {
    dim3 grid(ceil_div(T, 16), ceil_div(E, 16));
    MOE_LAUNCH("router_gemm_t16x16_k8", (k_router_gemm<1, 1, 8>), grid, dim3(512), 0, s, x, w, bias, logits, T, H, E);
  } else {
    dim3 grid(ceil_div(T, 32), ceil_div(E, 64));
    MOE_LAUNCH("router_gemm_t32x64_k2", (k_router_gemm<2, 4, 2>), grid, dim3(128), 0, s, x, w, bias, logits, T, H, E);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int32_t* idx, float* w, int T, int E, int k,
                       hipStream_t s) {
  MOE_LAUNCH("topk", k_topk, dim3(ceil_div(T, 4)), dim3(256), 0, s, logits, idx, w, T, E, k);
  return hipGetLastError();
}

}  // namespace moe
