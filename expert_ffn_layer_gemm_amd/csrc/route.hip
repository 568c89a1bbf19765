// Router: logits = x W_r^T (+ bias) on MFMA, then per-token top-k with
// renormalised softmax weights ("Lower latency and higher throughput with
// multi-node DeepSeek deployment", MoE Router section).
//
// Router GEMM.  x is bf16 (exact in fp32) and W_r is fp32.  Each fp32 weight is
// split exactly into three bf16 terms w = hi + mid + lo by truncation (hi the
// top 8 significant bits, mid the next 8, lo the remaining <= 8), and
// x W^T = x lo^T + x mid^T + x hi^T runs on the bf16 MFMA with fp32
// accumulation: three bf16 MFMAs per product, well above the fp32 MFMA rate,
// with products that are exact in fp32.
//
// The GEMM is LDS-pipelined like the expert GEMMs: a workgroup computes a
// 128-token x 128-expert tile over one slice of H, staging 64-wide K chunks
// of x (128 B per row) and W_r (256 B per row) with direct-to-LDS loads
// through a 3-stage ring.  H is split into KS slices so that the grid fills
// the chip; slice partial sums go to [KS][T][E] and the top-k kernel adds
// them in slice order (deterministic), adds the bias and writes the logits.
//
// Top-k.  One wave per token.  Each logit becomes a 64-bit key
// (order-preserving integer image of the fp32 value << 32 | ~expert), with
// -0 canonicalised to +0 first, so a wave-wide max picks the largest logit and
// the lower expert index among equal ones; k rounds of max + removal give the
// slots best first.  The result does not depend on reduction order.
#include <algorithm>

#include "dispatch.hpp"
#include "pipe.hpp"

namespace moe {

// ------------------------------------------------------------ router GEMM ----
constexpr int kRtTM = 128, kRtTE = 128, kRtNS = 3;
constexpr int kRtXB = kRtTM * 128;          // x bytes per stage (64 bf16 per row)
constexpr int kRtWB = kRtTE * 256;          // W bytes per stage (64 fp32 per row)
constexpr int kRtStage = kRtXB + kRtWB;     // 48 KB
constexpr int kRtWaves = 8;                 // 1 (tokens) x 8 (experts)
constexpr int kRtIPW = kRtStage / 1024 / kRtWaves;
static_assert(kRtIPW * kRtWaves * 1024 == kRtStage, "stage must split evenly over the waves");

// Exact three-way bf16 split of 8 fp32 weights (truncation at 8 and 16 bits).
__device__ __forceinline__ void split3(const u32x4_t w0, const u32x4_t w1, u32x4_t& hi, u32x4_t& mid,
                                       u32x4_t& lo) {
  uint32_t wb[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
  uint32_t mb[8], lb[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float r1 = __uint_as_float(wb[q]) - __uint_as_float(wb[q] & 0xFFFF0000u);
    const uint32_t r1b = __float_as_uint(r1);
    mb[q] = r1b;
    lb[q] = __float_as_uint(r1 - __uint_as_float(r1b & 0xFFFF0000u));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = (wb[2 * i] >> 16) | (wb[2 * i + 1] & 0xFFFF0000u);
    mid[i] = (mb[2 * i] >> 16) | (mb[2 * i + 1] & 0xFFFF0000u);
    lo[i] = (lb[2 * i] >> 16) | (lb[2 * i + 1] & 0xFFFF0000u);
  }
}

// Direct-to-LDS loads of K chunk c (relative to the slice) into its stage.
__device__ __forceinline__ void rt_dma(uint8_t* lds, int c, const uint8_t* const (&jb)[kRtIPW],
                                       const uint32_t (&soff)[kRtIPW],
                                       const uint32_t (&kstep)[kRtIPW], const bool (&jv)[kRtIPW],
                                       int wave) {
  uint8_t* st = lds + (c % kRtNS) * kRtStage;
#pragma unroll
  for (int j = 0; j < kRtIPW; ++j)
    if (jv[j]) dma16(jb[j] + (size_t)c * kstep[j] + soff[j], st + (wave * kRtIPW + j) * 1024);
}

// grid (ceil(T/128), ceil(E/128), KS), 512 threads.  parts[ks][t][e] = sum over
// the ks-th slice of H of x[t][h] * w[e][h].
__global__ __launch_bounds__(512) void k_router_tiled(const uint16_t* __restrict__ x,
                                                      const float* __restrict__ w,
                                                      float* __restrict__ parts, int T, int H,
                                                      int E, int KS, int32_t* zero_ctr) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (zero_ctr && threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) *zero_ctr = 0;
  // Waves 1 (tokens) x 8 (experts): each wave multiplies all 128 token rows
  // with its own 16 experts, so every W_r value of the stage is split into
  // its three bf16 terms by one wave only (with 2 x 4 waves each split was
  // done twice, and the split's vector ops outweighed the MFMAs).
  constexpr int WM = 1, WN = 8, MB = kRtTM / WM / 16, NB = kRtTE / WN / 16;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kRtNS * kRtStage];
  const int t0 = blockIdx.x * kRtTM, e0 = blockIdx.y * kRtTE, ks = blockIdx.z;
  const int nch = H / 64;
  const int c_begin = (int)((long long)nch * ks / KS);
  const int nk = (int)((long long)nch * (ks + 1) / KS) - c_begin;
  const int mrows = min(kRtTM, T - t0), ncols = min(kRtTE, E - e0);
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // DMA blocks: 0..15 hold x rows 8b..8b+7, 16..47 hold W rows 4(b-16)..+3.
  // Blocks wholly past T or E are not fetched; rows past them in a fetched
  // block re-read the last row.  Those rows are never stored.
  const uint8_t* jb[kRtIPW];
  uint32_t soff[kRtIPW], kstep[kRtIPW];
  bool jv[kRtIPW];
  int nv = 0;
#pragma unroll
  for (int j = 0; j < kRtIPW; ++j) {
    const int blk = wave * kRtIPW + j;
    if (blk < kRtXB / 1024) {
      const int row = blk * 8 + (lane >> 3);
      jv[j] = blk * 8 < mrows;
      jb[j] = reinterpret_cast<const uint8_t*>(x) + (size_t)t0 * H * 2 + (size_t)c_begin * 128;
      soff[j] = (uint32_t)min(row, mrows - 1) * (uint32_t)(H * 2) + (uint32_t)(slot8(row, lane & 7) * 16);
      kstep[j] = 128;
    } else {
      const int row = (blk - kRtXB / 1024) * 4 + (lane >> 4);
      jv[j] = (blk - kRtXB / 1024) * 4 < ncols;
      jb[j] = reinterpret_cast<const uint8_t*>(w) + (size_t)e0 * H * 4 + (size_t)c_begin * 256;
      soff[j] = (uint32_t)min(row, ncols - 1) * (uint32_t)(H * 4) + (uint32_t)(slot16(row, lane & 15) * 16);
      kstep[j] = 256;
    }
    nv += jv[j] ? 1 : 0;
  }

  const int rbase = wm * (kRtTM / WM), cbase = wn * (kRtTE / WN);
  const int nmb = max(0, min(MB, ceil_div(mrows - rbase, 16)));
  const int ncb = max(0, min(NB, ceil_div(ncols - cbase, 16)));

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int c = 0; c < kRtNS - 1; ++c)
    if (c < nk) rt_dma(lds, c, jb, soff, kstep, jv, wave);
  for (int kc = 0; kc < nk; ++kc) {
    wait_vmcnt_le<(kRtNS - 2) * kRtIPW>(min(kRtNS - 2, nk - 1 - kc) * nv);
    lds_barrier();
    if (kc + kRtNS - 1 < nk) rt_dma(lds, kc + kRtNS - 1, jb, soff, kstep, jv, wave);
    const uint8_t* Xs = lds + (kc % kRtNS) * kRtStage;
    const uint8_t* Ws = Xs + kRtXB;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4_t a[MB], bh[NB], bm[NB], bl[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int r = rbase + i * 16 + r16;
        a[i] = lds_read16(Xs + r * 128 + (slot8(r, s2 * 4 + (lane >> 4)) << 4));
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int e = cbase + j * 16 + r16;
        const int c0 = s2 * 8 + 2 * (lane >> 4);
        const u32x4_t w0 = lds_read16(Ws + e * 256 + (slot16(e, c0) << 4));
        const u32x4_t w1 = lds_read16(Ws + e * 256 + (slot16(e, c0 + 1) << 4));
        split3(w0, w1, bh[j], bm[j], bl[j]);
      }
      // Small terms first (lo, mid, hi into each accumulator in turn).  With
      // the three sweeps over all blocks of the 1 x 8 layout the compiler
      // spilled; an accumulator's three MFMAs issue back to back instead.
#pragma unroll
      for (int i = 0; i < MB; ++i)
        if (i < nmb) {
#pragma unroll
          for (int j = 0; j < NB; ++j)
            if (j < ncb) {
              acc[i][j] = mfma_bf16_16x16x32(a[i], bl[j], acc[i][j]);
              acc[i][j] = mfma_bf16_16x16x32(a[i], bm[j], acc[i][j]);
              acc[i][j] = mfma_bf16_16x16x32(a[i], bh[j], acc[i][j]);
            }
        }
    }
  }

  // Lane holds D[4*(lane/16) + q][lane%16] of each 16x16 block.
  float* out = parts + (size_t)ks * T * E;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + rbase + i * 16 + (lane >> 4) * 4 + q, e = e0 + cbase + j * 16 + r16;
        if (t < T && e < E) out[(size_t)t * E + e] = acc[i][j][q];
      }
#else
  (void)x; (void)w; (void)parts; (void)T; (void)H; (void)E; (void)KS; (void)zero_ctr;
#endif
}

// ------------------------------------------------------------------ top-k ----
// One wave per token (topk_token); NPL = logits per lane.
template <int NPL>
__global__ __launch_bounds__(256) void k_topk(const float* parts, int KS,
                                              const float* __restrict__ bias, float* logits_out,
                                              int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w, int T, int E, int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int e;
  float w;
  topk_token<NPL>(parts, KS, bias, logits_out, t, T, E, k, lane, e, w);
  if (lane < k) {
    topk_idx[(size_t)t * k + lane] = e;
    topk_w[(size_t)t * k + lane] = w;
  }
}

// ---------------------------------------------------------------- launchers ----
// Slices of H: about one workgroup per CU, each slice at least 4 K chunks
// (256 of H) long, so the top-k's sum over slice partials stays short (a
// 64-token decode batch with H = 7168 and 256 experts: 28 slices, not 112).
int router_splits(int T, int H, int E) {
  const long long tiles = (long long)ceil_div(T, kRtTM) * ceil_div(E, kRtTE);
  const long long want = (256 + tiles - 1) / tiles;    // one workgroup per CU
  return (int)std::max(1LL, std::min(want, (long long)(H / 256)));
}

size_t router_workspace_bytes(int T, int H, int E) {
  const int ks = router_splits(T, H, E);
  return ks > 1 ? (size_t)ks * T * E * sizeof(float) : 0;
}

hipError_t launch_router_gemm(const uint16_t* x, const float* w, float* parts, int T, int H, int E,
                              hipStream_t s, int32_t* zero_ctr) {
  const int ks = router_splits(T, H, E);
  dim3 grid(ceil_div(T, kRtTM), ceil_div(E, kRtTE), ks);
  MOE_LAUNCH("router_gemm", k_router_tiled, grid, dim3(64 * kRtWaves), 0, s, x, w, parts, T, H, E, ks,
             zero_ctr);
  return hipGetLastError();
}

hipError_t launch_topk(const float* parts, int KS, const float* bias, float* logits_out,
                       int32_t* idx, float* w, int T, int E, int k, hipStream_t s) {
  const dim3 grid(ceil_div(T, 4)), block(256);
  if (E <= 64) MOE_LAUNCH("topk", k_topk<1>, grid, block, 0, s, parts, KS, bias, logits_out, idx, w, T, E, k);
  else if (E <= 128) MOE_LAUNCH("topk", k_topk<2>, grid, block, 0, s, parts, KS, bias, logits_out, idx, w, T, E, k);
  else if (E <= 256) MOE_LAUNCH("topk", k_topk<4>, grid, block, 0, s, parts, KS, bias, logits_out, idx, w, T, E, k);
  else if (E <= 512) MOE_LAUNCH("topk", k_topk<8>, grid, block, 0, s, parts, KS, bias, logits_out, idx, w, T, E, k);
  else MOE_LAUNCH("topk", k_topk<16>, grid, block, 0, s, parts, KS, bias, logits_out, idx, w, T, E, k);
  return hipGetLastError();
}

}  // namespace moe
