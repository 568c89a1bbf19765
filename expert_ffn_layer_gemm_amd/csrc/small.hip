// Routing and dispatch of a small batch (T <= 256 tokens, the decode case)
// in ONE launch after the router GEMM: top-k with renormalised weights, the
// expert histogram, counts and offsets, the token-ascending ranks (dest,
// src_row) and the grouped-FFN work lists.  "CuTeDSL at Perplexity" (Grid
// sync; MoE Dispatch/Combine) fuses the decode dispatch into one kernel with a
// grid-wide barrier; here no workgroup ever waits for another:
//   - every workgroup computes the top-k of 4 tokens, one wave per token,
//     summing the router's slice partials in slice order (8-bit layers: its
//     other waves quantise those tokens' rows of x meanwhile);
//   - it publishes its routing (device-scope fence) and takes a ticket from a
//     counter; the workgroup that draws the last ticket has every token's
//     routing and runs the dispatch of the whole batch on its own (with
//     T <= 256 it fits one workgroup), the others exit;
//   - the counter is zeroed by the router GEMM launched just before on the
//     same stream, so each call starts from zero, also in a HIP-graph replay.
// The result does not depend on which workgroup finishes last.
#include "dispatch.hpp"

namespace moe {

constexpr int kSmallT = kSmallBatch;   // tokens: one 256-token rank tile
constexpr int kMaxK = 16;
// Tokens per workgroup in the top-k phase (one wave each; the other waves
// of the 1024-thread workgroup only take part in the dispatch): few tokens
// per workgroup spread the reduction of the router's slice partials over as
// many CUs as the separate top-k kernel used.
constexpr int kTokPerWg = 4;

// Histogram, counts and offsets, ranks and work lists of T <= 256 tokens from
// their routing topk_idx [T, k] (global memory), by one 1024-thread workgroup.
__device__ __forceinline__ void dispatch_small(const int32_t* topk_idx, int32_t* counts,
                                               int32_t* offsets, int32_t* dest, int32_t* src_row,
                                               const Sched& sc, int T, int E, int k, int n_shared,
                                               int e_first) {
  __shared__ int sidx[kSmallT * kMaxK];                 // expert of every (t, j)
  __shared__ int cnt[2048];
  __shared__ int offs[2049];
  __shared__ uint32_t mask[1024 * (kSmallT / 32)];      // one bit per token, per expert
  __shared__ int wave_sum[16];
  const int tid = threadIdx.x;
  const int G = E + n_shared;

  // 1. the routing of the batch into LDS.
  for (int i = tid; i < T * k; i += 1024) sidx[i] = topk_idx[i];
  for (int i = tid; i < 2048; i += 1024) cnt[i] = 0;
  for (int i = tid; i < E * (kSmallT / 32); i += 1024) mask[i] = 0u;
  __syncthreads();

  // 2. histogram and per-expert token masks (thread t = token t) of the
  //    experts held here (E of them, global ids e_first ..).
  const int word = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  if (tid < T)
    for (int j = 0; j < k; ++j) {
      const int e = sidx[tid * k + j] - e_first;
      if ((unsigned)e >= (unsigned)E) continue;
      atomicAdd(&cnt[e], 1);
      atomicOr(&mask[e * (kSmallT / 32) + word], bit);
    }
  __syncthreads();
  if (tid == 0 && n_shared) cnt[E] = T;
  __syncthreads();

  // 3. counts and offsets (also kept in LDS).
  scan_groups(cnt, G, counts, offsets, offs, wave_sum);
  __syncthreads();

  // 4. token-ascending ranks inside each group.
  if (tid < T) {
    for (int j = 0; j < k; ++j) {
      const int e = sidx[tid * k + j] - e_first;
      if ((unsigned)e >= (unsigned)E) {   // routed to another share's expert
        dest[tid * k + j] = -1;
        continue;
      }
      const uint32_t* m = mask + e * (kSmallT / 32);
      int rank = __popc(m[word] & (bit - 1u));
      for (int w = 0; w < word; ++w) rank += __popc(m[w]);
      const int d = offs[e] + rank;
      dest[tid * k + j] = d;
      src_row[d] = tid;
    }
    if (n_shared) src_row[offs[E] + tid] = tid;
  }

  // 5. grouped-FFN work lists from the offsets.
  plan_groups(offs, sc, wave_sum);
}

// E_all: experts the router scores; E: the routed experts held here.
// QM: 0 bf16 layer; 1 fp8 and 2 MXFP8 layers, whose GEMMs gather rows of x
// quantised per token: the workgroup's other waves quantise its tokens' rows
// of x into xq / xs meanwhile (fp8 scales K-block-major, xs[b * T + t];
// MXFP8 per token, xs[t * H/32 + b]).
template <int NPL, int QM>
__global__ __launch_bounds__(1024) void k_route_dispatch_small(
    const float* parts, int KS, const float* __restrict__ bias, int32_t* topk_idx, float* topk_w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ dest,
    int32_t* __restrict__ src_row, Sched sc, int T, int E_all, int k, int E, int n_shared,
    int e_first, int32_t* tickets, const uint16_t* __restrict__ x, uint8_t* __restrict__ xq,
    void* __restrict__ xs, int H) {
  __shared__ int is_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kTokPerWg + wave;
  if (wave < kTokPerWg) {
    if (t < T) {
      int e;
      float w;
      topk_token<NPL>(parts, KS, bias, nullptr, t, T, E_all, k, lane, e, w);
      if (lane < k) {
        topk_idx[(size_t)t * k + lane] = e;
        topk_w[(size_t)t * k + lane] = w;
      }
    }
  } else if constexpr (QM != 0) {
    const int qt = threadIdx.x - 64 * kTokPerWg, nq = 1024 - 64 * kTokPerWg;
    for (int j = 0; j < kTokPerWg; ++j) {
      const int tt = blockIdx.x * kTokPerWg + j;
      if (tt >= T) break;
      if constexpr (QM == 2) {
        uint8_t* srow = static_cast<uint8_t*>(xs) + (size_t)tt * (H / 32);
        quantize_row<true>(x + (size_t)tt * H, xq + (size_t)tt * H,
                           [&](int b, uint32_t e8, int li) { if (li == 0) srow[b] = (uint8_t)e8; },
                           H, qt, nq);
      } else {
        float* xsf = static_cast<float*>(xs);
        quantize_row<false>(x + (size_t)tt * H, xq + (size_t)tt * H,
                            [&](int b, float sc, int li) { if (li == 0) xsf[(size_t)b * T + tt] = sc; },
                            H, qt, nq);
      }
    }
  }
  // Publish this workgroup's routing, then draw a ticket (vector atomic).
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = atomicAdd(tickets, 1) == (int)gridDim.x - 1;
  __syncthreads();
  if (!is_last) return;
  __threadfence();                     // every other workgroup's routing is visible
  dispatch_small(topk_idx, counts, offsets, dest, src_row, sc, T, E, k, n_shared, e_first);
}

// Requires T <= kSmallBatch, k <= 16 and E_all <= 1024; tickets zeroed by the
// router GEMM launched before on stream s.
template <int NPL>
static void launch_rds(int qm, dim3 grid, const float* parts, int KS, const float* bias,
                       int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* dest,
                       int32_t* src_row, const Sched& sc, int T, int E_all, int k, int E,
                       int n_shared, int e_first, int32_t* tickets, const uint16_t* x, uint8_t* xq,
                       void* xs, int H, hipStream_t s) {
#define MOE_RDS(QM)                                                                                 \
  MOE_LAUNCH("route_dispatch_small", (k_route_dispatch_small<NPL, QM>), grid, dim3(1024), 0, s,     \
             parts, KS, bias, idx, w, counts, offsets, dest, src_row, sc, T, E_all, k, E, n_shared, \
             e_first, tickets, x, xq, xs, H)
  if (qm == 2) MOE_RDS(2);
  else if (qm == 1) MOE_RDS(1);
  else MOE_RDS(0);
#undef MOE_RDS
}

hipError_t launch_route_dispatch_small(const float* parts, int KS, const float* bias, int32_t* idx,
                                       float* w, int32_t* counts, int32_t* offsets, int32_t* dest,
                                       int32_t* src_row, const Sched& sc, int T, int E_all, int k,
                                       int E, int n_shared, int e_first, int32_t* tickets,
                                       const uint16_t* x, uint8_t* xq, void* xs, int H, bool fp8,
                                       bool mx, hipStream_t s) {
  const dim3 grid(ceil_div(T, kTokPerWg));
  const int qm = mx ? 2 : fp8 ? 1 : 0;
  if (E_all <= 64) launch_rds<1>(qm, grid, parts, KS, bias, idx, w, counts, offsets, dest, src_row, sc, T, E_all, k, E, n_shared, e_first, tickets, x, xq, xs, H, s);
  else if (E_all <= 128) launch_rds<2>(qm, grid, parts, KS, bias, idx, w, counts, offsets, dest, src_row, sc, T, E_all, k, E, n_shared, e_first, tickets, x, xq, xs, H, s);
  else if (E_all <= 256) launch_rds<4>(qm, grid, parts, KS, bias, idx, w, counts, offsets, dest, src_row, sc, T, E_all, k, E, n_shared, e_first, tickets, x, xq, xs, H, s);
  else if (E_all <= 512) launch_rds<8>(qm, grid, parts, KS, bias, idx, w, counts, offsets, dest, src_row, sc, T, E_all, k, E, n_shared, e_first, tickets, x, xq, xs, H, s);
  else launch_rds<16>(qm, grid, parts, KS, bias, idx, w, counts, offsets, dest, src_row, sc, T, E_all, k, E, n_shared, e_first, tickets, x, xq, xs, H, s);
  return hipGetLastError();
}

}  // namespace moe
