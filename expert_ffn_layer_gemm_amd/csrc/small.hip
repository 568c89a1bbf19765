// Dispatch of a small batch (T <= 256 tokens, the decode case) in ONE
// workgroup and one launch: the expert histogram, counts and offsets, the
// token-ascending ranks (dest, src_row) and the grouped-FFN work lists, from
// the top-k kernel's routing.  The same steps as the separate permute / plan
// kernels ("CuTeDSL at Perplexity", MoE Dispatch/Combine: the decode path
// fuses the dispatch steps into one launch); with T <= 256 all of them fit one
// workgroup, so no grid barrier is needed.  (The top-k stays a kernel of its
// own: it sums the router's slice partials, which wants many workgroups.)
#include "dispatch.hpp"

namespace moe {

constexpr int kSmallT = kSmallBatch;   // tokens: one 256-token rank tile
constexpr int kMaxK = 16;

__global__ __launch_bounds__(1024) void k_dispatch_small(
    const int32_t* __restrict__ topk_idx, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ dest, int32_t* __restrict__ src_row,
    Sched sc, int T, int E, int k, int n_shared, int e_first) {
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

// Requires T <= kSmallBatch, k <= 16 and E <= 1024.
hipError_t launch_dispatch_small(const int32_t* idx, int32_t* counts, int32_t* offsets,
                                 int32_t* dest, int32_t* src_row, const Sched& sc, int T, int E,
                                 int k, int n_shared, int e_first, hipStream_t s) {
  MOE_LAUNCH("dispatch_small", k_dispatch_small, dim3(1), dim3(1024), 0, s, idx, counts, offsets,
             dest, src_row, sc, T, E, k, n_shared, e_first);
  return hipGetLastError();
}

}  // namespace moe
