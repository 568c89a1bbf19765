// Combine: out[t] = bf16( sum_{j: dest[t,j] >= 0} w[t,j] * y_perm[dest[t,j]]
//                         (+ y_perm[shared_base + t]) )
// ("CuTeDSL at Perplexity", local combine: vectorised weighted accumulation in
// registers from the offsets the dispatch computed; an expert-parallel share
// sums only its local pairs, dest < 0 marking the others; the
// DeepSeek-deployment page's shared expert is added after the routed sum).
//
// A gather, not a scatter: each token reads its k rows, so no atomics are
// needed and the summation order (slot order, then the shared row) is fixed.
// Contraction is disabled so each term is one rounded product and one rounded
// add, which makes the result reproducible and checkable bit for bit.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

#pragma clang fp contract(off)

template <int TPB>
__global__ __launch_bounds__(TPB) void k_combine(const uint16_t* __restrict__ y_perm,
                                                 const int32_t* __restrict__ dest,
                                                 const float* __restrict__ topk_w,
                                                 const int32_t* __restrict__ shared_base,
                                                 uint16_t* __restrict__ out, int T, int H, int k,
                                                 int n_shared) {
  const int t = blockIdx.x;
  const int chunks = H / 8;
  const size_t srow = n_shared ? (size_t)*shared_base + t : 0;
  for (int c = threadIdx.x; c < chunks; c += TPB) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    // Slots in groups of 4: the group's row loads are issued before its
    // adds, which still run in slot order.  Each y_perm row is read once:
    // non-temporal loads (0.121 -> 0.105 ms on the DeepSeek-like layer; the
    // same hint on the GEMMs' weight loads made them 4-17 % slower).
    for (int j0 = 0; j0 < k; j0 += 4) {
      u32x4_t raw[4];
      float w[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u;
        const int row = j < k ? dest[(size_t)t * k + j] : -1;
        ok[u] = row >= 0;                      // row < 0: held by another share, adds nothing
        w[u] = ok[u] ? topk_w[(size_t)t * k + j] : 0.f;
        raw[u] = ok[u] ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(y_perm + (size_t)row * H) + c)
                       : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (ok[u]) {
          float v[8];
          unpack_bf16x8(raw[u], v);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] = acc[q] + w[u] * v[q];
        }
    }
    if (n_shared) {
      float v[8];
      unpack_bf16x8(__builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(y_perm + srow * H) + c), v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = acc[q] + v[q];
    }
    reinterpret_cast<u32x4_t*>(out + (size_t)t * H)[c] = pack_bf16x8(acc);
  }
}

hipError_t launch_combine(const uint16_t* y_perm, const int32_t* dest, const float* topk_w,
                          const int32_t* shared_base, uint16_t* out, int T, int H, int k,
                          int n_shared, hipStream_t s) {
  if (H / 8 <= 256)
    MOE_LAUNCH("combine", (k_combine<64>), dim3(T), dim3(64), 0, s, y_perm, dest, topk_w,
               shared_base, out, T, H, k, n_shared);
  else
    MOE_LAUNCH("combine", (k_combine<256>), dim3(T), dim3(256), 0, s, y_perm, dest, topk_w,
               shared_base, out, T, H, k, n_shared);
  return hipGetLastError();
}

}  // namespace moe
