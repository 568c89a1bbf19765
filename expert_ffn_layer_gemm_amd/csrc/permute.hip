// Dispatch: counting sort of (token, slot) pairs by expert and the row copy
// into unpadded expert-contiguous groups ("CuTeDSL at Perplexity", MoE
// Dispatch/Combine, local kernel: count per expert, a unique index per token
// inside its expert's list, then a copy launched on many more blocks to use
// the memory bandwidth).  The Ironwood page (section 4.2.1) makes the same
// point for its ragged gather: no padded per-expert tensor is built in HBM.
//
// Differences from the page's kernel, for gfx950 and for determinism:
//   - the unique index is the token-ascending rank, computed from LDS bit masks
//     (one bit per token of a 256-token tile per expert) with popcounts, instead
//     of atomically incremented counters, so dest / src_row / x_perm are
//     identical from run to run;
//   - an expert-parallel share keeps only the pairs routed to its experts
//     [e_first, e_first + L) (same page, tensor-parallel deployment: the local
//     dispatch selects the tokens assigned to this rank's experts); the others
//     get dest = -1, and the row copies stop at the share's row count;
//   - four launches: per-tile histograms (256-token tiles, LDS atomics), one
//     workgroup turning them into per-tile bases, counts and offsets (wave-level
//     prefix scan), a tile grid assigning ranks, and a wide grid gathering rows
//     (x_perm[r] = x[src_row[r]], 16-byte lanes), quantising each 128-channel
//     group to e4m3fn on the way for fp8 layers.
#include "dispatch.hpp"

namespace moe {


constexpr int kRankTile = 256;   // tokens per tile of the histogram and rank kernels
constexpr int kMaxTopK = 16;     // slots per token at most (the C ABI rejects k > 16)

// Routings per local expert inside each 256-token tile: tile_cnt[tile][e]
// (E = the share's experts, global ids e_first ..).
__global__ __launch_bounds__(kRankTile) void k_tile_hist(const int32_t* __restrict__ idx,
                                                         int32_t* __restrict__ tile_cnt, int T,
                                                         int E, int k, int e_first) {
  __shared__ int cnt[1024];
  const int tid = threadIdx.x;
  for (int i = tid; i < E; i += kRankTile) cnt[i] = 0;
  __syncthreads();
  const int t = blockIdx.x * kRankTile + tid;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j] - e_first;
      if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
    }
  __syncthreads();
  for (int i = tid; i < E; i += kRankTile) tile_cnt[(size_t)blockIdx.x * E + i] = cnt[i];
}

// One workgroup of 1024: turns tile_cnt into each tile's base row inside
// every expert's group (routings of that expert in earlier tiles, in place),
// then counts per group and their exclusive prefix sum.
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ tile_cnt, int n_tiles,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets, int T, int E,
                                               int n_shared) {
  __shared__ int cnt[2048];
  __shared__ int wave_sum[16];
  const int tid = threadIdx.x, G = E + n_shared;
  for (int i = tid; i < 2048; i += 1024) cnt[i] = 0;
  __syncthreads();
  if (tid < E) {
    // 16 tiles' counts loaded at a time before their bases are stored (a load
    // after a store to the same array would wait for it).
    int run = 0;
    for (int b0 = 0; b0 < n_tiles; b0 += 16) {
      int c[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) c[q] = b0 + q < n_tiles ? tile_cnt[(size_t)(b0 + q) * E + tid] : 0;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (b0 + q < n_tiles) {
          tile_cnt[(size_t)(b0 + q) * E + tid] = run;
          run += c[q];
        }
    }
    cnt[tid] = run;
  }
  if (tid == 0 && n_shared) cnt[E] = T;
  __syncthreads();
  scan_groups(cnt, G, counts, offsets, nullptr, wave_sum);
}

// Token-ascending rank of every (t, j) inside its expert's group: the tile's
// base (k_scan) plus the routings of earlier tokens of the tile, counted from
// an LDS bit mask per expert (one bit per token of the tile).  A thread's k
// expert ids are loaded once, and each expert's first row (offsets[e] + the
// tile's base) is staged in LDS beside the masks, so the per-slot lookups are
// LDS reads instead of k rounds of dependent global loads.
__global__ __launch_bounds__(kRankTile) void k_rank(const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ tile_base,
                                                    int32_t* __restrict__ dest,
                                                    int32_t* __restrict__ src_row, int T, int E,
                                                    int k, int n_shared, int e_first) {
  __shared__ uint32_t mask[1024 * (kRankTile / 32)];
  __shared__ int first_row[1024];
  const int tid = threadIdx.x;
  const int32_t* base = tile_base + (size_t)blockIdx.x * E;
  for (int i = tid; i < E; i += kRankTile) first_row[i] = offsets[i] + base[i];
  for (int i = tid; i < E * (kRankTile / 32); i += kRankTile) mask[i] = 0u;
  const int t = blockIdx.x * kRankTile + tid;
  const bool valid = t < T;
  int ev[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) ev[j] = valid && j < k ? idx[(size_t)t * k + j] - e_first : -1;
  __syncthreads();
  const int word = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if ((unsigned)ev[j] < (unsigned)E) atomicOr(&mask[ev[j] * (kRankTile / 32) + word], bit);
  __syncthreads();
  if (!valid) return;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k) break;
    const int e = ev[j];
    if ((unsigned)e >= (unsigned)E) {   // routed to another share's expert
      dest[(size_t)t * k + j] = -1;
      continue;
    }
    const uint32_t* m = mask + e * (kRankTile / 32);
    int rank = __popc(m[word] & (bit - 1u));
    for (int w = 0; w < word; ++w) rank += __popc(m[w]);
    const int d = first_row[e] + rank;
    dest[(size_t)t * k + j] = d;
    src_row[d] = t;
  }
  if (n_shared) src_row[offsets[E] + t] = t;
}

// x_perm[r] = x[src_row[r]] (bf16), 16 bytes per lane.
constexpr int kGatherRows = 4;
// Rows: R, or *n_rows when n_rows is non-null (a share's row count, read on
// the device).
__device__ __forceinline__ int gather_rows(int R, const int32_t* n_rows) {
  return n_rows ? min(R, *n_rows) : R;
}

__global__ __launch_bounds__(256) void k_gather_bf16(const int32_t* __restrict__ src_row,
                                                     const uint16_t* __restrict__ x,
                                                     uint16_t* __restrict__ x_perm, int R, int H,
                                                     const int32_t* __restrict__ n_rows) {
  const int chunks = H / 8;
  R = gather_rows(R, n_rows);
  for (int rr = 0; rr < kGatherRows; ++rr) {
    const int r = blockIdx.x * kGatherRows + rr;
    if (r >= R) return;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (size_t)src_row[r] * H);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(x_perm + (size_t)r * H);
    for (int c = threadIdx.x; c < chunks; c += 256) dst[c] = src[c];
  }
}

// x_perm[r] = e4m3 codes of x[src_row[r]] per 128-channel group, scale =
// amax/448 (quantize_row<false>), scales K-block-major: x_scale[b * ld + r].
__global__ __launch_bounds__(256) void k_gather_fp8(const int32_t* __restrict__ src_row,
                                                    const uint16_t* __restrict__ x,
                                                    uint8_t* __restrict__ x_perm,
                                                    float* __restrict__ x_scale, int R, int H, int ld,
                                                    const int32_t* __restrict__ n_rows) {
  R = gather_rows(R, n_rows);
  for (int rr = 0; rr < kGatherRows; ++rr) {
    const int r = blockIdx.x * kGatherRows + rr;
    if (r >= R) return;
    quantize_row<false>(x + (size_t)src_row[r] * H, x_perm + (size_t)r * H,
                        [&](int b, float sc, int li) { if (li == 0) x_scale[(size_t)b * ld + r] = sc; },
                        H, threadIdx.x, 256);
  }
}

// Per-token e4m3 codes of x (xq[t] = codes of x[t]) and their 128-channel
// scales, K-block-major per token: xs[b * T + t].
__global__ __launch_bounds__(256) void k_quantize_tokens_fp8(const uint16_t* __restrict__ x,
                                                             uint8_t* __restrict__ xq,
                                                             float* __restrict__ xs, int T, int H) {
  for (int tt = 0; tt < kGatherRows; ++tt) {
    const int t = blockIdx.x * kGatherRows + tt;
    if (t >= T) return;
    quantize_row<false>(x + (size_t)t * H, xq + (size_t)t * H,
                        [&](int b, float sc, int li) { if (li == 0) xs[(size_t)b * T + t] = sc; },
                        H, threadIdx.x, 256);
  }
}

// xs_perm[b * R + r] = xs_tok[b * T + src_row[r]] for the rows r < *n_rows:
// thread r of block (x, y) handles blocks 8 y .. 8 y + 7 of its row (stores
// of consecutive rows adjacent; the gathers stay inside one block's T scales).
constexpr int kScaleBlocksPerThread = 8;
__global__ __launch_bounds__(256) void k_permute_scales(const float* __restrict__ xs_tok,
                                                        const int32_t* __restrict__ src_row,
                                                        const int32_t* __restrict__ n_rows,
                                                        float* __restrict__ xs_perm, int T, int R,
                                                        int KB) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= min(R, *n_rows)) return;
  const int t = src_row[r];
  const int b0 = blockIdx.y * kScaleBlocksPerThread;
  const int b1 = min(KB, b0 + kScaleBlocksPerThread);
  for (int b = b0; b < b1; ++b) xs_perm[(size_t)b * R + r] = xs_tok[(size_t)b * T + t];
}

size_t permute_workspace_bytes(int T, int E) {
  return (size_t)ceil_div(T, kRankTile) * E * sizeof(int32_t);
}

// x_perm[r] = MXFP8 codes of x[src_row[r]] (x[r] when src_row is null):
// blocks of 32 channels (quantize_row<true>), E8M0 scales x_scale[r][b].
__global__ __launch_bounds__(256) void k_gather_mx(const int32_t* __restrict__ src_row,
                                                   const uint16_t* __restrict__ x,
                                                   uint8_t* __restrict__ x_perm,
                                                   uint8_t* __restrict__ x_scale, int R, int H,
                                                   const int32_t* __restrict__ n_rows) {
  R = gather_rows(R, n_rows);
  for (int rr = 0; rr < kGatherRows; ++rr) {
    const int r = blockIdx.x * kGatherRows + rr;
    if (r >= R) return;
    uint8_t* srow = x_scale + (size_t)r * (H / 32);
    quantize_row<true>(x + (size_t)(src_row ? src_row[r] : r) * H, x_perm + (size_t)r * H,
                       [&](int b, uint32_t e8, int li) { if (li == 0) srow[b] = (uint8_t)e8; },
                       H, threadIdx.x, 256);
  }
}

hipError_t launch_permute(const int32_t* topk_idx, const uint16_t* x, int32_t* counts,
                          int32_t* offsets, int32_t* dest, int32_t* src_row, void* x_perm,
                          void* x_perm_scale, int32_t* tile_cnt, int T, int H, int E, int k,
                          int n_shared, int e_first, bool share, bool fp8, bool mx,
                          hipStream_t s) {
  const int n_tiles = ceil_div(T, kRankTile);
  if (T > 0)
    MOE_LAUNCH_OR_RETURN("tile_hist", k_tile_hist, dim3(n_tiles), dim3(kRankTile), 0, s, topk_idx, tile_cnt,
               T, E, k, e_first);
  MOE_LAUNCH_OR_RETURN("scan", k_scan, dim3(1), dim3(1024), 0, s, tile_cnt, n_tiles, counts, offsets, T, E,
             n_shared);
  if (T == 0) return hipGetLastError();
  MOE_LAUNCH_OR_RETURN("rank", k_rank, dim3(n_tiles), dim3(kRankTile), 0, s, topk_idx, offsets, tile_cnt,
             dest, src_row, T, E, k, n_shared, e_first);
  if (x_perm == nullptr) return hipGetLastError();
  const int R = T * (k + n_shared);
  // A share has fewer rows than R; its count is offsets[G] on the device.
  const int32_t* n_rows = share ? offsets + E + n_shared : nullptr;
  const dim3 grid(ceil_div(R, kGatherRows));
  if (mx)
    MOE_LAUNCH("gather_mx", k_gather_mx, grid, dim3(256), 0, s, src_row, x,
               static_cast<uint8_t*>(x_perm), static_cast<uint8_t*>(x_perm_scale), R, H, n_rows);
  else if (fp8)
    MOE_LAUNCH("gather_fp8", k_gather_fp8, grid, dim3(256), 0, s, src_row, x,
               static_cast<uint8_t*>(x_perm), static_cast<float*>(x_perm_scale), R, H, R, n_rows);
  else
    MOE_LAUNCH("gather_bf16", k_gather_bf16, grid, dim3(256), 0, s, src_row, x,
               static_cast<uint16_t*>(x_perm), R, H, n_rows);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t* x, uint8_t* xq, void* xs, int T, int H, bool mx,
                                hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (mx)
    MOE_LAUNCH("quantize_rows_mx", k_gather_mx, dim3(ceil_div(T, kGatherRows)), dim3(256), 0, s,
               static_cast<const int32_t*>(nullptr), x, xq, static_cast<uint8_t*>(xs), T, H,
               static_cast<const int32_t*>(nullptr));
  else
    MOE_LAUNCH("quantize_rows_fp8", k_quantize_tokens_fp8, dim3(ceil_div(T, kGatherRows)), dim3(256),
               0, s, x, xq, static_cast<float*>(xs), T, H);
  return hipGetLastError();
}

hipError_t launch_permute_scales(const float* xs_tok, const int32_t* src_row, const int32_t* n_rows,
                                 float* xs_perm, int T, int R, int KB, hipStream_t s) {
  if (R == 0 || KB == 0) return hipSuccess;
  const dim3 grid(ceil_div(R, 256), ceil_div(KB, kScaleBlocksPerThread));
  MOE_LAUNCH("permute_scales", k_permute_scales, grid, dim3(256), 0, s, xs_tok, src_row, n_rows,
             xs_perm, T, R, KB);
  return hipGetLastError();
}

}  // namespace moe
