// Definitions shared by the grouped-FFN kernels (ffn.hip: schedule and
// weight-streaming kernels; tiled.hip: LDS-pipelined tiled kernel).
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace moe {

// Groups of at most skinny_max_rows(T) rows go to the weight-streaming
// kernels, larger ones to the tiled kernels: 64 when no group can be larger
// (T <= 64, the decode case: no tiled launch at all), else 48 (groups of
// 49-64 rows measured faster in the tiled kernels: Qwen3.5-like Zipf routing
// 1.51 -> 1.43 ms per step; DeepSeek-like and decode unchanged).
constexpr int kSkinnyMax = 64;
__host__ __device__ constexpr int skinny_max_rows(int T) { return T <= kSkinnyMax ? kSkinnyMax : 48; }
// Rows per tile of the tiled kernels: 256 for bf16; 160 for fp8 (a
// DeepSeek-like routed group of ~128 rows stays in one tile, so its weights
// are streamed once) and for bf16 layers with small mean groups (bf_stream:
// their few tiled groups are weight-streaming-bound and run the fp8 kernel's
// 3-stage form in bf16); 128 for MXFP8 (its B-row scales need the LDS).
__host__ __device__ constexpr int tile_rows(bool fp8, bool mx, bool bf_stream = false) {
  return mx ? 128 : fp8 ? 160 : bf_stream ? 160 : 256;
}

// bf16 layers whose mean group (T k / E rows) is at most twice the streaming
// kernels' row limit: most groups stream, the tiled ones are few.
__host__ __device__ constexpr bool bf16_stream_tiles(int T, int k, int E, bool fp8) {
  return !fp8 && (long long)T * k / (E > 0 ? E : 1) <= 2LL * skinny_max_rows(T);
}

// Rows per tile of a group of m rows: the group is cut into ceil(m / bm)
// tiles of equal height (rounded up to 16), so that the tiles of one group,
// which stream the same weights, take the same time and stay in step on an
// XCD's L2.  The last tile may be shorter; none is empty.
__host__ __device__ inline int group_tile_rows(int m, int bm) {
  const int n = (m + bm - 1) / bm;
  return ((m + n - 1) / n + 15) / 16 * 16;
}

// Consecutive row tiles of a group are taken in bands of up to kTileBand;
// the tiled kernels walk a band column tile by column tile, row tile fastest,
// so workgroups that stream the same weight slice are adjacent in dispatch
// order (and start together on one XCD's L2), and those that share a row
// tile are at most kTileBand apart.
constexpr int kTileBand = 8;

// Groups of at most skinny_max_rows(T) rows go to the weight-streaming kernels
// as 16-row slices (one MFMA row block each), slices of a group adjacent.
constexpr int kSliceRows = 16;

struct Sched {
  int32_t* n_skinny;  // number of skinny slices
  int32_t* n_tiles;
  int32_t* skinny;    // [max_slices][4] (group, first row, group's first slice, its slices)
  int32_t* tiles;     // [max_tiles][4] (group, first row, band's first tile, band size)
  int G;
  int tile_rows;      // rows per tiled-kernel tile
  int skinny_max;     // groups of 1 .. skinny_max rows are sliced, larger ones tiled
};

// Work item and column tile of this workgroup.  Blocks are renumbered so each
// XCD (own L2) takes a contiguous run of (item, column tile) pairs; within a
// band of items (the slices of a group, or up to kTileBand row tiles) the
// order is column tile major, item fastest, so workgroups that stream the
// same weights are dispatched back to back on one L2.  `items` holds 4 ints
// per item, the last two being the band's first item and its size.  Returns
// false for blocks past the valid pairs.
__device__ __forceinline__ bool band_item(const int32_t* items, int n_items, int n_ntile, int& item,
                                          int& nt, int bid) {
  constexpr int kXcd = 8;
  const int n_valid = n_items * n_ntile;
  const int per_xcd = (n_valid + kXcd - 1) / kXcd;
  const int logical = (bid % kXcd) * per_xcd + bid / kXcd;
  if (bid >= kXcd * per_xcd || logical >= n_valid) return false;
  const int band_first = items[4 * (logical / n_ntile) + 2];
  const int band_size = items[4 * (logical / n_ntile) + 3];
  const int local = logical - band_first * n_ntile;
  item = band_first + local % band_size;
  nt = local / band_size;
  return true;
}

__device__ __forceinline__ bool band_item(const int32_t* items, int n_items, int n_ntile, int& item,
                                          int& nt) {
  return band_item(items, n_items, n_ntile, item, nt, blockIdx.x);
}

// Grid size for band_item over at most max_items items: the renumbering
// needs up to 7 blocks past the valid pairs.
inline long long band_grid(long long max_items, int n_ntile) {
  return (max_items * n_ntile + 15) / 8 * 8;
}

// silu(g) * u with the hardware exp2 and reciprocal (about 1 ulp each; the
// result is rounded to bf16 or quantised right after).  Large negative g
// gives exp = inf and a zero reciprocal, so silu -> -0 as it should.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

// Operands of one grouped GEMM launch.  Row-major, K contiguous:
// A [R, K] (x_perm or h), B0/B1 [G, N, K] (gate/up or down), out [R, N].
struct GemmArgs {
  Sched sc;
  const int32_t* offsets;
  const int32_t* a_rows;   // optional: A row of permuted row r is a_rows[r] (gather on load)
  const uint8_t* A;
  // fp8: fp32 activation scales stored K-block-major, the scale of A row a
  // for K block kb at A_scale[kb * s_ld + a], a = s_rows ? s_rows[r] : r for
  // permuted row r (the scales one K step of a row tile needs are then
  // adjacent); mxfp8: [R, K/32] E8M0 bytes of row a_rows ? a_rows[r] : r.
  const void* A_scale;
  const uint8_t* B0;
  const uint8_t* B1;       // up weights (dual) or unused
  const void* s_B0;        // fp8: [G, N/128, K/128] fp32; mxfp8: [G, N, K/32] E8M0 bytes
  const void* s_B1;
  uint8_t* out;            // bf16 or e4m3 codes
  void* out_scale;         // dual: fp8 [N/128][R] fp32 (K-block-major for the next GEMM);
                           // mxfp8 [R, N/32] E8M0 bytes
  int K, N, n_ntile;
  // Split-K (bf16 streaming kernel): ksplit workgroups per (slice, column
  // tile) each sum K / ksplit of K into part [ksplit][R][dual ? 2N : N] fp32;
  // a reduce kernel adds the slices in order and applies the epilogue.
  int ksplit = 1;
  int R = 0;               // rows of the permuted matrix: stride of out_scale and of part
  const int32_t* s_rows = nullptr;
  int s_ld = 0;
  float* part = nullptr;
};

// Tiled kernel launches: bf16 (tiled.hip), fp8 and MXFP8 (tiled8.hip).
hipError_t launch_tiled(const char* name, bool dual, long long blocks, const GemmArgs& a, hipStream_t s);
hipError_t launch_tiled8_bf16(const char* name, bool dual, long long blocks, const GemmArgs& a,
                              hipStream_t s);
hipError_t launch_tiled8(const char* name, bool mx, bool dual, long long blocks, const GemmArgs& a,
                         hipStream_t s);

}  // namespace moe
