// Host-side launchers of the MoE kernels (one per kernel family).  Each one
// enqueues on the given stream and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// prof.hip: measurement hook (events around launches when enabled).
void prof_call_begin();
void prof_before(const char* name, hipStream_t s);
void prof_after(hipStream_t s);
// Per-launch timing is on: run concurrent kernel chains one after the other.
bool prof_serial();

// Launch a kernel, bracketed by the measurement hook.
#define MOE_LAUNCH(name, kernel, grid, block, shmem, stream, ...)          \
  do {                                                                   \
    ::moe::prof_before(name, stream);                                    \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__); \
    ::moe::prof_after(stream);                                           \
  } while (0)

// MOE_LAUNCH, then return the launch error (if any) from the enclosing
// launcher before anything else is enqueued.
#define MOE_LAUNCH_OR_RETURN(...)                                          \
  do {                                                                   \
    MOE_LAUNCH(__VA_ARGS__);                                             \
    if (hipError_t e_ = hipGetLastError(); e_ != hipSuccess) return e_;  \
  } while (0)

// route.hip
// The router GEMM splits H into router_splits() slices and writes their
// partial sums to parts [KS][T][E] (KS == 1: parts may be the logits buffer);
// router_workspace_bytes() is the size of parts when KS > 1, else 0.
int router_splits(int T, int H, int E);
size_t router_workspace_bytes(int T, int H, int E);
// zero_ctr (optional): a counter the kernel sets to 0 (read by the next
// launch on the stream, the small-batch routing + dispatch kernel).
hipError_t launch_router_gemm(const uint16_t* x, const float* w, float* parts, int T, int H, int E,
                              hipStream_t s, int32_t* zero_ctr = nullptr);
// Logits = sum of the KS partial planes in order (+ bias), written to
// logits_out when non-null (may alias parts when KS == 1), then top-k.
hipError_t launch_topk(const float* parts, int KS, const float* bias, float* logits_out,
                       int32_t* idx, float* w, int T, int E, int k, hipStream_t s);

// permute.hip
// E = the routed experts held here (global ids e_first ..); share: an
// expert-parallel share (pairs routed elsewhere get dest = -1, rows < R).
// tile_cnt: permute_workspace_bytes(T, E) of device scratch (per-tile counts).
// x_perm == nullptr skips the row copy (the GEMMs then gather rows through src_row).
size_t permute_workspace_bytes(int T, int E);
hipError_t launch_permute(const int32_t* topk_idx, const uint16_t* x, int32_t* counts,
                          int32_t* offsets, int32_t* dest, int32_t* src_row, void* x_perm,
                          void* x_perm_scale, int32_t* tile_cnt, int T, int H, int E, int k,
                          int n_shared, int e_first, bool share, bool fp8, bool mx,
                          hipStream_t s);
// Per-token quantisation of x (fp8: 128-channel groups, scales K-block-major
// per token, xs[b * T + t]; mxfp8: blocks of 32, xs[t * H/32 + b]): the rows
// the 8-bit GEMMs gather through src_row.
hipError_t launch_quantize_rows(const uint16_t* x, uint8_t* xq, void* xs, int T, int H, bool mx,
                                hipStream_t s);
// fp8 activation scales of the permuted rows from the per-token ones:
// xs_perm[b * R + r] = xs_tok[b * T + src_row[r]] for r < *n_rows (K-block-
// major both, so the GEMMs read one K block's scales of consecutive rows
// adjacent).
hipError_t launch_permute_scales(const float* xs_tok, const int32_t* src_row, const int32_t* n_rows,
                                 float* xs_perm, int T, int R, int KB, hipStream_t s);

// combine.hip
// shared_base: device pointer to the first row of the shared group (n_shared).
hipError_t launch_combine(const uint16_t* y_perm, const int32_t* dest, const float* topk_w,
                          const int32_t* shared_base, uint16_t* out, int T, int H, int k,
                          int n_shared, hipStream_t s);

// ffn.hip: the on-device schedule and the grouped GEMMs.
struct FfnArgs {
  int T, H, E, k, I, n_shared;
  bool fp8;
  const int32_t* offsets;
  const int32_t* a_rows;    // nullptr: x_perm holds the permuted rows; else rows of x_perm gathered
  const void* x_perm;
  const void* x_perm_scale;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* s_gate;
  const void* s_up;
  const void* s_down;
  void* y_perm;
  void* workspace;
  // Upper bound on the rows of any group: T when the groups come from a top-k
  // routing (a token picks an expert once), R for caller-given offsets.
  long long max_group_rows;
  // The work lists in the workspace were already built (by the small-batch
  // routing + dispatch kernel); skip the planner.
  bool planned;
  // MXFP8 operands (fp8 is then true as well: 8-bit codes).
  bool mx = false;
  // Run the tiled and the weight-streaming chains on the caller's stream
  // only (no side stream is created or used).
  bool one_stream = false;
  // fp8 activation scales, K-block-major: block kb of permuted row r at
  // x_perm_scale[kb * s_ld + (s_rows ? s_rows[r] : r)]; s_ld = 0 means R
  // (one scale per permuted row, the layout moe_grouped_ffn takes).
  const int32_t* s_rows = nullptr;
  int s_ld = 0;
};
size_t ffn_workspace_bytes(int T, int H, int E, int k, int I, int n_shared, bool fp8, bool mx);
hipError_t launch_grouped_ffn(const FfnArgs& a, hipStream_t s);

// A second stream per device and slot (default priority, non-blocking) with
// a fork and a join event, created on first use; null if it cannot be made.
// Slot 0: the grouped FFN's streaming chain; slot 1: the layer's per-token
// quantisation, run beside the router.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool tried = false, ok = false;
};
constexpr int kSideSlots = 2;
SideStream* side_stream(int slot);

// small.hip: top-k of a batch of at most kSmallBatch tokens (k <= 16) from the
// router's slice partials (8-bit layers: and x quantised per token into xq,
// xs), then histogram, offsets, ranks and the FFN work lists, in one launch (tickets: a counter zeroed by the preceding router
// GEMM on the same stream).  E_all: experts scored; E: routed experts held
// here (global ids e_first ..).
struct Sched;
Sched ffn_schedule(const FfnArgs& a);   // the work lists inside a's workspace
constexpr int kSmallBatch = 256;
hipError_t launch_route_dispatch_small(const float* parts, int KS, const float* bias, int32_t* idx,
                                       float* w, int32_t* counts, int32_t* offsets, int32_t* dest,
                                       int32_t* src_row, const Sched& sc, int T, int E_all, int k,
                                       int E, int n_shared, int e_first, int32_t* tickets,
                                       const uint16_t* x, uint8_t* xq, void* xs, int H, bool fp8,
                                       bool mx, hipStream_t s);

}  // namespace moe
