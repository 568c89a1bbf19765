// C ABI of libmoe.so (declared in include/moe.h): argument validation,
// workspace layout and the launch sequence of each entry point.  Everything
// here runs on the host; all arithmetic of the layer is in the kernels.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "ffn.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define MOE_NEED_PTR(p)                                                                   \
  do {                                                                                    \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);       \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s: %s not 16-byte aligned", fn, #p); \
  } while (0)

// Shape checks shared by every entry point.
int check_shape(const char* fn, const moe_shape* s, bool need_ffn_dims) {
  if (s == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: shape is NULL", fn);
  if (s->wdtype != MOE_BF16 && s->wdtype != MOE_FP8_E4M3_BLOCK128 && s->wdtype != MOE_MXFP8)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown wdtype %d", fn, s->wdtype);
  if (s->T < 0) return fail(MOE_ERR_UNSUPPORTED, "%s: T=%d < 0", fn, s->T);
  if (s->E < 1 || s->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d not in [1,1024]", fn, s->E);
  if (s->k < 1 || s->k > 16 || s->k > s->E)
    return fail(MOE_ERR_UNSUPPORTED, "%s: k=%d not in [1, min(E,16)]", fn, s->k);
  if (s->n_shared != 0 && s->n_shared != 1)
    return fail(MOE_ERR_UNSUPPORTED, "%s: n_shared=%d not 0 or 1", fn, s->n_shared);
  if ((long long)s->T * (s->k + s->n_shared) >= (1LL << 31))
    return fail(MOE_ERR_UNSUPPORTED, "%s: T*(k+n_shared) >= 2^31", fn);
  if (s->H < 128 || s->H % 128 || s->H > 131072)
    return fail(MOE_ERR_UNSUPPORTED, "%s: H=%d not a multiple of 128 in [128, 131072]", fn, s->H);
  if (need_ffn_dims && (s->I < 128 || s->I % 128))
    return fail(MOE_ERR_UNSUPPORTED, "%s: I=%d not a positive multiple of 128", fn, s->I);
  // One expert matrix must stay below 4 GB (32-bit in-matrix offsets) and K
  // below 131072 (fp8 block scales of a tile are staged in LDS).
  if (need_ffn_dims && ((long long)s->H * s->I >= (1LL << 31) || s->H > 131072 || s->I > 131072))
    return fail(MOE_ERR_UNSUPPORTED, "%s: H*I=%lld too large", fn, (long long)s->H * s->I);
  if (s->e_local < 0 || s->e_first < 0 || (s->e_local == 0 && s->e_first != 0) ||
      (long long)s->e_first + s->e_local > s->E)
    return fail(MOE_ERR_UNSUPPORTED, "%s: expert share e_first=%d e_local=%d not within E=%d", fn,
                s->e_first, s->e_local, s->E);
  return MOE_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// 8-bit codes with scales: per-128 fp32 block scales or MX E8M0 bytes.
bool is_8bit(const moe_shape* s) { return s->wdtype != MOE_BF16; }
bool is_mx(const moe_shape* s) { return s->wdtype == MOE_MXFP8; }

// Routed experts held here (the expert-parallel share, else all E).
int n_local(const moe_shape* s) { return s->e_local ? s->e_local : s->E; }
bool is_share(const moe_shape* s) { return s->e_local != 0; }

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// moe_forward workspace: routing, dispatch and expert intermediates.  The
// forward path never builds x_perm: the GEMMs gather their rows through
// src_row from x (bf16) or from x quantised once per token (fp8, mxfp8: xq,
// xs).  fp8 scales are K-block-major: per permuted row ([H/128][R], R slots
// per block) for large batches (quantised per token into xs_tok, then moved
// to the rows once the ranks are known), per token ([H/128][T]) for small
// ones, whose routing launch quantises before the rows are known.
struct FwdLayout {
  size_t logits, rpart, idx, w, counts, offsets, tcnt, tick, dest, src_row, xq, xs, xs_tok, y_perm, ffn,
      total;
};

FwdLayout fwd_layout(const moe_shape* s) {
  const bool fp8 = is_8bit(s), mx = is_mx(s);
  const size_t T = s->T, H = s->H, E = s->E, k = s->k, G = n_local(s) + s->n_shared;
  const size_t R = T * (k + s->n_shared);
  FwdLayout L{};
  size_t off = 0;
  L.logits = off;  off += align256(T * E * 4);
  L.rpart = off;   off += align256(moe::router_workspace_bytes(s->T, s->H, s->E));
  L.idx = off;     off += align256(T * k * 4);
  L.w = off;       off += align256(T * k * 4);
  L.counts = off;  off += align256(G * 4);
  L.offsets = off; off += align256((G + 1) * 4);
  L.tcnt = off;    off += align256(moe::permute_workspace_bytes(s->T, n_local(s)));
  L.tick = off;    off += 256;          // ticket counter of the small-batch routing + dispatch
  L.dest = off;    off += align256(T * k * 4);
  L.src_row = off; off += align256(R * 4);
  L.xq = off;      off += fp8 ? align256(T * H) : 0;
  L.xs = off;      off += mx ? align256(T * (H / 32)) : fp8 ? align256(R * (H / 128) * 4) : 0;
  L.xs_tok = off;  off += (fp8 && !mx) ? align256(T * (H / 128) * 4) : 0;
  L.y_perm = off;  off += align256(R * H * 2);
  L.ffn = off;
  off += moe::ffn_workspace_bytes(s->T, s->H, n_local(s), s->k, s->I, s->n_shared, fp8, mx);
  L.total = off;
  return L;
}

// Argument checks of the whole-layer entry points (everything but the workspace).
int check_forward_args(const char* fn, const moe_shape* shape, const void* x, const float* w_router,
                       const float* router_bias, const void* w_gate, const void* w_up,
                       const void* w_down, const void* s_gate, const void* s_up,
                       const void* s_down, const void* out, const int32_t* topk_idx_out,
                       const float* topk_w_out) {
  if (int rc = check_shape(fn, shape, true)) return rc;
  if ((long long)shape->T * shape->H * 2 >= (1LL << 32))   // 32-bit row offsets into x
    return fail(MOE_ERR_UNSUPPORTED, "%s: T*H*2 >= 2^32", fn);
  if (shape->T == 0) return MOE_OK;
  MOE_NEED_PTR(x);
  MOE_NEED_PTR(w_router);
  MOE_NEED_PTR(w_gate);
  MOE_NEED_PTR(w_up);
  MOE_NEED_PTR(w_down);
  MOE_NEED_PTR(out);
  if (is_8bit(shape)) {
    MOE_NEED_PTR(s_gate);
    MOE_NEED_PTR(s_up);
    MOE_NEED_PTR(s_down);
  }
  if (router_bias && !aligned16(router_bias))
    return fail(MOE_ERR_INVALID_ARG, "%s: router_bias not 16-byte aligned", fn);
  if (topk_idx_out && !aligned16(topk_idx_out))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_idx_out not 16-byte aligned", fn);
  if (topk_w_out && !aligned16(topk_w_out))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_w_out not 16-byte aligned", fn);
  return MOE_OK;
}

// The launch sequence of the whole layer on stream s, intermediates in ws
// (laid out by L).  one_stream: run the grouped FFN's two kernel chains on s
// alone (no side stream is created or used).
hipError_t forward_launch(const moe_shape* shape, const void* x, const float* w_router,
                          const float* router_bias, const void* w_gate, const void* w_up,
                          const void* w_down, const void* s_gate, const void* s_up,
                          const void* s_down, void* out, int32_t* topk_idx_out,
                          float* topk_w_out, uint8_t* ws, const FwdLayout& L, bool one_stream,
                          hipStream_t s) {
  const bool fp8 = is_8bit(shape), mx = is_mx(shape);
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  int32_t* idx = topk_idx_out ? topk_idx_out : reinterpret_cast<int32_t*>(ws + L.idx);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* dest = reinterpret_cast<int32_t*>(ws + L.dest);
  int32_t* src_row = reinterpret_cast<int32_t*>(ws + L.src_row);
  uint8_t* xq = fp8 ? ws + L.xq : nullptr;
  void* xs = fp8 ? static_cast<void*>(ws + L.xs) : nullptr;
  float* xs_tok = (fp8 && !mx) ? reinterpret_cast<float*>(ws + L.xs_tok) : nullptr;
  void* y_perm = ws + L.y_perm;

  // Router: slice partial sums (or, unsplit, the raw products in the logits
  // buffer), reduced in slice order by the top-k kernel.
  const int ks = moe::router_splits(shape->T, shape->H, shape->E);
  float* parts = ks > 1 ? reinterpret_cast<float*>(ws + L.rpart) : logits;
  const int nl = n_local(shape);
  moe::FfnArgs a{shape->T, shape->H, nl, shape->k, shape->I, shape->n_shared, fp8,
                 offsets, src_row, fp8 ? static_cast<const void*>(xq) : x, xs, w_gate, w_up,
                 w_down, s_gate, s_up, s_down, y_perm, ws + L.ffn, (long long)shape->T, false, mx};
  a.one_stream = one_stream;
  const bool small = shape->T <= moe::kSmallBatch;
  if (small) {                       // fp8 scales per token: rows map to tokens
    a.s_rows = src_row;
    a.s_ld = shape->T;
  }
  int32_t* tick = reinterpret_cast<int32_t*>(ws + L.tick);
  hipError_t e = hipSuccess;
  // Large 8-bit batches: the per-token quantisation of x needs no routing, so
  // it runs on a side stream beside the router GEMM, top-k and ranks (forked
  // after everything already on s, so an earlier call's GEMMs are done with
  // the buffers) and is joined before the FFN.
  void* xs_q = mx ? xs : static_cast<void*>(xs_tok);
  moe::SideStream* qs = nullptr;
  if (fp8 && !small && !one_stream && !moe::prof_serial()) qs = moe::side_stream(1);
  if (qs) {
    e = hipEventRecord(qs->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(qs->s, qs->fork, 0);
    if (e == hipSuccess)
      e = moe::launch_quantize_rows(static_cast<const uint16_t*>(x), xq, xs_q, shape->T, shape->H,
                                    mx, qs->s);
    if (e == hipSuccess) e = hipEventRecord(qs->join, qs->s);
    if (e != hipSuccess) return e;
  }
  e = moe::launch_router_gemm(static_cast<const uint16_t*>(x), w_router, parts,
                                         shape->T, shape->H, shape->E, s, small ? tick : nullptr);
  if (small) {
    // Small batch: top-k, dispatch tables and FFN work lists in one launch.
    if (e == hipSuccess)
      e = moe::launch_route_dispatch_small(parts, ks, router_bias, idx, w, counts, offsets, dest,
                                           src_row, moe::ffn_schedule(a), shape->T, shape->E,
                                           shape->k, nl, shape->n_shared, shape->e_first, tick,
                                           static_cast<const uint16_t*>(x), xq, xs, shape->H, fp8,
                                           mx, s);
    a.planned = true;
  } else {
    if (e == hipSuccess)
      e = moe::launch_topk(parts, ks, router_bias, nullptr, idx, w, shape->T, shape->E, shape->k, s);
    // Routing tables only: no row copy.
    if (e == hipSuccess)
      e = moe::launch_permute(idx, static_cast<const uint16_t*>(x), counts, offsets, dest, src_row,
                              nullptr, nullptr, reinterpret_cast<int32_t*>(ws + L.tcnt), shape->T,
                              shape->H, nl, shape->k, shape->n_shared, shape->e_first,
                              is_share(shape), fp8, mx, s);
  }
  if (e == hipSuccess && fp8 && !small) {   // (small batches: quantised in the routing launch)
    if (qs)
      e = hipStreamWaitEvent(s, qs->join, 0);
    else
      e = moe::launch_quantize_rows(static_cast<const uint16_t*>(x), xq, xs_q, shape->T, shape->H,
                                    mx, s);
    // fp8: the token scales moved to the permuted rows (of this share: offsets[G] rows)
    if (e == hipSuccess && !mx)
      e = moe::launch_permute_scales(xs_tok, src_row, offsets + nl + shape->n_shared,
                                     static_cast<float*>(xs), shape->T,
                                     shape->T * (shape->k + shape->n_shared), shape->H / 128, s);
  }
  if (e == hipSuccess) e = moe::launch_grouped_ffn(a, s);
  if (e == hipSuccess)
    e = moe::launch_combine(static_cast<const uint16_t*>(y_perm), dest, w, offsets + nl,
                            static_cast<uint16_t*>(out), shape->T, shape->H, shape->k,
                            shape->n_shared, s);
  return e;
}

// ------------------------------------------------ fixed device scratch ----
// The intermediates of moe_forward_noalloc live in this array, one copy per
// GPU, held from module load until the process ends.  Nothing in it has to
// start at zero: every kernel writes what a later one reads.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol); it passes the device address hipGetSymbolAddress returns,
// looked up once per device and kept.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(const char* fn, uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library tracks", fn, dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0)
      return fail(MOE_ERR_HIP, "%s: scratch symbol address %p unusable", fn, p);
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

int moe_abi_version(void) { return 5; }

size_t moe_forward_workspace_bytes(const moe_shape* shape) {
  if (check_shape("moe_forward_workspace_bytes", shape, true) != MOE_OK) return 0;
  return fwd_layout(shape).total;
}

size_t moe_workspace_bytes(const moe_shape* shape) { return moe_forward_workspace_bytes(shape); }

size_t moe_ffn_workspace_bytes(const moe_shape* shape) {
  if (check_shape("moe_ffn_workspace_bytes", shape, true) != MOE_OK) return 0;
  return moe::ffn_workspace_bytes(shape->T, shape->H, n_local(shape), shape->k, shape->I,
                                  shape->n_shared, is_8bit(shape), is_mx(shape));
}

size_t moe_route_workspace_bytes(const moe_shape* shape) {
  if (check_shape("moe_route_workspace_bytes", shape, false) != MOE_OK) return 0;
  return moe::router_workspace_bytes(shape->T, shape->H, shape->E);
}

int moe_route(const moe_shape* shape, const void* x, const float* w_router,
              const float* router_bias, float* logits, int32_t* topk_idx, float* topk_w,
              void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "moe_route";
  moe::prof_call_begin();
  if (int rc = check_shape(fn, shape, false)) return rc;
  if (shape->T == 0) return MOE_OK;
  MOE_NEED_PTR(x);
  MOE_NEED_PTR(w_router);
  MOE_NEED_PTR(logits);
  MOE_NEED_PTR(topk_idx);
  MOE_NEED_PTR(topk_w);
  if (router_bias && !aligned16(router_bias))
    return fail(MOE_ERR_INVALID_ARG, "%s: router_bias not 16-byte aligned", fn);
  const size_t need = moe::router_workspace_bytes(shape->T, shape->H, shape->E);
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
  if (need > 0 && !aligned16(workspace))
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace not 16-byte aligned", fn);
  const int ks = moe::router_splits(shape->T, shape->H, shape->E);
  float* parts = ks > 1 ? static_cast<float*>(workspace) : logits;
  hipError_t e = moe::launch_router_gemm(static_cast<const uint16_t*>(x), w_router, parts,
                                         shape->T, shape->H, shape->E, as_stream(stream));
  if (e == hipSuccess)
    e = moe::launch_topk(parts, ks, router_bias, logits, topk_idx, topk_w, shape->T, shape->E,
                         shape->k, as_stream(stream));
  return hip_status(e, fn);
}

int moe_route_from_logits(const moe_shape* shape, const float* logits, int32_t* topk_idx,
                          float* topk_w, void* stream) {
  const char* fn = "moe_route_from_logits";
  moe::prof_call_begin();
  if (shape == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: shape is NULL", fn);
  if (shape->T < 0) return fail(MOE_ERR_UNSUPPORTED, "%s: T < 0", fn);
  if (shape->E < 1 || shape->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "%s: E not in [1,1024]", fn);
  if (shape->k < 1 || shape->k > 16 || shape->k > shape->E)
    return fail(MOE_ERR_UNSUPPORTED, "%s: k not in [1, min(E,16)]", fn);
  if (shape->T == 0) return MOE_OK;
  MOE_NEED_PTR(logits);
  MOE_NEED_PTR(topk_idx);
  MOE_NEED_PTR(topk_w);
  return hip_status(moe::launch_topk(logits, 1, nullptr, nullptr, topk_idx, topk_w, shape->T,
                                     shape->E, shape->k,
                                     as_stream(stream)), fn);
}

size_t moe_permute_workspace_bytes(const moe_shape* shape) {
  if (check_shape("moe_permute_workspace_bytes", shape, false) != MOE_OK) return 0;
  return moe::permute_workspace_bytes(shape->T, n_local(shape));
}

int moe_permute(const moe_shape* shape, const int32_t* topk_idx, const void* x, int32_t* counts,
                int32_t* offsets, int32_t* dest, int32_t* src_row, void* x_perm,
                void* x_perm_scale, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "moe_permute";
  moe::prof_call_begin();
  if (int rc = check_shape(fn, shape, false)) return rc;
  const bool fp8 = is_8bit(shape), mx = is_mx(shape);
  MOE_NEED_PTR(counts);
  MOE_NEED_PTR(offsets);
  if (shape->T > 0) {
    MOE_NEED_PTR(topk_idx);
    MOE_NEED_PTR(x);
    MOE_NEED_PTR(dest);
    MOE_NEED_PTR(src_row);
    MOE_NEED_PTR(x_perm);
    if (fp8) MOE_NEED_PTR(x_perm_scale);
  }
  const size_t need = moe::permute_workspace_bytes(shape->T, n_local(shape));
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
  if (need > 0 && !aligned16(workspace))
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace not 16-byte aligned", fn);
  return hip_status(moe::launch_permute(topk_idx, static_cast<const uint16_t*>(x), counts, offsets,
                                        dest, src_row, x_perm, x_perm_scale,
                                        static_cast<int32_t*>(workspace), shape->T, shape->H,
                                        n_local(shape), shape->k, shape->n_shared, shape->e_first,
                                        is_share(shape), fp8, mx, as_stream(stream)), fn);
}

int moe_grouped_ffn(const moe_shape* shape, const int32_t* offsets, const void* x_perm,
                    const void* x_perm_scale, const void* w_gate, const void* w_up,
                    const void* w_down, const void* s_gate, const void* s_up,
                    const void* s_down, void* y_perm, void* workspace, size_t ws_bytes,
                    void* stream) {
  const char* fn = "moe_grouped_ffn";
  moe::prof_call_begin();
  if (int rc = check_shape(fn, shape, true)) return rc;
  const bool fp8 = is_8bit(shape);
  if (shape->T == 0) return MOE_OK;
  MOE_NEED_PTR(offsets);
  MOE_NEED_PTR(x_perm);
  MOE_NEED_PTR(w_gate);
  MOE_NEED_PTR(w_up);
  MOE_NEED_PTR(w_down);
  MOE_NEED_PTR(y_perm);
  if (fp8) {
    MOE_NEED_PTR(x_perm_scale);
    MOE_NEED_PTR(s_gate);
    MOE_NEED_PTR(s_up);
    MOE_NEED_PTR(s_down);
  }
  const size_t need = moe_ffn_workspace_bytes(shape);
  if (workspace == nullptr || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", fn);
  moe::FfnArgs a{shape->T, shape->H, n_local(shape), shape->k, shape->I, shape->n_shared, fp8,
                 offsets, nullptr, x_perm, x_perm_scale, w_gate, w_up, w_down, s_gate, s_up,
                 s_down, y_perm, workspace,
                 (long long)shape->T * (shape->k + shape->n_shared), false, is_mx(shape)};
  return hip_status(moe::launch_grouped_ffn(a, as_stream(stream)), fn);
}

int moe_combine(const moe_shape* shape, const void* y_perm, const int32_t* dest,
                const float* topk_w, const int32_t* offsets, void* out, void* stream) {
  const char* fn = "moe_combine";
  moe::prof_call_begin();
  if (int rc = check_shape(fn, shape, false)) return rc;
  if (shape->T == 0) return MOE_OK;
  MOE_NEED_PTR(y_perm);
  MOE_NEED_PTR(dest);
  MOE_NEED_PTR(topk_w);
  MOE_NEED_PTR(out);
  if (shape->n_shared) MOE_NEED_PTR(offsets);
  const int32_t* shared_base = shape->n_shared ? offsets + n_local(shape) : nullptr;
  return hip_status(moe::launch_combine(static_cast<const uint16_t*>(y_perm), dest, topk_w,
                                        shared_base, static_cast<uint16_t*>(out), shape->T,
                                        shape->H, shape->k, shape->n_shared, as_stream(stream)),
                    fn);
}

int moe_forward(const moe_shape* shape, const void* x, const float* w_router,
                const float* router_bias, const void* w_gate, const void* w_up,
                const void* w_down, const void* s_gate, const void* s_up, const void* s_down,
                void* out, int32_t* topk_idx_out, float* topk_w_out, void* workspace,
                size_t ws_bytes, void* stream) {
  const char* fn = "moe_forward";
  moe::prof_call_begin();
  if (int rc = check_forward_args(fn, shape, x, w_router, router_bias, w_gate, w_up, w_down, s_gate,
                                  s_up, s_down, out, topk_idx_out, topk_w_out))
    return rc;
  if (shape->T == 0) return MOE_OK;
  const FwdLayout L = fwd_layout(shape);
  if (workspace == nullptr || ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, L.total);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", fn);
  return hip_status(forward_launch(shape, x, w_router, router_bias, w_gate, w_up, w_down, s_gate,
                                   s_up, s_down, out, topk_idx_out, topk_w_out,
                                   static_cast<uint8_t*>(workspace), L, false, as_stream(stream)),
                    fn);
}

int moe_forward_noalloc(const moe_shape* shape, const void* x, const float* w_router,
                        const float* router_bias, const void* w_gate, const void* w_up,
                        const void* w_down, const void* s_gate, const void* s_up,
                        const void* s_down, void* out, int32_t* topk_idx_out, float* topk_w_out,
                        void* stream) {
  const char* fn = "moe_forward_noalloc";
  moe::prof_call_begin();
  if (int rc = check_forward_args(fn, shape, x, w_router, router_bias, w_gate, w_up, w_down, s_gate,
                                  s_up, s_down, out, topk_idx_out, topk_w_out))
    return rc;
  if (shape->T == 0) return MOE_OK;
  const FwdLayout L = fwd_layout(shape);
  if (L.total > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "%s: this shape needs %zu bytes of scratch, more than the library's fixed %zu "
                "(MOE_NOALLOC_SCRATCH_BYTES); call moe_forward with a workspace instead",
                fn, L.total, (size_t)kScratchBytes);
  uint8_t* ws = nullptr;
  if (int rc = scratch_of_current_device(fn, &ws)) return rc;
  return hip_status(forward_launch(shape, x, w_router, router_bias, w_gate, w_up, w_down, s_gate,
                                   s_up, s_down, out, topk_idx_out, topk_w_out, ws, L, true,
                                   as_stream(stream)),
                    fn);
}

}  // extern "C"
