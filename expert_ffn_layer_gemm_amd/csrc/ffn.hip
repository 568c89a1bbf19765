// Grouped expert FFN: for every non-empty group g (rows [offsets[g],
// offsets[g+1]) of the permuted matrix)
//     h = silu(X W_gate[g]^T) * (X W_up[g]^T)      (gate/up GEMM, SwiGLU epilogue)
//     y = h W_down[g]^T                            (down GEMM)
// with fp32 accumulation on the MFMA units.  SwiGLU is fused into the gate/up
// GEMM as in the Ironwood page's GMM v2 (section 4.2.2): the gate and up
// weights are two B streams of the same workgroup, so each output element has
// its gate and up sums in the same lane.  FP8 layers follow the DeepSeek
// deployment page (Quantization): e4m3 operands, one fp32 scale per 128x128
// weight block and per 128 activation channels, applied to the fp32
// accumulator once per 128-wide K block; the SwiGLU epilogue re-quantises h
// per row per 128 channels.
//
// Scheduling (DeepSeek-deployment page, Quantization and CUDA Graph
// sections: kernels read the routed token counts on the device instead of
// sizing work from the buffer's upper bound).  One small kernel reads
// `offsets` and writes two work lists into the workspace:
//   - skinny list: groups with 1..skinny_max_rows(T) rows.  Decode-sized groups are
//     bound by streaming their weights from HBM; the skinny kernel keeps the
//     few activation rows in registers (straight from L2) and streams each
//     weight byte exactly once, 16 bytes per lane, with the next K block's
//     weight loads in flight while the current one is multiplied.
//   - tile list: (group, first row) pairs covering groups with more rows, for
//     an LDS-tiled MFMA kernel (prefill-sized groups, compute bound).
// Both GEMM grids are sized on the host from upper bounds; workgroups past
// the device-side list length exit at once.  No host synchronisation.
#include <algorithm>

#include "dispatch.hpp"

namespace moe {

// ------------------------------------------------------------------ plan ----
__global__ __launch_bounds__(1024) void k_plan(const int32_t* __restrict__ offsets, Sched sc) {
  __shared__ int wave_sum[16];
  plan_groups(offsets, sc, wave_sum);
}

// ---------------------------------------------------------- skinny, bf16 ----
// Whether streaming work item b (split factor p.ksplit) exists.
__device__ __forceinline__ bool skinny_live(const GemmArgs& p, int b) {
  int slot, nt;
  return band_item(p.sc.skinny, *p.sc.n_skinny, p.n_ntile, slot, nt, b / p.ksplit);
}

// Workgroup = NW waves; wave w owns 16 h columns (DUAL) or 32 output columns and
// all (<= 16*MB) rows of its slice.  Lane l: row/column l%16 of each 16x16 MFMA block, 8
// consecutive k at offset 8*(l/16) of each 32-wide K step.
// Split-K (p.ksplit > 1; "Lower latency and higher throughput with multi-node
// DeepSeek deployment", GEMM kernels: split-K lowers the latency of some
// shapes at low batch): when few experts hold rows, K is cut into ksplit
// ranges, block b taking range b % ksplit of the work item b / ksplit, so
// ksplit times as many waves stream the weights; each writes its fp32
// partial sums and k_splitk_reduce adds them in range order.
template <bool DUAL, int NW, int MB>
__device__ __forceinline__ void skinny_bf16_item(const GemmArgs& p, const int bid, const int tid_) {
  int slot, nt;
  const int ks = bid % p.ksplit;
  if (!band_item(p.sc.skinny, *p.sc.n_skinny, p.n_ntile, slot, nt, bid / p.ksplit)) return;
  const int g = p.sc.skinny[4 * slot], s0 = p.sc.skinny[4 * slot + 1];
  const int row0 = p.offsets[g] + s0, m = min(16 * MB, p.offsets[g + 1] - row0);
  const int nmb = ceil_div(m, 16);
  const int lane = tid_ & 63, wave = tid_ >> 6;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const int K = p.K, N = p.N;
  // Two weight streams per wave: gate and up rows of 16 h columns (DUAL), or
  // the rows of 32 consecutive output columns (16 + 16).
  const int n0 = (nt * NW + wave) * (DUAL ? 16 : 32);

  // This block's K range [kbeg, kbeg + Kc).
  const int Kc = K / p.ksplit, kbeg = ks * Kc;
  const uint16_t* b0 = reinterpret_cast<const uint16_t*>(p.B0) + ((size_t)g * N + n0 + r16) * K + kq + kbeg;
  const uint16_t* b1 = DUAL ? reinterpret_cast<const uint16_t*>(p.B1) + ((size_t)g * N + n0 + r16) * K + kq + kbeg
                            : b0 + (size_t)16 * K;
  const uint16_t* arow[MB];
  bool aok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = mb * 16 + r16;
    aok[mb] = r < m;
    const int pr = row0 + (aok[mb] ? r : 0);
    arow[mb] = reinterpret_cast<const uint16_t*>(p.A) + (size_t)(p.a_rows ? p.a_rows[pr] : pr) * K + kq + kbeg;
  }

  f32x4_t acc0[MB], acc1[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc0[mb] = acc1[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int U = 4;  // 32-wide K steps per iteration (128 of K)
  u32x4_t cur0[U], cur1[U], nxt0[U], nxt1[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    cur0[u] = *reinterpret_cast<const u32x4_t*>(b0 + u * 32);
    cur1[u] = *reinterpret_cast<const u32x4_t*>(b1 + u * 32);
  }
  for (int k0 = 0; k0 < Kc; k0 += 32 * U) {
    const bool more = k0 + 32 * U < Kc;
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        nxt0[u] = *reinterpret_cast<const u32x4_t*>(b0 + k0 + 32 * U + u * 32);
        nxt1[u] = *reinterpret_cast<const u32x4_t*>(b1 + k0 + 32 * U + u * 32);
      }
    }
    // A fragments one 32-wide K step at a time (MB x 4 registers live), so
    // the 4-block variant keeps enough waves per SIMD to hide the weight
    // stream's latency.
#pragma unroll
    for (int u = 0; u < U; ++u) {
      u32x4_t a[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        if (mb < nmb)
          a[mb] = aok[mb] ? *reinterpret_cast<const u32x4_t*>(arow[mb] + k0 + u * 32)
                          : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        if (mb < nmb) {
          acc0[mb] = mfma_bf16_16x16x32(a[mb], cur0[u], acc0[mb]);
          acc1[mb] = mfma_bf16_16x16x32(a[mb], cur1[u], acc1[mb]);
        }
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        cur0[u] = nxt0[u];
        cur1[u] = nxt1[u];
      }
    }
  }

  if (p.ksplit > 1) {   // fp32 partials of this K range: gate | up, or two column blocks
    const int NP = DUAL ? 2 * N : N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      if (mb < nmb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = mb * 16 + (lane >> 4) * 4 + q;
          if (r < m) {
            float* o = p.part + ((size_t)ks * p.R + row0 + r) * NP + n0 + r16;
            o[0] = acc0[mb][q];
            o[DUAL ? N : 16] = acc1[mb][q];
          }
        }
      }
    return;
  }
  uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    if (mb < nmb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = mb * 16 + (lane >> 4) * 4 + q;
        if (r < m) {
          uint16_t* o = out + (size_t)(row0 + r) * N + n0 + r16;
          if (DUAL) {
            o[0] = (uint16_t)f32_to_bf16_bits(silu_mul(acc0[mb][q], acc1[mb][q]));
          } else {
            o[0] = (uint16_t)f32_to_bf16_bits(acc0[mb][q]);
            o[16] = (uint16_t)f32_to_bf16_bits(acc1[mb][q]);
          }
        }
      }
    }
}

// WALK = false: one workgroup per work item.  WALK = true (grid capped at
// kSkinnyGrid workgroups): each walks items b, b + grid, ... (same XCD: the
// grid is a multiple of 8 times the split factor) and stops at the first index
// past the list; the thread index is laundered per item so nothing derived
// from it is hoisted out of the walk into long-lived registers.
template <bool DUAL, int NW, int MB, bool WALK>
__global__ __launch_bounds__(64 * NW) void k_skinny_bf16(const GemmArgs p) {
  if constexpr (!WALK) {
    skinny_bf16_item<DUAL, NW, MB>(p, blockIdx.x, (int)threadIdx.x);
  } else {
    for (int b = blockIdx.x; skinny_live(p, b); b += (int)gridDim.x) {
      int tid = (int)threadIdx.x;
      asm volatile("" : "+v"(tid));
      skinny_bf16_item<DUAL, NW, MB>(p, b, tid);
      __syncthreads();                     // LDS of this item is read before the next one writes it
    }
  }
}

// Sum of the ksplit fp32 partial planes in plane order for rows below
// *n_rows, then the epilogue: DUAL h = bf16(silu(gate) * up), else bf16(y).
// 4 columns per thread.
template <bool DUAL>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int ksplit,
                                                       int R, int N, const int32_t* __restrict__ n_rows,
                                                       uint16_t* __restrict__ out) {
  const int r = blockIdx.y;
  if (r >= *n_rows) return;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= N) return;
  const int NP = DUAL ? 2 * N : N;
  float4 a = *reinterpret_cast<const float4*>(part + (size_t)r * NP + c);
  float4 b = DUAL ? *reinterpret_cast<const float4*>(part + (size_t)r * NP + N + c) : float4{};
  for (int s = 1; s < ksplit; ++s) {
    const float* pl = part + ((size_t)s * R + r) * NP;
    const float4 x = *reinterpret_cast<const float4*>(pl + c);
    a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
    if (DUAL) {
      const float4 y = *reinterpret_cast<const float4*>(pl + N + c);
      b.x += y.x; b.y += y.y; b.z += y.z; b.w += y.w;
    }
  }
  if (DUAL) {
    a.x = silu_mul(a.x, b.x); a.y = silu_mul(a.y, b.y);
    a.z = silu_mul(a.z, b.z); a.w = silu_mul(a.w, b.w);
  }
  const uint32_t lo = pack_bf16x2(a.x, a.y);
  const uint32_t hi = pack_bf16x2(a.z, a.w);
  *reinterpret_cast<uint2*>(out + (size_t)r * N + c) = make_uint2(lo, hi);
}

// Split-K reduce of an 8-bit gate/up GEMM: h = silu(sum of gate planes) *
// (sum of up planes), planes added in order, then h quantised per row like
// the one-pass epilogue: fp8 (MX = false) per 128 columns (scale = amax /
// 448, 32 threads of 4 columns per group; scales [N/128][R]), MXFP8 per 32
// columns (E8M0, 8 threads per block; [R][N/32]).  Rows below *n_rows; 4
// columns per thread.
template <bool MX>
__global__ __launch_bounds__(256) void k_splitk_reduce_q8(const float* __restrict__ part, int ksplit,
                                                          int R, int N, const int32_t* __restrict__ n_rows,
                                                          uint8_t* __restrict__ out, void* __restrict__ out_scale) {
  const int r = blockIdx.y;
  if (r >= *n_rows) return;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;   // N is a multiple of 128: whole groups per block
  if (c >= N) return;
  const int NP = 2 * N;
  float4 a = *reinterpret_cast<const float4*>(part + (size_t)r * NP + c);
  float4 b = *reinterpret_cast<const float4*>(part + (size_t)r * NP + N + c);
  for (int s2 = 1; s2 < ksplit; ++s2) {
    const float* pl = part + ((size_t)s2 * R + r) * NP;
    const float4 x = *reinterpret_cast<const float4*>(pl + c);
    const float4 y = *reinterpret_cast<const float4*>(pl + N + c);
    a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
    b.x += y.x; b.y += y.y; b.z += y.z; b.w += y.w;
  }
  float h[4] = {silu_mul(a.x, b.x), silu_mul(a.y, b.y), silu_mul(a.z, b.z), silu_mul(a.w, b.w)};
  float am = fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])), fmaxf(fabsf(h[2]), fabsf(h[3])));
  uint32_t word = 0;
  if constexpr (MX) {
    am = wave_max_xor(am, 8);
    const uint32_t e8 = mx_e8m0(am);
    const float inv = mx_inv_scale(e8);
#pragma unroll
    for (int q = 0; q < 4; ++q) word |= f32_to_e4m3(fminf(fmaxf(h[q] * inv, -448.f), 448.f)) << (8 * q);
    if ((c & 31) == 0) static_cast<uint8_t*>(out_scale)[(size_t)r * (N / 32) + c / 32] = (uint8_t)e8;
  } else {
    am = wave_max_xor(am, 32);
    const float scale = am == 0.f ? 1.f : am / 448.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) word |= f32_to_e4m3(fminf(fmaxf(h[q] / scale, -448.f), 448.f)) << (8 * q);
    if ((c & 127) == 0) static_cast<float*>(out_scale)[(size_t)(c / 128) * R + r] = scale;
  }
  *reinterpret_cast<uint32_t*>(out + (size_t)r * N + c) = word;
}

// ----------------------------------------------------------- skinny, fp8 ----
// Same scheme with the e4m3 16x16x128 MFMA: one MFMA per 128-wide K block;
// lane l supplies 32 codes at K offset 32*(l/16).  The block partial is scaled
// by (activation scale of its row) * (weight block scale) into fp32.
// DUAL needs NW = 8 so a workgroup covers one 128-column group of h, whose
// row maxima are combined across waves through LDS.
template <bool DUAL, int NW, int MB>
__device__ __forceinline__ void skinny_fp8_item(const GemmArgs& p, const int bid, const int tid_) {
  __shared__ float row_amax[NW][16 * MB];
  int slot, nt;
  // Split-K as in the bf16 kernel: block b sums K range b % ksplit of work
  // item b / ksplit (whole 128-K scale blocks) into fp32 partials.
  const int ks = bid % p.ksplit;
  if (!band_item(p.sc.skinny, *p.sc.n_skinny, p.n_ntile, slot, nt, bid / p.ksplit)) return;
  const int g = p.sc.skinny[4 * slot], s0 = p.sc.skinny[4 * slot + 1];
  const int row0 = p.offsets[g] + s0, m = min(16 * MB, p.offsets[g + 1] - row0);
  const int nmb = ceil_div(m, 16);
  const int lane = tid_ & 63, wave = tid_ >> 6;
  const int r16 = lane & 15, kq = (lane >> 4) * 32;
  const int K = p.K, N = p.N, KB = K / 128;
  const int n0 = (nt * NW + wave) * 16;
  const int nblk = n0 / 128;
  const int KBc = KB / p.ksplit, kb0 = ks * KBc;   // this block's 128-K blocks

  const uint8_t* b0 = p.B0 + ((size_t)g * N + n0 + r16) * K + kq;
  const uint8_t* b1 = DUAL ? p.B1 + ((size_t)g * N + n0 + r16) * K + kq : nullptr;
  const float* sb0 = static_cast<const float*>(p.s_B0) + ((size_t)g * (N / 128) + nblk) * KB;
  const float* sb1 = DUAL ? static_cast<const float*>(p.s_B1) + ((size_t)g * (N / 128) + nblk) * KB : nullptr;
  const uint8_t* arow[MB];
  bool aok[MB];
  const float* srow[MB][4];
  bool sok[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = mb * 16 + r16;
    aok[mb] = r < m;
    const int pr = row0 + (aok[mb] ? r : 0);
    arow[mb] = p.A + (size_t)(p.a_rows ? p.a_rows[pr] : pr) * K + kq;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = mb * 16 + (lane >> 4) * 4 + q;
      sok[mb][q] = rr < m;
      const int ps = row0 + (sok[mb][q] ? rr : 0);
      srow[mb][q] = static_cast<const float*>(p.A_scale) + (p.s_rows ? p.s_rows[ps] : ps);
    }
  }
  f32x4_t acc0[MB], acc1[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc0[mb] = acc1[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  i32x8_t cur0 = *reinterpret_cast<const i32x8_t*>(b0 + kb0 * 128), cur1{};
  if (DUAL) cur1 = *reinterpret_cast<const i32x8_t*>(b1 + kb0 * 128);
  for (int kb = kb0; kb < kb0 + KBc; ++kb) {
    const bool more = kb + 1 < kb0 + KBc;
    i32x8_t nxt0{}, nxt1{};
    if (more) {
      nxt0 = *reinterpret_cast<const i32x8_t*>(b0 + (kb + 1) * 128);
      if (DUAL) nxt1 = *reinterpret_cast<const i32x8_t*>(b1 + (kb + 1) * 128);
    }
    const float s0 = sb0[kb], s1 = DUAL ? sb1[kb] : 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      if (mb < nmb) {
        const i32x8_t a = aok[mb] ? *reinterpret_cast<const i32x8_t*>(arow[mb] + kb * 128) : i32x8_t{};
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        const f32x4_t p0 = mfma_fp8_16x16x128(a, cur0, z);
        f32x4_t p1 = z;
        if (DUAL) p1 = mfma_fp8_16x16x128(a, cur1, z);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sa = sok[mb][q] ? srow[mb][q][(size_t)kb * p.s_ld] : 0.f;
          acc0[mb][q] += p0[q] * (sa * s0);
          if (DUAL) acc1[mb][q] += p1[q] * (sa * s1);
        }
      }
    if (more) { cur0 = nxt0; if (DUAL) cur1 = nxt1; }
  }

  if (p.ksplit > 1) {   // fp32 partials of this K range: gate | up, or the columns
    const int NP = DUAL ? 2 * N : N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      if (mb < nmb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = mb * 16 + (lane >> 4) * 4 + q;
          if (r < m) {
            float* o = p.part + ((size_t)ks * p.R + row0 + r) * NP + n0 + r16;
            o[0] = acc0[mb][q];
            if (DUAL) o[N] = acc1[mb][q];
          }
        }
      }
    return;
  }

  if constexpr (DUAL) {
    // h = silu(g) * u, then per-row amax over the workgroup's 128 columns.
    float hv[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = mb * 16 + (lane >> 4) * 4 + q;
        hv[mb][q] = (mb < nmb && r < m) ? silu_mul(acc0[mb][q], acc1[mb][q]) : 0.f;
        const float am = row16_max(fabsf(hv[mb][q]));
        if (r16 == 0) row_amax[wave][r] = am;
      }
    __syncthreads();
    const int gcol = (nt * NW * 16) / 128;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      if (mb < nmb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = mb * 16 + (lane >> 4) * 4 + q;
          if (r < m) {
            float am = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) am = fmaxf(am, row_amax[w][r]);
            const float scale = am == 0.f ? 1.f : am / 448.f;
            const float qv = fminf(fmaxf(hv[mb][q] / scale, -448.f), 448.f);
            p.out[(size_t)(row0 + r) * N + n0 + r16] = (uint8_t)f32_to_e4m3(qv);
            if (wave == 0 && r16 == 0) static_cast<float*>(p.out_scale)[(size_t)gcol * p.R + row0 + r] = scale;
          }
        }
      }
  } else {
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      if (mb < nmb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = mb * 16 + (lane >> 4) * 4 + q;
          if (r < m) out[(size_t)(row0 + r) * N + n0 + r16] = (uint16_t)f32_to_bf16_bits(acc0[mb][q]);
        }
      }
  }
}

// WALK = false: one workgroup per work item.  WALK = true (grid capped at
// kSkinnyGrid workgroups): each walks items b, b + grid, ... (same XCD: the
// grid is a multiple of 8 times the split factor) and stops at the first index
// past the list; the thread index is laundered per item so nothing derived
// from it is hoisted out of the walk into long-lived registers.
template <bool DUAL, int NW, int MB, bool WALK>
__global__ __launch_bounds__(64 * NW) void k_skinny_fp8(const GemmArgs p) {
  if constexpr (!WALK) {
    skinny_fp8_item<DUAL, NW, MB>(p, blockIdx.x, (int)threadIdx.x);
  } else {
    for (int b = blockIdx.x; skinny_live(p, b); b += (int)gridDim.x) {
      int tid = (int)threadIdx.x;
      asm volatile("" : "+v"(tid));
      skinny_fp8_item<DUAL, NW, MB>(p, b, tid);
      __syncthreads();                     // LDS of this item is read before the next one writes it
    }
  }
}

// ----------------------------------------------------------- skinny, mxfp8 ----
// The 32 codes lane l contributes to an e4m3 MFMA 16x16x128 from a row whose
// 128-K block starts at ptr - 16*(l/16): 16 bytes at K 16*(l/16) and 16 at
// K 64 + 16*(l/16).
__device__ __forceinline__ i32x8_t ld32(const uint8_t* ptr) {
  const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(ptr);
  const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(ptr + 64);
  return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Weight streaming for MXFP8 layers (16-row slices).  Wave w owns CB blocks
// of 16 output columns; lane l loads its row's 32 codes of each 128-K block
// in the MFMA's layout (16 bytes at K 16*(l/16), 16 at K 64 + 16*(l/16)), the
// next block's codes in flight while the current one is multiplied.  The
// scaled MFMA applies the E8M0 scales of K block 4*kb + l/16 of the lane's A
// row and B rows, so the partial sums accumulate directly.  Each A fragment
// feeds CB (x2 for gate/up) MFMAs.  Scales: one 16-byte load per row and 4 K
// blocks (the lane picks byte l/16 of each dword); a byte per block and row
// re-fetched the row's scale line from memory for every block (measured:
// 0.76 GB of extra HBM reads on the decode workload).  Rows whose scale arrays
// are not 16-byte aligned (K not a multiple of 512) take the byte loads.
// DUAL: h = silu(g) * u is quantised per row in MX blocks of 32 columns:
// within the wave for CB = 2, else two adjacent waves combine their row
// maxima in LDS.
template <int NB>
__device__ __forceinline__ void mx_load(i32x8_t& a, i32x8_t (&b)[NB], int kb, bool aok,
                                        const uint8_t* arow, const uint8_t* const (&bp)[NB]) {
#pragma unroll
  for (int j = 0; j < NB; ++j) b[j] = ld32(bp[j] + (size_t)kb * 128);
  // Rows past the slice feed zero codes (outputs never stored).
  a = aok ? ld32(arow + (size_t)kb * 128) : i32x8_t{};
}

// Scale dwords of K blocks 4 g .. 4 g + 3 of the A row ([NB]) and B rows.
template <int NB>
__device__ __forceinline__ void mx_load_scales(u32x4_t (&sv)[NB + 1], int g, const uint8_t* sarow,
                                               const uint8_t* const (&sbrow)[NB]) {
#pragma unroll
  for (int j = 0; j < NB; ++j) sv[j] = *reinterpret_cast<const u32x4_t*>(sbrow[j] + 16 * g);
  sv[NB] = *reinterpret_cast<const u32x4_t*>(sarow + 16 * g);
}

// MXFP8 streaming shapes: waves per workgroup and 16-column blocks per wave
// (gate/up, down).
constexpr int kMxNW = 4, kMxCB = 2;
constexpr int kMxNWD = 4, kMxCBD = 2;

// Byte q of x.
__device__ __forceinline__ uint32_t byte_of(uint32_t x, int q) { return (x >> (8 * q)) & 0xFFu; }
// Element i (0..3, runtime) of a 4-dword vector.
__device__ __forceinline__ uint32_t dword_of(const u32x4_t v, int i) {
  return i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}

// Scale modes (SM): 0 one byte per row and block; 1 (rows 16-byte aligned,
// K a multiple of 512) one 16-byte load per row and 4 K blocks; 2 (also
// K <= 8192) the workgroup copies the scale rows of its A and B rows into
// LDS once (dynamic shared memory, rows padded by 16 bytes), so each scale
// line is read from memory once per workgroup.
template <bool DUAL, int NW, int CB, int SM>
__device__ __forceinline__ void skinny_mx_item(const GemmArgs& p, const int bid, const int tid_) {
  constexpr bool VEC = SM == 1;
  static_assert(!DUAL || CB == 2 || (CB == 1 && NW % 2 == 0), "an MX block of h is 32 columns");
  constexpr int NM = DUAL ? 2 : 1;          // weight matrices
  constexpr int NB = NM * CB;               // B streams per lane: [matrix][column block]
  __shared__ float row_amax[NW][16];
  int slot, nt;
  // Split-K: block b sums 128-K blocks [kb0, kb0 + KBc) of work item
  // b / ksplit (kb0 a multiple of 4, so the 16-byte scale loads stay aligned).
  const int ks = bid % p.ksplit;
  if (!band_item(p.sc.skinny, *p.sc.n_skinny, p.n_ntile, slot, nt, bid / p.ksplit)) return;
  const int g = p.sc.skinny[4 * slot], s0 = p.sc.skinny[4 * slot + 1];
  const int row0 = p.offsets[g] + s0, m = min(16, p.offsets[g + 1] - row0);
  const int lane = tid_ & 63, wave = tid_ >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int K = p.K, N = p.N, KB = K / 128, K32 = K / 32;
  const int n0 = (nt * NW + wave) * 16 * CB;
  const int KBc = KB / p.ksplit, kb0 = ks * KBc;

  // Per-lane stream bases: codes at the lane's 16-byte offset; scale rows.
  const uint8_t* bp[NB];
  const uint8_t* sbrow[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const size_t brow = (size_t)g * N + n0 + (j % CB) * 16 + r16;
    bp[j] = (j < CB ? p.B0 : p.B1) + brow * K + 16 * q4;
    sbrow[j] = static_cast<const uint8_t*>(j < CB ? p.s_B0 : p.s_B1) + brow * K32;
  }
  const bool aok = r16 < m;
  const int pr = row0 + (aok ? r16 : 0);
  const size_t arow_i = (size_t)(p.a_rows ? p.a_rows[pr] : pr);
  const uint8_t* arow = p.A + arow_i * K + 16 * q4;
  const uint8_t* sarow = static_cast<const uint8_t*>(p.A_scale) + arow_i * K32;

  // SM 2: LDS rows 0 .. NW*NB*16-1 hold the B rows (wave, stream, row), then
  // 16 A rows; row stride K32 + 16.
  extern __shared__ __attribute__((aligned(16))) uint8_t mxs[];
  const int RS = K32 + 16;
  if constexpr (SM == 2) {
    // Only the 16-byte pieces of this block's K range (4 K blocks each).
    constexpr int BR = NW * NB * 16;
    const int c_lo = kb0 / 4, c16 = KBc / 4, total = (BR + 16) * c16;
    for (int idx = tid_; idx < total; idx += 64 * NW) {
      const int R = idx / c16, cc = c_lo + idx % c16;
      const uint8_t* src;
      if (R < BR) {
        const int w = R / (NB * 16), j = (R / 16) % NB, r = R % 16;
        const size_t br = (size_t)g * N + (nt * NW + w) * 16 * CB + (j % CB) * 16 + r;
        src = static_cast<const uint8_t*>(j < CB ? p.s_B0 : p.s_B1) + br * K32;
      } else {
        const int r = row0 + min(R - BR, m - 1);
        src = static_cast<const uint8_t*>(p.A_scale) + (size_t)(p.a_rows ? p.a_rows[r] : r) * K32;
      }
      *reinterpret_cast<u32x4_t*>(mxs + R * RS + cc * 16) = *reinterpret_cast<const u32x4_t*>(src + cc * 16);
    }
    __syncthreads();
  }
  const uint8_t* lsa = mxs + (NW * NB * 16 + r16) * RS + q4;   // SM 2: this lane's A scale row

  f32x4_t acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Block kb's codes in (da, db); loads past the last block re-read it
  // (cache hits, never multiplied), which keeps them unconditional.
  i32x8_t da, db[NB], xa, xb[NB];
  const int kb1 = kb0 + KBc;                // end of this block's K range
  mx_load<NB>(da, db, kb0, aok, arow, bp);
  u32x4_t sv[NB + 1];
  if constexpr (VEC) mx_load_scales<NB>(sv, kb0 / 4, sarow, sbrow);
  for (int kb = kb0; kb < kb1; ++kb) {
    mx_load<NB>(xa, xb, min(kb + 1, kb1 - 1), aok, arow, bp);
    uint32_t sa, sb[NB];
    if constexpr (SM == 2) {
      sa = lsa[4 * kb];
#pragma unroll
      for (int j = 0; j < NB; ++j) sb[j] = mxs[((wave * NB + j) * 16 + r16) * RS + 4 * kb + q4];
    } else if constexpr (VEC) {
      sa = byte_of(dword_of(sv[NB], kb & 3), q4);
#pragma unroll
      for (int j = 0; j < NB; ++j) sb[j] = byte_of(dword_of(sv[j], kb & 3), q4);
    } else {
      sa = sarow[4 * kb + q4];
#pragma unroll
      for (int j = 0; j < NB; ++j) sb[j] = sbrow[j][4 * kb + q4];
    }
    if (!aok) sa = 127u;                    // zero codes with scale 1
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = mfma_mx8_16x16x128(da, db[j], acc[j], sa, sb[j]);
    // the next 4 blocks' scale dwords, after the last use of these
    if (VEC && (kb & 3) == 3) mx_load_scales<NB>(sv, min(kb + 1, kb1 - 4) / 4, sarow, sbrow);
    da = xa;
#pragma unroll
    for (int j = 0; j < NB; ++j) db[j] = xb[j];
  }

  if (p.ksplit > 1) {   // fp32 partials of this K range: gate | up, or the columns
    const int NP = DUAL ? 2 * N : N;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = q4 * 4 + q;
      if (r < m) {
        float* o = p.part + ((size_t)ks * p.R + row0 + r) * NP + n0 + r16;
#pragma unroll
        for (int j = 0; j < NB; ++j) o[(j / CB) * N + (j % CB) * 16] = acc[j][q];
      }
    }
    return;
  }

  if constexpr (DUAL) {
    float hv[4][CB], am[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = q4 * 4 + q;
      am[q] = 0.f;
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        hv[q][c] = r < m ? silu_mul(acc[c][q], acc[CB + c][q]) : 0.f;
        am[q] = fmaxf(am[q], fabsf(hv[q][c]));
      }
      am[q] = row16_max(am[q]);
      if (CB == 1 && r16 == 0) row_amax[wave][r] = am[q];
    }
    if (CB == 1) __syncthreads();
    const int N32 = N / 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = q4 * 4 + q;
      if (r < m) {
        const float a = CB == 1 ? fmaxf(row_amax[wave][r], row_amax[wave ^ 1][r]) : am[q];
        const uint32_t e8 = mx_e8m0(a);
        const float inv = mx_inv_scale(e8);
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          const float qv = fminf(fmaxf(hv[q][c] * inv, -448.f), 448.f);
          p.out[(size_t)(row0 + r) * N + n0 + c * 16 + r16] = (uint8_t)f32_to_e4m3(qv);
        }
        if ((CB == 2 || (wave & 1) == 0) && r16 == 0)
          static_cast<uint8_t*>(p.out_scale)[(size_t)(row0 + r) * N32 + n0 / 32] = (uint8_t)e8;
      }
    }
  } else {
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = q4 * 4 + q;
      if (r < m) {
#pragma unroll
        for (int c = 0; c < CB; ++c)
          out[(size_t)(row0 + r) * N + n0 + c * 16 + r16] = (uint16_t)f32_to_bf16_bits(acc[c][q]);
      }
    }
  }
}

// WALK = false: one workgroup per work item.  WALK = true (grid capped at
// kSkinnyGrid workgroups): each walks items b, b + grid, ... (same XCD: the
// grid is a multiple of 8 times the split factor) and stops at the first index
// past the list; the thread index is laundered per item so nothing derived
// from it is hoisted out of the walk into long-lived registers.
template <bool DUAL, int NW, int CB, int SM, bool WALK>
__global__ __launch_bounds__(64 * NW) void k_skinny_mx(const GemmArgs p) {
  if constexpr (!WALK) {
    skinny_mx_item<DUAL, NW, CB, SM>(p, blockIdx.x, (int)threadIdx.x);
  } else {
    for (int b = blockIdx.x; skinny_live(p, b); b += (int)gridDim.x) {
      int tid = (int)threadIdx.x;
      asm volatile("" : "+v"(tid));
      skinny_mx_item<DUAL, NW, CB, SM>(p, b, tid);
      __syncthreads();                     // LDS of this item is read before the next one writes it
    }
  }
}

// ------------------------------------------------------------------- host ----
namespace {
size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct WsLayout {
  size_t h, h_scale, n_skinny, n_tiles, skinny, tiles, part, total;
  int max_tiles, max_slices;
  int split_up, split_dn;   // split-K factors of the bf16 streaming GEMMs (1 = none)
};

// Split-K factor of a bf16 streaming GEMM whose at most `items` slices have
// `waves` waves each and stream [N, K] weights: the smallest power of two up
// to 8 that gives the chip about 4096 waves (16 per CU), keeping K / S a
// multiple of 128.  Below 32 MB of weights the launch latency dominates and
// the extra reduce launch would cost more than it saves: no split.
// elt: bytes per weight; kalign: each K range a multiple of kalign (128 for
// bf16 and fp8; 1024 for MXFP8: its scales come 4 K blocks at a time, and
// ranges of 512 measured slower than no split on an EP8 decode share).
int split_factor(long long items, long long waves, int N, int K, int elt, int kalign) {
  if (items * N * K * elt < (32LL << 20)) return 1;
  int S = 1;
  while (S < 8 && items * waves * S < 4096 && K % (2 * S * kalign) == 0) S *= 2;
  return S;
}

WsLayout ffn_layout(int T, int H, int E, int k, int I, int n_shared, bool fp8, bool mx) {
  (void)H;
  WsLayout L{};
  const long long R = (long long)T * (k + n_shared);
  const int G = E + n_shared;
  const long long big_groups = std::min<long long>(G, R / (skinny_max_rows(T) + 1));
  L.max_tiles = (int)(R / tile_rows(fp8, mx, bf16_stream_tiles(T, k, E, fp8)) + big_groups + 1);
  size_t off = 0;
  L.h = off;        off += align256((size_t)R * I * (fp8 ? 1 : 2));
  // h scales: fp8 one fp32 per 128 channels, mxfp8 one E8M0 byte per 32
  L.h_scale = off;  off += mx ? align256((size_t)R * (I / 32)) : fp8 ? align256((size_t)R * (I / 128) * 4) : 0;
  L.n_skinny = off; off += 256;
  L.n_tiles = off;  off += 256;
  L.max_slices = (int)std::min<long long>(4LL * G, R / kSliceRows + G);
  L.skinny = off;   off += align256((size_t)L.max_slices * 16);
  L.tiles = off;    off += align256((size_t)L.max_tiles * 16);
  // Split-K partials: layers whose groups all stay below kSkinnyMax rows
  // (T <= kSkinnyMax: no tiled work), when few slices would leave the chip
  // idle.  Waves per slice: bf16 gate/up I/16, down H/32; fp8 I/16, H/16;
  // MXFP8 I/32, H/32.
  L.split_up = L.split_dn = 1;
  if (T <= kSkinnyMax) {
    const long long items = std::min<long long>(G, R);
    const int elt = fp8 ? 1 : 2, ka = mx ? 1024 : 128;
    L.split_up = split_factor(items, mx ? I / 32 : I / 16, 2 * I, H, elt, ka);
    L.split_dn = split_factor(items, (fp8 && !mx) ? H / 16 : H / 32, H, I, elt, ka);
  }
  L.part = off;
  if (L.split_up > 1 || L.split_dn > 1)
    off += align256((size_t)R * 4 * std::max((size_t)L.split_up * 2 * I, (size_t)L.split_dn * H));
  L.total = off;
  return L;
}
}  // namespace

Sched ffn_schedule(const FfnArgs& f) {
  const WsLayout L = ffn_layout(f.T, f.H, f.E, f.k, f.I, f.n_shared, f.fp8, f.mx);
  uint8_t* ws = static_cast<uint8_t*>(f.workspace);
  return Sched{reinterpret_cast<int32_t*>(ws + L.n_skinny), reinterpret_cast<int32_t*>(ws + L.n_tiles),
               reinterpret_cast<int32_t*>(ws + L.skinny), reinterpret_cast<int32_t*>(ws + L.tiles),
               f.E + f.n_shared, tile_rows(f.fp8, f.mx, bf16_stream_tiles(f.T, f.k, f.E, f.fp8)),
               skinny_max_rows(f.T)};
}

size_t ffn_workspace_bytes(int T, int H, int E, int k, int I, int n_shared, bool fp8, bool mx) {
  return ffn_layout(T, H, E, k, I, n_shared, fp8, mx).total;
}

// A second stream per host thread and device, with a fork and a join event:
// the tiled kernels (groups > skinny_max_rows(T) rows) and the weight-streaming
// kernels (the other groups) touch disjoint groups, and each down GEMM needs
// only the gate/up rows of its own groups, so the two chains run concurrently.
// Created on first use with default priority and kept for the life of the
// process (host objects only; no device memory).  If creation fails the
// chains run one after the other on the caller's stream.
SideStream* side_stream(int slot) {
  constexpr int kMaxDev = 16;
  thread_local SideStream per_dev[kMaxDev][kSideSlots];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev || slot < 0 || slot >= kSideSlots)
    return nullptr;
  SideStream& x = per_dev[dev][slot];
  if (!x.tried) {
    x.tried = true;
    x.ok = hipStreamCreateWithFlags(&x.s, hipStreamNonBlocking) == hipSuccess &&
           hipEventCreateWithFlags(&x.fork, hipEventDisableTiming) == hipSuccess &&
           hipEventCreateWithFlags(&x.join, hipEventDisableTiming) == hipSuccess;
  }
  return x.ok ? &x : nullptr;
}

// When (nearly) every group is tiled, the streaming kernels' grid is capped
// at kSkinnyGrid workgroups (4 per CU; a multiple of 8 times every split
// factor) that walk the work list: the host-side bound on the items is loose
// (every group might be small), and a grid of that bound whose workgroups
// nearly all find nothing cost up to ~40 us of dispatch after the tiled chain
// of the DeepSeek-like layer (4096 walkers still 15 us, 1024 about a third of
// that: the DeepSeek-like layer and both prefills -0.3 to -0.6 %).  With real
// streaming work (decode, skewed routing) each workgroup keeps one item:
// walking measured 2-3 % slower there.
constexpr long long kSkinnyGrid = 1024;

template <typename Kern1, typename KernW>
static hipError_t launch_gemm(const char* name, Kern1 one, KernW walk_kern, int threads,
                              long long blocks, bool walk, const GemmArgs& a, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  if (walk && blocks > kSkinnyGrid) {
    MOE_LAUNCH(name, walk_kern, dim3((unsigned)kSkinnyGrid), dim3(threads), 0, s, a);
  } else {
    MOE_LAUNCH(name, one, dim3((unsigned)blocks), dim3(threads), 0, s, a);
  }
  return hipGetLastError();
}

template <bool DUAL, int NW, int CB>
static hipError_t launch_skinny_mx(const char* name, long long blocks, bool walk, const GemmArgs& a,
                                   hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  const bool w = walk && blocks > kSkinnyGrid;
  const dim3 grid((unsigned)(w ? kSkinnyGrid : blocks));
  const int K32 = a.K / 32;
#define MOE_SKMX(SM, SHM)                                                                          \
  {                                                                                                \
    if (w) MOE_LAUNCH(name, (k_skinny_mx<DUAL, NW, CB, SM, true>), grid, dim3(64 * NW), SHM, s, a); \
    else MOE_LAUNCH(name, (k_skinny_mx<DUAL, NW, CB, SM, false>), grid, dim3(64 * NW), SHM, s, a); \
  }
  if (a.K % 512 == 0 && a.K <= 8192) {
    constexpr int NB = (DUAL ? 2 : 1) * CB;
    const size_t shm = (size_t)(NW * NB * 16 + 16) * (K32 + 16);
    MOE_SKMX(2, shm)
  } else if (a.K % 512 == 0) {
    MOE_SKMX(1, 0)
  } else {
    MOE_SKMX(0, 0)
  }
#undef MOE_SKMX
  return hipGetLastError();
}

hipError_t launch_grouped_ffn(const FfnArgs& f, hipStream_t s) {
  const WsLayout L = ffn_layout(f.T, f.H, f.E, f.k, f.I, f.n_shared, f.fp8, f.mx);
  uint8_t* ws = static_cast<uint8_t*>(f.workspace);
  const Sched sc = ffn_schedule(f);
  const long long R = (long long)f.T * (f.k + f.n_shared);
  if (!f.planned) {
    MOE_LAUNCH("plan", k_plan, dim3(1), dim3(1024), 0, s, f.offsets, sc);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }

  uint8_t* h = ws + L.h;
  void* h_scale = f.fp8 ? static_cast<void*>(ws + L.h_scale) : nullptr;
  GemmArgs up{};
  up.sc = sc;
  up.offsets = f.offsets;
  up.a_rows = f.a_rows;
  up.A = static_cast<const uint8_t*>(f.x_perm);
  up.A_scale = f.x_perm_scale;
  up.B0 = static_cast<const uint8_t*>(f.w_gate);
  up.B1 = static_cast<const uint8_t*>(f.w_up);
  up.s_B0 = f.s_gate;
  up.s_B1 = f.s_up;
  up.out = h;
  up.out_scale = h_scale;
  up.K = f.H;
  up.N = f.I;
  up.R = (int)R;
  up.s_rows = f.s_rows;           // fp8 activation scales, K-block-major
  up.s_ld = f.s_ld ? f.s_ld : (int)R;

  GemmArgs dn = up;
  dn.a_rows = nullptr;            // h (and its scales, [I/128][R]) in permuted row order
  dn.s_rows = nullptr;
  dn.s_ld = (int)R;
  dn.A = h;
  dn.A_scale = h_scale;
  dn.B0 = static_cast<const uint8_t*>(f.w_down);
  dn.B1 = nullptr;
  dn.s_B0 = f.s_down;
  dn.s_B1 = nullptr;
  dn.out = static_cast<uint8_t*>(f.y_perm);
  dn.out_scale = nullptr;
  dn.K = f.I;
  dn.N = f.H;

  // No group above the skinny limit: no tiled work, skip its launches (decode).
  const bool tiled = f.max_group_rows > skinny_max_rows(f.T);
  // The streaming chain gets a stream of its own only when the routing is
  // expected to leave real work for it next to the tiled one (mean rows per
  // group at most twice the skinny limit, e.g. the Zipf-routed Qwen3.5-like
  // layer: 20); with larger groups nearly every group is tiled, and the
  // mostly empty streaming launches then cost more concurrently than after
  // the tiled chain on one stream (DeepSeek-like layer 2.86 -> 2.83 ms,
  // Qwen3-like prefill 2.66 -> 2.645; the Zipf layer 1.41 -> 1.44 on one).
  const long long mean_rows = (long long)f.T * f.k / std::max(1, f.E);
  const bool mixed = mean_rows <= 2LL * skinny_max_rows(f.T);
  SideStream* side = tiled && mixed && !prof_serial() && !f.one_stream ? side_stream(0) : nullptr;
  const bool walk = tiled && !mixed;   // streaming grids capped and walked (see kSkinnyGrid)
  hipStream_t ks = s;                // stream of the streaming chain
  if (side) {                        // fork after the plan
    hipError_t e = hipEventRecord(side->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
    if (e != hipSuccess) return e;
    ks = side->s;
  }

  // Every launch is checked before the next is enqueued; after a failed one
  // nothing more is launched, and the side stream is still joined back.
  hipError_t err = hipSuccess;
  auto run = [&](hipError_t e) { if (err == hipSuccess) err = e; return err == hipSuccess; };

  // The tiled chain runs on the caller's stream and is enqueued first: its
  // large workgroups (one per CU, each needing a CU free of other waves) start
  // before the weight-streaming workgroups, which wait for the fork event on
  // the side stream, fill the machine (Qwen3.5-like layer: 1.47 -> 1.42 ms
  // against the opposite assignment).
  const char* nm_tg = f.mx ? "tiled_gateup_mx" : f.fp8 ? "tiled_gateup_fp8" : "tiled_gateup_bf16";
  const char* nm_td = f.mx ? "tiled_down_mx" : f.fp8 ? "tiled_down_fp8" : "tiled_down_bf16";
  up.n_ntile = f.I / 128;
  dn.n_ntile = ceil_div(f.H, 256);
  // bf16 layers with small mean groups: the few tiled groups are
  // weight-streaming-bound and take the 3-stage 160-row kernel in bf16 (the
  // Qwen3.5-like layer 1.40 -> 1.36 ms, same bits); larger groups the
  // 256-row bf16 kernel.
  const bool bfs = bf16_stream_tiles(f.T, f.k, f.E, f.fp8);
  auto tiled_gemm = [&](const char* nm, bool dual, const GemmArgs& g) {
    const long long blocks = (long long)L.max_tiles * g.n_ntile;
    return f.fp8 ? launch_tiled8(nm, f.mx, dual, blocks, g, s)
                 : bfs ? launch_tiled8_bf16(nm, dual, blocks, g, s) : launch_tiled(nm, dual, blocks, g, s);
  };
  if (tiled && run(tiled_gemm(nm_tg, true, up))) run(tiled_gemm(nm_td, false, dn));

  // gate/up + SwiGLU, then down, of the groups of at most skinny_max_rows(T) rows
  if (err != hipSuccess) {
  } else if (f.fp8) {
    // Split-K only without tiled work (the layout reserved the partials then).
    const bool split = !tiled && (L.split_up > 1 || L.split_dn > 1);
    float* part = reinterpret_cast<float*>(ws + L.part);
    const int32_t* n_rows = f.offsets + (f.E + f.n_shared);
    up.ksplit = split ? L.split_up : 1;
    dn.ksplit = split ? L.split_dn : 1;
    up.R = dn.R = (int)R;
    up.part = dn.part = part;
    if (f.mx) {
      up.n_ntile = f.I / (16 * kMxCB * kMxNW);
      dn.n_ntile = f.H / (16 * kMxCBD * kMxNWD);
      run(launch_skinny_mx<true, kMxNW, kMxCB>("skinny_gateup_mx",
                                               band_grid(L.max_slices, up.n_ntile) * up.ksplit, walk, up, ks));
    } else {
      up.n_ntile = f.I / (16 * 8);
      dn.n_ntile = f.H / (16 * 4);
      run(launch_gemm("skinny_gateup_fp8", k_skinny_fp8<true, 8, 1, false>, k_skinny_fp8<true, 8, 1, true>,
                      512, band_grid(L.max_slices, up.n_ntile) * up.ksplit, walk, up, ks));
    }
    if (err == hipSuccess && up.ksplit > 1) {
      if (f.mx)
        MOE_LAUNCH("splitk_reduce_gateup", k_splitk_reduce_q8<true>, dim3(ceil_div(f.I, 1024), (unsigned)R),
                   dim3(256), 0, ks, part, up.ksplit, (int)R, f.I, n_rows, h, h_scale);
      else
        MOE_LAUNCH("splitk_reduce_gateup", k_splitk_reduce_q8<false>, dim3(ceil_div(f.I, 1024), (unsigned)R),
                   dim3(256), 0, ks, part, up.ksplit, (int)R, f.I, n_rows, h, h_scale);
      run(hipGetLastError());
    }
    if (err == hipSuccess) {
      if (f.mx)
        run(launch_skinny_mx<false, kMxNWD, kMxCBD>("skinny_down_mx",
                                                    band_grid(L.max_slices, dn.n_ntile) * dn.ksplit, walk, dn, ks));
      else
        run(launch_gemm("skinny_down_fp8", k_skinny_fp8<false, 4, 1, false>, k_skinny_fp8<false, 4, 1, true>,
                        256, band_grid(L.max_slices, dn.n_ntile) * dn.ksplit, walk, dn, ks));
    }
    if (err == hipSuccess && dn.ksplit > 1) {
      MOE_LAUNCH("splitk_reduce_down", k_splitk_reduce<false>, dim3(ceil_div(f.H, 1024), (unsigned)R),
                 dim3(256), 0, ks, part, dn.ksplit, (int)R, f.H, n_rows, static_cast<uint16_t*>(f.y_perm));
      run(hipGetLastError());
    }
  } else {
    // Split-K only without tiled work (the layout reserved the partials then).
    const bool split = !tiled && (L.split_up > 1 || L.split_dn > 1);
    float* part = reinterpret_cast<float*>(ws + L.part);
    const int32_t* n_rows = f.offsets + (f.E + f.n_shared);
    up.n_ntile = f.I / (16 * 4);
    up.ksplit = split ? L.split_up : 1;
    up.R = (int)R;
    up.part = part;
    dn.n_ntile = f.H / (32 * 4);
    dn.ksplit = split ? L.split_dn : 1;
    dn.R = (int)R;
    dn.part = part;
    if (run(launch_gemm("skinny_gateup_bf16", k_skinny_bf16<true, 4, 1, false>,
                        k_skinny_bf16<true, 4, 1, true>, 256,
                        band_grid(L.max_slices, up.n_ntile) * up.ksplit, walk, up, ks)) && up.ksplit > 1) {
      MOE_LAUNCH("splitk_reduce_gateup", k_splitk_reduce<true>, dim3(ceil_div(f.I, 1024), (unsigned)R),
                 dim3(256), 0, ks, part, up.ksplit, (int)R, f.I, n_rows, reinterpret_cast<uint16_t*>(h));
      run(hipGetLastError());
    }
    if (err == hipSuccess &&
        run(launch_gemm("skinny_down_bf16", k_skinny_bf16<false, 4, 1, false>,
                        k_skinny_bf16<false, 4, 1, true>, 256,
                        band_grid(L.max_slices, dn.n_ntile) * dn.ksplit, walk, dn, ks)) && dn.ksplit > 1) {
      MOE_LAUNCH("splitk_reduce_down", k_splitk_reduce<false>, dim3(ceil_div(f.H, 1024), (unsigned)R),
                 dim3(256), 0, ks, part, dn.ksplit, (int)R, f.H, n_rows,
                 static_cast<uint16_t*>(f.y_perm));
      run(hipGetLastError());
    }
  }
  if (side) {                        // join: the caller's stream waits for the streaming chain
    hipError_t e = hipEventRecord(side->join, side->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
    run(e);
  }
  return err;
}

}  // namespace moe
