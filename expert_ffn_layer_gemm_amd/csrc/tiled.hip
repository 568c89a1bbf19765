// LDS-pipelined tiled grouped GEMM for bf16 layers, for the groups too large
// for the weight-streaming kernels, more than 48 rows in batches of more than
// 64 tokens (prefill-sized groups, the shared expert, the hot experts of a
// skewed routing).  Computes, per (group, row tile, column tile):
//   DUAL:   h = silu(X W_gate^T) * (X W_up^T)    128 h columns (256 B rows)
//   single: y = h W_down^T                        256 output columns
// with fp32 accumulation.  SwiGLU in the epilogue follows the Ironwood page's
// GMM v2 (section 4.2.2): gate and up are two B streams of one workgroup.
// (8-bit layers have a kernel of their own, tiled8.hip.)
//
// gfx950 design:
//   - Row tile 256 x 256 staged B rows, 8 waves (2 per SIMD) laid out 2 x 4,
//     128 x 64 per wave: at 128 FLOP per staged byte the operand stream from
//     L2 stays below what the MFMA rate needs.
//   - K is staged in 128-byte chunks (64 bf16 per row) by direct-to-LDS loads
//     (global_load_lds_dwordx4) into two rings, activation rows and weight
//     rows, of 2 + 2 stages of 32 KB (one chunk in flight while one is
//     multiplied; 2 + 3 or 3 + 2 stages measured no faster).
//   - Software pipeline: a wave reads the LDS fragments of the next K step
//     while its MFMAs of the current one run (A row block i right after the
//     row block's last MFMA), and the chunk barrier sits inside a chunk's
//     second K step, after the wave's last read of the chunk and before its
//     first read of the next.  The direct-to-LDS loads are issued from inline
//     assembly so the compiler keeps exact lgkm-counter waits for the
//     interleaved reads (it cannot see a pending LDS write).  Measured 7-12 %
//     faster than reading a step's fragments then waiting, with bit-identical
//     output (same MFMA order per accumulator).
//   - A direct-to-LDS instruction writes 1 KB contiguously (lane i at +16 i),
//     8 staged rows; each block of 8 rows lies in A, B0 or B1 and has its own
//     wave-uniform base.  Each lane fetches global chunk c ^ (row & 7) of its
//     row so row r's chunk c sits in slot c ^ (r & 7).  Fragment reads (16
//     lanes on 16 consecutive rows, one chunk) with this slot map measured
//     conflict-free on gfx950 (the row-XOR variant (r ^ r >> 3) & 7 tried
//     first was not).
//   - Blocks are renumbered so each XCD (own L2) takes a contiguous run of
//     tiles, and within a band of up to 8 row tiles of a group the order is
//     column tile major, row tile fastest: the workgroups that stream one
//     weight slice are dispatched back to back and run in step on one L2
//     (measured: with row tiles 12-16 dispatches apart they drifted out of
//     step and every row tile re-read the weights from HBM).
//   - Rows past the group's end are not fetched (8-row blocks wholly past it)
//     or re-read its last row; they are never stored, and the fragment reads
//     and MFMAs of 16-row blocks wholly past the end are skipped.
#include "ffn.hpp"
#include "pipe.hpp"

namespace moe {
namespace {

constexpr int kBRows = 256;                       // staged B rows per tile
constexpr int kBf16NSA = 2, kBf16NSB = 2;        // bf16 A / B ring stages

// Slot of 16-byte chunk c of staged row r for rows of RB bytes: 128-byte rows
// c ^ (r & 7), 64-byte rows c ^ ((r >> 1) & 3) (both measured conflict-free
// for 16 lanes reading one chunk of 16 consecutive rows).
template <int RB>
__device__ __forceinline__ int slot(int r, int c) {
  if constexpr (RB == 128) return slot8(r, c);
  return c ^ ((r >> 1) & 3);
}

// Direct-to-LDS loads of this wave's IPW 1 KB blocks of one K chunk into a
// ring stage (wave-uniform base + 32-bit lane offset per block), through
// dma16_untracked: the compiler does not see these LDS writes, and the caller
// orders them with vm-counter waits and barriers.
template <int IPW>
__device__ __forceinline__ void dma_blocks_untracked(uint8_t* st, const uint8_t* const (&jb)[IPW],
                                                     const uint32_t (&soff)[IPW],
                                                     const bool (&jv)[IPW], size_t koff, int wave) {
#pragma unroll
  for (int j = 0; j < IPW; ++j)
    if (jv[j]) dma16_untracked(jb[j] + koff, soff[j], st + (wave * IPW + j) * 1024);
}

// Staged B row of 16-column block j (lane row r16) for wave column wn.
template <bool DUAL, int WN, int NB>
__device__ __forceinline__ int b_row(int j, int wn, int r16) {
  if constexpr (DUAL)
    return (j < NB / 2 ? wn * (128 / WN) + j * 16 : 128 + wn * (128 / WN) + (j - NB / 2) * 16) + r16;
  return wn * (256 / WN) + j * 16 + r16;
}

}  // namespace

template <bool DUAL, int WM, int WN, int BM, int NSA, int NSB, int RB>
__global__ __launch_bounds__(64 * WM * WN) void k_tiled3(const GemmArgs p) {
  // The body is device code only; the host pass needs just the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  // A (activation rows) and B (weight rows) have rings of their own: NSA and
  // NSB stages.  The vm-counter waits follow from the issue order: at every
  // chunk boundary A is issued before B.
  static_assert(NSA >= 2 && NSB >= 2 && (NSB == NSA || NSB == NSA + 1 || NSA == NSB + 1), "ring depths");
  constexpr int kRB = RB;                         // bytes of K per staged row and chunk
  constexpr int RPB = 1024 / RB;                  // staged rows per 1 KB DMA block
  constexpr int LPR = RB / 16;                    // lanes per staged row
  constexpr int kBM = BM;                         // rows per tile
  constexpr int NW = WM * WN;                     // waves per workgroup
  constexpr int MB = kBM / WM / 16;               // 16-row blocks per wave
  constexpr int NB = kBRows / WN / 16;            // 16-column blocks per wave
  constexpr int A_BYTES = kBM * kRB, B_BYTES = kBRows * kRB;
  constexpr int IPWA = A_BYTES / 1024 / NW;       // direct-to-LDS instructions per wave and chunk
  constexpr int IPWB = B_BYTES / 1024 / NW;
  static_assert(IPWA * NW * 1024 == A_BYTES && IPWB * NW * 1024 == B_BYTES,
                "a chunk must split evenly over the waves");
  constexpr int A_STAGE = A_BYTES;
  constexpr int B_STAGE = B_BYTES;
  constexpr int B_RING = NSA * A_STAGE;           // byte offset of the B ring
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSA * A_STAGE + NSB * B_STAGE];

  int tslot, nt;
  if (!band_item(p.sc.tiles, *p.sc.n_tiles, p.n_ntile, tslot, nt)) return;
  const int g = p.sc.tiles[4 * tslot], m0 = p.sc.tiles[4 * tslot + 1];
  const int row0 = p.offsets[g] + m0;
  const int gm = p.offsets[g + 1] - p.offsets[g];
  const int mrows = min(group_tile_rows(gm, kBM), gm - m0);
  const int K = p.K, N = p.N;
  const size_t Kb = 2 * (size_t)K;                 // bytes per row
  const int nk = (int)(Kb / kRB);
  const int tid = threadIdx.x, lane = tid & 63;
  // Wave index as a scalar: keeps every per-wave condition a scalar branch.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int n0 = nt * (DUAL ? 128 : 256);
  const int ncols = DUAL ? 128 : min(256, N - n0);
  const int r16 = lane & 15;

  // Sources of the 1 KB blocks (RPB staged rows each) this wave moves per
  // chunk: A block a = wave * IPWA + j holds tile rows RPB a .., B block
  // b = wave * IPWB + j staged B rows RPB b .., all in B0 or all in B1; each
  // has a wave-uniform base plus a 32-bit lane offset.  A blocks wholly past
  // the group's end are not fetched (their LDS rows keep stale data from
  // earlier chunks; those outputs are never stored).
  const uint8_t* ab[IPWA];
  uint32_t aoff[IPWA];
  bool av[IPWA];
  int nva = 0;                                     // vm instructions per A chunk of this wave
#pragma unroll
  for (int j = 0; j < IPWA; ++j) {
    const int brow0 = (wave * IPWA + j) * RPB;
    const int row = brow0 + lane / LPR;
    const uint32_t sl = (uint32_t)(slot<RB>(row, lane % LPR) * 16);
    av[j] = brow0 < mrows;
    const int r = min(row, mrows - 1);
    // With a_rows the tile's rows are gathered from the unpermuted matrix.
    ab[j] = p.a_rows ? p.A : p.A + (size_t)row0 * Kb;
    aoff[j] = (p.a_rows ? (uint32_t)p.a_rows[row0 + r] : (uint32_t)r) * (uint32_t)Kb + sl;
    nva += av[j] ? 1 : 0;
  }
  const uint8_t* bb[IPWB];
  uint32_t boff[IPWB];
  bool bv[IPWB];
#pragma unroll
  for (int j = 0; j < IPWB; ++j) {
    int br = (wave * IPWB + j) * RPB;
    const uint8_t* B = p.B0;
    if (DUAL && br >= 128) { B = p.B1; br -= 128; }
    const int row = (wave * IPWB + j) * RPB + lane / LPR;
    const uint32_t sl = (uint32_t)(slot<RB>(row, lane % LPR) * 16);
    bv[j] = true;
    bb[j] = B + (size_t)g * N * Kb;
    // Rows past the matrix (ragged last column tile) re-read its last row.
    boff[j] = (uint32_t)min(n0 + br + lane / LPR, N - 1) * (uint32_t)Kb + sl;
  }

  // 16-row blocks of the wave holding valid rows.
  const int rbase = wm * (kBM / WM);
  const int nmb = max(0, min(MB, ceil_div(mrows - rbase, 16)));
  const bool has_cols = DUAL || wn * (256 / WN) < ncols;
  const bool active = nmb > 0 && has_cols;

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  {
  // bf16: the software-pipelined main loop (file header), for the wave's
  // valid row blocks only.
  static_assert(RB == 128 && MB == 8, "bf16 pipeline layout");
  // chunk c: A in stage c % NSA of the A ring, B in stage c % NSB of the B ring
  auto sa = [&](int c) { return lds + (c % NSA) * A_STAGE; };
  auto sb = [&](int c) { return lds + B_RING + (c % NSB) * B_STAGE; };
  auto issue_a = [&](int c) { dma_blocks_untracked<IPWA>(sa(c), ab, aoff, av, (size_t)c * kRB, wave); };
  auto issue_b = [&](int c) { dma_blocks_untracked<IPWB>(sb(c), bb, boff, bv, (size_t)c * kRB, wave); };
  // Prologue: A chunks 0 .. NSA-1 and B chunks 0 .. NSB-1, A before B per chunk.
#pragma unroll
  for (int c = 0; c < (NSA > NSB ? NSA : NSB); ++c) {
    if (c < NSA && c < nk) issue_a(c);
    if (c < NSB && c < nk) issue_b(c);
  }
  // Chunk c >= 1 is awaited at the boundary of chunk c - 1.  Loads complete
  // in issue order, so the wave may leave in flight what it issued after the
  // later of A(c), B(c): with NSB >= NSA that is A(c) (A(c+1 .. c+NSA-2) and
  // B(c+1 .. c+NSB-2) follow it), with NSA = NSB + 1 it is B(c)
  // (A(c+2 .. c+NSA-2) and B(c+1 .. c+NSB-2) follow it); chunks past the
  // last are never issued.
  constexpr int XA = NSA <= NSB ? NSA - 2 : NSA - 3;
  constexpr int XB = NSB - 2;
  auto wait_chunk = [&](int c) {   // A and B of chunk c landed (this wave's share)
    const int xa = NSA <= NSB ? min(XA, nk - 1 - c) : min(XA, nk - 2 - c);
    wait_vmcnt_le<XA * IPWA + XB * IPWB>(max(0, xa) * nva + max(0, min(XB, nk - 1 - c)) * IPWB);
  };
  // Chunk 0: the prologue issued A(1 .. NSA-1) and B(1 .. NSB-1) after it.
  wait_vmcnt_le<(NSA - 1) * IPWA + (NSB - 1) * IPWB>(min(NSA - 1, nk - 1) * nva +
                                                     min(NSB - 1, nk - 1) * IPWB);
  lds_barrier();
  auto rd_b = [&](const uint8_t* st, int ks, u32x4_t (&b)[NB]) {
    const int c = ks * 4 + (lane >> 4);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int br = b_row<DUAL, WN, NB>(j, wn, r16);
      b[j] = lds_read16(st + br * kRB + (slot<RB>(br, c) << 4));
    }
  };
  auto rd_a = [&](const uint8_t* st, int ks, int i) {
    const int c = ks * 4 + (lane >> 4);
    const int r = rbase + i * 16 + r16;
    return lds_read16(st + r * kRB + (slot<RB>(r, c) << 4));
  };
  auto boundary = [&](int kc) {   // after every wave's last read of chunk kc
    if (kc + 1 < nk) wait_chunk(kc + 1);
    lds_barrier();
    if (kc + NSA < nk) issue_a(kc + NSA);
    if (kc + NSB < nk) issue_b(kc + NSB);
  };
  // The main loop, compiled once per count NMB of valid row blocks of the
  // wave (0: the wave only takes part in the loads and barriers).
  auto main_loop = [&](auto nm) {
    constexpr int NMB = decltype(nm)::value;
    if constexpr (NMB == 0) {
      for (int kc = 0; kc < nk; ++kc) boundary(kc);
    } else {
      constexpr int H = NMB / 2;   // row blocks of K step 1 multiplied before the boundary
      u32x4_t a[MB], bc[NB], bn[NB];
      rd_b(sb(0), 0, bc);
#pragma unroll
      for (int i = 0; i < NMB; ++i) a[i] = rd_a(sa(0), 0, i);
      // sched_barrier(0) keeps the compiler from regrouping the reads and
      // MFMAs: each read is issued while the MFMA pipe works on the row block
      // before it.
      auto chunk = [&](int kc, auto last_c) {
        constexpr bool last = decltype(last_c)::value;
        const uint8_t* st = sa(kc);
        const uint8_t* sn = sa(kc + 1);
        const uint8_t* bt = sb(kc);
        const uint8_t* bnx = sb(kc + 1);
        // K step 0 of chunk kc; reads of step 1 (B over the first two row
        // blocks, or all of it after the first when there is one).
#pragma unroll
        for (int i = 0; i < NMB; ++i) {
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = mfma_bf16_16x16x32(a[i], bc[j], acc[i][j]);
          if (i < 2) {
            const int c = 4 + (lane >> 4);
            constexpr int JB = NMB >= 2 ? NB / 2 : NB;
#pragma unroll
            for (int j = JB * i; j < JB * i + JB; ++j) {
              const int br = b_row<DUAL, WN, NB>(j, wn, r16);
              bn[j] = lds_read16(bt + br * kRB + (slot<RB>(br, c) << 4));
            }
          }
          a[i] = rd_a(st, 1, i);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) bc[j] = bn[j];
        // K step 1: first half, the chunk boundary, then the second half with
        // the reads of the next chunk's step 0.
#pragma unroll
        for (int i = 0; i < H; ++i) {
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = mfma_bf16_16x16x32(a[i], bc[j], acc[i][j]);
          __builtin_amdgcn_sched_barrier(0);
        }
        boundary(kc);
        if constexpr (!last) {
          rd_b(bnx, 0, bn);
#pragma unroll
          for (int i = 0; i < H; ++i) a[i] = rd_a(sn, 0, i);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = H; i < NMB; ++i) {
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = mfma_bf16_16x16x32(a[i], bc[j], acc[i][j]);
          if constexpr (!last) a[i] = rd_a(sn, 0, i);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) bc[j] = bn[j];
      };
      for (int kc = 0; kc + 1 < nk; ++kc) chunk(kc, std::false_type{});
      chunk(nk - 1, std::true_type{});
    }
  };
  with_count<MB>(active ? nmb : 0, main_loop);
  }

  // Epilogue.  Lane holds rows rbase + 16 i + 4 (lane/16) + q of its blocks.
  // The output tile is assembled in LDS (the ring stages are free once every
  // wave is past its last read) and written out in 16-byte row pieces rather
  // than the lanes' own 2-byte elements (8x fewer store instructions, no
  // partial-line writes).
  constexpr int OUT_B = 2;                           // bytes per output element (bf16)
  constexpr int OCOLS = DUAL ? 128 : 256;            // output columns per tile
  constexpr int ROWB = OCOLS * OUT_B;                // bytes per tile row: 256 or 512
  constexpr int NCH = ROWB / 16;                     // 16-byte pieces per row
  static_assert(kBM * ROWB <= (int)sizeof(lds), "output tile fits in LDS");
  uint8_t* const tile = lds;
  // Piece (r, c / (16 / OUT_B)) sits at piece index c16 ^ (r % NCH): the
  // 4 rows a store instruction covers (4 apart) fall on different banks.
  auto tile_at = [&](int r, int c) {
    const int byte = c * OUT_B;
    return tile + r * ROWB + ((((byte >> 4) ^ (r % NCH))) << 4) + (byte & 15);
  };
  lds_barrier();                                      // every wave is past its last stage read
  if (active) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
      if (i < nmb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rbase + i * 16 + (lane >> 4) * 4 + q;
          if constexpr (DUAL) {
#pragma unroll
            for (int j = 0; j < NB / 2; ++j)
              *reinterpret_cast<uint16_t*>(tile_at(r, wn * (128 / WN) + j * 16 + r16)) =
                  (uint16_t)f32_to_bf16_bits(silu_mul(acc[i][j][q], acc[i][j + NB / 2][q]));
          } else {
#pragma unroll
            for (int j = 0; j < NB; ++j)
              *reinterpret_cast<uint16_t*>(tile_at(r, wn * (256 / WN) + j * 16 + r16)) =
                  (uint16_t)f32_to_bf16_bits(acc[i][j][q]);
          }
        }
      }
  }
  lds_barrier();
  // Rows past the group's end and columns past the matrix are not written.
  const int nch = ncols * OUT_B / 16;
  uint8_t* const out = p.out + ((size_t)row0 * N + n0) * OUT_B;
  for (int idx = tid; idx < mrows * NCH; idx += 64 * NW) {
    const int r = idx / NCH, ch = idx % NCH;
    if (ch < nch)
      *reinterpret_cast<u32x4_t*>(out + (size_t)r * N * OUT_B + ch * 16) =
          *reinterpret_cast<const u32x4_t*>(tile + r * ROWB + ((ch ^ (r % NCH)) << 4));
  }
#else
  (void)p;
#endif
}

hipError_t launch_tiled(const char* name, bool dual, long long blocks, const GemmArgs& a, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)band_grid(blocks, 1));
  // 256-row tiles (compute-bound prefill groups), 2 + 2 stages.  The row
  // count matches tile_rows() used by the schedule.
  static_assert(tile_rows(false, false) == 256, "bf16 tile height");
  if (dual) MOE_LAUNCH(name, (k_tiled3<true, 2, 4, 256, kBf16NSA, kBf16NSB, 128>), grid, dim3(512), 0, s, a);
  else MOE_LAUNCH(name, (k_tiled3<false, 2, 4, 256, kBf16NSA, kBf16NSB, 128>), grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
