// LDS-pipelined tiled grouped GEMM for 8-bit layers (e4m3 codes with fp32
// 128 x 128 block scales, or MXFP8 with E8M0 scales per 32 values), for the
// groups too large for the weight-streaming kernels.  Per (group, row tile,
// column tile) it computes
//   DUAL:   h = silu(X W_gate^T) * (X W_up^T)    128 h columns, re-quantised
//   single: y = h W_down^T                        256 output columns, bf16
// with fp32 accumulation.  fp8: each 128-wide K block's MFMA partial is scaled
// by the row's activation scale times the weight block's scale ("Lower latency
// and higher throughput with multi-node DeepSeek deployment", Quantization);
// MXFP8: the E8M0 scales ride the scaled MFMA ("Hosting Qwen on Blackwell",
// Quantization).  SwiGLU in the epilogue follows the Ironwood page's GMM v2
// (section 4.2.2): gate and up are two B streams of one workgroup.
//
// gfx950 design.  These layers are memory-bound (a ~128-row expert group
// reads 29 MB of weights for 7.5 GFLOP, about 256 FLOP per byte against the
// 625 of fp8's ridge), so the kernel is a load pipeline that keeps two
// chunks of whole 128-byte row pieces in flight per CU with the MFMAs, the
// per-block scaling and the epilogue overlapped as far as its LDS allows:
//   - Row tile BM (MXFP8 128, fp8 160) x 256 staged B rows, 8 waves (2 per SIMD) laid
//     out 2 x 4; K staged in 128-byte chunks (one 16x16x128 MFMA step) by
//     direct-to-LDS loads of whole 128-byte row pieces into a 3-stage A ring
//     and a 3-stage B ring (two chunks in flight while one is multiplied).
//     A 160-row tile keeps a DeepSeek-like routed group (mean 128 rows) in
//     one tile, so its weights are streamed once.
//   - Scales travel in groups of SG chunks: every SG-th chunk, the first
//     waves load, per A row (and per B row for MX, or the two weight-block
//     scale rows for fp8), the scales of the next SG chunks.  fp8 activation
//     scales are stored K-block-major (one K block's scales of consecutive
//     rows adjacent), so a chunk's row scales are a few whole cache lines
//     instead of one line per row (3 % per DeepSeek-like layer).  MXFP8 with K a
//     multiple of 512 uses SG = 4 (one 16-byte request per row per 4 chunks
//     instead of four 4-byte ones); fp8 uses SG = 1, since 160-row tiles
//     leave no LDS for 4-chunk scale stages.  A scale stage is reused SG
//     chunks later, so NSS = ceil((NS + SG - 1) / SG) stages suffice.
//   - Chunk c's loads are issued after the boundary of chunk c - NS (the
//     workgroup barrier that ends every wave's reads of those stages), one
//     part between each two columns of the second half's MFMAs; each wave
//     waits with explicit vm-counter counts (its own loads land in issue
//     order), then an LDS-only barrier publishes the chunk.
//   - Every wave issues the same number of loads for every chunk index: A
//     blocks past the tile and the scale loads of waves (or chunks) without
//     one go to a 1 KB LDS sink (MX scale stand-ins read one line with all
//     lanes), and the chunks after the last re-read the last one.  All waits
//     are then compile-time counts, and the loop carries
//     no per-wave or per-chunk bookkeeping (a scalar branch tree per wait,
//     stage indices by division, masked scale loads): with one loop copy per
//     count of valid row blocks it runs about 40 % fewer instructions per
//     chunk, which is what the waves' issue slots were spent on.
//   - fp8 computes D = B A^T (weights times activations): a lane's four
//     outputs of a 16 x 16 block are then four consecutive columns of one
//     row, so one activation scale times one weight-block scale rescales them
//     (one multiply per block instead of four; 6 % faster per layer, same
//     bits), and the epilogue writes 4 or 8 bytes per block and lane.
//   - Software pipeline: a wave reads the A fragments of the second half of
//     its row blocks before the boundary, multiplies the first half, passes
//     the boundary, reads the next chunk's A fragments of the first half, and
//     multiplies the second half column by column, reading the next chunk's B
//     fragment j as soon as column j is done.  Row blocks past the group's end
//     are not multiplied: the loop is compiled once per count of valid row
//     blocks.
//   - A direct-to-LDS instruction writes 1 KB (8 staged rows of 128 B; lane i
//     at +16 i); row r's 16-byte piece c sits in slot c ^ (r & 7), which makes
//     the fragment reads (16 lanes on 16 rows, one piece) conflict-free.
//   - XCD-contiguous block numbering and band order as in the bf16 kernel.
#include "ffn.hpp"
#include "pipe.hpp"

namespace moe {
namespace {

constexpr int k8BRows = 256;   // staged B rows per tile
constexpr int k8NS = 3;        // ring stages of A and of B
constexpr int kPersistGrid = 256;   // persistent fp8 kernel: one workgroup per CU

// Direct-to-LDS load of `BYTES` (4 or 16) bytes per lane from the lane's own
// address: lane i writes dst + BYTES * i.  Issued from inline assembly, like
// dma16_untracked (the caller orders it with vm-counter waits and barriers).
template <int BYTES>
__device__ __forceinline__ void dma_addr_untracked(const void* src, uint8_t* dst) {
  const uint32_t la = (uint32_t)(size_t)(lds_ptr_t)dst;
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(la), "v"(src) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :: "s"(la), "v"(src) : "memory", "m0");
}

// Staged B row of 16-column block j (lane row r16) for wave column wn
// (4 wave columns, 4 blocks each).
template <bool DUAL>
__device__ __forceinline__ int b8_row(int j, int wn, int r16) {
  if constexpr (DUAL) return (j < 2 ? wn * 32 + j * 16 : 128 + wn * 32 + (j - 2) * 16) + r16;
  return wn * 64 + j * 16 + r16;
}

}  // namespace

// LDS bytes of one configuration (static: checked against the 160 KB limit).
template <bool MX, int BM, int SG>
struct Tiled8Lds {
  static constexpr int A_BYTES = BM * 128;
  static constexpr int B_BYTES = k8BRows * 128;
  static constexpr int SROWS = MX ? BM + k8BRows : BM + 2;   // scale rows of a stage
  static constexpr int SB = 4 * SG;                           // bytes per scale row and stage
  static constexpr int NSC = (SROWS + 63) / 64;               // waves that load scales
  // A scale stage has a slot for every lane of those waves (lanes past the
  // scale rows load a duplicate into their own slot, so no lane is masked).
  static constexpr int SSTAGE = (NSC * 64 * SB + 255) / 256 * 256;
  static constexpr int NSS = (k8NS + SG - 1 + SG - 1) / SG;  // scale stages
  // 1 KB sink for the loads that only keep every wave's load count equal.
  static constexpr int SINK = k8NS * A_BYTES + k8NS * B_BYTES + NSS * SSTAGE;
  static constexpr int TOTAL = SINK + 1024;
};

template <bool MX, bool DUAL, int BM, int SG, bool BF = false>
__global__ __launch_bounds__(512) void k_tiled8(const GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using L = Tiled8Lds<MX, BM, SG>;
  static_assert(L::TOTAL <= 160 * 1024, "LDS budget");
  static_assert(SG == 1 || (SG == 4 && L::NSS == 2), "4-byte scale loads, or 16-byte ones in 2 stages");
  constexpr int NS = k8NS;
  constexpr int NW = 8, WN = 4;
  constexpr int MB = BM / 32;                       // 16-row blocks per wave (2 wave rows)
  constexpr int NB = 4;                             // 16-column blocks per wave
  constexpr int HA = MB / 2;                        // row blocks multiplied before the boundary
  constexpr int A_BLK = BM / 8;                     // 1 KB DMA blocks of an A chunk
  constexpr int IPWA = (A_BLK + NW - 1) / NW;       // A blocks per wave (block j * NW + wave)
  constexpr int IPWB = L::B_BYTES / 1024 / NW;
  constexpr int NSC = L::NSC;
  static_assert(NSC <= NW, "scale rows");
  static_assert(IPWB == NB && IPWA <= NB, "one load part per column");
  // Every wave issues exactly OPS loads for every chunk index: A blocks past
  // the tile and scale loads of waves or chunks without one go to the sink,
  // chunks past the end re-read the last chunk.  Every vm-counter wait is then
  // a compile-time count (no per-wave or per-chunk bookkeeping in the loop).
  static_assert(!(BF && MX), "bf16 operands carry no scales");
  constexpr int OPS = IPWA + IPWB + (BF ? 0 : 1);
  constexpr int B_RING = NS * L::A_BYTES;
  constexpr int S_RING = B_RING + NS * L::B_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::TOTAL];
  uint8_t* const sink = lds + L::SINK;

  int tslot, nt;
  if (!band_item(p.sc.tiles, *p.sc.n_tiles, p.n_ntile, tslot, nt)) return;
  const int g = p.sc.tiles[4 * tslot], m0 = p.sc.tiles[4 * tslot + 1];
  const int row0 = p.offsets[g] + m0;
  const int gm = p.offsets[g + 1] - p.offsets[g];
  const int mrows = min(group_tile_rows(gm, BM), gm - m0);
  const int K = p.K, N = p.N;
  const int KBY = BF ? 2 * K : K;                   // bytes per operand row
  const int nk = KBY / 128;
  const int KB = K / 128;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int n0 = nt * (DUAL ? 128 : 256);
  const int ncols = DUAL ? 128 : min(256, N - n0);
  const int r16 = lane & 15;

  // A DMA blocks of this wave: block a = j * NW + wave holds tile rows
  // 8a .. 8a+7; rows past the group's end re-read its last row (never
  // stored), blocks past the tile load into the sink.
  const uint8_t* const ab = p.a_rows ? p.A : p.A + (size_t)row0 * KBY;
  uint32_t aoff[IPWA];
  bool ain[IPWA];
#pragma unroll
  for (int j = 0; j < IPWA; ++j) {
    const int blk = j * NW + wave;
    const int row = blk * 8 + lane / 8;
    const uint32_t sl = (uint32_t)(slot8(row, lane % 8) * 16);
    ain[j] = blk < A_BLK;
    const int r = min(row, mrows - 1);
    aoff[j] = (p.a_rows ? (uint32_t)p.a_rows[row0 + r] : (uint32_t)r) * (uint32_t)KBY + sl;
  }
  // B: this wave's 32 staged rows come from one matrix (DUAL: waves 0-3 the
  // gate rows, 4-7 the up rows).
  const uint8_t* bb;
  uint32_t boff[IPWB];
  {
    int br0 = wave * IPWB * 8;
    const uint8_t* B = p.B0;
    if (DUAL && br0 >= 128) { B = p.B1; br0 -= 128; }
    bb = B + (size_t)g * N * KBY;
#pragma unroll
    for (int j = 0; j < IPWB; ++j) {
      const int row = (wave * IPWB + j) * 8 + lane / 8;
      const uint32_t sl = (uint32_t)(slot8(row, lane % 8) * 16);
      // Rows past the matrix (ragged last column tile) re-read its last row.
      boff[j] = (uint32_t)min(n0 + br0 + j * 8 + lane / 8, N - 1) * (uint32_t)KBY + sl;
    }
  }

  // Scale row of this lane (waves < NSC; sr = srow clamped to the rows
  // there are): sr < BM the A row's scales; fp8: sr = BM, BM+1 the two
  // weight-block scale rows of the tile (DUAL: gate, up; single: the tile's
  // two 128-column blocks); MX: sr = BM + b the E8M0 row of staged B row b.
  // A stage holds SB bytes per lane: chunks SG*q .. SG*q+SG-1 of the row's
  // scales (4 bytes per chunk).  Waves >= NSC compute a valid address too
  // (their loads go to the sink).
  const int srow = wave * 64 + lane;
  const int sr = min(srow, L::SROWS - 1);
  const bool swave = wave < NSC;
  const uint8_t* ssrc = nullptr;
  uint32_t sstep = 4;                                // bytes from one chunk's scale to the next
  if constexpr (!BF) {
    const int N128 = N / 128;
    if (sr < BM) {
      const int r = row0 + min(sr, mrows - 1);
      if constexpr (MX) {
        const size_t ar = (size_t)(p.a_rows ? p.a_rows[r] : r);
        ssrc = static_cast<const uint8_t*>(p.A_scale) + ar * (size_t)(4 * KB);
      } else {                                       // K-block-major: a chunk's row scales adjacent
        const size_t ar = (size_t)(p.s_rows ? p.s_rows[r] : r);
        ssrc = static_cast<const uint8_t*>(p.A_scale) + ar * 4;
        sstep = 4u * (uint32_t)p.s_ld;
      }
    } else if constexpr (MX) {
      int br = sr - BM;
      const uint8_t* sB = static_cast<const uint8_t*>(p.s_B0);
      if (DUAL && br >= 128) { sB = static_cast<const uint8_t*>(p.s_B1); br -= 128; }
      ssrc = sB + ((size_t)g * N + min(n0 + br, N - 1)) * (size_t)(K / 32);
    } else {
      const int which = sr - BM;
      if (DUAL)
        ssrc = static_cast<const uint8_t*>(which ? p.s_B1 : p.s_B0) +
               ((size_t)g * N128 + nt) * (size_t)(4 * KB);
      else
        ssrc = static_cast<const uint8_t*>(p.s_B0) +
               ((size_t)g * N128 + min(n0 / 128 + which, N128 - 1)) * (size_t)(4 * KB);
    }
  }

  // Ring positions: chunk c sits in A and B stage c % NS (kept as a running
  // stage index, not recomputed) and in scale stage (c / SG) % NSS.
  auto a_st = [&](int st) { return lds + st * L::A_BYTES; };
  auto b_st = [&](int st) { return lds + B_RING + st * L::B_BYTES; };
  auto s_st = [&](int c, int st) {
    const int ss = SG == 1 ? st : ((c >> 2) & 1);
    return lds + S_RING + ss * L::SSTAGE;
  };
  // Part j (of NB) of chunk c's loads into stage st: the scale load with part
  // 0, A block j (if any), B block j.  Chunk kc+NS's parts are issued between
  // the columns of chunk kc's second half (after its boundary, so its stages
  // are free): spread out, not as one burst after the barrier (measured 5 %
  // faster on the DeepSeek-like layer, same output bits).
  // MX: three chunks in four have no scale load of their own (16-byte loads
  // cover SG = 4 chunks); the loads that stand in for them only keep the
  // counts, and have every lane read what lane 63 reads for the chunk group,
  // one line instead of 64 (MXFP8 prefill 2.25 -> 1.94 ms).  fp8 (SG = 1)
  // has stand-ins only in the waves past the scale rows, whose lanes all
  // read one address anyway.
  const uint8_t* const ssrc_pad = reinterpret_cast<const uint8_t*>(
      ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(reinterpret_cast<uint64_t>(ssrc) >> 32), 63) << 32) |
      (uint32_t)__builtin_amdgcn_readlane((int)reinterpret_cast<uint64_t>(ssrc), 63));
  auto issue_part = [&](int c, int st, int j) {
    const int cc = min(c, nk - 1);
    if (!BF && j == 0) {
      const bool real = swave && c % SG == 0;
      uint8_t* const dst = real ? s_st(c, st) + wave * 64 * L::SB : sink;
      const size_t sk = (size_t)(cc - cc % SG);
      dma_addr_untracked<L::SB>((real || !MX ? ssrc : ssrc_pad) + sk * sstep, dst);
    }
    if (j < IPWA) {
      const int ja = j < IPWA ? j : 0;
      uint8_t* const dst = ain[ja] ? a_st(st) + (ja * NW + wave) * 1024 : sink;
      dma16_untracked(ab + (size_t)cc * 128, aoff[ja], dst);
    }
    dma16_untracked(bb + (size_t)cc * 128, boff[j], b_st(st) + (wave * IPWB + j) * 1024);
  };
#pragma unroll
  for (int c = 0; c < NS; ++c)
#pragma unroll
    for (int j = 0; j < NB; ++j) issue_part(c, c, j);
  wait_vmcnt<(NS - 1) * OPS>();                      // chunk 0 is in
  lds_barrier();

  // Valid 16-row blocks of this wave (0 for a wave without columns).
  const int rbase = wm * (BM / 2);
  const bool has_cols = DUAL || wn * 64 < ncols;
  const int nmb = has_cols ? max(0, min(MB, ceil_div(mrows - rbase, 16))) : 0;

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A lane's 32 codes: K bytes 16*(lane/16) .. +16 and 64 + 16*(lane/16) .. +16
  // (the same positions for A and B, so the pairing inside the MFMA is right).
  // Every 16-row block starts at a multiple of 8 rows, so the slot map of the
  // lane's row depends on r16 only: a fragment read is a per-stage base (one
  // add per stage and ring) plus a compile-time offset per block.
  const int c0 = lane >> 4, c1 = 4 + (lane >> 4);
  const int sh = 8 * (lane >> 4);                  // MX: byte of this lane's K block
  const uint32_t a_lo0 = (uint32_t)((rbase + r16) * 128 + (slot8(r16, c0) << 4));
  const uint32_t a_hi0 = (uint32_t)((rbase + r16) * 128 + (slot8(r16, c1) << 4));
  const int brow0 = b8_row<DUAL>(0, wn, r16);
  const uint32_t b_lo0 = (uint32_t)(B_RING + brow0 * 128 + (slot8(r16, c0) << 4));
  const uint32_t b_hi0 = (uint32_t)(B_RING + brow0 * 128 + (slot8(r16, c1) << 4));
  const uint32_t s_a0 = (uint32_t)(S_RING + (rbase + r16) * L::SB);   // A row scales
  const uint32_t s_b0 = (uint32_t)(S_RING + (BM + brow0) * L::SB);    // MX: B row scales
  // opaque to the compiler, so the per-block offsets stay immediates
  auto opq = [](uint32_t v) { asm volatile("" : "+v"(v)); return v; };
  auto frag_at = [&](uint32_t lo, uint32_t hi) {
    const u32x4_t x = lds_read16(lds + lo), y = lds_read16(lds + hi);
    return i32x8_t{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                   (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
  };
  // LDS byte offset of scale stage of chunk c (ring stage st) plus the chunk's
  // dword inside a scale slot
  auto s_off = [&](int c, int st) {
    const int ss = SG == 1 ? st : ((c >> 2) & 1);
    return (uint32_t)(ss * L::SSTAGE + (c % SG) * 4);
  };
  auto ld32 = [&](uint32_t off) { return *reinterpret_cast<const uint32_t*>(lds + off); };

  i32x8_t a[MB], b[NB];
  uint32_t sam[MB], sbm[NB];                       // MX: E8M0 bytes
  // fp8 multiplies weights by activations (D = B A^T: a lane's four outputs
  // are four consecutive columns of one row, so one row scale and one block
  // scale cover them); MXFP8 activations by weights.
  float saf[MB];                                   // fp8: activation scale of the lane's row
  float sb_lo = 0.f, sb_hi = 0.f;                  // fp8: weight block scales
  // Per-stage read bases of chunk c in ring stage st.
  struct Bases { uint32_t alo, ahi, blo, bhi, sa, sb; };
  auto bases = [&](int c, int st) {
    const uint32_t so = s_off(c, st);
    return Bases{opq(a_lo0 + st * L::A_BYTES), opq(a_hi0 + st * L::A_BYTES),
                 opq(b_lo0 + st * L::B_BYTES), opq(b_hi0 + st * L::B_BYTES),
                 opq(s_a0 + so), MX ? opq(s_b0 + so) : 0u};
  };
  // Fragment reads (read unconditionally, also for the chunk after the last:
  // in-bounds LDS, never used).
  auto next_a = [&](const Bases& q, int i) {
    a[i] = frag_at(q.alo + i * 2048, q.ahi + i * 2048);
    if constexpr (MX) sam[i] = (ld32(q.sa + i * 16 * L::SB) >> sh) & 0xFFu;
    else if constexpr (!BF) saf[i] = __uint_as_float(ld32(q.sa + i * 16 * L::SB));
  };
  auto next_b = [&](const Bases& q, int j) {
    const int dr = b8_row<DUAL>(j, 0, 0);          // row offset of block j
    b[j] = frag_at(q.blo + dr * 128, q.bhi + dr * 128);
    if constexpr (MX) sbm[j] = (ld32(q.sb + dr * L::SB) >> sh) & 0xFFu;
  };
  auto rd_bsc = [&](int c, int st) {
    if constexpr (!MX && !BF) {
      const uint32_t o = S_RING + s_off(c, st) + BM * L::SB;
      const float s0 = __uint_as_float(ld32(o)), s1 = __uint_as_float(ld32(o + L::SB));
      sb_lo = DUAL ? s0 : (wn < 2 ? s0 : s1);
      sb_hi = DUAL ? s1 : sb_lo;
    }
  };

  // Partial tiles of the current column for the row blocks of one half.
  constexpr int HMAX = MB - HA;
  f32x4_t pr[2][HMAX];
  // MFMAs of row blocks [i0, i1) with B block j (blocks below the count nm)
  auto col = [&](int i0, int i1, int j, auto nm) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
      if (i < count_value(nm)) {
        if constexpr (MX) {
          acc[i][j] = mfma_mx8_16x16x128(a[i], b[j], acc[i][j], sam[i], sbm[j]);
        } else if constexpr (BF) {
          // The chunk's 64 bf16 values as two K = 32 steps: the lane's low 16
          // bytes are elements 8 (lane/16) .. +8, its high ones 32 + the same.
          const i32x8_t x = a[i], y = b[j];
          acc[i][j] = mfma_bf16_16x16x32(u32x4_t{(uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]},
                                         u32x4_t{(uint32_t)y[0], (uint32_t)y[1], (uint32_t)y[2], (uint32_t)y[3]},
                                         acc[i][j]);
          acc[i][j] = mfma_bf16_16x16x32(u32x4_t{(uint32_t)x[4], (uint32_t)x[5], (uint32_t)x[6], (uint32_t)x[7]},
                                         u32x4_t{(uint32_t)y[4], (uint32_t)y[5], (uint32_t)y[6], (uint32_t)y[7]},
                                         acc[i][j]);
        } else {
          pr[j & 1][i - i0] = mfma_fp8_16x16x128(b[j], a[i], f32x4_t{0.f, 0.f, 0.f, 0.f});
        }
      }
  };
  // fp8: acc += partial * (row scale * block scale)
  auto scale_col = [&](int i0, int i1, int j, auto nm) {
    if constexpr (!MX && !BF) {
      const float sbv = j < NB / 2 ? sb_lo : sb_hi;
#pragma unroll
      for (int i = i0; i < i1; ++i)
        if (i < count_value(nm)) {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][j][q] += pr[j & 1][i - i0][q] * (saf[i] * sbv);
        }
    }
  };

  auto main_loop = [&](auto nm) {
  // Prologue reads: chunk 0's B fragments, A of the first half, block scales.
  {
    const Bases q0 = bases(0, 0);
#pragma unroll
    for (int j = 0; j < NB; ++j) next_b(q0, j);
#pragma unroll
    for (int i = 0; i < HA; ++i) next_a(q0, i);
  }
  rd_bsc(0, 0);
  int st = 0;                                      // stage of chunk kc
  for (int kc = 0; kc < nk; ++kc) {
    const int sn = st == NS - 1 ? 0 : st + 1;      // stage of chunk kc + 1
    // A fragments of the second half (the stage is refilled at the boundary).
    {
      const Bases qk = bases(kc, st);
#pragma unroll
      for (int i = HA; i < MB; ++i) next_a(qk, i);
    }
    // First half: row blocks [0, HA), column by column; a column's partials
    // are scaled into the accumulators one column later.
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      col(0, HA, j, nm);
      if (j > 0) scale_col(0, HA, j - 1, nm);
    }
    scale_col(0, HA, NB - 1, nm);
    // Keep the first half ahead of the boundary (the compiler would sink it
    // past the wait and barrier otherwise): it runs while the wave waits.
#pragma unroll
    for (int i = 0; i < HA; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) asm volatile("" : "+v"(acc[i][j]));
    // Boundary of chunk kc: wait for chunk kc+1 (chunk kc+2's loads may be
    // in flight), barrier; then chunk kc+NS goes into the stages chunk kc used.
    wait_vmcnt<(NS - 2) * OPS>();
    lds_barrier();
    // The next chunk's A fragments of the first half (registers just freed).
    const Bases qn = bases(kc + 1, sn);
#pragma unroll
    for (int i = 0; i < HA; ++i) next_a(qn, i);
    __builtin_amdgcn_sched_barrier(0);
    // Second half, column by column; B fragment j of the next chunk is read
    // as soon as column j is done.
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      col(HA, MB, j, nm);
      issue_part(kc + NS, st, j);
      if (j > 0) scale_col(HA, MB, j - 1, nm);
      next_b(qn, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    scale_col(HA, MB, NB - 1, nm);
    rd_bsc(kc + 1, sn);
    st = sn;
  }
  };
  // One copy of the loop per count of valid row blocks: no row-block branch
  // inside (with the uniform load counts, the DeepSeek-like layer went from
  // 3.20 to 2.87 ms; runtime checks there cost a scalar branch per block and
  // column).
  with_count<MB>(nmb, main_loop);
  // The loads of the chunks past the end (re-reads into the ring and the
  // sink) land before the epilogue reuses the ring.
  wait_vmcnt<0>();

  // Epilogue.  MXFP8: the lane holds rows rbase + 16 i + 4 (lane/16) + q of
  // its blocks, column lane % 16; fp8: see below.
  // The output tile is assembled in LDS (the ring stages are free once every
  // wave is past its last read) and written out in 16-byte row pieces.
  constexpr int OUT_B = (DUAL && !BF) ? 1 : 2;       // bytes per output element
  constexpr int OCOLS = DUAL ? 128 : 256;            // output columns per tile
  constexpr int ROWB = OCOLS * OUT_B;                // bytes per tile row: 128 or 512
  constexpr int NCH = ROWB / 16;                     // 16-byte pieces per row
  constexpr int AMAX_BYTES = (DUAL && !MX && !BF) ? WN * BM * 4 : 0;
  static_assert(AMAX_BYTES + BM * ROWB <= L::TOTAL, "output tile fits in LDS");
  float* amax_s = reinterpret_cast<float*>(lds);     // [WN][BM]
  uint8_t* const tile = lds + AMAX_BYTES;
  auto tile_at = [&](int r, int c) {
    const int byte = c * OUT_B;
    return tile + r * ROWB + ((((byte >> 4) ^ (r % NCH))) << 4) + (byte & 15);
  };
  lds_barrier();                                      // every wave is past its last stage read
  if constexpr (MX && DUAL) {
    // The wave's 32 h columns are one MX block of each of its rows.
    const int N32 = N / 32;
    const int hc0 = n0 + wn * 32;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = rbase + i * 16 + (lane >> 4) * 4 + q;
        float hv[2], am = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          hv[j] = silu_mul(acc[i][j][q], acc[i][j + 2][q]);
          am = fmaxf(am, fabsf(hv[j]));
        }
        am = row16_max(am);
        if (i < nmb && r < mrows) {
          const uint32_t e8 = mx_e8m0(am);
          const float inv = mx_inv_scale(e8);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float qv = fminf(fmaxf(hv[j] * inv, -448.f), 448.f);
            *tile_at(r, wn * 32 + j * 16 + r16) = (uint8_t)f32_to_e4m3(qv);
          }
          if (r16 == 0) static_cast<uint8_t*>(p.out_scale)[(size_t)(row0 + r) * N32 + hc0 / 32] = (uint8_t)e8;
        }
      }
  } else if constexpr (DUAL && BF) {
    // bf16: the lane holds rows rbase + 16 i + 4 (lane/16) + q of its blocks,
    // column lane % 16; h = silu(g) * u rounded to bf16.
#pragma unroll
    for (int i = 0; i < MB; ++i)
      if (i < nmb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rbase + i * 16 + (lane >> 4) * 4 + q;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            *reinterpret_cast<uint16_t*>(tile_at(r, wn * 32 + j * 16 + r16)) =
                (uint16_t)f32_to_bf16_bits(silu_mul(acc[i][j][q], acc[i][j + 2][q]));
        }
      }
  } else if constexpr (DUAL) {
    // fp8 (D = B A^T): per row block i and column block j the lane holds row
    // m = rbase + 16 i + lane % 16 and columns 4 (lane / 16) + q of the block.
    // h = silu(g) * u; per-row maxima over the tile's 128 columns: the lane's
    // 8 values, the 4 lanes of the row, then the 4 waves of the row.
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int m = rbase + i * 16 + r16;
      float am = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float h = (i < nmb && m < mrows) ? silu_mul(acc[i][j][q], acc[i][j + 2][q]) : 0.f;
          acc[i][j][q] = h;
          am = fmaxf(am, fabsf(h));
        }
      am = fmaxf(am, __shfl_xor(am, 16));
      am = fmaxf(am, __shfl_xor(am, 32));
      if (lane < 16) amax_s[wn * BM + m] = am;
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < MB; ++i)
      if (i < nmb) {
        const int m = rbase + i * 16 + r16;
        if (m < mrows) {
          float am = 0.f;
#pragma unroll
          for (int w = 0; w < WN; ++w) am = fmaxf(am, amax_s[w * BM + m]);
          const float scale = am == 0.f ? 1.f : am / 448.f;
          float qd[2][4];
          if (scale >= kDivFastMin) {       // the row's eight quotients from one reciprocal
            const float y = 1.f / scale;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) qd[j][q] = div_rn_by(acc[i][j][q], scale, y);
          } else {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) qd[j][q] = acc[i][j][q] / scale;
          }
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float qv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) qv[q] = fminf(fmaxf(qd[j][q], -448.f), 448.f);
            // four e4m3 codes, columns 4 (lane / 16) .. +3 of block j
            int w4 = __builtin_amdgcn_cvt_pk_fp8_f32(qv[0], qv[1], 0, false);
            w4 = __builtin_amdgcn_cvt_pk_fp8_f32(qv[2], qv[3], w4, true);
            *reinterpret_cast<uint32_t*>(tile_at(m, wn * 32 + j * 16 + 4 * (lane >> 4))) = (uint32_t)w4;
          }
          if (wn == 0 && lane < 16) static_cast<float*>(p.out_scale)[(size_t)nt * p.R + row0 + m] = scale;
        }
      }
  } else if constexpr (MX || BF) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
      if (i < nmb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = rbase + i * 16 + (lane >> 4) * 4 + q;
#pragma unroll
          for (int j = 0; j < NB; ++j)
            *reinterpret_cast<uint16_t*>(tile_at(r, wn * 64 + j * 16 + r16)) =
                (uint16_t)f32_to_bf16_bits(acc[i][j][q]);
        }
      }
  } else {
    // fp8 (D = B A^T): four consecutive output columns of row m per block.
#pragma unroll
    for (int i = 0; i < MB; ++i)
      if (i < nmb) {
        const int m = rbase + i * 16 + r16;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const uint32_t lo = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          const uint32_t hi = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
          *reinterpret_cast<u32x2_t*>(tile_at(m, wn * 64 + j * 16 + 4 * (lane >> 4))) = u32x2_t{lo, hi};
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

// Persistent form of the 8-bit kernel for large launches (the DeepSeek-like
// layer's fp8 GEMMs, the Qwen3-like MXFP8 prefill).  Per item the plain
// kernel spends 3.5-4.5 us before its first MFMA (the chain tile count ->
// band entry -> tile entry -> group offsets -> A rows, then the first chunk)
// and 2.5-5 us in the epilogue, with a workgroup launch in between: 12 % of
// a DeepSeek-like gate/up item, a quarter of its down item (16 chunks), a
// fifth and a third of the MXFP8 prefill's.  Here one workgroup per CU walks
// its items (blockIdx.x + k * gridDim.x, the same XCD-contiguous band order):
//   - the lanes of every wave look up the workgroup's items once, in
//     parallel (lane l: item l, at most 64), and keep them in registers;
//   - the last NS iterations of an item's K loop load the next item's first
//     chunks into the ring, so the next item starts on data already in LDS;
//   - the epilogue writes from registers (no staging tile): MXFP8 multiplies
//     with the operands swapped (D = B A^T, as fp8), so a lane holds four
//     consecutive columns of one row and a 32-column E8M0 block of h is one
//     wave's, reduced across its lanes.  The next item's third chunk is held
//     back until after the stores (the last iteration's loads go to the sink
//     instead, keeping the counts): fp8 gate/up passes the per-row maxima of
//     four waves through the stage the last chunk freed, and the wait for
//     the next item's first chunk then retires neither the stores nor that
//     chunk;
//   - gathered A rows (gate/up; MXFP8 also their scale rows) are looked up
//     two items ahead, right after an epilogue, when only loads issued long
//     before are in flight;
//   - MXFP8 scale stages alternate per 4-chunk group across items (a
//     running parity), as within one.
// fp8: same arithmetic and bits as k_tiled8<false, DUAL, 160, 1>; MXFP8: the
// same products as k_tiled8<true, DUAL, 128, 4>, taken transposed.
template <bool MX, bool DUAL>
__global__ __launch_bounds__(512) void k_tiled8p(const GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = MX ? 128 : 160, SG = MX ? 4 : 1;
  using L = Tiled8Lds<MX, BM, SG>;
  static_assert(L::TOTAL <= 160 * 1024, "LDS budget");
  static_assert(SG == 1 || L::NSS == 2, "MXFP8: two 4-chunk scale stages");
  constexpr int NS = k8NS;
  constexpr int NW = 8, WN = 4;
  constexpr int MB = BM / 32;
  constexpr int NB = 4;
  constexpr int HA = MB / 2;
  constexpr int A_BLK = BM / 8;
  constexpr int IPWA = (A_BLK + NW - 1) / NW;
  constexpr int IPWB = L::B_BYTES / 1024 / NW;
  constexpr int NSC = L::NSC;
  static_assert(NSC <= NW && IPWB == NB && IPWA <= NB, "load parts");
  constexpr int OPS = IPWA + IPWB + 1;
  constexpr int B_RING = NS * L::A_BYTES;
  constexpr int S_RING = B_RING + NS * L::B_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::TOTAL];
  uint8_t* const sink = lds + L::SINK;

  const int K = p.K, N = p.N;
  const int nk = K / 128, KB = K / 128;
  const int N128 = N / 128;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  // fp8: the second wave row's columns pace each chunk (the first row's waves
  // wait for them at the chunk barrier), so its waves take issue priority
  // (DeepSeek-like layer -0.9 %; MXFP8 measured 0.5 % slower with it).
  if constexpr (!MX) {
    if (wm == 1) __builtin_amdgcn_s_setprio(1);
  }
  const int r16 = lane & 15;

  // Items of this workgroup (blockIdx.x + k * gridDim.x, k < 64; the host
  // sizes the grid for that): lane k holds item k as (group | rows << 16,
  // first row | column tile << 24).
  uint32_t mw0, mw1;
  int n_items;
  {
    int tslot = 0, ntv = 0;
    const bool ok = band_item(p.sc.tiles, *p.sc.n_tiles, p.n_ntile, tslot, ntv,
                              (int)blockIdx.x + lane * (int)gridDim.x);
    uint32_t w0 = 0, w1 = 0;
    if (ok) {
      const int g = p.sc.tiles[4 * tslot], m0 = p.sc.tiles[4 * tslot + 1];
      const int o0 = p.offsets[g], gm = p.offsets[g + 1] - o0;
      const int mr = min(group_tile_rows(gm, BM), gm - m0);
      w0 = (uint32_t)g | ((uint32_t)mr << 16);
      w1 = (uint32_t)(o0 + m0) | ((uint32_t)ntv << 24);
    }
    mw0 = w0;
    mw1 = w1;
    // band_item is monotone in k: the valid items are a prefix.
    n_items = __builtin_amdgcn_readfirstlane(__popcll(__ballot(ok)));
  }
  if (n_items == 0) return;
  struct Item { int g, row0, mrows, nt; };
  auto item = [&](int i) {
    const uint32_t w0 = (uint32_t)__builtin_amdgcn_readlane((int)mw0, i);
    const uint32_t w1 = (uint32_t)__builtin_amdgcn_readlane((int)mw1, i);
    return Item{(int)(w0 & 0xFFFFu), (int)(w1 & 0xFFFFFFu), (int)(w0 >> 16), (int)(w1 >> 24)};
  };

  // Per-lane load geometry (item independent).  A block j * NW + wave holds
  // tile rows 8 (j * NW + wave) .. +7 (blocks past the tile go to the sink);
  // B: this wave's 32 staged rows from one matrix (DUAL: waves 0-3 gate,
  // 4-7 up); scales: lane row sr as in the plain kernel.
  bool ain[IPWA];
  int arow[IPWA];
  uint32_t asl[IPWA];
#pragma unroll
  for (int j = 0; j < IPWA; ++j) {
    const int blk = j * NW + wave;
    arow[j] = blk * 8 + lane / 8;
    asl[j] = (uint32_t)(slot8(arow[j], lane % 8) * 16);
    ain[j] = blk < A_BLK;
  }
  int br0 = wave * IPWB * 8;
  const uint8_t* Bm = p.B0;
  if (DUAL && br0 >= 128) { Bm = p.B1; br0 -= 128; }
  uint32_t bsl[IPWB];
#pragma unroll
  for (int j = 0; j < IPWB; ++j)
    bsl[j] = (uint32_t)(slot8((wave * IPWB + j) * 8 + lane / 8, lane % 8) * 16);
  const int srow = wave * 64 + lane;
  const int sr = min(srow, L::SROWS - 1);
  const bool swave = wave < NSC;
  const uint32_t sstep = (!MX && sr < BM) ? 4u * (uint32_t)p.s_ld : 4u;

  // Load sources of one item.  spad (MXFP8): what lane 63 reads, for the
  // scale loads that only keep the counts (one line instead of 64).
  struct Src {
    const uint8_t* ab;
    const uint8_t* bb;
    const uint8_t* ssrc;
    const uint8_t* spad;
    uint32_t aoff[IPWA];
    uint32_t boff[IPWB];
  };
  // A rows of an item (the gathered ones, if any) as offsets, and for MXFP8
  // the lane's activation scale row.
  struct ARows { uint32_t off[IPWA]; uint32_t srow; };
  auto a_rows_of = [&](const Item& it) {
    ARows ar;
#pragma unroll
    for (int j = 0; j < IPWA; ++j) {
      const int r = min(arow[j], it.mrows - 1);
      ar.off[j] = (p.a_rows ? (uint32_t)p.a_rows[it.row0 + r] : (uint32_t)r) * (uint32_t)K + asl[j];
    }
    ar.srow = 0;
    if constexpr (MX) {
      const int r = it.row0 + min(sr, it.mrows - 1);
      ar.srow = (uint32_t)((p.a_rows && sr < BM) ? p.a_rows[r] : r);
    }
    return ar;
  };
  auto make_src = [&](const Item& it, const ARows& ar) {
    Src s;
    s.ab = p.a_rows ? p.A : p.A + (size_t)it.row0 * K;
#pragma unroll
    for (int j = 0; j < IPWA; ++j) s.aoff[j] = ar.off[j];
    s.bb = Bm + (size_t)it.g * N * K;
    const int n0 = it.nt * (DUAL ? 128 : 256);
#pragma unroll
    for (int j = 0; j < IPWB; ++j)
      s.boff[j] = (uint32_t)min(n0 + br0 + j * 8 + lane / 8, N - 1) * (uint32_t)K + bsl[j];
    if constexpr (MX) {
      if (sr < BM) {
        s.ssrc = static_cast<const uint8_t*>(p.A_scale) + (size_t)ar.srow * (size_t)(4 * KB);
      } else {
        int br = sr - BM;
        const uint8_t* sB = static_cast<const uint8_t*>(p.s_B0);
        if (DUAL && br >= 128) { sB = static_cast<const uint8_t*>(p.s_B1); br -= 128; }
        s.ssrc = sB + ((size_t)it.g * N + min(n0 + br, N - 1)) * (size_t)(K / 32);
      }
      s.spad = reinterpret_cast<const uint8_t*>(
          ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(reinterpret_cast<uint64_t>(s.ssrc) >> 32), 63) << 32) |
          (uint32_t)__builtin_amdgcn_readlane((int)reinterpret_cast<uint64_t>(s.ssrc), 63));
    } else {
      if (sr < BM) {
        s.ssrc = static_cast<const uint8_t*>(p.A_scale) + (size_t)(it.row0 + min(sr, it.mrows - 1)) * 4;
      } else {
        const int which = sr - BM;
        if (DUAL)
          s.ssrc = static_cast<const uint8_t*>(which ? p.s_B1 : p.s_B0) +
                   ((size_t)it.g * N128 + it.nt) * (size_t)(4 * KB);
        else
          s.ssrc = static_cast<const uint8_t*>(p.s_B0) +
                   ((size_t)it.g * N128 + min(n0 / 128 + which, N128 - 1)) * (size_t)(4 * KB);
      }
      s.spad = s.ssrc;
    }
    return s;
  };

  auto a_st = [&](int st) { return lds + st * L::A_BYTES; };
  auto b_st = [&](int st) { return lds + B_RING + st * L::B_BYTES; };
  // Scale stage of chunk c in ring stage st: fp8 the ring stage; MXFP8 the
  // parity of the chunk's 4-chunk group counted from the walk's start (sgo:
  // the item's first group's parity).
  auto s_stage = [&](int c, int st, int sgo) { return MX ? (((c >> 2) + sgo) & 1) : st; };
  // Part j of chunk c of source s into stage st (to_sink: every load of the
  // part goes to the sink; it only keeps the counts).
  auto issue_part = [&](const Src& s, int c, int st, int sgo, int j, bool to_sink) {
    const int cc = min(c, nk - 1);
    if (j == 0) {
      const bool real = swave && c % SG == 0 && !to_sink;
      uint8_t* const dst = real ? lds + S_RING + s_stage(c, st, sgo) * L::SSTAGE + wave * 64 * L::SB : sink;
      const size_t sk = (size_t)(cc - cc % SG);
      dma_addr_untracked<L::SB>((real || !MX ? s.ssrc : s.spad) + sk * sstep, dst);
    }
    if (j < IPWA) {
      const int ja = j < IPWA ? j : 0;
      uint8_t* const dst = (ain[ja] && !to_sink) ? a_st(st) + (ja * NW + wave) * 1024 : sink;
      dma16_untracked(s.ab + (size_t)cc * 128, s.aoff[ja], dst);
    }
    uint8_t* const dst = to_sink ? sink : b_st(st) + (wave * IPWB + j) * 1024;
    dma16_untracked(s.bb + (size_t)cc * 128, s.boff[j], dst);
  };

  // First items: sources of items 0 and 1, A rows of item 2, then the first
  // NS chunks of item 0.
  Src cur, nxt;
  ARows ar2;
  {
    const Item i0 = item(0);
    cur = make_src(i0, a_rows_of(i0));
    if (n_items > 1) {
      const Item i1 = item(1);
      nxt = make_src(i1, a_rows_of(i1));
    } else {
      nxt = cur;
    }
    ar2 = a_rows_of(item(n_items > 2 ? 2 : 0));
  }
  int sgo = 0;                                       // MXFP8: scale-group parity of the item's chunk 0
  const int sgo_step = (nk / 4) & 1;
#pragma unroll
  for (int c = 0; c < NS; ++c)
#pragma unroll
    for (int j = 0; j < NB; ++j) issue_part(cur, c, c, 0, j, false);
  wait_vmcnt<(NS - 1) * OPS>();
  lds_barrier();

  // Fragment reads and MFMAs, as in the plain kernel.
  const int rbase = wm * (BM / 2);
  // Epilogue column of a lane after the pair exchange: c even starts at 4c
  // of its first block, c odd at 4 (c - 1) of the next (c = lane / 16).
  const bool ceven = ((lane >> 4) & 1) == 0;
  const int pcol = ceven ? 4 * (lane >> 4) : 16 + 4 * ((lane >> 4) - 1);
  const int c0 = lane >> 4, c1 = 4 + (lane >> 4);
  const int sh = 8 * (lane >> 4);                    // MXFP8: byte of this lane's K block
  const uint32_t a_lo0 = (uint32_t)((rbase + r16) * 128 + (slot8(r16, c0) << 4));
  const uint32_t a_hi0 = (uint32_t)((rbase + r16) * 128 + (slot8(r16, c1) << 4));
  const int brow0 = b8_row<DUAL>(0, wn, r16);
  const uint32_t b_lo0 = (uint32_t)(B_RING + brow0 * 128 + (slot8(r16, c0) << 4));
  const uint32_t b_hi0 = (uint32_t)(B_RING + brow0 * 128 + (slot8(r16, c1) << 4));
  const uint32_t s_a0 = (uint32_t)(S_RING + (rbase + r16) * L::SB);
  const uint32_t s_b0 = (uint32_t)(S_RING + (BM + brow0) * L::SB);   // MXFP8: B row scales
  auto opq = [](uint32_t v) { asm volatile("" : "+v"(v)); return v; };
  auto frag_at = [&](uint32_t lo, uint32_t hi) {
    const u32x4_t x = lds_read16(lds + lo), y = lds_read16(lds + hi);
    return i32x8_t{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                   (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
  };
  auto ld32 = [&](uint32_t off) { return *reinterpret_cast<const uint32_t*>(lds + off); };

  f32x4_t acc[MB][NB];
  i32x8_t a[MB], b[NB];
  float saf[MB];                                     // fp8: activation scale of the lane's row
  uint32_t sam[MB], sbm[NB];                         // MXFP8: E8M0 bytes
  float sb_lo = 0.f, sb_hi = 0.f;
  struct Bases { uint32_t alo, ahi, blo, bhi, sa, sb; };
  auto bases = [&](int c, int st, int sgo_) {
    const uint32_t so = (uint32_t)(s_stage(c, st, sgo_) * L::SSTAGE + (MX ? (c & 3) * 4 : 0));
    return Bases{opq(a_lo0 + st * L::A_BYTES), opq(a_hi0 + st * L::A_BYTES),
                 opq(b_lo0 + st * L::B_BYTES), opq(b_hi0 + st * L::B_BYTES), opq(s_a0 + so),
                 MX ? opq(s_b0 + so) : 0u};
  };
  auto next_a = [&](const Bases& q, int i) {
    a[i] = frag_at(q.alo + i * 2048, q.ahi + i * 2048);
    if constexpr (MX) sam[i] = (ld32(q.sa + i * 16 * L::SB) >> sh) & 0xFFu;
    else saf[i] = __uint_as_float(ld32(q.sa + i * 16 * L::SB));
  };
  auto next_b = [&](const Bases& q, int j) {
    const int dr = b8_row<DUAL>(j, 0, 0);
    b[j] = frag_at(q.blo + dr * 128, q.bhi + dr * 128);
    if constexpr (MX) sbm[j] = (ld32(q.sb + dr * L::SB) >> sh) & 0xFFu;
  };
  auto rd_bsc = [&](int st) {
    if constexpr (!MX) {
      const uint32_t o = S_RING + (uint32_t)(st * L::SSTAGE) + BM * L::SB;
      const float s0 = __uint_as_float(ld32(o)), s1 = __uint_as_float(ld32(o + L::SB));
      sb_lo = DUAL ? s0 : (wn < 2 ? s0 : s1);
      sb_hi = DUAL ? s1 : sb_lo;
    }
  };
  constexpr int HMAX = MB - HA;
  f32x4_t pr[2][HMAX];
  auto col = [&](int i0, int i1, int j, auto nm) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
      if (i < count_value(nm)) {
        if constexpr (MX) acc[i][j] = mfma_mx8_16x16x128(b[j], a[i], acc[i][j], sbm[j], sam[i]);
        else pr[j & 1][i - i0] = mfma_fp8_16x16x128(b[j], a[i], f32x4_t{0.f, 0.f, 0.f, 0.f});
      }
  };
  auto scale_col = [&](int i0, int i1, int j, auto nm) {
    if constexpr (!MX) {
      const float sbv = j < NB / 2 ? sb_lo : sb_hi;
#pragma unroll
      for (int i = i0; i < i1; ++i)
        if (i < count_value(nm)) {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][j][q] += pr[j & 1][i - i0][q] * (saf[i] * sbv);
        }
    }
  };

  int st = 0;                                        // ring stage of the current chunk
  for (int it_i = 0;; ++it_i) {
    const Item it = item(it_i);
    const bool has_next = it_i + 1 < n_items;
    const int n0 = it.nt * (DUAL ? 128 : 256);
    const int ncols = DUAL ? 128 : min(256, N - n0);
    const bool has_cols = DUAL || wn * 64 < ncols;
    const int nmb = has_cols ? max(0, min(MB, ceil_div(it.mrows - rbase, 16))) : 0;
    // The tail's loads: the next item's chunks 0 .. NS-1, or re-reads of
    // this item's last chunk after the last item.
    Src tsrc;
    tsrc.ab = has_next ? nxt.ab : cur.ab;
    tsrc.bb = has_next ? nxt.bb : cur.bb;
    tsrc.ssrc = has_next ? nxt.ssrc : cur.ssrc;
    tsrc.spad = has_next ? nxt.spad : cur.spad;
#pragma unroll
    for (int j = 0; j < IPWA; ++j) tsrc.aoff[j] = has_next ? nxt.aoff[j] : cur.aoff[j];
#pragma unroll
    for (int j = 0; j < IPWB; ++j) tsrc.boff[j] = has_next ? nxt.boff[j] : cur.boff[j];
    const int tshift = has_next ? nk : 0;
    const int sgo_n = (sgo + sgo_step) & 1;          // MXFP8: the next item's
    const int tsgo = has_next ? sgo_n : sgo;

#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto main_loop = [&](auto nm) {
      {
        const Bases q0 = bases(0, st, sgo);
#pragma unroll
        for (int j = 0; j < NB; ++j) next_b(q0, j);
#pragma unroll
        for (int i = 0; i < HA; ++i) next_a(q0, i);
      }
      rd_bsc(st);
      // One chunk: its loads are issued by issue(j) between the second
      // half's columns.
      auto step = [&](int kc, auto&& issue) {
        const int sn = st == NS - 1 ? 0 : st + 1;
        {
          const Bases qk = bases(kc, st, sgo);
#pragma unroll
          for (int i = HA; i < MB; ++i) next_a(qk, i);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          col(0, HA, j, nm);
          if (j > 0) scale_col(0, HA, j - 1, nm);
        }
        scale_col(0, HA, NB - 1, nm);
#pragma unroll
        for (int i = 0; i < HA; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) asm volatile("" : "+v"(acc[i][j]));
        wait_vmcnt<(NS - 2) * OPS>();
        lds_barrier();
        // (After the last chunk these read the next item's chunk 0, unused.)
        const Bases qn = bases(kc + 1, sn, sgo);
#pragma unroll
        for (int i = 0; i < HA; ++i) next_a(qn, i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          col(HA, MB, j, nm);
          issue(j);
          if (j > 0) scale_col(HA, MB, j - 1, nm);
          next_b(qn, j);
          __builtin_amdgcn_sched_barrier(0);
        }
        scale_col(HA, MB, NB - 1, nm);
        rd_bsc(sn);
        st = sn;
      };
      for (int kc = 0; kc < nk - NS; ++kc)
        step(kc, [&](int j) { issue_part(cur, kc + NS, st, sgo, j, false); });
      for (int kc = nk - NS; kc < nk; ++kc) {
        // The next item's chunk NS-1 is held back (see below).
        const bool to_sink = has_next && kc == nk - 1;
        step(kc, [&](int j) { issue_part(tsrc, kc + NS - tshift, st, tsgo, j, to_sink); });
      }
    };
    with_count<MB>(nmb, main_loop);
    // st is now the stage of the next item's chunk 0; the last chunk's
    // stage (free: every wave is past the last boundary) is st_last.
    const int st_last = st == 0 ? NS - 1 : st - 1;
    if (!has_next) wait_vmcnt<0>();                  // the tail's re-reads land before the exit

    if constexpr (DUAL) {
      // h = silu(g) * u per lane: row m, columns 4 c + q of blocks 0 and 1
      // (c = lane / 16).  MXFP8: one E8M0 scale per row and 32 columns (the
      // wave's); fp8: per 128 columns (four waves, through the free stage),
      // scale amax / 448.
      uint32_t w4[MB][2];
      float scl[MB];
      uint32_t e8s[MB];
      float* amax_s = reinterpret_cast<float*>(b_st(st_last));   // fp8: [WN][BM]
      if constexpr (!MX) lds_barrier();
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int m = rbase + i * 16 + r16;
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float h;
            if constexpr (MX) h = silu_mul(acc[i][j][q], acc[i][j + 2][q]);
            else h = (i < nmb && m < it.mrows) ? silu_mul(acc[i][j][q], acc[i][j + 2][q]) : 0.f;
            acc[i][j][q] = h;
            am = fmaxf(am, fabsf(h));
          }
        am = fmaxf(am, __shfl_xor(am, 16));
        am = fmaxf(am, __shfl_xor(am, 32));
        if constexpr (MX) {
          const uint32_t e8 = mx_e8m0(am);
          const float inv = mx_inv_scale(e8);
          e8s[i] = e8;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            uint32_t v = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              v |= ((uint32_t)f32_to_e4m3(fminf(fmaxf(acc[i][j][q] * inv, -448.f), 448.f)) & 0xFFu) << (8 * q);
            w4[i][j] = v;
          }
        } else {
          if (lane < 16) amax_s[wn * BM + m] = am;
        }
      }
      if constexpr (!MX) {
        lds_barrier();
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int m = rbase + i * 16 + r16;
          float am = 0.f;
#pragma unroll
          for (int w = 0; w < WN; ++w) am = fmaxf(am, amax_s[w * BM + m]);
          const float scale = am == 0.f ? 1.f : am / 448.f;
          scl[i] = scale;
          float qd[2][4];
          if (scale >= kDivFastMin) {       // the row's eight quotients from one reciprocal
            const float y = 1.f / scale;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) qd[j][q] = div_rn_by(acc[i][j][q], scale, y);
          } else {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) qd[j][q] = acc[i][j][q] / scale;
          }
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float qv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) qv[q] = fminf(fmaxf(qd[j][q], -448.f), 448.f);
            int v = __builtin_amdgcn_cvt_pk_fp8_f32(qv[0], qv[1], 0, false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(qv[2], qv[3], v, true);
            w4[i][j] = (uint32_t)v;
          }
        }
      }
      if (has_next && it_i + 2 < n_items) ar2 = a_rows_of(item(it_i + 2));
      // Lanes c and c ^ 1 trade codes so that each holds eight consecutive
      // columns of its row (c even of block 0, c odd of block 1): one 8-byte
      // store per lane and row block.
#pragma unroll
      for (int i = 0; i < MB; ++i)
        if (i < nmb) {
          const int m = rbase + i * 16 + r16;
          const uint32_t got = (uint32_t)__shfl_xor((int)(ceven ? w4[i][1] : w4[i][0]), 16);
          if (m < it.mrows) {
            const u32x2_t o = ceven ? u32x2_t{w4[i][0], got} : u32x2_t{got, w4[i][1]};
            *reinterpret_cast<u32x2_t*>(p.out + (size_t)(it.row0 + m) * N + n0 + wn * 32 + pcol) = o;
            if constexpr (MX) {
              if (lane < 16)
                static_cast<uint8_t*>(p.out_scale)[(size_t)(it.row0 + m) * (N / 32) + (n0 + wn * 32) / 32] =
                    (uint8_t)e8s[i];
            } else {
              if (wn == 0 && lane < 16)
                static_cast<float*>(p.out_scale)[(size_t)it.nt * p.R + it.row0 + m] = scl[i];
            }
          }
        }
      if (!MX && has_next) lds_barrier();            // the maxima are read: the stage is free
    } else {
      if (has_next && it_i + 2 < n_items) ar2 = a_rows_of(item(it_i + 2));
      // A lane holds four consecutive bf16 columns of row m per block; lanes
      // c and c ^ 1 trade halves so that each holds eight (c even of block j,
      // c odd of block j + 1): one 16-byte store per lane and block pair.
#pragma unroll
      for (int i = 0; i < MB; ++i)
        if (i < nmb) {
          const int m = rbase + i * 16 + r16;
          uint8_t* const orow = p.out + ((size_t)(it.row0 + m) * N + n0 + wn * 64) * 2;
#pragma unroll
          for (int jp = 0; jp < NB; jp += 2) {
            uint32_t v[2][2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              v[t][0] = pack_bf16x2(acc[i][jp + t][0], acc[i][jp + t][1]);
              v[t][1] = pack_bf16x2(acc[i][jp + t][2], acc[i][jp + t][3]);
            }
            const uint32_t g0 = (uint32_t)__shfl_xor((int)(ceven ? v[1][0] : v[0][0]), 16);
            const uint32_t g1 = (uint32_t)__shfl_xor((int)(ceven ? v[1][1] : v[0][1]), 16);
            const int cidx = jp * 16 + pcol;
            if (m < it.mrows && wn * 64 + cidx < ncols)
              *reinterpret_cast<u32x4_t*>(orow + (size_t)cidx * 2) =
                  ceven ? u32x4_t{v[0][0], v[0][1], g0, g1} : u32x4_t{g0, g1, v[1][0], v[1][1]};
          }
        }
    }
    if (!has_next) break;
    // The next item's chunk NS-1 into the free stage, after the stores: the
    // vm counter retires in issue order, so the wait for the next item's
    // chunk 0 (chunks 1, the sink loads and NS-1 came later) need not wait
    // for the stores, nor for this last chunk.
#pragma unroll
    for (int j = 0; j < NB; ++j) issue_part(nxt, NS - 1, st_last, sgo_n, j, false);
    cur = nxt;
    if (it_i + 2 < n_items) nxt = make_src(item(it_i + 2), ar2);
    sgo = sgo_n;
    wait_vmcnt<NS * OPS>();                          // the new item's chunk 0 is in
    lds_barrier();
  }
#else
  (void)p;
#endif
}

hipError_t launch_tiled8_bf16(const char* name, bool dual, long long blocks, const GemmArgs& a,
                              hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)band_grid(blocks, 1));
  static_assert(tile_rows(false, false, true) == 160, "bf16 streaming tile height");
  if (dual) MOE_LAUNCH(name, (k_tiled8<false, true, 160, 1, true>), grid, dim3(512), 0, s, a);
  else MOE_LAUNCH(name, (k_tiled8<false, false, 160, 1, true>), grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tiled8(const char* name, bool mx, bool dual, long long blocks, const GemmArgs& a,
                         hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)band_grid(blocks, 1));
  // Scales in groups of 4 chunks when a row's scale array splits into 16-byte
  // pieces (K a multiple of 512), else one 4-byte load per chunk.
  const bool g4 = a.K % 512 == 0;
  static_assert(tile_rows(true, true) == 128, "MXFP8 tile height");
  static_assert(tile_rows(true, false) == 160, "fp8 tile height");
  // Persistent walk for large launches: one workgroup per CU (more when a
  // workgroup would exceed the 64 items its lanes hold), a multiple of 8 so
  // that every workgroup stays on one XCD's band run.  Needs K of at least
  // NS chunks, no ragged column tile, the packed item fields (rows < 2^24,
  // column tiles < 256), and fp8 ungathered activation scales, MXFP8 scales
  // in 4-chunk groups.
  const long long pairs = (long long)band_grid(blocks, 1);
  const int ncw = dual ? 128 : 256;
  if (pairs >= 4 * kPersistGrid && a.K >= 128 * k8NS && a.N % ncw == 0 && a.n_ntile < 256 &&
      a.R < (1 << 24) && (mx ? g4 : a.s_rows == nullptr)) {
    const long long need = (pairs + 8 + 63) / 64;
    const dim3 pgrid((unsigned)(((need > kPersistGrid ? need : kPersistGrid) + 7) / 8 * 8));
    if (mx) {
      if (dual) MOE_LAUNCH(name, (k_tiled8p<true, true>), pgrid, dim3(512), 0, s, a);
      else MOE_LAUNCH(name, (k_tiled8p<true, false>), pgrid, dim3(512), 0, s, a);
    } else {
      if (dual) MOE_LAUNCH(name, (k_tiled8p<false, true>), pgrid, dim3(512), 0, s, a);
      else MOE_LAUNCH(name, (k_tiled8p<false, false>), pgrid, dim3(512), 0, s, a);
    }
    return hipGetLastError();
  }
  if (mx) {
    if (dual) {
      if (g4) MOE_LAUNCH(name, (k_tiled8<true, true, 128, 4>), grid, dim3(512), 0, s, a);
      else MOE_LAUNCH(name, (k_tiled8<true, true, 128, 1>), grid, dim3(512), 0, s, a);
    } else {
      if (g4) MOE_LAUNCH(name, (k_tiled8<true, false, 128, 4>), grid, dim3(512), 0, s, a);
      else MOE_LAUNCH(name, (k_tiled8<true, false, 128, 1>), grid, dim3(512), 0, s, a);
    }
  } else {
    if (dual) MOE_LAUNCH(name, (k_tiled8<false, true, 160, 1>), grid, dim3(512), 0, s, a);
    else MOE_LAUNCH(name, (k_tiled8<false, false, 160, 1>), grid, dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
