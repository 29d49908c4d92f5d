// FlashAttention-2 forward pass on 16-bit inputs (bf16 or fp16 in, the same
// type out, fp32 accumulation), for gfx950 (MI355X).  This header holds the
// kernel template; fa2_fwd_bf16.hip and fa2_fwd_fp16.hip instantiate it.
//
// The algorithm (pages "FlashAttention学习笔记(2)" and "Flash Attention V2原理解读",
// forward sections; "flash-attention123和ring-attention", 优化1-优化4):
//   outer loop: one work item per block of kBlockM = 32 * WAVES query rows
//               (128, or 256 with eight wavefronts) of one (batch, head);
//               items are independent;
//   inner loop: K_j, V_j blocks of BN keys, staged in LDS and shared by the
//               workgroup's wavefronts;
//   per block:  S = scale * Q_i K_j^T on MFMA, online row max / row sum, the
//               running O rescaled by exp(m_old - m_new) and P~ V_j added on
//               MFMA, no division by l inside the loop;
//   after:      O = O / l once, L = m + ln(l); K/V blocks that the causal mask
//               covers entirely are neither loaded nor computed.
//   lengths:    Q has Nq rows, K and V Nk (the grid follows the query length,
//               page "FlashAttention学习笔记(2)", section "V2中的thread blocks
//               排布"); the causal mask is aligned bottom-right, key j hidden
//               from query i when j > i + Nk - Nq, so a query that sees no key
//               at all (Nq > Nk) gets O = 0 and L = -inf.
//
// Persistent grid.  The page's grid has one thread block per (query block,
// batch, head).  Here as many workgroups run as fit on the chip at once and
// each walks a fixed sequence of work items: the items of one XCD are the
// query blocks of a contiguous range of heads (which read the same K/V and so
// share that XCD's L2), dealt to its workgroups in a snake order so that heavy
// and light causal blocks balance.  While the last K/V block of an item is
// processed, the next item's Q rows and first K/V blocks are already loading.
//
// Issue priority.  Where two workgroups share a CU (four wavefronts each), the
// SIMDs' arbitration favours the older one: with the same number of blocks
// each, the younger finished up to 15% later and then ran alone on its CU.
// Each wavefront therefore lowers its priority (s_setprio 3, 2, 1, 0) as its
// workgroup passes each quarter of its blocks, so that the partner that is
// behind wins the arbitration until it reaches the same quarter.  The
// eight-wavefront form has its CU to itself and keeps the default priority
// (the test and branch per block cost it 1-2%).
//
// Wavefront layout (the pages' split-Q warp scheme, re-derived for 64-wide
// wavefronts and 32x32 MFMA tiles): each wavefront owns 32 query rows against
// the shared K/V block and never exchanges partial results with another.
// WAVES = 4 (two or three workgroups per CU, as OCC, the wavefronts per SIMD
// that the registers allow, permits) or 8 (d = 128 on large grids: one
// workgroup per CU, both wavefronts of a SIMD in it, each K/V block staged
// once per CU).
//
// MFMA orientation.  v_mfma_f32_32x32x16_{bf16,f16} produces a 32x32 fp32 tile
// where lane l holds column (l % 32) and rows 8*(r/4) + 4*(l/32) + (r%4),
// r = 0..15.  The kernel computes S^T = K Q^T, so that a lane holds 16 keys of
// ONE query row: the row max and row sum are in-lane, plus one exchange with
// the lane 32 positions away.  The output is accumulated transposed too,
// O^T += V^T P^T, so each lane's accumulators all belong to its one query row
// (the rescale and the final 1/l are per-lane scalars).  The P^T operand comes
// straight from the S^T registers: the contraction index may be permuted
// freely as long as both operands use the same order, and the V^T operand is
// read in exactly the order in which S^T's accumulator rows sit in a lane.
//
// Memory pipeline.  K and V blocks go from HBM straight into LDS
// (global_load_lds_dwordx4, no register staging), double-buffered: while
// block j is consumed, blocks j+1 (V) and j+2 (K) are in flight, with one
// workgroup barrier per block.  Each direct load writes 1 KB of LDS.  K: whole
// key rows in 1 KB pieces that sit 1040 bytes apart, with the rows that share
// a piece chosen so that the K fragment reads (16 rows x 16 bytes per pass)
// touch every LDS bank once.  V: 128-byte blocks of 4 key rows x 16 dims, so
// that each 16-lane group of a transposing read (ds_read_b64_tr_b16) reads
// one contiguous block, the pattern the LDS serves fastest.  Every fragment
// address is one per-lane base plus a compile-time offset.  With eight
// wavefronts the next item's Q rows take the same route, into 8 KB of LDS per
// wavefront: they go out in the current item's prologue, once its own rows
// have been read from there, and the next item's prologue reads them in the
// operand layout.  The
// direct loads, and the waits and barriers that order them, are inline
// assembly, so the compiler does not serialise them against the LDS reads in
// between.
//
// Epilogue.  O and L go straight from registers to global memory through
// buffer stores whose resource covers only the rows < Nq: rows past the end
// are dropped by the hardware, and every wavefront issues the same number of
// stores, which the next item's first wait counts past.
//
// Overlap.  Block j's row max is formed while block j-1 is finished, so that
// the one branch of a step (the rescale test) comes first; after it, block
// j+1's S = K Q^T MFMAs, block j's exp2, row sum and 16-bit packing, block
// j's PV MFMAs and block j+1's row max all sit in one basic block, where the
// compiler interleaves the vector ALU work with both MFMA streams.
//
// Rescaling.  The running reference max m only moves when a block's row max
// exceeds it by more than kTau (in log2 units); otherwise O and l keep their
// scale and P~ = exp2(c s - c m) stays <= 2^kTau.  O / l and L = m + ln(l) are
// unchanged by the choice of reference, so this is the same online softmax
// with fewer rescales of O.
//
// Rounding.  P~ is rounded to the input type (nearest even) for the PV
// product; l sums the unrounded fp32 values.  For fp16, P~ <= 2^kTau stays far
// below the type's largest value, and a value below its normal range loses at
// most 2^-25 against l >= 1.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "fa2_device.h"
#include "fa2_internal.h"
#include "fa2_schedule.h"

namespace fa2 {
namespace {

using namespace dev;


constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units

// Keys per K/V block and wavefronts per SIMD for each head dimension.
template <int D> struct Cfg {
  static constexpr int BN = mfma_block_n(D);
};
// Workgroups resident per CU with WAVES wavefronts each.
template <int WAVES, int OCC> constexpr int groups_per_cu() { return OCC * 4 / WAVES; }

// LDS layout of a K block: key row r lives in 1 KB piece blk(r) at row slot
// slot(r); pieces are kPiece bytes apart, so piece b starts 16*b bytes further
// into the 256-byte bank cycle.  Rows 0..15 of any aligned group get 16
// different bank offsets (for the K reads, 16 lanes x 16 bytes per pass).
//   D = 32:  4 pieces of 16 rows, blk = r % 4, slot = r / 4 (bank offset
//            16*blk + 64*(slot % 4));
//   D = 64:  8 pieces of 8 rows;
//   D = 96, 128, 256: 16 pieces of 4, 4 and 2 rows (a D = 96 piece holds 768
//            bytes of rows).
// piece_row(b) + slot_row(s) inverts blk/slot: it is the row at slot s of
// piece b, which the direct loads need.
constexpr int kPiece = 1024 + 16;
template <int D> __host__ __device__ constexpr int blk(int r) {
  if constexpr (D == 32) return r & 3;
  else if constexpr (D == 64) return ((r >> 2) & 3) + 4 * (r & 1);
  else return 4 * (r & 3) + ((r >> 2) & 3);
}
template <int D> __host__ __device__ constexpr int slot(int r) {
  if constexpr (D == 32) return r >> 2;
  else if constexpr (D == 64) return 2 * (r >> 4) + ((r >> 1) & 1);
  else return r >> 4;
}
template <int D> __host__ __device__ constexpr int piece_row(int b) {
  if constexpr (D == 32) return b;
  else return 4 * (b & 3) + (b >> 2);
}
template <int D> __host__ __device__ constexpr int slot_row(int s) {
  if constexpr (D == 32) return 4 * s;
  else if constexpr (D == 64) return 16 * (s >> 1) + 2 * (s & 1);
  else return 16 * s;
}
template <int D> __host__ __device__ constexpr int rows_per_piece() {
  return D == 96 ? 4 : 1024 / (2 * D);
}
template <int D> __host__ __device__ constexpr int lds_off(int r) {
  return blk<D>(r) * kPiece + slot<D>(r) * 2 * D;
}
// Every row of a block has one (piece, slot) inside the block, piece_row +
// slot_row finds it again, and the rows of each aligned group of 16 sit at 16
// different bank offsets.
template <int D, int BN> __host__ __device__ constexpr bool k_layout_ok() {
  constexpr int RPP = rows_per_piece<D>();
  for (int r = 0; r < BN; ++r) {
    if (blk<D>(r) < 0 || blk<D>(r) >= BN / RPP || slot<D>(r) < 0 || slot<D>(r) >= RPP) return false;
    if (piece_row<D>(blk<D>(r)) + slot_row<D>(slot<D>(r)) != r) return false;
  }
  for (int g = 0; g < BN; g += 16)
    for (int a = g; a < g + 16; ++a)
      for (int b = a + 1; b < g + 16; ++b)
        if ((lds_off<D>(a) / 16) % 16 == (lds_off<D>(b) / 16) % 16) return false;
  return true;
}
// V layout: element (key row r, dim d) at (r/4)*4*2D + (d/16)*128 + 32*(r%4) + 2*(d%16):
// 128-byte blocks of 4 key rows x 16 dims.  Direct load n of a V block fills
// blocks 8n .. 8n+7; lane l writes 16 bytes of block 8n + l/8: row (l%8)/2 of
// its group of 4, dims 8*(l%2) .. +8 of its 16-dim segment.
template <int D> __host__ __device__ constexpr int v_row(int n, int l) {
  return 4 * ((8 * n + l / 8) / (D / 16)) + (l % 8) / 2;
}
template <int D> __host__ __device__ constexpr int v_dim(int n, int l) {
  return 16 * ((8 * n + l / 8) % (D / 16)) + 8 * (l % 2);
}
template <int D> __host__ __device__ constexpr int v_off(int r, int d) {
  return (r / 4) * (8 * D) + (d / 16) * 128 + 32 * (r % 4) + 2 * (d % 16);
}
// V^T fragment reads (the A operand of O^T += V^T P^T, PV k-step u of 16 keys,
// head-dimension tile t of 32 dims) through ds_read_b64_tr_b16: lane l reads 8
// bytes at v_read_base(l) + v_read_off(u, t, e), e = 0 for operand slots 0..3
// and e = 1 for slots 4..7.  Within each 16-lane group the hardware hands lane
// i element j (j = 0..3) of its result from element i % 4 of the 8 bytes that
// lane 4j + i/4 of the group addressed.
template <int D> __host__ __device__ __forceinline__ constexpr int v_read_base(int l) {
  return ((l >> 4) >> 1) * 4 * (2 * D) + ((l >> 4) & 1) * 128 + 8 * (l & 15);
}
template <int D> __host__ __device__ __forceinline__ constexpr int v_read_off(int u, int t, int e) {
  return u * 32 * D + e * 16 * D + t * 256;
}
// Compile-time proof of the V layout of a block of BN keys:
//  - the direct loads (load n, lane l: 16 bytes at n*1024 + 16*l, key row
//    v_row, dims v_dim .. +7) stay inside the block, land where v_off puts
//    them and write every (row, 8 dims) exactly once; where the kernel splits
//    the load address into a per-load and a per-lane part (8 blocks of a load
//    and the 16-dim segments of a row nest), the parts add up to it;
//  - every transposing read is 8-byte aligned and inside the block, each
//    16-lane group reads one 128-byte span with 16 distinct 8-byte slots, and
//    slot s of lane l's operand receives V[key][32t + l%32] for the key that
//    slot s of the P~ operand holds: 16u + 8*(s/4) + 4*(l/32) + s%4 (P~ is
//    packed from the S^T accumulators, whose register r of lane l is key
//    8*(r/4) + 4*(l/32) + r%4 of its 32-key sub-block).
template <int D, int BN> __host__ __device__ constexpr bool v_layout_ok() {
  constexpr int TBV = BN * 2 * D, NSEG = D / 16;
  constexpr bool SEP = 8 % NSEG == 0 || NSEG % 8 == 0;
  bool seen[BN * D / 8] = {};
  for (int n = 0; n < TBV / 1024; ++n)
    for (int l = 0; l < 64; ++l) {
      const int r = v_row<D>(n, l), d = v_dim<D>(n, l);
      if (r < 0 || r >= BN || d < 0 || d + 8 > D || d % 8 != 0) return false;
      for (int k = 0; k < 8; ++k)
        if (v_off<D>(r, d + k) != n * 1024 + 16 * l + 2 * k) return false;
      if (seen[(r * D + d) / 8]) return false;
      seen[(r * D + d) / 8] = true;
      if (SEP && v_row<D>(n, 0) * D + v_dim<D>(n, 0) + v_row<D>(0, l) * D + v_dim<D>(0, l) !=
                     r * D + d)
        return false;
    }
  for (int u = 0; u < BN / 16; ++u)
    for (int t = 0; t < D / 32; ++t)
      for (int e = 0; e < 2; ++e)
        for (int grp = 0; grp < 4; ++grp) {
          int lo = 1 << 30;
          for (int l = 16 * grp; l < 16 * grp + 16; ++l) {
            const int a = v_read_base<D>(l) + v_read_off<D>(u, t, e);
            lo = a < lo ? a : lo;
            if (a < 0 || a + 8 > TBV || a % 8 != 0) return false;
          }
          bool used[16] = {};
          for (int l = 16 * grp; l < 16 * grp + 16; ++l) {
            const int a = v_read_base<D>(l) + v_read_off<D>(u, t, e);
            if (a - lo >= 128 || used[(a - lo) / 8]) return false;
            used[(a - lo) / 8] = true;
            const int i = l & 15;
            for (int j = 0; j < 4; ++j) {
              const int src = 16 * grp + 4 * j + i / 4;  // the lane whose address serves slot j
              const int s = 4 * e + j;
              const int key = 16 * u + 8 * (s / 4) + 4 * (l / 32) + s % 4;
              const int dim = 32 * t + (l & 31);
              if (v_read_base<D>(src) + v_read_off<D>(u, t, e) + 2 * (i % 4) != v_off<D>(key, dim))
                return false;
            }
          }
        }
  return true;
}
// Q rows staged in LDS (a wavefront's 32 rows of 2D bytes, QC = D/8 chunks of
// 16 bytes each): chunk c of row r sits at slot c ^ q_swz(r) of the row.
template <int D> __host__ __device__ constexpr int q_swz(int r) {
  return (r * (D / 8) / 16) & (D / 8 - 1);
}
// Compile-time proof of that layout: direct load n, lane l (16 bytes at
// n*1024 + 16*l) fills slot l % QC of row QRPL*n + l / QC with the chunk that
// belongs there, every (row, chunk) exactly once; the operand read of k-step
// ks (lane l: chunk 2*ks + l/32 of row l%32) finds that chunk; and each
// 16-lane group of a read meets 16 different 16-byte bank groups.
template <int D> __host__ __device__ constexpr bool q_layout_ok() {
  constexpr int ROWB = 2 * D, QC = D / 8, QRPL = 1024 / ROWB;
  if (QC < 4 || QC > 16 || (QC & (QC - 1)) != 0 || QRPL * QC != 64) return false;
  int where[32 * 16] = {};
  for (int i = 0; i < 32 * QC; ++i) where[i] = -1;
  for (int n = 0; n < 32 * ROWB / 1024; ++n)
    for (int l = 0; l < 64; ++l) {
      const int r = QRPL * n + l / QC, c = (l % QC) ^ q_swz<D>(r), off = n * 1024 + 16 * l;
      if (off != r * ROWB + (l % QC) * 16 || where[r * QC + c] != -1) return false;
      where[r * QC + c] = off;
    }
  for (int ks = 0; ks < D / 16; ++ks)
    for (int grp = 0; grp < 4; ++grp) {
      bool used[16] = {};
      for (int l = 16 * grp; l < 16 * grp + 16; ++l) {
        const int qc = l & 31, c = 2 * ks + (l >> 5);
        const int off = qc * ROWB + ((c ^ q_swz<D>(qc)) * 16);
        if (where[qc * QC + c] != off || used[(off / 16) % 16]) return false;
        used[(off / 16) % 16] = true;
      }
    }
  return true;
}
static_assert(q_layout_ok<128>(), "Q LDS layout");

template <typename T, int D, bool CAUSAL, bool SPLIT, int WAVES, int OCC>
__global__ void __launch_bounds__(64 * WAVES, (groups_per_cu<WAVES, OCC>()))
fa2_fwd_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
               const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
               float* __restrict__ Lg, float* __restrict__ Ow, float* __restrict__ Lw,
               int Nq, int Nk, int BH, int num_m_block, int num_splits, int total_items,
               float c, float scale_abs, uint32_t qsign, uint32_t qkeep) {
  typedef typename Vec16<T>::x8 t8_t;
  typedef typename Vec16<T>::x4 t4_t;
  constexpr int BN = Cfg<D>::BN;
  constexpr int kWaves = WAVES;              // wavefronts per workgroup
  constexpr int kBM = 32 * WAVES;            // query rows per work item
  static_assert((WAVES == 4 || WAVES == 8) && groups_per_cu<WAVES, OCC>() >= 1, "wavefronts");
  constexpr int CH = D / 8;                  // 16-byte chunks per key row
  constexpr int KT = BN / 32;                // 32-key sub-blocks per block
  constexpr int KS = D / 16;                 // MFMA k-steps over the head dimension
  constexpr int DT = D / 32;                 // 32-wide tiles of the head dimension
  constexpr int U = BN / 16;                 // 16-key MFMA k-steps of the PV product
  constexpr int ROWB = D * 2;                // bytes per key row
  constexpr int RPP = rows_per_piece<D>();   // key rows per 1 KB piece
  constexpr int PIECES = BN / RPP;           // pieces per K block
  constexpr int LOADS = PIECES / kWaves;     // direct loads per thread per block
  constexpr int TB = PIECES * kPiece;        // bytes per K block buffer
  constexpr int TBV = BN * ROWB;             // bytes per V block buffer
  constexpr int LOADS_V = TBV / 1024 / kWaves;  // direct V loads per thread per block
  constexpr int NSEG = D / 16;               // 16-dim segments per V row
  // V load addresses split into a per-lane part and a per-load part unless the
  // 16-dim segments of a row and the 8 blocks of a load do not nest (D = 96).
  constexpr bool V_SEP = 8 % NSEG == 0 || NSEG % 8 == 0;
  constexpr int KTSTEP = lds_off<D>(32) - lds_off<D>(0); // 32 keys further in a K block
  constexpr int NSTORE = DT * (SPLIT ? 4 : 2) + 1;  // O and L stores per wavefront per item
  static_assert(LOADS >= 1 && PIECES % kWaves == 0, "block must split evenly over wavefronts");
  static_assert(BN % 32 == 0 && BN % RPP == 0 && RPP * ROWB <= 1024, "piece geometry");
  static_assert(k_layout_ok<D, BN>(), "K LDS layout: rows, pieces and banks");
  static_assert(lds_off<D>(BN - 1) + ROWB <= TB, "K rows stay inside their buffer");
  static_assert(LOADS_V >= 1 && TBV % (1024 * kWaves) == 0, "V block must split evenly");
  static_assert(v_layout_ok<D, BN>(), "V LDS layout: direct loads and transposing reads");
  // Eight-wavefront form (d = 128): the next item's Q rows go by direct loads
  // of whole rows into QB bytes of LDS (8 KB per wavefront), and the prologue
  // reads them from there in the MFMA operand layout.  (Loaded in that layout
  // straight from memory, each lane reads its own row: 32 rows per load
  // instruction, which held the last block of every item up by thousands of
  // cycles.)  The four-wavefront forms, whose two or three workgroups per CU
  // cover each other's item edges, keep the per-lane loads.
  constexpr bool QT = WAVES == 8;
  constexpr int QB = QT ? kBM * ROWB : 0;
  constexpr int QC = ROWB / 16;             // 16-byte chunks per Q row
  constexpr int QRPL = 1024 / ROWB;         // Q rows per direct load
  constexpr int QLOADS = 32 * ROWB / 1024;  // direct loads of a wavefront's 32 Q rows
  static_assert(!QT || q_layout_ok<D>(), "Q LDS layout: direct loads and operand reads");
  static_assert(groups_per_cu<WAVES, OCC>() * (2 * TBV + 2 * TB + QB) <= 160 * 1024,
                "the resident workgroups' LDS fits a CU");
  static_assert(TBV + 16 * ROWB * (U - 1) + 8 * ROWB + 256 * (DT - 1) < 65536 &&
                    2 * TBV + TB + KTSTEP * (KT - 1) + 32 * (KS - 1) < 65536,
                "LDS offsets fit the 16-bit instruction offset");

  __shared__ __attribute__((aligned(1024))) char smem[2 * TBV + 2 * TB + QB];  // V0 V1 K0 K1 Q
  char* const Vb0 = smem;
  char* const Kb0 = smem + 2 * TBV;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
  const int col = lane & 31;  // this lane's query row within the wavefront's 32
  // The wavefront's group of 32 query rows in a work item.  With eight
  // wavefronts, w and w + 4 share a SIMD; they take groups w and 7 - w, so
  // that each SIMD holds one early and one late group of the item and the
  // causal diagonal's work (and the blocks it hides) splits evenly over the
  // SIMDs.
  const int rgrp = kWaves == 8 && wave >= 4 ? 11 - wave : wave;
  const int half = lane >> 5;

  // Causal offset: key j is visible to query i when j <= i + off.
  const int off = Nk - Nq;
  const int nkb = (Nk + BN - 1) / BN;  // K/V blocks of a (batch, head)

  // ---- work schedule.  The grid is persistent: each workgroup processes a
  // sequence of work items (query block, batch*head).  Workgroup ids reach the
  // 8 XCDs round-robin; XCD x takes a contiguous range of logical items (the
  // query blocks of the same few heads, which read the same K/V and so share
  // that XCD's L2), ordered head by head with a head's heaviest causal query
  // block first.  The workgroups of an XCD walk that range in groups, in a
  // snake order (group k: slot s takes position s, or P-1-s when k is odd), so
  // that heavy and light causal blocks alternate per workgroup.
  // (With fewer than 8 workgroups the ranges are split over that many.)
  // (The walk and the item mapping are in fa2_schedule.h, shared with the
  // library's host-side schedule queries.)
  const sched::Walk walk = sched::walk_of(total_items, (int)gridDim.x, (int)blockIdx.x);
  auto logical_of = [&](int k) -> int {  // the k-th item of this workgroup, or -1
    return sched::item_of(walk, k);
  };

  // ---- per-item state
  int bh = 0, m = 0, q0 = 0, qrow = 0, j_beg = 0, j_end = 0, j_mask = 0, j_cend = 0;
  int g0 = 0;      // running block count of this workgroup at the current item's first block
  int k_item = 0;  // index of the current item in this workgroup's sequence
  const uint16_t *Qh = Qg, *Kh = Kg, *Vh = Vg;
  // O and L of the item's query block as buffer resources whose size covers
  // only the rows < Nq: the hardware drops stores to rows past the end, so
  // every wavefront issues the same number of stores for every item.
  __amdgpu_buffer_rsrc_t o_rsrc, l_rsrc;
  int gb = 0;  // buffer parity base: block j uses K and V buffers (gb + j) & 1
  // logical item -> (batch*head, query block, split): splits fastest, then the
  // query blocks of a head (heaviest causal block first), then the heads.
  auto decode = [&](int logical, int& bh_, int& m_, int& s_) __attribute__((always_inline)) {
    const sched::Item it = sched::decode(logical, num_m_block, num_splits, CAUSAL, SPLIT);
    bh_ = it.bh;
    m_ = it.m;
    s_ = it.split;
  };
  // K/V blocks up to the last key that query block m sees.  A query block
  // whose last row sees no key has none: with splits its items are empty;
  // without, it runs block 0 fully masked, which leaves every row with l = 0
  // (O = 0, L = -inf) and keeps the empty-item path out of the plain kernel.
  // (Nk >= 1 here; the host handles Nk == 0.)
  auto blocks_of = [&](int m_) __attribute__((always_inline)) -> int {
    return sched::blocks_of(m_, Nq, off, nkb, kBM, BN, CAUSAL, SPLIT);
  };
  // KV blocks [beg, end) of split s of query block m.
  auto range_of = [&](int m_, int s_, int& beg, int& end) __attribute__((always_inline)) {
    const sched::Range r = sched::range_of(blocks_of(m_), s_, num_splits, SPLIT);
    beg = r.beg;
    end = r.end;
  };
  auto set_item = [&](int logical) __attribute__((always_inline)) {
    int sp;
    decode(logical, bh, m, sp);
    range_of(m, sp, j_beg, j_end);
    const size_t qslice = (size_t)bh * (size_t)Nq * D;
    const size_t kslice = (size_t)bh * (size_t)Nk * D;
    Qh = Qg + qslice;
    Kh = Kg + kslice;
    Vh = Vg + kslice;
    const int rows = min(kBM, Nq - m * kBM);
    if constexpr (SPLIT) {
      const size_t prow = ((size_t)sp * BH + bh) * Nq + (size_t)m * kBM;  // first partial row
      o_rsrc = __builtin_amdgcn_make_buffer_rsrc(Ow + prow * D, (short)0, rows * D * 4,
                                                 kBufferFlags);
      l_rsrc = __builtin_amdgcn_make_buffer_rsrc(Lw + prow, (short)0, rows * 4, kBufferFlags);
    } else {
      o_rsrc = __builtin_amdgcn_make_buffer_rsrc(Og + qslice + (size_t)m * kBM * D, (short)0,
                                                 rows * ROWB, kBufferFlags);
      l_rsrc = __builtin_amdgcn_make_buffer_rsrc(Lg + (size_t)bh * Nq + (size_t)m * kBM, (short)0,
                                                 rows * 4, kBufferFlags);
    }
    q0 = m * kBM + rgrp * 32;  // first query row of this wavefront
    qrow = q0 + col;
    gb = g0 - j_beg;
    // Blocks before j_mask need no mask for this wavefront (every key visible
    // to every one of its rows: below the first row's diagonal, and whole).
    const int seen = q0 + off + 1;  // keys visible to the wavefront's first row
    j_mask = CAUSAL ? (seen <= 0 ? 0 : min(seen / BN, Nk / BN)) : Nk / BN;
    // Blocks from j_cend on are hidden from every row of this wavefront (past
    // its last row's diagonal; the item's later rows need them): it takes part
    // in their loads and barriers only.  At least one block is computed (a
    // wavefront whose rows see no key computes one block fully masked).
    const int last_seen = q0 + 31 + off;  // last key visible to the wavefront's last row
    j_cend = CAUSAL ? max(j_beg + 1, min(j_end, last_seen < 0 ? 0 : last_seen / BN + 1)) : j_end;
  };

  // Q fragments (the B operand of S^T = K Q^T), kept in registers for an item.
  // A negative scale flips Q's sign (exact); a zero scale zeroes Q, which gives
  // the same all-zero logits.
  t8_t qf[KS];
  auto load_q = [&](const uint16_t* qh, int row) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t t = {0u, 0u, 0u, 0u};
      if (row < Nq) t = *(const u32x4_t*)(qh + (size_t)row * D + ks * 16 + 8 * half);
      qf[ks] = __builtin_bit_cast(t8_t, t);
    }
  };
  // Whole-row direct loads into this wavefront's 32 * ROWB bytes of LDS:
  // load n fills rows QRPL*n .. QRPL*n + QRPL-1 of the wavefront's 32, lane l
  // the 16-byte slot l % QC of row r = QRPL*n + l / QC.  Row r's chunk c sits
  // at slot c ^ q_swz(r), so lane l fetches chunk (l % QC) ^ q_swz(r).  The
  // operand reads below take one chunk index of 16 consecutive rows per 16
  // lanes; those rows span 16 * ROWB bytes, and q_swz gives the rows that
  // fall on the same 16-byte bank group of a 256-byte line distinct slots, so
  // the 16 lanes meet 16 different bank groups.  Rows past Nq are clamped to
  // row Nq-1: their results are never stored.  Only this wavefront touches
  // its area.
  char* const q_area = smem + 2 * TBV + 2 * TB + wave * 32 * ROWB;
  auto load_q_lds = [&](const uint16_t* qh, int row0) __attribute__((always_inline)) {
    const int ql = fresh_lane();
    const int rl = ql / QC, sl = ql % QC;
    if (row0 + 32 <= Nq) {
#pragma unroll
      for (int n = 0; n < QLOADS; ++n) {
        const uint32_t voff = (uint32_t)(rl * D + (sl ^ q_swz<D>(QRPL * n + rl)) * 8) * 2;
        lds_dma(qh + (size_t)(row0 + QRPL * n) * D, voff, lds_addr(q_area + n * 1024));
      }
    } else {
#pragma unroll
      for (int n = 0; n < QLOADS; ++n) {
        const int r = QRPL * n + rl;
        lds_dma(qh + (size_t)min(row0 + r, Nq - 1) * D + (sl ^ q_swz<D>(r)) * 8,
                lds_addr(q_area + n * 1024));
      }
    }
  };
  // ... read in the operand layout once they have landed (prologue).
  auto read_q = [&]() __attribute__((always_inline)) {
    if constexpr (QT) {
      const int ql = fresh_lane();
      const int qc = ql & 31, qhf = ql >> 5;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[ks] = *(const t8_t*)(q_area + qc * ROWB + (((2 * ks + qhf) ^ q_swz<D>(qc)) * 16));
    }
  };
  // After the sign/zero fix, the fragments pass through an empty asm
  // statement: the compiler waits for the Q loads there, once per item, and
  // from then on sees register values with no load pending (it cannot see the
  // direct LDS loads, so a pending Q load inside the KV loop would make it
  // wait for every load in flight).
  auto fix_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t t = (__builtin_bit_cast(u32x4_t, qf[ks]) & qkeep) ^ qsign;
      asm volatile("" : "+v"(t));
      qf[ks] = __builtin_bit_cast(t8_t, t);
    }
  };

  // ---- global -> LDS staging.  K: load i of this thread fills piece
  // b = wave*LOADS + i, whose lane L writes bytes 16L.. of the piece: row slot
  // L / CH, 16-byte chunk L % CH of the key row r with blk(r) = b and
  // slot(r) = L / CH.  That row is piece_row(b) (wave-uniform) plus
  // slot_row(L / CH) (per lane).  For D = 96 a piece holds 4 rows (lanes
  // 0..47); lanes 48..63 repeat the loads of lanes 0..15 into the piece's
  // unread last 256 bytes, so every lane's address stays inside the tensor.
  auto k_src_lane = [](int l) { return D == 96 && l >= 48 ? l - 48 : l; };
  auto k_lane_row = [&](int l) { return slot_row<D>(k_src_lane(l) / CH); };
  auto k_lane_col = [&](int l) { return (k_src_lane(l) % CH) * 8; };
  const uint32_t lane_bytes = (uint32_t)(k_lane_row(lane) * D + k_lane_col(lane)) * 2;
  // k0 goes through an empty asm statement: for the constant first blocks of an
  // item the compiler would otherwise precompute the clamped tail addresses
  // once, outside the item loop, and keep them in (spilled) registers.
  auto issue_k = [&](const uint16_t* head, int k0, char* buf) __attribute__((always_inline)) {
    asm volatile("" : "+s"(k0));
    if (k0 + BN <= Nk) {
      // Scalar base (the piece's first row) plus a constant 32-bit per-lane offset.
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int b = wave * LOADS + i;
        lds_dma(head + (size_t)(k0 + piece_row<D>(b)) * D, lane_bytes,
                lds_addr(buf + b * kPiece));
      }
    } else {
      // Ragged last block: rows past Nk are clamped to row Nk-1 (their keys are masked).
      const int tl = fresh_lane();
      const int lane_row = k_lane_row(tl), lane_col = k_lane_col(tl);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int b = wave * LOADS + i;
        const int r = min(k0 + piece_row<D>(b) + lane_row, Nk - 1);
        lds_dma(head + (size_t)r * D + lane_col, lds_addr(buf + b * kPiece));
      }
    }
  };
  // V: load i of this thread fills 1 KB chunk n = wave*LOADS_V + i of the
  // block (v_row / v_dim above).  Where the geometry nests, the lane's share of
  // the row and dims is the same for every n and n adds a wave-uniform offset;
  // otherwise each load keeps its own per-lane offset.
  uint32_t vlane[V_SEP ? 1 : LOADS_V];
  if constexpr (V_SEP) {
    vlane[0] = (uint32_t)(v_row<D>(0, lane) * D + v_dim<D>(0, lane)) * 2;
  } else {
#pragma unroll
    for (int i = 0; i < LOADS_V; ++i)
      vlane[i] = (uint32_t)(v_row<D>(wave * LOADS_V + i, lane) * D +
                            v_dim<D>(wave * LOADS_V + i, lane)) * 2;
  }
  auto issue_v = [&](const uint16_t* head, int k0, char* buf) __attribute__((always_inline)) {
    asm volatile("" : "+s"(k0));
    const char* base = (const char*)(head + (size_t)k0 * D);
    if (k0 + BN <= Nk) {
#pragma unroll
      for (int i = 0; i < LOADS_V; ++i) {
        const int n = wave * LOADS_V + i;
        if constexpr (V_SEP)
          lds_dma(base + (v_row<D>(n, 0) * D + v_dim<D>(n, 0)) * 2, vlane[0],
                  lds_addr(buf + n * 1024));
        else
          lds_dma(base, vlane[i], lds_addr(buf + n * 1024));
      }
    } else {
      // Ragged last block: rows past Nk are clamped to row Nk-1 (P~ is 0 there).
      const int tl = fresh_lane();
#pragma unroll
      for (int i = 0; i < LOADS_V; ++i) {
        const int n = wave * LOADS_V + i;
        const int r = min(k0 + v_row<D>(n, tl), Nk - 1);
        lds_dma(head + (size_t)r * D + v_dim<D>(n, tl), lds_addr(buf + n * 1024));
      }
    }
  };
  // The first blocks of an item (blocks beg, beg+1, ... of its range): Q rows,
  // K_beg and V_beg, and K_beg+1 if the range has it.  g is the running block
  // count of this workgroup: block g of the sequence uses buffers g & 1.
  auto issue_item_q = [&](const uint16_t* qh, int row0) __attribute__((always_inline)) {
    if constexpr (QT) load_q_lds(qh, row0);
    else load_q(qh, row0 + col);
  };
  auto issue_item_kv = [&](const uint16_t* kh, const uint16_t* vh, int beg, int blocks,
                           int g) __attribute__((always_inline)) {
    issue_k(kh, beg * BN, Kb0 + (g & 1) * TB);
    issue_v(vh, beg * BN, Vb0 + (g & 1) * TBV);
    if (blocks > 1) issue_k(kh, (beg + 1) * BN, Kb0 + ((g + 1) & 1) * TB);
  };
  auto issue_item_start = [&](const uint16_t* qh, const uint16_t* kh, const uint16_t* vh, int row0,
                              int beg, int blocks, int g) __attribute__((always_inline)) {
    issue_item_q(qh, row0);
    issue_item_kv(kh, vh, beg, blocks, g);
  };

  // ---- LDS fragment addresses (bytes within a block buffer).
  // K (A operand of S^T): key row kt*32 + col, dims 16*ks + 8*half ..+8.
  const uint32_t kaddr = lds_off<D>(col) + 16 * half;
  // V^T (A operand of O^T += V^T P^T) through ds_read_b64_tr_b16: within each
  // group of 16 lanes, lane 4*r + c supplies the address of 4 consecutive dims
  // (d0 + 4c ..) of key row (kbase + r); the hardware hands lane t of the
  // group the 4 keys kbase..kbase+3 of dim d0 + t.  kbase = 16u + 4*half (the
  // first 4 slots of the operand) or 16u + 8 + 4*half (the last 4), matching
  // the keys 8*(r/4) + 4*half + r%4 that a lane's S^T accumulators hold.  With
  // the V layout, the 16 lanes of a group read one contiguous 128-byte block:
  // lane i at byte 8i of the block of rows kbase.. and dims d0..d0+15.
  const uint32_t vaddr = (uint32_t)v_read_base<D>(lane);

  // Issue priority: lowered by one each time another prio_step blocks of this
  // workgroup's sequence have started (set before the first item).
  int prio_step = 1, prio_next = 1, prio_level = 3;

  f32x16_t o[DT];
  float m_ref = kNegInf;  // reference max of the (sign-adjusted) raw logits
  float mc = 0.f;         // c * m_ref (0 while m_ref = -inf)
  float m_lim = kNegInf;  // m_ref + kTau / c: a larger row max moves the reference
  float l_part = 0.f;     // running sum over this lane's half of the keys
  const float tau_raw = kTau / c;
  // Row max of the block about to be consumed, formed while the block before
  // it was finished (over the unmasked logits; a masked block forms it again).
  float mx_c = kNegInf;

  auto compute_S = [&](const char* kb, f32x16_t (&S)[KT]) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      S[kt] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const t8_t a = *(const t8_t*)(kb + kaddr + kt * KTSTEP + ks * 32);
        S[kt] = mfma32x32x16(a, qf[ks], S[kt]);
      }
    }
  };

  // Row max over the lane's keys and the lane 32 positions away.
  auto row_max = [&](const f32x16_t(&S)[KT]) __attribute__((always_inline)) -> float {
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kt][r]);
    return halves_max(mx);
  };

  // Block j's step of the online softmax (new running max, rescaled running
  // sum, unnormalised probabilities) and the rescaled O update.  `during`
  // issues independent MFMA work (the next block's S) after the rescale test,
  // where it can overlap this block's exps; `after` forms the next block's
  // row max while the PV product runs.  The row max of block j (mx_c) was
  // formed by the previous step's `after` (or the item's prologue); a masked
  // block forms it again after masking.
  auto consume = [&](auto masked_tag, int j, f32x16_t(&S)[KT], auto&& during,
                     auto&& after) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = j * BN;
    if constexpr (MASKED) {
      // key = k0 + cr + 4*half with cr = kt*32 + 8*(r/4) + r%4 (a constant):
      // it is hidden when cr + (k0 - q0 - off) > col - 4*half (after the lane's
      // query row's diagonal) or cr + (k0 - Nk) >= -4*half (past the keys),
      // i.e. when cr exceeds one per-lane threshold.
      const int ml = fresh_lane();
      const int mh = -4 * (ml >> 5);
      int th = mh - (k0 - Nk) - 1;
      if (CAUSAL) th = min(th, (ml & 31) + mh - (k0 - q0 - off));
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = kt * 32 + 8 * (r / 4) + (r % 4);
          S[kt][r] = cr > th ? kNegInf : S[kt][r];
        }
      mx_c = row_max(S);
    }
    const float mx = mx_c;
    // The reference moves when the block's row max exceeds m_lim = m_ref +
    // kTau / c.  The first block with a visible key always moves it (m_lim =
    // -inf; alpha = exp2(-inf) = 0 then: O and l are still zero).  A block can
    // hold no key a row sees (mx = -inf: a split's range, or a row that sees
    // no key at all): the reference then stays at -inf and the block adds
    // nothing, without forming exp2(-inf + inf).  Moves are rare, so the test
    // is one compare and a branch that the whole wavefront takes together.
    if (__builtin_amdgcn_ballot_w64(mx > m_lim)) {
      const bool move = mx > m_lim;
      const float alpha = move ? __builtin_amdgcn_exp2f(c * (m_ref - mx)) : 1.f;
      m_ref = move ? mx : m_ref;
      mc = move ? c * mx : mc;
      m_lim = move ? mx + tau_raw : m_lim;
      l_part *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] *= alpha;
    }
    during();
    float ls[2] = {0.f, 0.f};  // two chains: shorter dependency, same sum in every form
    t8_t pb[U];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kt][r], c, -mc));
        ls[r / 8] += p;
        pb[kt * 2 + r / 8][r % 8] = (T)p;  // round to nearest even
      }
    l_part += ls[0] + ls[1];
    const char* vb = Vb0 + ((gb + j) & 1) * TBV + vaddr;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr_t)(vb + v_read_off<D>(u, t, 0)));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr_t)(vb + v_read_off<D>(u, t, 1)));
        const t8_t a =
            __builtin_bit_cast(t8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[t] = mfma32x32x16(a, pb[u], o[t]);
      }
    after();
    // The row sum and the next row max are due before the next block's
    // barrier: formed here they overlap the PV product (left to itself, the
    // compiler moves both past the barrier, where nothing overlaps them).
    asm volatile("" : "+v"(l_part), "+v"(mx_c));
  };

  // One barrier per block: block j's V and block j+1's K have landed in LDS,
  // and every wavefront is done with the buffers of block j-1, which the loads
  // for blocks j+2 (K) and j+1 (V) issued right after reuse.
  // k_known / v_known: the caller knows that block j+2 (K) / j+1 (V) exists
  // (the loops of block pairs below), so the test is left out of the loop.
  // Eight-wavefront form: the next item's Q rows go out in the current
  // item's prologue (the Q area is free once it has been read), so that an
  // item's last block issues only K/V loads; the first block's wait then
  // leaves those rows in flight.
  bool q_early = false;
  auto advance = [&](int j, auto k_known, auto v_known) __attribute__((always_inline)) {
    // At an item's first block the previous item's O and L stores, issued
    // last, need not have completed.  (The eight-wavefront form waits for
    // them too: by then they have had the item edge to complete, and the
    // block loop without the test runs 0-1% faster.)
    if constexpr (QT) {
      if (j == j_beg && q_early) wait_vmcnt<QLOADS>();
      else wait_vmcnt<0>();
    } else {
      if (kWaves == 4 && j == j_beg && k_item > 0) wait_vmcnt<NSTORE>();
      else wait_vmcnt<0>();
    }
    lds_barrier();
    if (kWaves == 4 && g0 + (j - j_beg) >= prio_next) {  // a quarter of the blocks passed
      prio_next += prio_step;
      --prio_level;
      if (prio_level == 2) __builtin_amdgcn_s_setprio(2);
      else if (prio_level == 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    if (decltype(k_known)::value || j + 2 < j_end) issue_k(Kh, (j + 2) * BN, Kb0 + ((gb + j) & 1) * TB);
    if (decltype(v_known)::value || j + 1 < j_end) issue_v(Vh, (j + 1) * BN, Vb0 + ((gb + j + 1) & 1) * TBV);
  };

  // The item after the current one, and its key range.
  int next = -1, nbh = 0, nm = 0, nsp = 0, nbeg = 0, nend = 0;
  auto look_ahead = [&]() __attribute__((always_inline)) {
    next = logical_of(k_item + 1);
    if (next >= 0) {
      decode(next, nbh, nm, nsp);
      range_of(nm, nsp, nbeg, nend);
    }
  };
  // ---- item prologue: wait for Q and K_beg, then S for the first block.
  // Vector memory operations complete in issue order, and V_beg and K_beg+1
  // (and, after the first item, the previous item's O and L stores) were
  // issued after K_beg, so the wait leaves that many operations in flight;
  // then a barrier.  The first item's prologue is separate from the later
  // items' (at the end of the loop), so that the compiler's own wait for the
  // Q registers counts the stores on the later path instead of draining
  // everything.
  f32x16_t S_cur[KT];
  auto prologue = [&](auto later_tag) __attribute__((always_inline)) {
    const bool two = j_end - j_beg > 1;
    if constexpr (QT) {
      // The Q rows (the oldest loads in flight) have landed; K, V and the
      // stores may still be in flight.
      if constexpr (decltype(later_tag)::value) {
        if (two) wait_vmcnt<LOADS_V + 2 * LOADS + NSTORE>();
        else wait_vmcnt<LOADS_V + LOADS + NSTORE>();
      } else {
        if (two) wait_vmcnt<LOADS_V + 2 * LOADS>();
        else wait_vmcnt<LOADS_V + LOADS>();
      }
      read_q();
    }
    fix_q();
    if constexpr (decltype(later_tag)::value) {
      if (two) wait_vmcnt<LOADS_V + LOADS + NSTORE>();
      else wait_vmcnt<LOADS_V + NSTORE>();
    } else {
      if (two) wait_vmcnt<LOADS_V + LOADS>();
      else wait_vmcnt<LOADS_V>();
    }
    lds_barrier();
    if constexpr (QT) {
      look_ahead();
      q_early = next >= 0 && nend > nbeg;
      if (q_early) issue_item_q(Qg + (size_t)nbh * (size_t)Nq * D, nm * kBM + rgrp * 32);
    }
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = f32x16_t{};
    m_ref = kNegInf;
    mc = 0.f;
    m_lim = kNegInf;
    l_part = 0.f;
    compute_S(Kb0 + (g0 & 1) * TB, S_cur);
    mx_c = row_max(S_cur);
  };
  // The next item's Q (with eight wavefronts, only its K/V: the Q rows went
  // out in the prologue) and first K/V blocks; issued while this item's last
  // block is processed (or at once, for an empty item).
  auto prefetch_next = [&]() __attribute__((always_inline)) {
    if (next >= 0 && nend > nbeg) {
      const size_t nqs = (size_t)nbh * (size_t)Nq * D, nks = (size_t)nbh * (size_t)Nk * D;
      if constexpr (QT)
        issue_item_kv(Kg + nks, Vg + nks, nbeg, nend - nbeg, g0 + (j_end - j_beg));
      else
        issue_item_start(Qg + nqs, Kg + nks, Vg + nks, nm * kBM + rgrp * 32, nbeg,
                         nend - nbeg, g0 + (j_end - j_beg));
    }
  };
  // The same in two parts, for a wavefront whose rows see none of the item's
  // last blocks: its Q registers are free from its last computed block on, so
  // its share of the next item's Q goes out then (with eight wavefronts it
  // went out in the prologue), and the next item's first K/V blocks (whose
  // buffers free up only at the item's last block) later.
  auto prefetch_next_q = [&]() __attribute__((always_inline)) {
    if constexpr (!QT) {
      if (next >= 0 && nend > nbeg)
        issue_item_q(Qg + (size_t)nbh * (size_t)Nq * D, nm * kBM + rgrp * 32);
    }
  };
  auto prefetch_next_kv = [&]() __attribute__((always_inline)) {
    if (next >= 0 && nend > nbeg) {
      const size_t nks = (size_t)nbh * (size_t)Nk * D;
      issue_item_kv(Kg + nks, Vg + nks, nbeg, nend - nbeg, g0 + (j_end - j_beg));
    }
  };
  // ---- item epilogue, after the KV loop: O = O / l once, L = m + ln(l).
  // (A row that saw no key has l = 0: O = 0 and L = -inf.)
  auto store_result = [&]() __attribute__((always_inline)) {
    const float l_tot = halves_sum(l_part);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int lrow = rgrp * 32 + col;  // this lane's row in the query block
    if constexpr (SPLIT) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dim = t * 32 + 8 * g + 4 * half;
          f32x4_t w;
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = o[t][g * 4 + r] * inv;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, w), o_rsrc,
                                                 (lrow * D + dim) * 4, 0, 0);
        }
    } else {
      // Lane half h holds dims 32t + 8g + 4h .. +3 of its row for g = 0..3.
      // For each pair (2i, 2i+1), one swap across the halves leaves half h
      // with all 8 dims 32t + 8(2i + h) .. +7: 16-byte stores, half as many.
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          t4_t w0, w1;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            w0[r] = (T)(o[t][(2 * i) * 4 + r] * inv);
            w1[r] = (T)(o[t][(2 * i + 1) * 4 + r] * inv);
          }
          u32x2_t a = __builtin_bit_cast(u32x2_t, w0), b = __builtin_bit_cast(u32x2_t, w1);
          uint32_t a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
          swap_halves(a0, b0);
          swap_halves(a1, b1);
          const u32x4_t v = {a0, a1, b0, b1};
          __builtin_amdgcn_raw_buffer_store_b128(v, o_rsrc,
                                                 lrow * ROWB + (t * 32 + 8 * (2 * i + half)) * 2,
                                                 0, 0);
        }
    }
    // Both halves of a row hold the same l and m: they store the same L.
    __builtin_amdgcn_raw_buffer_store_b32(
        __builtin_bit_cast(uint32_t,
                           __builtin_fmaf(__builtin_amdgcn_logf(l_tot), kLn2, scale_abs * m_ref)),
        l_rsrc, lrow * 4, 0, 0);
  };
  // Split items whose key range is empty (a split past the keys its rows see,
  // or a query block that sees no key at all) are finished here (O_s = 0,
  // L_s = -inf), so that the KV loop below is only ever entered through a
  // prologue.  Returns false when the workgroup's sequence ends.
  auto finish_empty_items = [&]() __attribute__((always_inline)) -> bool {
    if constexpr (SPLIT) {
      while (j_end == j_beg) {
        look_ahead();
        prefetch_next();
#pragma unroll
        for (int t = 0; t < DT; ++t) o[t] = f32x16_t{};
        m_ref = kNegInf;
        l_part = 0.f;
        store_result();
        if (next < 0) return false;
        ++k_item;
        set_item(next);
      }
    }
    return true;
  };

  int logical = logical_of(0);
  if (logical < 0) return;  // uniform for the workgroup
  {
    int blocks = 0;  // this workgroup's K/V blocks over all its items
    for (int k = 0, lg = logical; lg >= 0; lg = logical_of(++k)) {
      int b_, m_, s_, beg_, end_;
      decode(lg, b_, m_, s_);
      range_of(m_, s_, beg_, end_);
      blocks += end_ - beg_;
    }
    prio_step = max(1, (blocks + 3) / 4);
    prio_next = prio_step;
    if constexpr (kWaves == 4) __builtin_amdgcn_s_setprio(3);
  }
  set_item(logical);
  if (!finish_empty_items()) return;
  if (k_item == 0) {
    issue_item_start(Qh, Kh, Vh, q0, j_beg, j_end - j_beg, g0);
    prologue(std::false_type{});
  } else {
    prologue(std::true_type{});  // prefetched by the last empty item, stores after it
  }

  for (;;) {
    if constexpr (!QT) look_ahead();
    const int j_unmasked = min(j_mask, j_cend - 1);  // unmasked blocks that have a successor
    f32x16_t SB[KT];
    int j = j_beg;
    // Unrolled by two so that the S registers alternate between S_cur and SB
    // instead of being copied every block.
    for (; j + 2 <= j_unmasked; j += 2) {
      advance(j, std::true_type{}, std::true_type{});
      consume(std::false_type{}, j, S_cur,
              [&]() { compute_S(Kb0 + ((gb + j + 1) & 1) * TB, SB); },
              [&]() { mx_c = row_max(SB); });
      advance(j + 1, std::false_type{}, std::true_type{});
      consume(std::false_type{}, j + 1, SB,
              [&]() { compute_S(Kb0 + ((gb + j) & 1) * TB, S_cur); },
              [&]() { mx_c = row_max(S_cur); });
    }
    if (j < j_unmasked) {
      advance(j, std::false_type{}, std::false_type{});
      consume(std::false_type{}, j, S_cur,
              [&]() { compute_S(Kb0 + ((gb + j + 1) & 1) * TB, SB); },
              [&]() { mx_c = row_max(SB); });
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) S_cur[kt] = SB[kt];
      ++j;
    }
    for (; j + 2 < j_cend; j += 2) {
      advance(j, std::true_type{}, std::true_type{});
      consume(std::true_type{}, j, S_cur,
              [&]() { compute_S(Kb0 + ((gb + j + 1) & 1) * TB, SB); }, [] {});
      advance(j + 1, std::false_type{}, std::true_type{});
      consume(std::true_type{}, j + 1, SB,
              [&]() { compute_S(Kb0 + ((gb + j) & 1) * TB, S_cur); }, [] {});
    }
    if (j + 1 < j_cend) {
      advance(j, std::false_type{}, std::false_type{});
      consume(std::true_type{}, j, S_cur,
              [&]() { compute_S(Kb0 + ((gb + j + 1) & 1) * TB, SB); }, [] {});
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) S_cur[kt] = SB[kt];
      ++j;
    }
    // Last block that this wavefront computes.  At the item's last block both
    // K buffers and the other V buffer are free, and so are the Q registers:
    // the next item's Q (unless it went out in the prologue), K_beg, V_beg and
    // K_beg+1 go out there and overlap that block's softmax, its PV product
    // and the O stores.
    advance(j, std::false_type{}, std::false_type{});
    if (j + 1 == j_end) prefetch_next();
    // Always the masked form: one copy of the code, and for an unmasked block
    // the threshold test hides nothing.
    consume(std::true_type{}, j, S_cur, [] {}, [] {});
    // Blocks hidden from all of this wavefront's rows: loads and barriers.
    // Its next Q rows go out after the first of them (its Q registers are
    // free; the item's last block then issues less at once).
    if (++j < j_end) {
      advance(j, std::false_type{}, std::false_type{});
      prefetch_next_q();
      if (j + 1 == j_end) prefetch_next_kv();
      for (++j; j < j_end; ++j) {
        advance(j, std::false_type{}, std::false_type{});
        if (j + 1 == j_end) prefetch_next_kv();
      }
    }
    store_result();
    if (next < 0) break;
    g0 += j_end - j_beg;
    ++k_item;
    set_item(next);
    if (!finish_empty_items()) break;
    prologue(std::true_type{});
  }
}

// OCC: wavefronts per SIMD that the kernel's registers allow (1: up to 512
// VGPRs, 2: up to 256, 3: up to 168, 4: up to 128).
template <typename T, int D, bool CAUSAL, bool SPLIT, int WAVES, int OCC>
hipError_t launch(const FwdArgs& a) {
  if (a.block_m != 32 * WAVES) return hipErrorInvalidValue;  // num_m_block counts other blocks
  const int splits = SPLIT ? a.num_splits : 1;
  const int total = a.num_m_block * a.BH * splits;
  // Persistent grid: as many workgroups as fit on the chip at once (a 4-wave
  // workgroup puts one wave on each SIMD of a CU, so mfma_waves_per_simd
  // workgroups per CU; an 8-wave one two, so one workgroup per CU), each
  // walking its share of the work items.
  int cus = 0;
  const hipError_t e = cu_count(&cus);
  if (e != hipSuccess) return e;
  const int resident = groups_per_cu<WAVES, OCC>() * cus;
  const int grid = total < resident ? total : resident;
  // The kernel works with c = |scale| * log2(e) > 0: a negative scale flips the
  // sign of Q and a zero scale zeroes Q (both exact), with |scale| = 1 then.
  const bool zero = a.scale == 0.f;
  const float sa = zero ? 1.f : (a.scale < 0.f ? -a.scale : a.scale);
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  const uint32_t qkeep = zero ? 0u : 0xFFFFFFFFu;
  hipLaunchKernelGGL((fa2_fwd_kernel<T, D, CAUSAL, SPLIT, WAVES, OCC>), dim3(grid), dim3(64 * WAVES), 0,
                     a.stream, (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (uint16_t*)a.O, a.L, a.ws_O, a.ws_L, a.Nq, a.Nk, a.BH, a.num_m_block,
                     splits, total, sa * kLog2e, sa, qsign, qkeep);
  return hipGetLastError();
}

// Enqueue the kernel for element type T: one instantiation per head
// dimension, mask and split setting.
template <typename T>
hipError_t dispatch_fwd_mfma(const FwdArgs& a) {
  const bool split = a.num_splits > 0;
  switch ((a.d * 2 + a.causal) * 2 + split) {
#define FA2_CASE(D, C, OCC)                                                  \
  case (D * 2 + C) * 2 + 0: return launch<T, D, (bool)C, false, 4, OCC>(a); \
  case (D * 2 + C) * 2 + 1: return launch<T, D, (bool)C, true, 4, OCC>(a);
    // d = 32 fits 128 VGPRs without splits (four wavefronts per SIMD) and
    // 168 with them (three).
  case (32 * 2 + 0) * 2 + 0: return launch<T, 32, false, false, 4, 4>(a);
  case (32 * 2 + 0) * 2 + 1: return launch<T, 32, false, true, 4, 3>(a);
  case (32 * 2 + 1) * 2 + 0: return launch<T, 32, true, false, 4, 4>(a);
  case (32 * 2 + 1) * 2 + 1: return launch<T, 32, true, true, 4, 3>(a);
    // d = 64 without splits: 153-155 VGPRs, so three wavefronts per SIMD too;
    // the split form needs more and keeps two.
  case (64 * 2 + 0) * 2 + 0: return launch<T, 64, false, false, 4, 3>(a);
  case (64 * 2 + 0) * 2 + 1: return launch<T, 64, false, true, 4, 2>(a);
  case (64 * 2 + 1) * 2 + 0: return launch<T, 64, true, false, 4, 3>(a);
  case (64 * 2 + 1) * 2 + 1: return launch<T, 64, true, true, 4, 2>(a);
    FA2_CASE(96, 0, 2)
    FA2_CASE(96, 1, 2)
#undef FA2_CASE
    // d = 128 without splits: eight wavefronts per workgroup on large grids.
#define FA2_CASE_128(C)                                                         \
  case (128 * 2 + C) * 2 + 0:                                                   \
    return a.block_m == kBlockM_wide ? launch<T, 128, (bool)C, false, 8, 2>(a)  \
                                     : launch<T, 128, (bool)C, false, 4, 2>(a); \
  case (128 * 2 + C) * 2 + 1: return launch<T, 128, (bool)C, true, 4, 2>(a);
    FA2_CASE_128(0)
    FA2_CASE_128(1)
#undef FA2_CASE_128
    // d = 256: two wavefronts per SIMD (256 VGPRs, a few spilled) when the
    // items fill two workgroups on every CU; otherwise, and with splits, one
    // (512 VGPRs, no spill), which is faster for a workgroup alone on its CU.
#define FA2_CASE_256(C)                                                            \
  case (256 * 2 + C) * 2 + 0: {                                                    \
    int cus = 0;                                                                   \
    const hipError_t e = cu_count(&cus);                                           \
    if (e != hipSuccess) return e;                                                 \
    return (int64_t)a.num_m_block * a.BH >= 2 * (int64_t)cus                       \
               ? launch<T, 256, (bool)C, false, 4, 2>(a)                           \
               : launch<T, 256, (bool)C, false, 4, 1>(a);                          \
  }                                                                                \
  case (256 * 2 + C) * 2 + 1: return launch<T, 256, (bool)C, true, 4, 1>(a);
    FA2_CASE_256(0)
    FA2_CASE_256(1)
#undef FA2_CASE_256
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace fa2
