// FlashAttention-2 forward pass, bf16 in / bf16 out, for gfx950 (MI355X).
//
// The algorithm (pages "FlashAttention学习笔记(2)" and "Flash Attention V2原理解读",
// forward sections; "flash-attention123和ring-attention", 优化1-优化4):
//   outer loop: one work item per block of kBlockM = 128 query rows of one
//               (batch, head); items are independent;
//   inner loop: K_j, V_j blocks of BN keys, staged in LDS and shared by the
//               workgroup's four wavefronts;
//   per block:  S = scale * Q_i K_j^T on MFMA, online row max / row sum, the
//               running O rescaled by exp(m_old - m_new) and P~ V_j added on
//               MFMA, no division by l inside the loop;
//   after:      O = O / l once, L = m + ln(l); K/V blocks that the causal mask
//               covers entirely are neither loaded nor computed.
//
// Persistent grid.  The page's grid has one thread block per (query block,
// batch, head).  Here as many workgroups run as fit on the chip at once and
// each walks a fixed sequence of work items: the items of one XCD are the
// query blocks of a contiguous range of heads (which read the same K/V and so
// share that XCD's L2), dealt to its workgroups in a snake order so that heavy
// and light causal blocks balance.  While the last K/V block of an item is
// processed, the next item's Q rows and first K/V blocks are already loading.
//
// Wavefront layout (the pages' split-Q warp scheme, re-derived for 64-wide
// wavefronts and 32x32 MFMA tiles): each wavefront owns 32 query rows against
// the shared K/V block and never exchanges partial results with another.
//
// MFMA orientation.  v_mfma_f32_32x32x16_bf16 produces a 32x32 fp32 tile
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
// address is one per-lane base plus a compile-time offset.  The direct loads,
// and the waits and barriers that order them, are inline assembly, so the
// compiler does not serialise them against the LDS reads in between.
//
// Epilogue.  O and L go straight from registers to global memory through
// buffer stores whose resource covers only the rows < N: rows past the end
// are dropped by the hardware, and every wavefront issues the same number of
// stores, which the next item's first wait counts past.
//
// Overlap.  The MFMAs of block j+1's S = K Q^T are issued in the same basic
// block as block j's softmax (vector ALU: exp2, row max/sum, bf16 packing), so
// the matrix cores and the vector ALUs work concurrently; the PV MFMAs of
// block j follow.
//
// Rescaling.  The running reference max m only moves when a block's row max
// exceeds it by more than kTau (in log2 units); otherwise O and l keep their
// scale and P~ = exp2(c s - c m) stays <= 2^kTau.  O / l and L = m + ln(l) are
// unchanged by the choice of reference, so this is the same online softmax
// with fewer rescales of O.
#include <hip/hip_runtime.h>

#include <atomic>

#include <stdint.h>

#include <type_traits>

#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
static_assert(kBM == kBlockM_bf16, "kBlockM mismatch");

constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units

// Keys per K/V block and wavefronts per SIMD for each head dimension.
template <int D> struct Cfg;
template <> struct Cfg<64> { static constexpr int BN = 64, kWavesPerSimd = 2; };
template <> struct Cfg<128> { static constexpr int BN = 64, kWavesPerSimd = 2; };
template <> struct Cfg<256> { static constexpr int BN = 32, kWavesPerSimd = 1; };
static_assert(Cfg<64>::BN == bf16_block_n(64) && Cfg<128>::BN == bf16_block_n(128) &&
                  Cfg<256>::BN == bf16_block_n(256),
              "host view of the block size");

// LDS layout of a K or V block: key row r lives in 1 KB piece blk(r) at row
// slot slot(r); pieces are kPiece bytes apart.  Rows 0..15 of any aligned group
// fall in 16 different pieces (16 different bank offsets, for the K reads),
// and the 4 rows of an aligned group of 4 fall in pieces 4 apart (64-byte bank
// offsets apart, for the transposing V reads).
constexpr int kPiece = 1024 + 16;
template <int D>
__host__ __device__ constexpr int blk(int r) {
  if constexpr (D == 64) return ((r >> 2) & 3) + 4 * (r & 1);
  else return 4 * (r & 3) + ((r >> 2) & 3);
}
template <int D>
__host__ __device__ constexpr int slot(int r) {
  if constexpr (D == 64) return 2 * (r >> 4) + ((r >> 1) & 1);
  else return r >> 4;
}
template <int D>
__host__ __device__ constexpr int lds_off(int r) { return blk<D>(r) * kPiece + slot<D>(r) * 2 * D; }
// V layout: element (key row r, dim d) at (r/4)*4*2D + (d/16)*128 + 32*(r%4) + 2*(d%16).

template <int D, bool CAUSAL, bool SPLIT>
__global__ void __launch_bounds__(kThreads, Cfg<D>::kWavesPerSimd)
fa2_fwd_bf16_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                    const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                    float* __restrict__ Lg, float* __restrict__ Ow, float* __restrict__ Lw,
                    int N, int BH, int num_m_block, int num_splits, int total_items,
                    float c, float scale_abs, uint32_t qsign, uint32_t qkeep) {
  constexpr int BN = Cfg<D>::BN;
  constexpr int CH = D / 8;                  // 16-byte chunks per key row
  constexpr int KT = BN / 32;                // 32-key sub-blocks per block
  constexpr int KS = D / 16;                 // MFMA k-steps over the head dimension
  constexpr int DT = D / 32;                 // 32-wide tiles of the head dimension
  constexpr int U = BN / 16;                 // 16-key MFMA k-steps of the PV product
  constexpr int ROWB = D * 2;                // bytes per key row
  constexpr int RPP = 1024 / ROWB;           // key rows per 1 KB piece
  constexpr int PIECES = BN / RPP;           // pieces per K or V block
  constexpr int LOADS = PIECES / kWaves;     // direct loads per thread per block
  constexpr int TB = PIECES * kPiece;        // bytes per K block buffer
  constexpr int TBV = BN * ROWB;             // bytes per V block buffer
  constexpr int LOADS_V = TBV / 1024 / kWaves;  // direct V loads per thread per block
  constexpr int NSEG = D / 16;               // 16-dim segments per V row
  constexpr int KTSTEP = lds_off<D>(32) - lds_off<D>(0); // 32 keys further in a K block
  constexpr int NSTORE = DT * 4 + 1;         // O and L stores per wavefront per item
  static_assert(LOADS >= 1 && PIECES % kWaves == 0, "block must split evenly over wavefronts");
  // blk()/slot() place the rows of a K block on exactly 16 pieces (8 for D = 64)
  // of RPP rows each; any other block size would address rows and pieces
  // outside the block and its buffer.
  static_assert(PIECES == (D == 64 ? 8 : 16) && BN == PIECES * RPP,
                "K LDS layout is defined for BN = 64 (D = 64, 128) and BN = 32 (D = 256) only");
  static_assert(lds_off<D>(BN - 1) + ROWB <= TB, "K rows stay inside their buffer");
  static_assert(LOADS_V >= 1 && TBV % (1024 * kWaves) == 0, "V block must split evenly");
  static_assert(TBV + 16 * ROWB * (U - 1) + 8 * ROWB + 256 * (DT - 1) < 65536 &&
                    2 * TBV + TB + KTSTEP * (KT - 1) + 32 * (KS - 1) < 65536,
                "LDS offsets fit the 16-bit instruction offset");

  __shared__ __attribute__((aligned(1024))) char smem[2 * TBV + 2 * TB];  // V0 V1 K0 K1
  char* const Vb0 = smem;
  char* const Kb0 = smem + 2 * TBV;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
  const int col = lane & 31;  // this lane's query row within the wavefront's 32
  const int half = lane >> 5;

  // ---- work schedule.  The grid is persistent: each workgroup processes a
  // sequence of work items (query block, batch*head).  Workgroup ids reach the
  // 8 XCDs round-robin; XCD x takes a contiguous range of logical items (the
  // query blocks of the same few heads, which read the same K/V and so share
  // that XCD's L2), ordered head by head with a head's heaviest causal query
  // block first.  The workgroups of an XCD walk that range in groups, in a
  // snake order (group k: slot s takes position s, or P-1-s when k is odd), so
  // that heavy and light causal blocks alternate per workgroup.
  // (With fewer than 8 workgroups the ranges are split over that many.)
  const int nx = gridDim.x < 8 ? (int)gridDim.x : 8;
  const int xcd = blockIdx.x % nx;
  const int lslot = blockIdx.x / nx;
  const int P = ((int)gridDim.x - xcd + nx - 1) / nx;  // workgroups on this XCD
  const int per = total_items / nx, rem = total_items % nx;
  const int x_base = xcd * per + (xcd < rem ? xcd : rem);
  const int x_items = per + (xcd < rem ? 1 : 0);
  auto logical_of = [&](int k) -> int {  // the k-th item of this workgroup, or -1
    const int pos = k * P + ((k & 1) ? P - 1 - lslot : lslot);
    return pos < x_items ? x_base + pos : -1;
  };

  // ---- per-item state
  int bh = 0, m = 0, q0 = 0, qrow = 0, j_beg = 0, j_end = 0, j_mask = 0;
  int g0 = 0;      // running block count of this workgroup at the current item's first block
  int k_item = 0;  // index of the current item in this workgroup's sequence
  const uint16_t *Qh = Qg, *Kh = Kg, *Vh = Vg;
  // O and L of the item's query block as buffer resources whose size covers
  // only the rows < N: the hardware drops stores to rows past the end, so
  // every wavefront issues the same number of stores for every item.
  __amdgpu_buffer_rsrc_t o_rsrc, l_rsrc;
  int gb = 0;  // buffer parity base: block j uses K and V buffers (gb + j) & 1
  // logical item -> (batch*head, query block, split): splits fastest, then the
  // query blocks of a head (heaviest causal block first), then the heads.
  auto decode = [&](int logical, int& bh_, int& m_, int& s_) __attribute__((always_inline)) {
    int mi = logical;
    s_ = 0;
    if constexpr (SPLIT) {
      mi = logical / num_splits;
      s_ = logical - mi * num_splits;
    }
    bh_ = mi / num_m_block;
    mi -= bh_ * num_m_block;
    m_ = CAUSAL ? num_m_block - 1 - mi : mi;
  };
  auto blocks_of = [&](int m_) __attribute__((always_inline)) -> int {
    if (CAUSAL) return (min(N, (m_ + 1) * kBM) - 1) / BN + 1;
    return (N + BN - 1) / BN;
  };
  // KV blocks [beg, end) of split s of query block m: ceil(blocks / num_splits)
  // blocks per split, so split 0 is never empty (and holds key 0, which every
  // row sees); later splits can be.
  auto range_of = [&](int m_, int s_, int& beg, int& end) __attribute__((always_inline)) {
    const int jt = blocks_of(m_);
    if constexpr (SPLIT) {
      const int per = (jt + num_splits - 1) / num_splits;
      beg = min(s_ * per, jt);
      end = min(beg + per, jt);
    } else {
      beg = 0;
      end = jt;
    }
  };
  auto set_item = [&](int logical) __attribute__((always_inline)) {
    int sp;
    decode(logical, bh, m, sp);
    range_of(m, sp, j_beg, j_end);
    const size_t slice = (size_t)bh * (size_t)N * D;
    Qh = Qg + slice;
    Kh = Kg + slice;
    Vh = Vg + slice;
    const int rows = min(kBM, N - m * kBM);
    if constexpr (SPLIT) {
      const size_t prow = ((size_t)sp * BH + bh) * N + (size_t)m * kBM;  // first partial row
      o_rsrc = __builtin_amdgcn_make_buffer_rsrc(Ow + prow * D, (short)0, rows * D * 4,
                                                 kBufferFlags);
      l_rsrc = __builtin_amdgcn_make_buffer_rsrc(Lw + prow, (short)0, rows * 4, kBufferFlags);
    } else {
      o_rsrc = __builtin_amdgcn_make_buffer_rsrc(Og + slice + (size_t)m * kBM * D, (short)0,
                                                 rows * ROWB, kBufferFlags);
      l_rsrc = __builtin_amdgcn_make_buffer_rsrc(Lg + (size_t)bh * N + (size_t)m * kBM, (short)0,
                                                 rows * 4, kBufferFlags);
    }
    q0 = m * kBM + wave * 32;  // first query row of this wavefront
    qrow = q0 + col;
    gb = g0 - j_beg;
    // Blocks before j_mask need no mask for this wavefront (every key visible
    // to every one of its rows).
    j_mask = CAUSAL ? min((q0 + 1) / BN, N / BN) : N / BN;
  };

  // Q fragments (the B operand of S^T = K Q^T), kept in registers for an item.
  // A negative scale flips Q's sign (exact); a zero scale zeroes Q, which gives
  // the same all-zero logits.
  bf16x8_t qf[KS];
  auto load_q = [&](const uint16_t* qh, int row) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t t = {0u, 0u, 0u, 0u};
      if (row < N) t = *(const u32x4_t*)(qh + (size_t)row * D + ks * 16 + 8 * half);
      qf[ks] = __builtin_bit_cast(bf16x8_t, t);
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
      qf[ks] = __builtin_bit_cast(bf16x8_t, t);
    }
  };

  // ---- global -> LDS staging.  K: load i of this thread fills piece
  // b = wave*LOADS + i, whose lane L writes bytes 16L.. of the piece: row slot
  // L / CH, 16-byte chunk L % CH of the key row r with blk(r) = b and
  // slot(r) = L / CH.  That row splits into a per-lane part and a per-piece
  // (wave-uniform) part 4*(b&3) + (b>>2).
  auto k_lane_row = [](int l) { const int sl = l / CH; return D == 64 ? 16 * (sl >> 1) + 2 * (sl & 1) : 16 * sl; };
  auto k_lane_col = [](int l) { return (l % CH) * 8; };
  const uint32_t lane_bytes = (uint32_t)(k_lane_row(lane) * D + k_lane_col(lane)) * 2;
  // k0 goes through an empty asm statement: for the constant first blocks of an
  // item the compiler would otherwise precompute the clamped tail addresses
  // once, outside the item loop, and keep them in (spilled) registers.
  auto issue_k = [&](const uint16_t* head, int k0, char* buf) __attribute__((always_inline)) {
    asm volatile("" : "+s"(k0));
    if (k0 + BN <= N) {
      // Scalar base (the piece's first row) plus a constant 32-bit per-lane offset.
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int b = wave * LOADS + i;
        lds_dma(head + (size_t)(k0 + 4 * (b & 3) + (b >> 2)) * D, lane_bytes,
                lds_addr(buf + b * kPiece));
      }
    } else {
      // Ragged last block: rows past N are clamped to row N-1 (their keys are masked).
      const int tl = fresh_lane();
      const int lane_row = k_lane_row(tl), lane_col = k_lane_col(tl);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int b = wave * LOADS + i;
        const int r = min(k0 + 4 * (b & 3) + (b >> 2) + lane_row, N - 1);
        lds_dma(head + (size_t)r * D + lane_col, lds_addr(buf + b * kPiece));
      }
    }
  };
  // V: load i of this thread fills 1 KB chunk n = wave*LOADS_V + i, whose lane
  // L writes 16 bytes: 128-byte block bk = 8n + L/8 (row group bk / NSEG, dim
  // segment bk % NSEG), row (L%8)/2 of that group, dims 8*(L%2) ..+8 of that
  // segment.  The lane's share of the key row and dims is the same for every
  // n; n only adds a wave-uniform row / dim offset.
  auto v_lane_row = [](int l) { return NSEG <= 8 ? 4 * ((l / 8) / NSEG) + (l % 8) / 2 : (l % 8) / 2; };
  auto v_lane_dim = [](int l) {
    return NSEG <= 8 ? 16 * ((l / 8) % NSEG) + 8 * (l % 2) : 16 * (l / 8) + 8 * (l % 2);
  };
  const uint32_t vlane = (uint32_t)(v_lane_row(lane) * D + v_lane_dim(lane)) * 2;
  auto issue_v = [&](const uint16_t* head, int k0, char* buf) __attribute__((always_inline)) {
    asm volatile("" : "+s"(k0));
    const char* base = (const char*)(head + (size_t)k0 * D);
    if (k0 + BN <= N) {
#pragma unroll
      for (int i = 0; i < LOADS_V; ++i) {
        const int n = wave * LOADS_V + i;
        const int row_u = NSEG <= 8 ? 4 * n * (8 / NSEG) : 4 * (n / 2);
        const int dim_u = NSEG <= 8 ? 0 : 128 * (n % 2);
        lds_dma(base + (row_u * D + dim_u) * 2, vlane, lds_addr(buf + n * 1024));
      }
    } else {
      // Ragged last block: rows past N are clamped to row N-1 (P~ is 0 there).
      const int tl = fresh_lane();
      const int vrow_l = v_lane_row(tl), vdim_l = v_lane_dim(tl);
#pragma unroll
      for (int i = 0; i < LOADS_V; ++i) {
        const int n = wave * LOADS_V + i;
        const int row_u = NSEG <= 8 ? 4 * n * (8 / NSEG) : 4 * (n / 2);
        const int dim_u = NSEG <= 8 ? 0 : 128 * (n % 2);
        const int r = min(k0 + row_u + vrow_l, N - 1);
        lds_dma(head + (size_t)r * D + dim_u + vdim_l, lds_addr(buf + n * 1024));
      }
    }
  };
  // The first blocks of an item (blocks beg, beg+1, ... of its range): Q rows,
  // K_beg and V_beg, and K_beg+1 if the range has it.  g is the running block
  // count of this workgroup: block g of the sequence uses buffers g & 1.
  auto issue_item_start = [&](const uint16_t* qh, const uint16_t* kh, const uint16_t* vh, int row,
                              int beg, int blocks, int g) __attribute__((always_inline)) {
    load_q(qh, row);
    issue_k(kh, beg * BN, Kb0 + (g & 1) * TB);
    issue_v(vh, beg * BN, Vb0 + (g & 1) * TBV);
    if (blocks > 1) issue_k(kh, (beg + 1) * BN, Kb0 + ((g + 1) & 1) * TB);
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
  const uint32_t vaddr =
      (uint32_t)(((lane >> 4) >> 1) * 4 * ROWB + ((lane >> 4) & 1) * 128 + 8 * (lane & 15));

  f32x16_t o[DT];
  float m_ref = kNegInf;  // reference max of the (sign-adjusted) raw logits
  float l_part = 0.f;     // running sum over this lane's half of the keys

  auto compute_S = [&](const char* kb, f32x16_t (&S)[KT]) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      S[kt] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a = *(const bf16x8_t*)(kb + kaddr + kt * KTSTEP + ks * 32);
        S[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], S[kt], 0, 0, 0);
      }
    }
  };

  // Block j's step of the online softmax (new running max, rescaled running
  // sum, unnormalised probabilities) and the rescaled O update;
  // `during` issues independent MFMA work (the next block's S) alongside.
  auto consume = [&](auto masked_tag, int j, f32x16_t(&S)[KT],
                     auto&& during) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = j * BN;
    if constexpr (MASKED) {
      // key = k0 + cr + 4*half with cr = kt*32 + 8*(r/4) + r%4 (a constant):
      // it is hidden when cr + (k0 - q0) > col - 4*half (after the lane's query
      // row) or cr + (k0 - N) >= -4*half (past the sequence), i.e. when cr
      // exceeds one per-lane threshold.
      const int ml = fresh_lane();
      const int mh = -4 * (ml >> 5);
      int th = mh - (k0 - N) - 1;
      if (CAUSAL) th = min(th, (ml & 31) + mh - (k0 - q0));
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = kt * 32 + 8 * (r / 4) + (r % 4);
          S[kt][r] = cr > th ? kNegInf : S[kt][r];
        }
    }
    during();
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kt][r]);
    mx = halves_max(mx);
    // The first block with a visible key always moves the reference (alpha =
    // exp2(-inf) = 0 then: O and l are still zero).  A split's range can hold
    // no key a row sees (mx = -inf): the reference then stays at -inf and the
    // block adds nothing, without forming exp2(-inf + inf).
    bool move;
    if constexpr (SPLIT) move = m_ref == kNegInf ? mx != kNegInf : c * (mx - m_ref) > kTau;
    else move = m_ref == kNegInf || c * (mx - m_ref) > kTau;
    const float alpha = move ? __builtin_amdgcn_exp2f(c * (m_ref - mx)) : 1.f;
    m_ref = move ? mx : m_ref;
    const float mc = m_ref == kNegInf ? 0.f : c * m_ref;
    float ls = 0.f;
    bf16x8_t pb[U];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kt][r], c, -mc));
        ls += p;
        pb[kt * 2 + r / 8][r % 8] = (__bf16)p;
      }
    l_part = alpha * l_part + ls;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] *= alpha;
    }
    const char* vb = Vb0 + ((gb + j) & 1) * TBV + vaddr;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr_t)(vb + u * 16 * ROWB + t * 256));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr_t)(vb + 8 * ROWB + u * 16 * ROWB + t * 256));
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[u], o[t], 0, 0, 0);
      }
  };

  // One barrier per block: block j's V and block j+1's K have landed in LDS,
  // and every wavefront is done with the buffers of block j-1, which the loads
  // for blocks j+2 (K) and j+1 (V) issued right after reuse.
  auto advance = [&](int j) __attribute__((always_inline)) {
    // At an item's first block the previous item's O and L stores, issued
    // last, need not have completed.
    if (j == j_beg && k_item > 0) wait_vmcnt<NSTORE>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (j + 2 < j_end) issue_k(Kh, (j + 2) * BN, Kb0 + ((gb + j) & 1) * TB);
    if (j + 1 < j_end) issue_v(Vh, (j + 1) * BN, Vb0 + ((gb + j + 1) & 1) * TBV);
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
    fix_q();
    const bool two = j_end - j_beg > 1;
    if constexpr (decltype(later_tag)::value) {
      if (two) wait_vmcnt<LOADS_V + LOADS + NSTORE>();
      else wait_vmcnt<LOADS_V + NSTORE>();
    } else {
      if (two) wait_vmcnt<LOADS_V + LOADS>();
      else wait_vmcnt<LOADS_V>();
    }
    lds_barrier();
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = f32x16_t{};
    m_ref = kNegInf;
    l_part = 0.f;
    compute_S(Kb0 + (g0 & 1) * TB, S_cur);
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
  // The next item's Q and first K/V blocks; issued while this item's last
  // block is processed (or at once, for an empty item).
  auto prefetch_next = [&]() __attribute__((always_inline)) {
    if (next >= 0 && nend > nbeg) {
      const size_t nslice = (size_t)nbh * (size_t)N * D;
      issue_item_start(Qg + nslice, Kg + nslice, Vg + nslice, nm * kBM + wave * 32 + col, nbeg,
                       nend - nbeg, g0 + (j_end - j_beg));
    }
  };
  // ---- item epilogue, after the KV loop: O = O / l once, L = m + ln(l).
  // (A split row that saw no key has l = 0: O_s = 0 and L_s = -inf.)
  auto store_result = [&]() __attribute__((always_inline)) {
    const float l_tot = halves_sum(l_part);
    float inv = 1.f / l_tot;
    if constexpr (SPLIT) inv = l_tot > 0.f ? inv : 0.f;
    const int lrow = wave * 32 + col;  // this lane's row in the query block
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = t * 32 + 8 * g + 4 * half;
        if constexpr (SPLIT) {
          f32x4_t w;
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = o[t][g * 4 + r] * inv;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, w), o_rsrc,
                                                 (lrow * D + dim) * 4, 0, 0);
        } else {
          bf16x4_t w;
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = (__bf16)(o[t][g * 4 + r] * inv);
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, w), o_rsrc,
                                                lrow * ROWB + dim * 2, 0, 0);
        }
      }
    // Both halves of a row hold the same l and m: they store the same L.
    __builtin_amdgcn_raw_buffer_store_b32(
        __builtin_bit_cast(uint32_t,
                           __builtin_fmaf(__builtin_amdgcn_logf(l_tot), kLn2, scale_abs * m_ref)),
        l_rsrc, lrow * 4, 0, 0);
  };
  // Split items whose key range is empty are finished here (O_s = 0,
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
  set_item(logical);
  if (!finish_empty_items()) return;
  if (k_item == 0) {
    issue_item_start(Qh, Kh, Vh, qrow, j_beg, j_end - j_beg, g0);
    prologue(std::false_type{});
  } else {
    prologue(std::true_type{});  // prefetched by the last empty item, stores after it
  }

  for (;;) {
    look_ahead();
    const int j_unmasked = min(j_mask, j_end - 1);  // unmasked blocks that have a successor
    f32x16_t SB[KT];
    int j = j_beg;
    // Unrolled by two so that the S registers alternate between S_cur and SB
    // instead of being copied every block.
    for (; j + 2 <= j_unmasked; j += 2) {
      advance(j);
      consume(std::false_type{}, j, S_cur,
              [&]() { compute_S(Kb0 + ((gb + j + 1) & 1) * TB, SB); });
      advance(j + 1);
      consume(std::false_type{}, j + 1, SB,
              [&]() { compute_S(Kb0 + ((gb + j) & 1) * TB, S_cur); });
    }
    if (j < j_unmasked) {
      advance(j);
      consume(std::false_type{}, j, S_cur,
              [&]() { compute_S(Kb0 + ((gb + j + 1) & 1) * TB, SB); });
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) S_cur[kt] = SB[kt];
      ++j;
    }
    for (; j + 2 < j_end; j += 2) {
      advance(j);
      consume(std::true_type{}, j, S_cur,
              [&]() { compute_S(Kb0 + ((gb + j + 1) & 1) * TB, SB); });
      advance(j + 1);
      consume(std::true_type{}, j + 1, SB,
              [&]() { compute_S(Kb0 + ((gb + j) & 1) * TB, S_cur); });
    }
    if (j + 1 < j_end) {
      advance(j);
      consume(std::true_type{}, j, S_cur,
              [&]() { compute_S(Kb0 + ((gb + j + 1) & 1) * TB, SB); });
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) S_cur[kt] = SB[kt];
      ++j;
    }
    // Last block of the item.  Both K buffers and the other V buffer are free
    // now, and so are the Q registers: the next item's Q, K_beg, V_beg,
    // K_beg+1 go out here and overlap this block's softmax, its PV product and
    // the O stores.
    advance(j);
    prefetch_next();
    // Always the masked form: one copy of the code, and for an unmasked block
    // the threshold test hides nothing.
    consume(std::true_type{}, j, S_cur, [] {});
    store_result();
    if (next < 0) break;
    g0 += j_end - j_beg;
    ++k_item;
    set_item(next);
    if (!finish_empty_items()) break;
    prologue(std::true_type{});
  }
}

// Compute units of the current device, queried once per device.
hipError_t cu_count(int* cus) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && (*cus = cache[dev].load(std::memory_order_relaxed)) > 0)
    return hipSuccess;
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (*cus < 1) *cus = 1;
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(*cus, std::memory_order_relaxed);
  return hipSuccess;
}

template <int D, bool CAUSAL, bool SPLIT>
hipError_t launch(const FwdArgs& a) {
  const int splits = SPLIT ? a.num_splits : 1;
  const int total = a.num_m_block * a.BH * splits;
  // Persistent grid: as many workgroups as fit on the chip at once (a 4-wave
  // workgroup puts one wave on each SIMD of a CU, so kWavesPerSimd workgroups
  // per CU), each walking its share of the work items.
  int cus = 0;
  const hipError_t e = cu_count(&cus);
  if (e != hipSuccess) return e;
  const int resident = Cfg<D>::kWavesPerSimd * cus;
  const int grid = total < resident ? total : resident;
  // The kernel works with c = |scale| * log2(e) > 0: a negative scale flips the
  // sign of Q and a zero scale zeroes Q (both exact), with |scale| = 1 then.
  const bool zero = a.scale == 0.f;
  const float sa = zero ? 1.f : (a.scale < 0.f ? -a.scale : a.scale);
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  const uint32_t qkeep = zero ? 0u : 0xFFFFFFFFu;
  hipLaunchKernelGGL((fa2_fwd_bf16_kernel<D, CAUSAL, SPLIT>), dim3(grid), dim3(kThreads), 0,
                     a.stream, (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (uint16_t*)a.O, a.L, a.ws_O, a.ws_L, a.N, a.BH, a.num_m_block, splits, total,
                     sa * kLog2e, sa, qsign, qkeep);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  const bool split = a.num_splits > 0;
  switch ((a.d * 2 + a.causal) * 2 + split) {
#define FA2_CASE(D, C)                                                  \
  case (D * 2 + C) * 2 + 0: return launch<D, (bool)C, false>(a);       \
  case (D * 2 + C) * 2 + 1: return launch<D, (bool)C, true>(a);
    FA2_CASE(64, 0)
    FA2_CASE(64, 1)
    FA2_CASE(128, 0)
    FA2_CASE(128, 1)
    FA2_CASE(256, 0)
    FA2_CASE(256, 1)
#undef FA2_CASE
  }
  return hipErrorInvalidValue;
}

hipError_t bf16_resident_workgroups(int d, int* slots) {
  int cus = 0;
  const hipError_t e = cu_count(&cus);
  if (e != hipSuccess) return e;
  *slots = (d == 256 ? Cfg<256>::kWavesPerSimd : Cfg<128>::kWavesPerSimd) * cus;
  return hipSuccess;
}

}  // namespace fa2
