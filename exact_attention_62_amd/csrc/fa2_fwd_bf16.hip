// FlashAttention-2 forward pass, bf16 in / bf16 out, for gfx950 (MI355X).
//
// The algorithm (pages "FlashAttention学习笔记(2)" and "Flash Attention V2原理解读",
// forward sections; "flash-attention123和ring-attention", 优化1-优化4):
//   outer loop: one workgroup per block of kBlockM = 128 query rows, grid over
//               (query block, batch, head);
//   inner loop: K_j, V_j blocks of BN keys, staged in LDS and shared by the
//               workgroup's four wavefronts;
//   per block:  S = scale * Q_i K_j^T on MFMA, online row max / row sum, the
//               running O rescaled by exp(m_old - m_new) and P~ V_j added on
//               MFMA, no division by l inside the loop;
//   after:      O = O / l once, L = m + ln(l); K/V blocks that the causal mask
//               covers entirely are neither loaded nor computed.
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
// address is one per-lane base plus a compile-time offset.
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

#include <stdint.h>

#include <type_traits>

#include "fa2_internal.h"

namespace fa2 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr_t;
typedef __attribute__((address_space(1))) const void* global_ptr_t;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
static_assert(kBM == kBlockM_bf16, "kBlockM mismatch");

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units

// Keys per K/V block and wavefronts per SIMD for each head dimension.
template <int D> struct Cfg;
template <> struct Cfg<64> { static constexpr int BN = 64, kWavesPerSimd = 2; };
template <> struct Cfg<128> { static constexpr int BN = 64, kWavesPerSimd = 2; };
template <> struct Cfg<256> { static constexpr int BN = 32, kWavesPerSimd = 1; };

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

// Value of x combined with the one held 32 lanes away (the two lane halves of
// a 32x32 MFMA tile hold different keys of the same query row).
__device__ __forceinline__ float halves_max(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }
__device__ __forceinline__ float halves_sum(float x) { return x + __shfl_xor(x, 32, 64); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, Cfg<D>::kWavesPerSimd)
fa2_fwd_bf16_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                    const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                    float* __restrict__ Lg, int N, int num_m_block, int total_blocks,
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

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
  const int col = lane & 31;  // this lane's query row within the wavefront's 32
  const int half = lane >> 5;

  // Workgroup -> (query block, batch*head).  Consecutive workgroup ids are
  // dispatched round-robin over the 8 XCDs; remap so that each XCD receives a
  // contiguous range of logical blocks, i.e. the query blocks of the same few
  // heads, which read the same K/V and so share that XCD's L2.  With the causal
  // mask, a head's heaviest (last) query block is issued first.
  int logical;
  {
    const int p = blockIdx.x;
    const int per = total_blocks / 8, rem = total_blocks % 8;
    const int x = p % 8, s = p / 8;
    logical = x * per + (x < rem ? x : rem) + s;
  }
  const int bh = logical / num_m_block;
  const int mi = logical - bh * num_m_block;
  const int m = CAUSAL ? num_m_block - 1 - mi : mi;

  const size_t slice = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Qg + slice;
  const uint16_t* Kh = Kg + slice;
  const uint16_t* Vh = Vg + slice;
  uint16_t* Oh = Og + slice;
  float* Lh = Lg + (size_t)bh * N;

  const int q0 = m * kBM + wave * 32;  // first query row of this wavefront
  const int qrow = q0 + col;

  // Q fragments (the B operand of S^T = K Q^T), kept in registers for the whole
  // loop.  A negative scale flips Q's sign (exact); a zero scale zeroes Q, which
  // gives the same all-zero logits.
  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4_t t = {0u, 0u, 0u, 0u};
    if (qrow < N) t = *(const u32x4_t*)(Qh + (size_t)qrow * D + ks * 16 + 8 * half);
    t = (t & qkeep) ^ qsign;
    qf[ks] = __builtin_bit_cast(bf16x8_t, t);
  }

  // ---- global -> LDS staging map: load i of this thread fills piece
  // b = wave*LOADS + i, whose lane L writes bytes 16L.. of the piece: row slot
  // L / CH, 16-byte chunk L % CH of the key row r with blk(r) = b and
  // slot(r) = L / CH.  That row splits into a per-lane part and a per-piece
  // (wave-uniform) part 4*(b&3) + (b>>2).
  int lane_row, lane_col;
  {
    const int sl = lane / CH;
    lane_row = D == 64 ? 16 * (sl >> 1) + 2 * (sl & 1) : 16 * sl;
    lane_col = (lane % CH) * 8;
  }
  const uint32_t lane_bytes = (uint32_t)(lane_row * D + lane_col) * 2;
  auto issue_block = [&](const uint16_t* head, int k0, char* buf) {
    if (k0 + BN <= N) {
      // Scalar base (the piece's first row) plus a constant 32-bit per-lane offset.
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int b = wave * LOADS + i;
        const char* base = (const char*)(head + (size_t)(k0 + 4 * (b & 3) + (b >> 2)) * D);
        __builtin_amdgcn_global_load_lds((global_ptr_t)(base + lane_bytes),
                                         (lds_ptr_t)(buf + b * kPiece), 16, 0, 0);
      }
    } else {
      // Ragged last block: rows past N are clamped to row N-1 (their keys are masked).
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int b = wave * LOADS + i;
        const int r = min(k0 + 4 * (b & 3) + (b >> 2) + lane_row, N - 1);
        __builtin_amdgcn_global_load_lds((global_ptr_t)(head + (size_t)r * D + lane_col),
                                         (lds_ptr_t)(buf + b * kPiece), 16, 0, 0);
      }
    }
  };

  // V staging: load i of this thread fills 1 KB chunk n = wave*LOADS_V + i,
  // whose lane L writes 16 bytes: 128-byte block bk = 8n + L/8 (row group
  // bk / NSEG, dim segment bk % NSEG), row (L%8)/2 of that group, dims
  // 8*(L%2) ..+8 of that segment.  The lane's share of the key row and dims is
  // the same for every n; n only adds a wave-uniform row / dim offset.
  int vrow_l, vdim_l;
  {
    const int x = lane / 8;
    if constexpr (NSEG <= 8) {
      vrow_l = 4 * (x / NSEG) + (lane % 8) / 2;
      vdim_l = 16 * (x % NSEG) + 8 * (lane % 2);
    } else {
      vrow_l = (lane % 8) / 2;
      vdim_l = 16 * x + 8 * (lane % 2);
    }
  }
  const uint32_t vlane = (uint32_t)(vrow_l * D + vdim_l) * 2;
  auto issue_v = [&](int k0, char* buf) __attribute__((always_inline)) {
    const char* base = (const char*)(Vh + (size_t)k0 * D);
    const bool tail = k0 + BN > N;  // rows past N are clamped to row N-1 (P~ is 0 there)
#pragma unroll
    for (int i = 0; i < LOADS_V; ++i) {
      const int n = wave * LOADS_V + i;
      const int row_u = NSEG <= 8 ? 4 * n * (8 / NSEG) : 4 * (n / 2);
      const int dim_u = NSEG <= 8 ? 0 : 128 * (n % 2);
      const char* src = base + (row_u * D + dim_u) * 2 + vlane;
      if (tail) src += (ptrdiff_t)(min(k0 + row_u + vrow_l, N - 1) - (k0 + row_u + vrow_l)) * ROWB;
      __builtin_amdgcn_global_load_lds((global_ptr_t)src, (lds_ptr_t)(buf + n * 1024), 16, 0, 0);
    }
  };

  // ---- LDS fragment addresses (bytes within a block buffer).
  // K (A operand of S^T): key row kt*32 + col, dims 16*ks + 8*half ..+8.
  const uint32_t kaddr = lds_off<D>(col) + 16 * half;
  // V^T (A operand of O^T += V^T P^T) through ds_read_b64_tr_b16: within each
  // group of 16 lanes, lane 4*r + c supplies the address of 4 consecutive dims
  // (d0 + 4c ..) of key row (kbase + r); the hardware hands lane t of the
  // group the 4 keys kbase..kbase+3 of dim d0 + t.  kbase = 16u + 4*half (the
  // first 4 slots of the operand) or 16u + 8 + 4*half (the last 4), matching
  // the keys 8*(r/4) + 4*half + r%4 that a lane's S^T accumulators hold.
  // With the V layout, the 16 lanes of a group read one contiguous 128-byte
  // block: lane i at byte 8i of the block of rows kbase.. and dims d0..d0+15.
  const uint32_t vaddr = (uint32_t)(((lane >> 4) >> 1) * 4 * ROWB + ((lane >> 4) & 1) * 128 + 8 * (lane & 15));

  f32x16_t o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16_t{};
  float m_ref = kNegInf;  // reference max of the (sign-adjusted) raw logits
  float l_part = 0.f;     // running sum over this lane's half of the keys

  const int n_blocks = (N + BN - 1) / BN;
  int j_end = n_blocks;
  if (CAUSAL) {
    const int last = min(N, (m + 1) * kBM) - 1;
    j_end = last / BN + 1;
  }

  char* const Vb0 = smem;
  char* const Kb0 = smem + 2 * TBV;

  auto compute_S = [&](const char* kb, f32x16_t (&S)[KT]) {
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

  // Softmax of block j (pseudo-code line 9) and the O update (line 10);
  // `during` issues independent MFMA work (the next block's S) alongside.
  auto consume = [&](auto masked_tag, int j, f32x16_t(&S)[KT], auto&& during) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int k0 = j * BN;
    if constexpr (MASKED) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kt * 32 + 8 * (r / 4) + 4 * half + (r % 4);
          const bool hide = (CAUSAL && key > qrow) || key >= N;
          S[kt][r] = hide ? kNegInf : S[kt][r];
        }
    }
    during();
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kt][r]);
    mx = halves_max(mx);
    float alpha = 1.f;
    if (m_ref == kNegInf) {  // first block with a visible key: O and l are still zero
      m_ref = mx;
      alpha = 0.f;
    } else if (c * (mx - m_ref) > kTau) {
      alpha = __builtin_amdgcn_exp2f(c * (m_ref - mx));
      m_ref = mx;
    }
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
    const char* vb = Vb0 + (j & 1) * TBV + vaddr;
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

  // ---- prologue: K0, V0 and K1 in flight; S for block 0.
  issue_block(Kh, 0, Kb0);
  issue_v(0, Vb0);
  if (j_end > 1) {
    issue_block(Kh, BN, Kb0 + TB);
    wait_vmcnt<LOADS_V + LOADS>();
  } else {
    wait_vmcnt<LOADS_V>();
  }
  __syncthreads();
  f32x16_t S_cur[KT];
  compute_S(Kb0, S_cur);

  // One barrier per block: block j's V and block j+1's K have landed in LDS,
  // and every wavefront is done with the buffers of block j-1, which the loads
  // for blocks j+2 (K) and j+1 (V) issued right after reuse.
  auto advance = [&](int j) {
    wait_vmcnt<0>();
    __syncthreads();
    if (j + 2 < j_end) issue_block(Kh, (j + 2) * BN, Kb0 + (j & 1) * TB);
    if (j + 1 < j_end) issue_v((j + 1) * BN, Vb0 + ((j + 1) & 1) * TBV);
  };
  // Blocks before j_mask need no mask for this wavefront (all keys visible to
  // all of its rows); the loop runs in three stretches so that each loop body
  // holds a single variant: unmasked, masked (causal diagonal, ragged tail),
  // and the last block, which has no successor to overlap with.
  const int j_mask = CAUSAL ? min((q0 + 1) / BN, N / BN) : N / BN;
  const int j_unmasked = min(j_mask, j_end - 1);  // unmasked blocks that have a successor
  f32x16_t SB[KT];
  int j = 0;
  // Unrolled by two so that the S registers alternate between S_cur and SB
  // instead of being copied every block.
  for (; j + 2 <= j_unmasked; j += 2) {
    advance(j);
    consume(std::false_type{}, j, S_cur, [&]() { compute_S(Kb0 + ((j + 1) & 1) * TB, SB); });
    advance(j + 1);
    consume(std::false_type{}, j + 1, SB, [&]() { compute_S(Kb0 + (j & 1) * TB, S_cur); });
  }
  if (j < j_unmasked) {
    advance(j);
    consume(std::false_type{}, j, S_cur, [&]() { compute_S(Kb0 + ((j + 1) & 1) * TB, SB); });
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) S_cur[kt] = SB[kt];
    ++j;
  }
  for (; j + 2 < j_end; j += 2) {
    advance(j);
    consume(std::true_type{}, j, S_cur, [&]() { compute_S(Kb0 + ((j + 1) & 1) * TB, SB); });
    advance(j + 1);
    consume(std::true_type{}, j + 1, SB, [&]() { compute_S(Kb0 + (j & 1) * TB, S_cur); });
  }
  if (j + 1 < j_end) {
    advance(j);
    consume(std::true_type{}, j, S_cur, [&]() { compute_S(Kb0 + ((j + 1) & 1) * TB, SB); });
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) S_cur[kt] = SB[kt];
    ++j;
  }
  advance(j);
  if (j < j_mask) consume(std::false_type{}, j, S_cur, [] {});
  else consume(std::true_type{}, j, S_cur, [] {});

  // ---- epilogue (lines 12-13): O = O / l once, L = m + ln(l).
  // The wavefront's 32 output rows are one contiguous stretch of O.  They go
  // through LDS (16-byte chunks XOR-swizzled by row against bank conflicts) so
  // that the global stores are whole rows, 16 bytes per lane.  The K buffers
  // are free once the last barrier has passed (the last block reads only V);
  // with D = 256 the staging needs all of LDS and waits for the last V reads.
  const float l_tot = halves_sum(l_part);
  const float inv = 1.f / l_tot;
  constexpr int CHK = D / 8;                    // 16-byte chunks per output row
  constexpr int SWZ = CHK < 16 ? CHK - 1 : 15;  // swizzle mask
  constexpr int STAGE = 32 * ROWB;              // bytes per wavefront
  constexpr bool IN_K = kWaves * STAGE <= 2 * TB;
  static_assert(kWaves * STAGE <= 2 * TBV + 2 * TB, "staging fits in LDS");
  if constexpr (!IN_K) __syncthreads();
  char* const stage = (IN_K ? Kb0 : smem) + wave * STAGE;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4_t w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = (__bf16)(o[t][g * 4 + r] * inv);
      const int d = t * 32 + 8 * g + 4 * half;
      *(bf16x4_t*)(stage + col * ROWB + (((d >> 3) ^ (col & SWZ)) << 4) + (d & 7) * 2) = w;
    }
  __builtin_amdgcn_s_waitcnt((15 << 0) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  constexpr int RPI = 64 / CHK;  // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = i * RPI + lane / CHK;
    const int ch = lane % CHK;
    const u32x4_t v = *(const u32x4_t*)(stage + row * ROWB + ((ch ^ (row & SWZ)) << 4));
    if (q0 + row < N) *(u32x4_t*)(Oh + (size_t)(q0 + row) * D + ch * 8) = v;
  }
  if (qrow < N && half == 0)
    Lh[qrow] = __builtin_fmaf(__builtin_amdgcn_logf(l_tot), kLn2, scale_abs * m_ref);
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  const int total = a.num_m_block * a.BH;
  // The kernel works with c = |scale| * log2(e) > 0: a negative scale flips the
  // sign of Q and a zero scale zeroes Q (both exact), with |scale| = 1 then.
  const bool zero = a.scale == 0.f;
  const float sa = zero ? 1.f : (a.scale < 0.f ? -a.scale : a.scale);
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  const uint32_t qkeep = zero ? 0u : 0xFFFFFFFFu;
  hipLaunchKernelGGL((fa2_fwd_bf16_kernel<D, CAUSAL>), dim3(total), dim3(kThreads), 0, a.stream,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (uint16_t*)a.O, a.L, a.N, a.num_m_block, total, sa * kLog2e, sa, qsign,
                     qkeep);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  switch (a.d * 2 + a.causal) {
    case 64 * 2 + 0: return launch<64, false>(a);
    case 64 * 2 + 1: return launch<64, true>(a);
    case 128 * 2 + 0: return launch<128, false>(a);
    case 128 * 2 + 1: return launch<128, true>(a);
    case 256 * 2 + 0: return launch<256, false>(a);
    case 256 * 2 + 1: return launch<256, true>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa2
