// FlashAttention-2 backward pass, bf16 or fp16 in / the same type out, fp32
// accumulation, for gfx950 (MI355X).
//
// The pages fix the structure (page "FlashAttention学习笔记(2)", sections on the
// forward and on the forward/backward thread-block split; page "Flash Attention
// V2原理解读", the backward discussion; page "flash-attention123和ring-attention",
// 优化1): the backward recomputes S and P block by block from the stored
// L = m + ln(l) alone (exp(S - L) is already the normalised weight), and runs
// with K/V outer and Q inner, so that dK and dV accumulate along a K/V block
// while dQ accumulates across K/V blocks.  The gradient formulas are the plain
// chain rule of softmax attention:
//   P = exp(scale * Q K^T - L),  dV = P^T dO,  dP = dO V^T,
//   D = rowsum(dO * O),  dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Q, O, dO, L and dQ have Nq rows, K, V, dK and dV Nk; the causal mask is
// aligned bottom-right as in the forward pass (key j visible to query i when
// j <= i + Nk - Nq), and a query that sees no key (L = -inf) contributes
// nothing (its P is masked to 0).
//
// Three kernels:
//   fa2_bwd_prep     D per row (bandwidth-bound).
//   fa2_bwd_dkdv     one workgroup per block of 128 keys (the pages' K/V-outer
//                    worker); each wavefront owns 32 keys and walks every query
//                    block that sees them, so its dK and dV stay in its own
//                    registers and no wavefronts exchange partial sums (the
//                    inter-warp reduction the pages point out for a split-Q
//                    warp layout does not arise).
//   fa2_bwd_dq       one workgroup per block of 128 queries, walking the K/V
//                    blocks like the forward pass, for dQ; this recomputes S
//                    and dP once more instead of accumulating dQ with atomics
//                    across workgroups, so the result is deterministic.
//
// Every product is a 32x32x16 bf16 or fp16 MFMA with fp32 accumulation.  As in the
// forward pass, accumulators are kept transposed where that puts one output
// row in one lane: lane l of a 32x32 tile holds column l % 32 and rows
// 8*(r/4) + 4*(l/32) + r%4.  Tiles staged in LDS use one layout (128-byte
// blocks of 4 rows x 16 dims) that serves both 16-byte row reads (the A
// operand of S and dP) and transposing reads (ds_read_b64_tr_b16, the A operand
// of dV^T, dK^T and dQ^T).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "fa2_device.h"
#include "fa2_internal.h"
#include "fa2_schedule.h"

namespace fa2 {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // keys (dK/dV) or queries (dQ) per workgroup
constexpr int kStep = 64;           // queries (dK/dV) or keys (dQ) per inner step

// Byte offset of element (row r, dim c) of a staged [rows][D] 16-bit tile.
// Rows go in groups of 4 (g = r/4, 8D bytes each) and dims in 16-dim segments of
// 128 bytes; a segment holds two 64-byte halves (its dims 0-7 and 8-15), each
// 4 rows x 16 bytes.  Odd row groups swap adjacent segments and row groups
// with bit 1 set swap the halves.  The 16 lanes of one pass of a 16-byte row
// read (4 row groups x 4 rows, one 16-dim segment) then reach all 64 banks
// once, and each 16-lane group of a transposing read still reads one whole
// 128-byte segment.
template <int D>
__device__ __forceinline__ constexpr int toff(int r, int c) {
  return (r >> 2) * (8 * D) + ((c >> 4) ^ ((r >> 2) & 1)) * 128 +
         64 * (((c >> 3) & 1) ^ ((r >> 3) & 1)) + 16 * (r & 3) + 2 * (c & 7);
}

// What the direct loads that stage a tile read.  Direct load n fills 1 KB
// chunk n of the tile: its lane L writes the 16 bytes at slot L%8 of 128-byte
// block bk = 8n + L/8, which is segment position bk % NSEG of row group
// g = bk / NSEG: row 4g + L%4, dims 16*((bk % NSEG) ^ (g%2)) + 8*((L%8)/4 ^ (g/2)%2).
// The row is stage_row(n, 0) (uniform) plus a non-negative per-lane part.
template <int D>
__device__ __forceinline__ constexpr int stage_row(int n, int L) {
  return 4 * ((8 * n + L / 8) / (D / 16)) + L % 4;
}
template <int D>
__device__ __forceinline__ constexpr int stage_col(int n, int L) {
  constexpr int NSEG = D / 16;
  const int bk = 8 * n + L / 8, g = bk / NSEG;
  return 16 * ((bk % NSEG) ^ (g & 1)) + 8 * (((L % 8) / 4) ^ ((g >> 1) & 1));
}

// The direct loads of a [ROWS][D] tile: NL loads of 1 KB.  When they split
// evenly over the wavefronts, wavefront w issues loads w*PER .. w*PER + PER-1;
// otherwise (d = 32 and 96) load i*kWaves + w for i < PER while it exists, a
// wave-uniform test.
template <int D, int ROWS>
struct TileLoads {
  static constexpr int NL = ROWS * D * 2 / 1024;
  static constexpr bool EVEN = NL % kWaves == 0;
  static constexpr int PER = (NL + kWaves - 1) / kWaves;
  static_assert(ROWS * D * 2 % 1024 == 0 && NL >= 1, "the tile is whole 1 KB loads");
  __device__ static constexpr int load(int wave, int i) {
    return EVEN ? wave * PER + i : i * kWaves + wave;
  }
  __device__ static constexpr bool issued(int wave, int i) { return EVEN || i * kWaves + wave < NL; }
};

// Stage rows [r0, r0 + ROWS) of a [N][D] 16-bit slice into LDS in the tile
// layout (this wavefront's loads, TileLoads).  With CLAMP, rows past N are
// clamped to row N - 1 (callers mask them); without, every row must exist, and
// each load is a scalar base (the row stage_row(n, 0)) plus a per-lane byte
// offset.
template <int D, int ROWS, bool CLAMP>
__device__ __forceinline__ void stage_tile(const uint16_t* head, int r0, int N, char* buf,
                                           int wave) {
  typedef TileLoads<D, ROWS> TL;
  const int lane = fresh_lane();  // recomputed here: not kept in registers across the loop
#pragma unroll
  for (int i = 0; i < TL::PER; ++i) {
    if (!TL::issued(wave, i)) continue;
    const int n = TL::load(wave, i);
    if constexpr (CLAMP) {
      const int r = min(r0 + stage_row<D>(n, lane), N - 1);
      lds_dma(head + (size_t)r * D + stage_col<D>(n, lane), lds_addr(buf + n * 1024));
    } else {
      const uint32_t voff =
          (uint32_t)(((stage_row<D>(n, lane) - stage_row<D>(n, 0)) * D + stage_col<D>(n, lane)) * 2);
      lds_dma(head + (size_t)(r0 + stage_row<D>(n, 0)) * D, voff, lds_addr(buf + n * 1024));
    }
  }
}

// The per-lane byte offsets of stage_tile without CLAMP, computed once by a
// kernel that keeps them in registers across its loop.
template <int D, int ROWS>
struct StageOffsets {
  static constexpr int LOADS = TileLoads<D, ROWS>::PER;
  uint32_t tile[LOADS];
  uint32_t vec;  // 4 * lane, for stage_vec
};
template <int D, int ROWS>
__device__ __forceinline__ StageOffsets<D, ROWS> stage_offsets(int wave) {
  typedef TileLoads<D, ROWS> TL;
  StageOffsets<D, ROWS> o;
  const int lane = fresh_lane();
#pragma unroll
  for (int i = 0; i < o.LOADS; ++i) {
    const int n = TL::load(wave, i);
    o.tile[i] = TL::issued(wave, i)
                    ? (uint32_t)(((stage_row<D>(n, lane) - stage_row<D>(n, 0)) * D +
                                  stage_col<D>(n, lane)) * 2)
                    : 0u;
  }
  o.vec = (uint32_t)(4 * lane);
  return o;
}
template <int D, int ROWS>
__device__ __forceinline__ void stage_tile_at(const uint16_t* head, int r0, char* buf, int wave,
                                              const StageOffsets<D, ROWS>& o) {
  typedef TileLoads<D, ROWS> TL;
#pragma unroll
  for (int i = 0; i < o.LOADS; ++i) {
    if (!TL::issued(wave, i)) continue;
    const int n = TL::load(wave, i);
    lds_dma(head + (size_t)(r0 + stage_row<D>(n, 0)) * D, o.tile[i], lds_addr(buf + n * 1024));
  }
}

// Stage 64 floats v[r0 .. r0+64) into LDS: one 4-byte direct load per lane.
// With CLAMP the index is clamped to N - 1; without, all 64 must exist.
__device__ __forceinline__ void stage_vec(const float* v, int r0, int N, char* buf) {
  const float* src = v + min(r0 + fresh_lane(), N - 1);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               : : "s"(lds_addr(buf)), "v"(src) : "memory", "m0");
}
// The same without clamping (all 64 must exist); voff = 4 * lane.
__device__ __forceinline__ void stage_vec_at(const float* v, int r0, uint32_t voff, char* buf) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               : : "s"(lds_addr(buf)), "v"(voff), "s"(v + r0) : "memory", "m0");
}

// LDS addresses of fragments in a staged tile, as two per-lane bases (computed
// once) plus compile-time offsets.
//
// Row fragment: the A operand of a 32x32x16 MFMA, rows m = row0 + lane%32
// (row0 a multiple of 32) and dims 16*ks + 8*(lane/32) .. +8, one 16-byte read
// at base[ks % 2] + (row0/4)*8D + 256*(ks/2), with g = (lane%32)/4 and
//   base[p](lane) = g*8D + 128*(p ^ g%2) + 64*(lane/32 ^ (g/2)%2) + 16*(lane%4).
template <int D>
__device__ __forceinline__ constexpr int row_base(int lane, int p) {
  const int g = (lane & 31) >> 2;
  return g * (8 * D) + 128 * (p ^ (g & 1)) + 64 * ((lane >> 5) ^ ((g >> 1) & 1)) + 16 * (lane & 3);
}
template <int D>
struct Bases {
  uint32_t row[2], tr[2];
};
template <typename T, int D>
__device__ __forceinline__ typename Vec16<T>::x8 row_frag(const char* tile, const Bases<D>& b,
                                                          int row0, int ks) {
  return *(const typename Vec16<T>::x8*)(tile + b.row[ks & 1] + (row0 / 4) * (8 * D) +
                                         256 * (ks >> 1));
}
// Transposed fragment: the A operand (dims x rows) for rows 16u .. 16u+15 of
// the tile and dims 32t .. 32t+31, in the permuted row order that matches a B
// operand packed from accumulator registers 8*(u%2) .. 8*(u%2)+7 of the
// 32-row tile u/2.  Within each 16-lane group (sb = (lane/16)%2, i = lane%16),
// lane 4*r + c points at dims 32t + 16sb + 4c .. +3 of row kbase + r;
// ds_read_b64_tr_b16 hands lane t of the group the 4 rows kbase .. kbase+3 of
// dim t.  kbase = 16u + 4*half (first 4 slots, e = 0) and 16u + 8 + 4*half
// (last 4, e = 1): row group g = 4u + half + 2e, so the group reads one whole
// 128-byte segment, at
//   base.tr[e](lane) = half*8D + 16D*e + 128*(sb ^ half) + 64*(c/2 ^ e) + 16*r + 8*(c%2),
//   + 32D*u + 256*t.
template <int D>
__device__ __forceinline__ constexpr int tr_base(int lane, int e) {
  const int half = lane >> 5, sb = (lane >> 4) & 1, i = lane & 15, c = i & 3;
  return half * (8 * D) + 16 * D * e + 128 * (sb ^ half) + 64 * ((c >> 1) ^ e) + 16 * (i >> 2) +
         8 * (c & 1);
}
template <int D>
__device__ __forceinline__ Bases<D> bases(int lane) {
  Bases<D> b;
#pragma unroll
  for (int p = 0; p < 2; ++p) b.row[p] = (uint32_t)row_base<D>(lane, p);
#pragma unroll
  for (int e = 0; e < 2; ++e) b.tr[e] = (uint32_t)tr_base<D>(lane, e);
  return b;
}
template <typename T, int D>
__device__ __forceinline__ typename Vec16<T>::x8 tr_frag(const char* tile, const Bases<D>& b, int u,
                                                         int t) {
  const int o = 32 * D * u + 256 * t;
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr_t)(tile + b.tr[0] + o));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr_t)(tile + b.tr[1] + o));
  return __builtin_bit_cast(typename Vec16<T>::x8,
                            __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Compile-time proof of the layout for a [ROWS][D] tile: the direct loads of
// stage_tile stay inside the tile (rows < ROWS, dims < D, 16-byte chunks) and
// fill every (row, 8 dims) exactly once, where toff puts it; row and
// transposing fragment reads are aligned (16 and 8 bytes), stay inside the
// tile and their addresses equal toff of the (row, dims) the MFMA operand
// needs; each 16-lane pass of a row read reaches 16 distinct 16-byte bank
// groups (64 banks of 4 bytes) and each 16-lane group of a transposing read 16
// distinct 8-byte slots of one 128-byte span.
template <int D, int ROWS>
__device__ __forceinline__ constexpr bool tile_layout_ok() {
  constexpr int BYTES = ROWS * D * 2;
  bool seen[ROWS * D / 8] = {};
  for (int n = 0; n < BYTES / 1024; ++n)
    for (int L = 0; L < 64; ++L) {
      const int r = stage_row<D>(n, L), c = stage_col<D>(n, L);
      if (r < 0 || r >= ROWS || c < 0 || c + 8 > D || c % 8 != 0) return false;
      if (seen[(r * D + c) / 8]) return false;
      seen[(r * D + c) / 8] = true;
      if (r < stage_row<D>(n, 0)) return false;  // the per-lane part of the address is >= 0
      for (int k = 0; k < 8; ++k)
        if (toff<D>(r, c + k) != n * 1024 + 16 * L + 2 * k) return false;
    }
  for (int row0 = 0; row0 < ROWS; row0 += 32)
    for (int ks = 0; ks < D / 16; ++ks)
      for (int pass = 0; pass < 4; ++pass) {
        bool used[16] = {};
        for (int l = 16 * pass; l < 16 * pass + 16; ++l) {
          const int a = row_base<D>(l, ks & 1) + (row0 / 4) * (8 * D) + 256 * (ks >> 1);
          if (a < 0 || a + 16 > BYTES || a % 16 != 0) return false;
          for (int k = 0; k < 8; ++k)
            if (toff<D>(row0 + (l & 31), 16 * ks + 8 * (l >> 5) + k) != a + 2 * k) return false;
          if (used[(a / 16) % 16]) return false;
          used[(a / 16) % 16] = true;
        }
      }
  for (int u = 0; u < ROWS / 16; ++u)
    for (int t = 0; t < D / 32; ++t)
      for (int e = 0; e < 2; ++e)
        for (int grp = 0; grp < 4; ++grp) {
          bool used[16] = {};
          int lo = 1 << 30;
          for (int l = 16 * grp; l < 16 * grp + 16; ++l) {
            const int a = tr_base<D>(l, e) + 32 * D * u + 256 * t;
            lo = a < lo ? a : lo;
            if (a < 0 || a + 8 > BYTES || a % 8 != 0) return false;
          }
          for (int l = 16 * grp; l < 16 * grp + 16; ++l) {
            const int a = tr_base<D>(l, e) + 32 * D * u + 256 * t, i = l & 15;
            const int row = 16 * u + 4 * (l >> 5) + 8 * e + (i >> 2);
            const int dim = 32 * t + 16 * ((l >> 4) & 1) + 4 * (i & 3);
            for (int k = 0; k < 4; ++k)
              if (toff<D>(row, dim + k) != a + 2 * k) return false;
            if (a - lo >= 128 || used[(a - lo) / 8]) return false;
            used[(a - lo) / 8] = true;
          }
        }
  return true;
}
static_assert(tile_layout_ok<32, 32>() && tile_layout_ok<32, 64>() && tile_layout_ok<32, 128>(),
              "tile layout, d = 32");
static_assert(tile_layout_ok<64, 32>() && tile_layout_ok<64, 64>() && tile_layout_ok<64, 128>(),
              "tile layout, d = 64");
static_assert(tile_layout_ok<96, 32>() && tile_layout_ok<96, 64>() && tile_layout_ok<96, 128>(),
              "tile layout, d = 96");
static_assert(tile_layout_ok<128, 32>() && tile_layout_ok<128, 64>() &&
                  tile_layout_ok<128, 128>(),
              "tile layout, d = 128");
static_assert(tile_layout_ok<256, 32>() && tile_layout_ok<256, 64>() &&
                  tile_layout_ok<256, 128>(),
              "tile layout, d = 256");

// B operand fragments of a [N][D] 16-bit slice held in registers: for k-step ks,
// lane l holds row r0 + l%32, dims 16*ks + 8*(l/32) .. +8 (zero past N).
template <typename T, int D>
__device__ __forceinline__ void load_frags(typename Vec16<T>::x8 (&f)[D / 16], const uint16_t* head,
                                           int row, int N, int half) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4_t t = {0u, 0u, 0u, 0u};
    if (row < N) t = *(const u32x4_t*)(head + (size_t)row * D + 16 * ks + 8 * half);
    f[ks] = __builtin_bit_cast(typename Vec16<T>::x8, t);
  }
}

// Wait for the fragment loads issued before a kernel's main loop and pass the
// registers through an empty asm statement.  The compiler then sees them
// defined by that statement rather than by pending loads, and puts no
// vmcnt wait inside the loop, where it would also wait for the direct loads
// that stage the next step (they are invisible to it).
template <typename V, int KS>
__device__ __forceinline__ void hold_loaded(V (&a)[KS], V (&b)[KS]) {
  wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(a[ks]), "+v"(b[ks]));
}
template <typename V, int KS>
__device__ __forceinline__ void hold_loaded(V (&a)[KS]) {
  wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(a[ks]));
}

// Store a transposed accumulator (DT tiles of 32 dims x 32 rows; lane = row)
// times `mul` as rows [row0, row0+32) of a [N][D] slice of type T, through a
// buffer resource bounded to rows < N.
template <typename T, int D>
__device__ __forceinline__ void store_rows(const f32x16_t (&acc)[D / 32], float mul,
                                           uint16_t* head, int row0, int N, int lane) {
  // 0 rows for a wavefront past the end: no store lands.  Both values are
  // uniform; readfirstlane keeps the resource in scalar registers (otherwise
  // the compiler wraps every store in a loop over distinct resources).
  const int rows = __builtin_amdgcn_readfirstlane(max(0, min(32, N - row0)));
  const uint64_t base = (uint64_t)(head + (size_t)row0 * D);
  const uint64_t ubase = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(base >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ubase, (short)0, rows * D * 2, kBufferFlags);
  const int half = lane >> 5, col = lane & 31;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      typename Vec16<T>::x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = (T)(acc[t][g * 4 + r] * mul);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, w), rs,
                                            (col * D + t * 32 + 8 * g + 4 * half) * 2, 0, 0);
    }
}

// Workgroup ids are dealt to the 8 XCDs round-robin (id % 8), and each XCD has
// its own L2.  The logical block index (sched::xcd_block, fa2_schedule.h) gives
// XCD x a contiguous range of blocks, so the blocks of one head (which read the
// same Q/dO or K/V tiles) run on one XCD and share its L2.  A bijection on
// [0, G) for any G; only speed depends on the dispatcher actually dealing ids
// this way.
using sched::xcd_block;

// ---------------------------------------------------------------- D = rowsum(dO * O)
// Writes -D (the dK/dV kernel starts its dP accumulators from it) and
// L*log2(e).  Rows are padded per head to Npad (a multiple of the dK/dV
// kernel's query step): padded rows get D = 0 and L*log2(e) = +inf, so
// exp2(c*S - L*log2(e)) is 0 there and the dK/dV kernel needs no test for
// queries past Nq.
// Threads per row of the prep kernel: one per 8 dims, rounded up to a power of
// two for the butterfly sum (d = 96: 16, of which 12 load).
template <int D>
constexpr int prep_tpr() {
  return D == 96 ? 16 : D / 8;
}
template <typename T, int D>
__global__ void __launch_bounds__(kThreads)
fa2_bwd_prep_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                    const float* __restrict__ L, float* __restrict__ Dv, float* __restrict__ L2v,
                    int Nq, int Npad, int rows) {
  typedef typename Vec16<T>::x8 t8_t;
  constexpr int TPR = prep_tpr<D>();  // threads per row, 8 dims each (the last idle for d = 96)
  const int row = blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  const int bh = row / Npad, q = row - bh * Npad;
  const bool valid = row < rows && q < Nq;
  const size_t src = (size_t)bh * Nq + q;
  float acc = 0.f;
  if (valid && t < D / 8) {
    const t8_t o = *(const t8_t*)(O + src * D + 8 * t);
    const t8_t g = *(const t8_t*)(dO + src * D + 8 * t);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += (float)o[i] * (float)g[i];
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m, 64);
  if (row < rows && t == 0) {
    Dv[row] = -acc;
    L2v[row] = valid ? L[src] * kLog2e : __builtin_inff();
  }
}

// ---------------------------------------------------------------- dK, dV
// Queries per step of the K/V-outer kernel: one 32-query tile, which keeps the
// live registers (K and V fragments, dK and dV accumulators, one S and one dP
// tile) within 256 so that two wavefronts share each SIMD.
constexpr int kQStep = 32;

// OCC: workgroups per CU (two, or one for d = 256, whose dK and dV
// accumulators alone take 256 registers).
template <typename T, int D, bool CAUSAL, int OCC>
__global__ void __launch_bounds__(kThreads, OCC)
fa2_bwd_dkdv_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                    const uint16_t* __restrict__ Vg, const uint16_t* __restrict__ dOg,
                    const float* __restrict__ L2g, const float* __restrict__ Dg,
                    uint16_t* __restrict__ dKg, uint16_t* __restrict__ dVg, int Nq, int Nk,
                    int Npad, int num_k_block, float c, float scale) {
  typedef typename Vec16<T>::x8 t8_t;
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int TILE = kQStep * D * 2;  // bytes of one staged [32][D] tile
  // Q, dO tiles, then 64 L and 64 D values (32 used), for two steps; and the
  // block's V rows (the B operand of dP), staged once.
  __shared__ __attribute__((aligned(1024))) char smem[2 * (2 * TILE + 512)];
  __shared__ __attribute__((aligned(1024))) char vtile[kRows * D * 2];
  static_assert(tile_layout_ok<D, kQStep>() && tile_layout_ok<D, kRows>(), "staged tiles");
  // L and D of a step: 64 floats each, 256 bytes after the two tiles; the reads
  // take 4 floats at 8g + 4*half (g < 4), the last ending at float 32.
  static_assert(4 * (8 * 3 + 4 + 4) <= 256, "L and D reads stay inside their 256 bytes");
  static_assert(OCC * (2 * (2 * TILE + 512) + kRows * D * 2) <= 160 * 1024,
                "the resident workgroups' LDS fits a CU");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  // The key blocks of a head are consecutive logical blocks, so they run side by
  // side on one XCD; with the causal mask the first (heaviest) goes out first.
  const int blk = xcd_block(blockIdx.x, gridDim.x);
  const int kb = blk % num_k_block;
  const int bh = blk / num_k_block;
  const size_t qslice = (size_t)bh * Nq * D, kslice = (size_t)bh * Nk * D;
  const uint16_t *Qh = Qg + qslice, *dOh = dOg + qslice;
  // L*log2(e) and D, Npad rows per head (padded rows: +inf and 0).
  const float *Lh = L2g + (size_t)bh * Npad, *Dh = Dg + (size_t)bh * Npad;
  const int off = Nk - Nq;                // key j visible to query i when j <= i + off
  const int k0 = kb * kRows + 32 * wave;  // this wavefront's first key
  const Bases<D> lb = bases<D>(lane);

  // K fragments stay in registers (the B operand of S); V is read from LDS,
  // which leaves registers for the dP accumulators to start from -D.
  t8_t kf[KS];
  load_frags<T, D>(kf, Kg + kslice, k0 + col, Nk, half);
  hold_loaded(kf);
  f32x16_t dk[DT], dv[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dk[t] = dv[t] = f32x16_t{};

  // Query steps: those from the first that can see the block's keys to the end,
  // walked from the last down.  Every key block of a head then starts at the
  // same query step, and the blocks running side by side read each staged Q/dO
  // tile at about the same time (from L2), whatever their first step.
  const int first_q = kb * kRows - off;  // the first query that sees the block's first key
  const int i_beg = CAUSAL ? (first_q > 0 ? first_q / kQStep : 0) : 0;
  const int i_end = (Nq + kQStep - 1) / kQStep;
  auto buf = [&](int i) { return smem + (i & 1) * (2 * TILE + 512); };
  // Only the first step walked (the last one) can reach past Nq; the others are
  // staged with scalar bases, no clamping and per-lane offsets held in registers.
  const StageOffsets<D, kQStep> so = stage_offsets<D, kQStep>(wave);
  auto stage = [&](int i, auto clamp) {
    char* b = buf(i);
    if constexpr (decltype(clamp)::value) {
      stage_tile<D, kQStep, true>(Qh, i * kQStep, Nq, b, wave);
      stage_tile<D, kQStep, true>(dOh, i * kQStep, Nq, b + TILE, wave);
      if (wave == 0) stage_vec(Lh, i * kQStep, Npad, b + 2 * TILE);
      if (wave == 1) stage_vec(Dh, i * kQStep, Npad, b + 2 * TILE + 256);
    } else {
      stage_tile_at<D, kQStep>(Qh, i * kQStep, b, wave, so);
      stage_tile_at<D, kQStep>(dOh, i * kQStep, b + TILE, wave, so);
      if (wave == 0) stage_vec_at(Lh, i * kQStep, so.vec, b + 2 * TILE);
      if (wave == 1) stage_vec_at(Dh, i * kQStep, so.vec, b + 2 * TILE + 256);
    }
  };
  if (i_beg < i_end) {
    // Rows past Nk are clamped copies: their dK and dV rows are never stored.
    stage_tile<D, kRows, true>(Vg + kslice, kb * kRows, Nk, vtile, wave);
    stage(i_end - 1, std::true_type{});
  }
  auto step = [&](int i, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    wait_vmcnt<0>();
    lds_barrier();
    if (i > i_beg) stage(i - 1, std::false_type{});
    const char* b = buf(i);
    const char* qtile = b;
    const char* dtile = b + TILE;
    const float* lv = (const float*)(b + 2 * TILE);
    const float* dvec = (const float*)(b + 2 * TILE + 256);
    const int q_base = i * kQStep;
    // dP starts from -D of each accumulator's query (the workspace holds -D),
    // so the products leave dP - D in it.
    f32x16_t S = f32x16_t{}, dP;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4_t D4 = *(const f32x4_t*)(dvec + 8 * g + 4 * half);
#pragma unroll
      for (int r = 0; r < 4; ++r) dP[g * 4 + r] = D4[r];
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      S = mfma32x32x16(row_frag<T, D>(qtile, lb, 0, ks), kf[ks], S);
      dP = mfma32x32x16(row_frag<T, D>(dtile, lb, 0, ks), row_frag<T, D>(vtile, lb, 32 * wave, ks),
                        dP);
    }
    // This lane's key is k0 + col; accumulator r holds query
    // q_base + cr + 4*half with cr = 8*(r/4) + r%4 (a constant).  With the
    // causal mask the query is visible to the key when cr >= lo
    // (key <= query + off); steps whose queries all see every key of the
    // wavefront run without the test (MASK false).  A query that sees no key
    // at all has L = -inf; every one of its entries is masked.  Queries past
    // Nq have L*log2(e) = +inf and so P = 0.
    const int lo = k0 + col - off - q_base - 4 * half;
    t8_t pb[2], sb[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int qr = 8 * g + 4 * half;  // first of 4 consecutive queries
      const f32x4_t L4 = *(const f32x4_t*)(lv + qr);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int cr = 8 * g + r;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[g * 4 + r], c, -L4[r]));
        if constexpr (MASK) p = cr < lo ? 0.f : p;
        pb[g / 2][(g % 2) * 4 + r] = (T)p;
        sb[g / 2][(g % 2) * 4 + r] = (T)(p * dP[g * 4 + r]);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        dv[t] = mfma32x32x16(tr_frag<T, D>(dtile, lb, u, t), pb[u], dv[t]);
        dk[t] = mfma32x32x16(tr_frag<T, D>(qtile, lb, u, t), sb[u], dk[t]);
      }
  };
  // Steps from i_clean up see every key of this wavefront (q_base + off >= k0 + 31):
  // they run without the mask; the rest (walked last) with it.
  const int need = k0 + 31 - off;
  const int i_clean = !CAUSAL ? i_beg : min(i_end, max(i_beg, need <= 0 ? 0 : (need + 31) / 32));
  for (int i = i_end - 1; i >= i_clean; --i) step(i, std::false_type{});
  for (int i = i_clean - 1; i >= i_beg; --i) step(i, std::true_type{});
  store_rows<T, D>(dv, 1.f, dVg + kslice, k0, Nk, lane);
  store_rows<T, D>(dk, scale, dKg + kslice, k0, Nk, lane);
}

// ---------------------------------------------------------------- dQ
template <typename T, int D, bool CAUSAL, int OCC>
__global__ void __launch_bounds__(kThreads, OCC)
fa2_bwd_dq_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                  const uint16_t* __restrict__ Vg, const uint16_t* __restrict__ dOg,
                  const float* __restrict__ L2g, const float* __restrict__ Dg,
                  uint16_t* __restrict__ dQg, int Nq, int Nk, int Npad, int num_m_block, float c,
                  float scale) {
  typedef typename Vec16<T>::x8 t8_t;
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int TILE = kStep * D * 2;
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * TILE];  // K, V tiles, two steps
  static_assert(tile_layout_ok<D, kStep>(), "staged tiles");
  static_assert(OCC * (2 * 2 * TILE) <= 160 * 1024, "the resident workgroups' LDS fits a CU");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  // The query blocks of a head are consecutive logical blocks (one XCD, one
  // L2 for the K/V tiles they all walk from key 0); heaviest causal block first.
  const int blk = xcd_block(blockIdx.x, gridDim.x);
  const int mi = blk % num_m_block;
  const int m = CAUSAL ? num_m_block - 1 - mi : mi;
  const int bh = blk / num_m_block;
  const size_t qslice = (size_t)bh * Nq * D, kslice = (size_t)bh * Nk * D;
  const uint16_t *Kh = Kg + kslice, *Vh = Vg + kslice;
  const int off = Nk - Nq;  // key j visible to query i when j <= i + off
  const int q0 = m * kRows + 32 * wave;
  const int qrow = q0 + col;
  const Bases<D> lb = bases<D>(lane);

  t8_t qf[KS], df[KS];
  load_frags<T, D>(qf, Qg + qslice, qrow, Nq, half);
  load_frags<T, D>(df, dOg + qslice, qrow, Nq, half);
  // L*log2(e) and -D of this lane's query (Npad rows per head).
  float l2 = qrow < Nq ? L2g[(size_t)bh * Npad + qrow] : 0.f;
  float dd = qrow < Nq ? Dg[(size_t)bh * Npad + qrow] : 0.f;  // -D
  hold_loaded(qf, df);
  asm volatile("" : "+v"(l2), "+v"(dd));
  // Every dP accumulator starts from -D of the lane's query, so the products
  // leave dP - D in it (one register tile, held across the loop).
  f32x16_t neg_d;
#pragma unroll
  for (int r = 0; r < 16; ++r) neg_d[r] = dd;
  f32x16_t dq[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dq[t] = f32x16_t{};

  // K/V blocks up to the last key the workgroup's last query sees (none when
  // it sees no key: dQ = 0).
  const int nkb = (Nk + kStep - 1) / kStep;
  const int last_key = min(Nq, (m + 1) * kRows) - 1 + off;
  const int j_end = CAUSAL ? (last_key < 0 ? 0 : min(last_key / kStep + 1, nkb)) : nkb;
  auto buf = [&](int j) { return smem + (j & 1) * (2 * TILE); };
  // Blocks wholly before Nk are staged with scalar bases; only a ragged last
  // block needs clamped per-lane addresses.
  auto stage = [&](int j) __attribute__((always_inline)) {
    if ((j + 1) * kStep <= Nk) {
      stage_tile<D, kStep, false>(Kh, j * kStep, Nk, buf(j), wave);
      stage_tile<D, kStep, false>(Vh, j * kStep, Nk, buf(j) + TILE, wave);
    } else {
      stage_tile<D, kStep, true>(Kh, j * kStep, Nk, buf(j), wave);
      stage_tile<D, kStep, true>(Vh, j * kStep, Nk, buf(j) + TILE, wave);
    }
  };
  // Blocks before j_clean need no mask for this wavefront: all their keys
  // precede Nk and every query of the wavefront sees them.  Walking up, they
  // come first, and a loop of their own runs them without any test, so that
  // each of their steps is one basic block.
  const int seen = q0 + off + 1;  // keys the wavefront's first query sees
  const int j_clean =
      min(j_end, min(Nk / kStep, CAUSAL ? (seen <= 0 ? 0 : seen / kStep) : Nk / kStep));
  auto step = [&](int j, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    wait_vmcnt<0>();
    lds_barrier();
    if (j + 1 < j_end) stage(j + 1);
    const char* kt_ = buf(j);
    const char* vt = buf(j) + TILE;
    t8_t sb[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16_t S = f32x16_t{}, dP = neg_d;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        S = mfma32x32x16(row_frag<T, D>(kt_, lb, 32 * kt, ks), qf[ks], S);
        dP = mfma32x32x16(row_frag<T, D>(vt, lb, 32 * kt, ks), df[ks], dP);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], c, -l2));
      if constexpr (MASKED) {
        // This lane's query is qrow; accumulator r holds key
        // j*64 + 32*kt + cr + 4*half with cr = 8*(r/4) + r%4 (a constant),
        // visible when cr <= th (key <= query + off, key < Nk); a query that
        // sees no key (L = -inf) has every entry masked.
        const int kb0 = j * kStep + 32 * kt + 4 * half;
        int th = Nk - 1 - kb0;
        if (CAUSAL) th = min(th, qrow + off - kb0);
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] = 8 * (r / 4) + (r % 4) > th ? 0.f : S[r];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sb[kt * 2 + r / 8][r % 8] = (T)(S[r] * dP[r]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < DT; ++t)
        dq[t] = mfma32x32x16(tr_frag<T, D>(kt_, lb, u, t), sb[u], dq[t]);
  };
  if (j_end > 0) stage(0);
  int j = 0;
  for (; j < j_clean; ++j) step(j, std::false_type{});
  for (; j < j_end; ++j) step(j, std::true_type{});
  store_rows<T, D>(dq, scale, dQg + qslice, q0, Nq, lane);
}

template <typename T, int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a) {
  constexpr int OCC = D == 256 ? 1 : 2;
  const float c = a.scale * kLog2e;
  const int Npad = (int)bwd_rows(a.Nq);
  const int qrows = a.BH * Npad;
  float* L2v = a.Dvec + (size_t)qrows;
  constexpr int RPB = kThreads / prep_tpr<D>();
  // Kernels with nothing to do are not launched: no queries leaves dK = dV = 0
  // (written by the dK/dV kernel, which then walks no query step); no keys
  // leaves dQ = 0 (written by the dQ kernel, which then walks no key block).
  if (qrows > 0)
    hipLaunchKernelGGL((fa2_bwd_prep_kernel<T, D>), dim3((qrows + RPB - 1) / RPB), dim3(kThreads),
                       0, a.stream, (const uint16_t*)a.O, (const uint16_t*)a.dO, a.L, a.Dvec, L2v,
                       a.Nq, Npad, qrows);
  const int nkb = (a.Nk + kRows - 1) / kRows;
  if (nkb * a.BH > 0)
    hipLaunchKernelGGL((fa2_bwd_dkdv_kernel<T, D, CAUSAL, OCC>), dim3(nkb * a.BH), dim3(kThreads), 0,
                       a.stream, (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (const uint16_t*)a.dO, L2v, a.Dvec, (uint16_t*)a.dK, (uint16_t*)a.dV, a.Nq,
                       a.Nk, Npad, nkb, c, a.scale);
  const int nmb = (a.Nq + kRows - 1) / kRows;
  if (nmb * a.BH > 0)
    hipLaunchKernelGGL((fa2_bwd_dq_kernel<T, D, CAUSAL, OCC>), dim3(nmb * a.BH), dim3(kThreads), 0,
                       a.stream, (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (const uint16_t*)a.dO, L2v, a.Dvec, (uint16_t*)a.dQ, a.Nq, a.Nk, Npad, nmb,
                       c, a.scale);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const BwdArgs& a) {
  switch (a.d * 2 + a.causal) {
    case 32 * 2 + 0: return launch<T, 32, false>(a);
    case 32 * 2 + 1: return launch<T, 32, true>(a);
    case 64 * 2 + 0: return launch<T, 64, false>(a);
    case 64 * 2 + 1: return launch<T, 64, true>(a);
    case 96 * 2 + 0: return launch<T, 96, false>(a);
    case 96 * 2 + 1: return launch<T, 96, true>(a);
    case 128 * 2 + 0: return launch<T, 128, false>(a);
    case 128 * 2 + 1: return launch<T, 128, true>(a);
    case 256 * 2 + 0: return launch<T, 256, false>(a);
    case 256 * 2 + 1: return launch<T, 256, true>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.elem == kBF16) return dispatch<__bf16>(a);
  if (a.elem == kFP16) return dispatch<_Float16>(a);
  return hipErrorInvalidValue;
}

}  // namespace fa2
