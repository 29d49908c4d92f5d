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
// ONE query row: the row max and row sum are in-lane, plus one
// v_permlane32_swap to combine the two lane halves.  The output is likewise
// accumulated transposed, O^T += V^T P^T, so each lane's accumulators all
// belong to its one query row (the rescale by alpha and the final 1/l are
// per-lane scalars).  The P^T operand comes straight from the S^T registers:
// the contraction index may be permuted freely as long as both operands use
// the same order, so V^T is stored in LDS with its keys permuted (bits 2 and
// 3 of the key index swapped within each group of 16) to match the order in
// which S^T's accumulator rows sit in a lane.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "fa2_internal.h"

namespace fa2 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
static_assert(kBM == kBlockM_bf16, "kBlockM mismatch");

// Keys per K/V block for each head dimension.  Each thread stages four
// consecutive keys x 8 dims of K and of V per block: BN * D = 4 * 8 * 256.
template <int D> struct KvBlock;
template <> struct KvBlock<64> { static constexpr int BN = 128, kWavesPerSimd = 2; };
template <> struct KvBlock<128> { static constexpr int BN = 64, kWavesPerSimd = 2; };
template <> struct KvBlock<256> { static constexpr int BN = 32, kWavesPerSimd = 1; };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Position of key k (within a block) in the V^T rows in LDS: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Combine a per-lane value with the one held 32 lanes away (the two lane halves
// of a 32x32 MFMA tile hold different keys of the same query row).
// (__builtin_amdgcn_permlane32_swap is not used here: with both of its results
// feeding one commutative operation, hipcc 7.2 keeps only the first result.)
__device__ __forceinline__ float halves_max(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }
__device__ __forceinline__ float halves_sum(float x) { return x + __shfl_xor(x, 32, 64); }

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, KvBlock<D>::kWavesPerSimd)
fa2_fwd_bf16_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                    const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                    float* __restrict__ Lg, int N, int num_m_block, int total_blocks,
                    float c, float scale_abs, uint32_t qsign) {
  constexpr int BN = KvBlock<D>::BN;
  constexpr int KST = D + 8;   // K row stride in LDS (elements): +16 bytes against bank conflicts
  constexpr int VST = BN + 8;  // V^T row stride in LDS (elements)
  constexpr int KS = D / 16;   // MFMA k-steps over the head dimension
  constexpr int DT = D / 32;   // 32-wide tiles of the head dimension
  constexpr int KT = BN / 32;  // 32-key sub-blocks per K/V block
  constexpr int CH = D / 8;    // 16-byte chunks per row
  static_assert(BN * D == 4 * 8 * kThreads, "each thread stages 4 rows x 8 elements");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[D * VST];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // Q fragments (the B operand of S^T = K Q^T), kept in registers for the whole loop.
  bf16x8_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4_t t = {0u, 0u, 0u, 0u};
    if (qrow < N) t = *(const u32x4_t*)(Qh + (size_t)qrow * D + ks * 16 + 8 * half);
    t ^= qsign;  // exact sign flip when the scale is negative
    qf[ks] = __builtin_bit_cast(bf16x8_t, t);
  }

  f32x16_t o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = f32x16_t{};
  float m_run = kNegInf;  // running max of the unscaled logits (sign-adjusted)
  float l_part = 0.f;     // running sum over this lane's half of the keys

  const int n_blocks = (N + BN - 1) / BN;
  int j_end = n_blocks;
  if (CAUSAL) {
    const int last = min(N, (m + 1) * kBM) - 1;
    j_end = last / BN + 1;
  }

  // Staging map: thread -> 16-byte column chunk cc of rows 4*rg .. 4*rg+3.
  const int cc = tid % CH;
  const int rg = tid / CH;
  u32x4_t kr[4], vr[4];
  auto load_block = [&](int j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = j * BN + rg * 4 + r;
      if (row < N) {
        kr[r] = *(const u32x4_t*)(Kh + (size_t)row * D + cc * 8);
        vr[r] = *(const u32x4_t*)(Vh + (size_t)row * D + cc * 8);
      } else {
        kr[r] = u32x4_t{0u, 0u, 0u, 0u};
        vr[r] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };

  load_block(0);
  for (int j = 0; j < j_end; ++j) {
    __syncthreads();  // every wavefront has finished reading the previous block
#pragma unroll
    for (int r = 0; r < 4; ++r) *(u32x4_t*)(Ks + (rg * 4 + r) * KST + cc * 8) = kr[r];
    {
      // V^T: for each of the thread's 8 dims, its 4 keys form 8 contiguous bytes.
      const int pos = vt_pos(rg * 4);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x2_t ev, od;
        ev[0] = __builtin_amdgcn_perm(vr[1][w], vr[0][w], 0x05040100u);
        ev[1] = __builtin_amdgcn_perm(vr[3][w], vr[2][w], 0x05040100u);
        od[0] = __builtin_amdgcn_perm(vr[1][w], vr[0][w], 0x07060302u);
        od[1] = __builtin_amdgcn_perm(vr[3][w], vr[2][w], 0x07060302u);
        *(u32x2_t*)(Vs + (cc * 8 + 2 * w) * VST + pos) = ev;
        *(u32x2_t*)(Vs + (cc * 8 + 2 * w + 1) * VST + pos) = od;
      }
    }
    __syncthreads();
    if (j + 1 < j_end) load_block(j + 1);  // in flight while this block is computed

    const int k0 = j * BN;
    if (CAUSAL && k0 > q0 + 31) continue;  // block entirely masked for this wavefront

    // S^T = K_j Q_i^T (line 8 of the pseudo-code), fp32 accumulation.
    f32x16_t sacc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      sacc[kt] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a = *(const bf16x8_t*)(Ks + (kt * 32 + col) * KST + ks * 16 + 8 * half);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kt], 0, 0, 0);
      }
    }

    const bool masked = (CAUSAL && k0 + BN - 1 > q0) || (k0 + BN > N);
    if (masked) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kt * 32 + 8 * (r / 4) + 4 * half + (r % 4);
          const bool hide = (CAUSAL && key > qrow) || key >= N;
          sacc[kt][r] = hide ? kNegInf : sacc[kt][r];
        }
    }

    // Online softmax (line 9): new running max, rescale factor, P~ and row sum.
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float mc = m_new == kNegInf ? 0.f : c * m_new;
    const float alpha = m_run == kNegInf ? 0.f : __builtin_amdgcn_exp2f(c * m_run - mc);
    m_run = m_new;

    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r], c, -mc));
        if (masked) p = sacc[kt][r] == kNegInf ? 0.f : p;
        sacc[kt][r] = p;
        ls += p;
      }
    l_part = alpha * l_part + ls;

    // O^T = diag(alpha) O^T + V_j^T P~^T (line 10), no division by l.
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] *= alpha;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        bf16x8_t pb;
#pragma unroll
        for (int s = 0; s < 8; ++s) pb[s] = (__bf16)sacc[kt][hk * 8 + s];
        const int u = kt * 2 + hk;  // 16-key step
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const bf16x8_t a = *(const bf16x8_t*)(Vs + (t * 32 + col) * VST + u * 16 + 8 * half);
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[t], 0, 0, 0);
        }
      }
  }

  // Epilogue (lines 12-13): O = O / l once, L = m + ln(l).
  const float l_tot = halves_sum(l_part);
  const float inv = 1.f / l_tot;
  if (qrow < N) {
    uint16_t* orow = Oh + (size_t)qrow * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
        bf16x4_t w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (__bf16)(o[t][g * 4 + r] * inv);
        *(bf16x4_t*)(orow + t * 32 + 8 * g + 4 * half) = w;
      }
    if (half == 0) Lh[qrow] = __builtin_fmaf(__builtin_amdgcn_logf(l_tot), kLn2, scale_abs * m_run);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  const int total = a.num_m_block * a.BH;
  const float sa = a.scale < 0.f ? -a.scale : a.scale;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fa2_fwd_bf16_kernel<D, CAUSAL>), dim3(total), dim3(kThreads), 0, a.stream,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (uint16_t*)a.O, a.L, a.N, a.num_m_block, total, sa * kLog2e, sa, qsign);
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
