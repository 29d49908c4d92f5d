// Decoding: FlashAttention-2 forward pass for one query per (batch, head) over a
// long key/value sequence, bf16 or fp16 in, for gfx950 (MI355X).
//
// The result is the same as the general kernel's: with one query row and the
// causal mask aligned bottom-right, the row sees every key, so the mask plays
// no part.  The pages' method is followed block by block (page "Flash
// Attention V2原理解读", the forward loop; page "FlashAttention学习笔记(2)",
// the online softmax with the 1/l division deferred to the end): keys are
// walked in blocks of 64, a running maximum and a running sum are kept, the
// weighted sum of V rows is rescaled when the maximum moves, and the division
// by the sum comes once at the end.  With splits, each split is one part of
// the key sequence and writes its normalised float32 partial result and its
// logsumexp, which the split-KV merge combines (page "Flash Attention
// V2原理解读", the split-KV discussion).
//
// Why a kernel of its own: one query row is one flop per byte of K and V, so
// the pass is bound by HBM, not by the matrix cores.  The general kernel pads
// the row to a 128-row MFMA tile (127 padding rows of exp and MFMA work) and
// keeps about one 32 KB block in flight per workgroup.  Here:
//   * a workgroup (4 wavefronts, one per SIMD) streams its key range through a
//     ring of kBuf staged K/V blocks with direct global->LDS loads, so that
//     kBuf - 1 blocks (96 KB at d = 128) are in flight per CU;
//   * wavefront w takes keys 16w .. 16w+15 of each block.  For q.k each key
//     is split over 4 lanes, each holding a quarter of q in registers and
//     using v_dot2 on pairs of 16-bit values; 2 lane exchanges finish the sum;
//   * for the weighted sum of V rows the lanes hold dims instead (D/64 each);
//     each key's weight is broadcast with readlane, and the wavefront reads
//     the key's V row from LDS in one 256-byte (d = 128) access;
//   * each wavefront keeps its own running maximum, sum and D/64 accumulators
//     per lane; the 4 wavefronts' states are merged through LDS at the end.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {
namespace {

using namespace dev;

constexpr int kThreads = 256;
constexpr int kKeys = 64;  // keys per staged block; 16 per wavefront

template <int D>
struct DecCfg {
  static_assert(D == 64 || D == 128 || D == 256, "decoding kernel head dimension");
  static constexpr int kBlockBytes = kKeys * D * 2;              // one of K or V
  static constexpr int kBuf = D == 256 ? 2 : 4;                  // staged blocks
  static constexpr int kLoads = kBlockBytes / 1024 / 4;          // direct loads per wave per tensor
  static constexpr int kRowsPerLoad = 512 / D;                   // rows per 1 KB load
  static constexpr int kLanesPerRow = D / 8;                     // 16-byte pieces per row
  static constexpr int kQuarter = D / 4;                         // dims per q.k lane
  static constexpr int kPieces = kQuarter / 8;                   // 16-byte pieces per q.k lane
  static constexpr int kDimsPerLane = D / 64;                    // dims per lane for P.V
};

template <typename T>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);
template <>
__device__ __forceinline__ float dot2<__bf16>(uint32_t a, uint32_t b, float c) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, a), __builtin_bit_cast(bf2, b), c,
                                         false);
}
template <>
__device__ __forceinline__ float dot2<_Float16>(uint32_t a, uint32_t b, float c) {
  typedef __attribute__((ext_vector_type(2))) _Float16 h2;
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}
template <typename T>
__device__ __forceinline__ float lo16(uint32_t w);
template <>
__device__ __forceinline__ float lo16<__bf16>(uint32_t w) {
  return __builtin_bit_cast(float, w << 16);
}
template <>
__device__ __forceinline__ float lo16<_Float16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <typename T>
__device__ __forceinline__ float hi16(uint32_t w);
template <>
__device__ __forceinline__ float hi16<__bf16>(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}
template <>
__device__ __forceinline__ float hi16<_Float16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// grid = BH * S workgroups: workgroup (bh, s) takes keys [s*chunk, (s+1)*chunk)
// of head bh (chunk a multiple of 64; a range past Nk is empty).  With
// partial (S splits, or the float32 partial-result entry point) it writes
// Ow[(s*BH + bh)*D ..] (normalised) and Lw[s*BH + bh]; otherwise O (type T)
// and L of row bh.  An empty range gives O = 0 and L = -inf.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads, 1)
fa2_decode_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                  const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                  float* __restrict__ Lg, float* __restrict__ Ow, float* __restrict__ Lw, int Nk,
                  int BH, int S, int chunk, int partial, float scale) {
  using C = DecCfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[C::kBuf * 2 * C::kBlockBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = blockIdx.x / S, s = blockIdx.x - bh * S;
  const int k_beg = s * chunk;
  const int k_end = min(Nk, k_beg + chunk);
  const int nblk = k_end > k_beg ? (k_end - k_beg + kKeys - 1) / kKeys : 0;
  const uint16_t* Kh = Kg + (size_t)bh * Nk * D;
  const uint16_t* Vh = Vg + (size_t)bh * Nk * D;

  // Stage block b (keys k_beg + 64b ..) into ring slot b % kBuf: load i of this
  // wavefront fills 1 KB chunk n = wave*kLoads + i of K (and of V), rows
  // kRowsPerLoad*n + lane / kLanesPerRow, bytes 16 * (lane % kLanesPerRow);
  // rows past Nk are clamped to row Nk - 1 (their keys are masked).
  auto issue = [&](int b) __attribute__((always_inline)) {
    const int r0 = k_beg + b * kKeys;
    char* kb = smem + (b % C::kBuf) * 2 * C::kBlockBytes;
    const int tl = fresh_lane();
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int n = wave * C::kLoads + i;
      const int r = min(r0 + C::kRowsPerLoad * n + tl / C::kLanesPerRow, Nk - 1);
      const size_t off = (size_t)r * D + 8 * (tl % C::kLanesPerRow);
      lds_dma(Kh + off, lds_addr(kb + n * 1024));
      lds_dma(Vh + off, lds_addr(kb + C::kBlockBytes + n * 1024));
    }
  };
  constexpr int kPerBlock = 2 * C::kLoads;  // direct loads per wavefront per block

  // This lane's quarter of q (q.k layout: key 16*wave + lane/4, quarter lane%4).
  const int kq = lane >> 2, qq = lane & 3;
  uint32_t qv[C::kQuarter / 2];
  {
    const uint32_t* qp = (const uint32_t*)(Qg + (size_t)bh * D + qq * C::kQuarter);
#pragma unroll
    for (int i = 0; i < C::kQuarter / 2; ++i) qv[i] = qp[i];
  }
  // Wait for q here, before any block is staged, and hand the registers through
  // an empty asm statement: the compiler then puts no wait of its own inside the
  // loop, where it would also wait for the staged blocks it cannot see.
  wait_vmcnt<0>();
#pragma unroll
  for (int i = 0; i < C::kQuarter / 2; ++i) asm volatile("" : "+v"(qv[i]));
  for (int b = 0; b < C::kBuf - 1 && b < nblk; ++b) issue(b);

  float m_run = -__builtin_inff();  // running maximum of the scaled logits
  float l_lane = 0.f;               // this lane's share of the running sum
  float acc[C::kDimsPerLane];       // dims lane*kDimsPerLane .. of the weighted V sum
#pragma unroll
  for (int e = 0; e < C::kDimsPerLane; ++e) acc[e] = 0.f;

  for (int b = 0; b < nblk; ++b) {
    // Block b has landed once at most min(kBuf - 2, nblk - 1 - b) later blocks
    // are still in flight (vector memory operations complete in issue order).
    switch (min(C::kBuf - 2, nblk - 1 - b)) {
      case 6: wait_vmcnt<(6 * kPerBlock < 63 ? 6 * kPerBlock : 63)>(); break;
      case 5: wait_vmcnt<(5 * kPerBlock < 63 ? 5 * kPerBlock : 63)>(); break;
      case 4: wait_vmcnt<(4 * kPerBlock < 63 ? 4 * kPerBlock : 63)>(); break;
      case 3: wait_vmcnt<(3 * kPerBlock < 63 ? 3 * kPerBlock : 63)>(); break;
      case 2: wait_vmcnt<(2 * kPerBlock < 63 ? 2 * kPerBlock : 63)>(); break;
      case 1: wait_vmcnt<kPerBlock>(); break;
      default: wait_vmcnt<0>();
    }
    lds_barrier();
    // Every wavefront is done with block b - 1: its slot takes block b + kBuf - 1.
    if (b + C::kBuf - 1 < nblk) issue(b + C::kBuf - 1);
    const char* kb = smem + (b % C::kBuf) * 2 * C::kBlockBytes;
    const char* vb = kb + C::kBlockBytes;

    // q.k for key 16*wave + kq, this lane's quarter; the 16-byte pieces are read
    // in an order rotated by the key, so the 16 lanes of a read pass reach
    // different banks.
    const int key = 16 * wave + kq;
    const char* krow = kb + key * (D * 2) + qq * (C::kQuarter * 2);
    float sdot = 0.f;
#pragma unroll
    for (int p = 0; p < C::kPieces; ++p) {
      const int pp = p ^ (kq % C::kPieces);
      const u32x4_t kv = *(const u32x4_t*)(krow + 16 * pp);
#pragma unroll
      for (int w = 0; w < 4; ++w) sdot = dot2<T>(kv[w], qv[pp * 4 + w], sdot);
    }
    sdot += __shfl_xor(sdot, 1, 64);
    sdot += __shfl_xor(sdot, 2, 64);
    const int kidx = k_beg + b * kKeys + key;
    const float t = kidx < k_end ? sdot * scale : -__builtin_inff();
    float mb = t;
#pragma unroll
    for (int x = 4; x < 64; x *= 2) mb = fmaxf(mb, __shfl_xor(mb, x, 64));
    const float m_new = fmaxf(m_run, mb);
    // Nothing seen yet (m_new = -inf): weights 0, nothing to rescale.
    const float ref = m_new == -__builtin_inff() ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - ref) * kLog2e);
    const float p = __builtin_amdgcn_exp2f((t - ref) * kLog2e);
    m_run = m_new;
    l_lane = l_lane * alpha + (qq == 0 ? p : 0.f);
#pragma unroll
    for (int e = 0; e < C::kDimsPerLane; ++e) acc[e] *= alpha;

    // Weighted V rows: lanes hold dims now; key k's weight sits in lane 4k.
    const char* vrow = vb + (16 * wave) * (D * 2) + lane * (C::kDimsPerLane * 2);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float pk =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), 4 * k));
      if constexpr (C::kDimsPerLane == 1) {
        const uint32_t w = *(const uint16_t*)(vrow + k * (D * 2));
        acc[0] = __builtin_fmaf(pk, lo16<T>(w), acc[0]);
      } else if constexpr (C::kDimsPerLane == 2) {
        const uint32_t w = *(const uint32_t*)(vrow + k * (D * 2));
        acc[0] = __builtin_fmaf(pk, lo16<T>(w), acc[0]);
        acc[1] = __builtin_fmaf(pk, hi16<T>(w), acc[1]);
      } else {
        const u32x2_t w = *(const u32x2_t*)(vrow + k * (D * 2));
        acc[0] = __builtin_fmaf(pk, lo16<T>(w[0]), acc[0]);
        acc[1] = __builtin_fmaf(pk, hi16<T>(w[0]), acc[1]);
        acc[2] = __builtin_fmaf(pk, lo16<T>(w[1]), acc[2]);
        acc[3] = __builtin_fmaf(pk, hi16<T>(w[1]), acc[3]);
      }
    }
  }

  // Merge the 4 wavefronts' (maximum, sum, accumulators) through LDS.
  float l_w = l_lane;
#pragma unroll
  for (int x = 1; x < 64; x *= 2) l_w += __shfl_xor(l_w, x, 64);
  __syncthreads();  // every wavefront is done with the staged blocks
  float* sm = (float*)smem;  // [4] maxima, [4] sums, then [4][D] accumulators
  if (lane == 0) {
    sm[wave] = m_run;
    sm[4 + wave] = l_w;
  }
#pragma unroll
  for (int e = 0; e < C::kDimsPerLane; ++e) sm[8 + wave * D + lane * C::kDimsPerLane + e] = acc[e];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < D) {
    float m = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < 4; ++w) m = fmaxf(m, sm[w]);
    const float ref = m == -__builtin_inff() ? 0.f : m;
    float tot = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f((sm[w] - ref) * kLog2e);
      tot += f * sm[4 + w];
      o += f * sm[8 + w * D + t];
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    const float lse = tot > 0.f ? __builtin_fmaf(__builtin_amdgcn_logf(tot), kLn2, m)
                                : -__builtin_inff();
    if (partial) {
      Ow[((size_t)s * BH + bh) * D + t] = o * inv;
      if (t == 0) Lw[(size_t)s * BH + bh] = lse;
    } else {
      Og[(size_t)bh * D + t] = __builtin_bit_cast(uint16_t, (T)(o * inv));
      if (t == 0) Lg[bh] = lse;
    }
  }
}

template <typename T, int D>
hipError_t launch(const FwdArgs& a) {
  const int S = a.num_splits > 0 ? a.num_splits : 1;
  // Keys per split, a whole number of 64-key blocks.
  const int per = (a.Nk + S - 1) / S;
  const int chunk = (per + kKeys - 1) / kKeys * kKeys;
  hipLaunchKernelGGL((fa2_decode_kernel<T, D>), dim3(a.BH * S), dim3(kThreads), 0, a.stream,
                     (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                     (uint16_t*)a.O, a.L, a.ws_O, a.ws_L, a.Nk, a.BH, S, chunk,
                     a.num_splits > 0 ? 1 : 0, a.scale);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const FwdArgs& a) {
  switch (a.d) {
    case 64: return launch<T, 64>(a);
    case 128: return launch<T, 128>(a);
    case 256: return launch<T, 256>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_supported(int d, int elem) {
  return (d == 64 || d == 128 || d == 256) && (elem == kBF16 || elem == kFP16);
}

hipError_t launch_decode(const FwdArgs& a) {
  return a.elem == kFP16 ? dispatch<_Float16>(a) : dispatch<__bf16>(a);
}

}  // namespace fa2
