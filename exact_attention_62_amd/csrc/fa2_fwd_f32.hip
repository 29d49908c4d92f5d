// FlashAttention-2 forward pass in float32 ("exact mode") for gfx950.
//
// Same algorithm as the bf16 kernel (Q block outer, K/V blocks inner, online
// row max and row sum, one division by l after the loop, L = m + ln(l),
// causally masked K/V blocks skipped: pages "FlashAttention学习笔记(2)" and
// "Flash Attention V2原理解读", forward sections; "flash-attention123和
// ring-attention", 优化1-优化3), but every step stays in float32 so that the
// result agrees with exact attention to about 1e-6.  gfx950 has no reduced-
// precision fp32 matrix path to fall into, and this mode is meant for small
// problems, so it runs on the vector ALUs: each wavefront owns one query row
// (its Q block), each lane one key of the current 64-key block, and the lanes
// share the output row's head dimension for the P~ V_j update.  Q has Nq rows
// and K, V Nk; the causal mask is aligned bottom-right (key j hidden from query
// i when j > i + Nk - Nq), and a query that sees no key gets O = 0, L = -inf.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "fa2_internal.h"

namespace fa2 {
namespace {

constexpr int kWaves = kBlockM_f32;  // one query row per wavefront
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;              // keys per K/V block: one per lane

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads)
fa2_fwd_f32_kernel(const float* __restrict__ Qg, const float* __restrict__ Kg,
                   const float* __restrict__ Vg, float* __restrict__ Og, float* __restrict__ Lg,
                   int Nq, int Nk, int num_m_block, float scale) {
  constexpr int R = (D + 63) / 64;  // output dims per lane (dims lane + 64 r < D)
  __shared__ float qs[kWaves][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int bh = blockIdx.x / num_m_block;
  const int m = blockIdx.x - bh * num_m_block;
  const int q = m * kWaves + wave;  // this wavefront's query row

  const size_t qslice = (size_t)bh * (size_t)Nq * D;
  const size_t kslice = (size_t)bh * (size_t)Nk * D;
  const float* Kh = Kg + kslice;
  const float* Vh = Vg + kslice;

  for (int t = lane; t < D; t += 64) qs[wave][t] = q < Nq ? Qg[qslice + (size_t)q * D + t] : 0.f;
  __syncthreads();
  if (q >= Nq) return;

  float o[R];
#pragma unroll
  for (int r = 0; r < R; ++r) o[r] = 0.f;
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  // Keys past the diagonal are never visited; with Nq > Nk the first queries
  // see none (the loop does not run: O = 0, L = -inf below).
  const int n_keys = CAUSAL ? min(Nk, q + 1 + (Nk - Nq)) : Nk;
  for (int k0 = 0; k0 < n_keys; k0 += kBN) {
    const int key = k0 + lane;
    float s = -__builtin_inff();
    if (key < n_keys) {
      const float* krow = Kh + (size_t)key * D;
      float acc = 0.f;
#pragma unroll 8
      for (int t = 0; t < D; t += 4) {
        const float4 kv = *(const float4*)(krow + t);
        acc = __builtin_fmaf(qs[wave][t + 0], kv.x, acc);
        acc = __builtin_fmaf(qs[wave][t + 1], kv.y, acc);
        acc = __builtin_fmaf(qs[wave][t + 2], kv.z, acc);
        acc = __builtin_fmaf(qs[wave][t + 3], kv.w, acc);
      }
      s = acc * scale;
    }
    const float m_new = fmaxf(m_run, wave_max(s));  // finite: key k0 is always visible
    const float alpha = expf(m_run - m_new);        // exp(-inf) = 0 on the first block
    const float p = key < n_keys ? expf(s - m_new) : 0.f;
    l_run = alpha * l_run + wave_sum(p);
    m_run = m_new;
#pragma unroll
    for (int r = 0; r < R; ++r) o[r] *= alpha;
    const int nk = min(kBN, n_keys - k0);
    for (int kk = 0; kk < nk; ++kk) {
      const float pk = __shfl(p, kk, 64);
      const float* vrow = Vh + (size_t)(k0 + kk) * D;
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane + 64 * r < D) o[r] = __builtin_fmaf(pk, vrow[lane + 64 * r], o[r]);
    }
  }

  float* orow = Og + qslice + (size_t)q * D;
  const bool seen = n_keys > 0;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (lane + 64 * r < D) orow[lane + 64 * r] = seen ? o[r] / l_run : 0.f;
  if (lane == 0) Lg[(size_t)bh * Nq + q] = seen ? m_run + logf(l_run) : -__builtin_inff();
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  const int total = a.num_m_block * a.BH;
  hipLaunchKernelGGL((fa2_fwd_f32_kernel<D, CAUSAL>), dim3(total), dim3(kThreads), 0, a.stream,
                     (const float*)a.Q, (const float*)a.K, (const float*)a.V, (float*)a.O, a.L,
                     a.Nq, a.Nk, a.num_m_block, a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
  switch (a.d * 2 + a.causal) {
    case 32 * 2 + 0: return launch<32, false>(a);
    case 32 * 2 + 1: return launch<32, true>(a);
    case 96 * 2 + 0: return launch<96, false>(a);
    case 96 * 2 + 1: return launch<96, true>(a);
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
