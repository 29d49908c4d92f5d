// Merge of split-KV partial results into O and L, for gfx950 (MI355X).
//
// When the key/value sequence is split across work items, each row of O gets
// one part from every split, and the parts have to be combined once more to
// reach the global softmax result (page "Flash Attention V2原理解读", the
// thread-block grid section).  Split s delivers, per row, O_s (normalised
// within its keys) and L_s = m_s + ln(l_s), so exp(L_s) is its share of the
// row's softmax denominator:
//   L = ln sum_s exp(L_s)   (as Lmax + ln sum_s exp(L_s - Lmax)),
//   O = sum_s exp(L_s - L) O_s.
// A split that saw no key of the row has L_s = -inf and weight 0; split 0
// always holds key 0, which every row sees, so Lmax is finite.
//
// The merge reads num_splits * d fp32 values per row and writes d bf16 values:
// it is bound by HBM bandwidth, so it is plain coalesced vector loads.  Each
// thread owns 4 consecutive dimensions of one row (d/4 threads per row).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "fa2_internal.h"

namespace fa2 {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;

template <int D>
__global__ void __launch_bounds__(kThreads)
fa2_combine_kernel(const float* __restrict__ Ow, const float* __restrict__ Lw,
                   uint16_t* __restrict__ O, float* __restrict__ L, int rows, int num_splits) {
  constexpr int TPR = D / 4;               // threads per row
  constexpr int RPB = kThreads / TPR;      // rows per workgroup
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  if (row >= rows) return;

  float lmax = -INFINITY;
  for (int s = 0; s < num_splits; ++s) lmax = fmaxf(lmax, Lw[(size_t)s * rows + row]);
  float tot = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < num_splits; ++s) {
    const float w = __builtin_amdgcn_exp2f((Lw[(size_t)s * rows + row] - lmax) * kLog2e);
    const f32x4_t o = *(const f32x4_t*)(Ow + ((size_t)s * rows + row) * D + 4 * t);
    tot += w;
    acc += w * o;
  }
  const float inv = 1.f / tot;
  bf16x4_t out;
#pragma unroll
  for (int r = 0; r < 4; ++r) out[r] = (__bf16)(acc[r] * inv);
  *(bf16x4_t*)(O + (size_t)row * D + 4 * t) = out;
  if (t == 0) L[row] = __builtin_fmaf(__builtin_amdgcn_logf(tot), kLn2, lmax);
}

template <int D>
hipError_t launch(const FwdArgs& a) {
  constexpr int RPB = kThreads / (D / 4);
  const int rows = a.BH * a.N;
  const int grid = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((fa2_combine_kernel<D>), dim3(grid), dim3(kThreads), 0, a.stream, a.ws_O,
                     a.ws_L, (uint16_t*)a.O, a.L, rows, a.num_splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_bf16(const FwdArgs& a) {
  switch (a.d) {
    case 64: return launch<64>(a);
    case 128: return launch<128>(a);
    case 256: return launch<256>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa2
