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
// A split that saw no key of the row has L_s = -inf and weight 0.  A row that
// saw no key in any split (a causal query before the first key, Nq > Nk) has
// an empty sum: O = 0 and L = -inf.
//
// The merge reads num_splits * d fp32 values per row and writes d values
// (bf16, fp16, or fp32 for fa2_merge): it is bound by HBM bandwidth, so it is
// plain coalesced vector loads.  Each thread owns 4 consecutive dimensions of
// one row (d/4 threads per row).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {
namespace {

using namespace dev;

constexpr int kThreads = 256;

template <typename T, int D>
__global__ void __launch_bounds__(kThreads)
fa2_combine_kernel(const float* __restrict__ Ow, const float* __restrict__ Lw,
                   void* __restrict__ O, float* __restrict__ L, int rows, int num_splits) {
  constexpr int TPR = D / 4;               // threads per row
  constexpr int RPB = kThreads / TPR;      // rows per workgroup
  if ((int)threadIdx.x >= RPB * TPR) return;  // d = 96: 240 of the 256 threads have a row
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  if (row >= rows) return;

  float lmax = kNegInf;
  for (int s = 0; s < num_splits; ++s) lmax = fmaxf(lmax, Lw[(size_t)s * rows + row]);
  const float ref = lmax == kNegInf ? 0.f : lmax;  // every weight is 0 for an empty row
  float tot = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < num_splits; ++s) {
    const float w = __builtin_amdgcn_exp2f((Lw[(size_t)s * rows + row] - ref) * kLog2e);
    const f32x4_t o = *(const f32x4_t*)(Ow + ((size_t)s * rows + row) * D + 4 * t);
    tot += w;
    acc += w * o;
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  if constexpr (std::is_same<T, float>::value) {
    *((f32x4_t*)O + ((size_t)row * D / 4 + t)) = acc * inv;
  } else {
    typedef typename Vec16<T>::x4 t4_t;
    t4_t out;
#pragma unroll
    for (int r = 0; r < 4; ++r) out[r] = (T)(acc[r] * inv);
    *((t4_t*)O + ((size_t)row * D / 4 + t)) = out;
  }
  if (t == 0) L[row] = tot > 0.f ? __builtin_fmaf(__builtin_amdgcn_logf(tot), kLn2, lmax) : kNegInf;
}

template <typename T, int D>
hipError_t launch(const FwdArgs& a) {
  constexpr int RPB = kThreads / (D / 4);
  const int rows = a.BH * a.Nq;
  const int grid = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((fa2_combine_kernel<T, D>), dim3(grid), dim3(kThreads), 0, a.stream, a.ws_O,
                     a.ws_L, a.O, a.L, rows, a.num_splits);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const FwdArgs& a) {
  switch (a.d) {
    case 32: return launch<T, 32>(a);
    case 64: return launch<T, 64>(a);
    case 96: return launch<T, 96>(a);
    case 128: return launch<T, 128>(a);
    case 256: return launch<T, 256>(a);
  }
  return hipErrorInvalidValue;
}

// Rows with no key at all (Nk == 0): O = 0, L = -inf.  One thread per 16
// bytes of O (every row is a multiple of 64 bytes) and per row of L, in a
// grid-stride loop over 64-bit indices (B*H*Nq may exceed 2^31).
__global__ void __launch_bounds__(kThreads)
fa2_fill_no_keys_kernel(u32x4_t* __restrict__ O, float* __restrict__ L, int64_t o_chunks,
                        int64_t rows) {
  const int64_t n = o_chunks > rows ? o_chunks : rows;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    if (i < o_chunks) O[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (i < rows) L[i] = kNegInf;
  }
}

}  // namespace

hipError_t launch_fill_no_keys(const FwdArgs& a) {
  constexpr int64_t kMaxBlocks = 2048;  // the loop strides over the rest
  const int64_t rows = (int64_t)a.BH * a.Nq;
  const int64_t o_chunks = rows * a.d * (a.elem == kFP32 ? 4 : 2) / 16;
  const int64_t n = o_chunks > rows ? o_chunks : rows;
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  hipLaunchKernelGGL(fa2_fill_no_keys_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                     (u32x4_t*)a.O, a.L, o_chunks, rows);
  return hipGetLastError();
}

hipError_t launch_combine(const FwdArgs& a) {
  if (a.elem == kBF16) return dispatch<__bf16>(a);
  if (a.elem == kFP16) return dispatch<_Float16>(a);
  if (a.elem == kFP32) return dispatch<float>(a);
  return hipErrorInvalidValue;
}

}  // namespace fa2
