// Internal interface between the host API (fa2_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa2 {

// Query rows per workgroup (the pages' kBlockM).  bf16: four wavefronts of 32
// rows each.  fp32 exact mode: four wavefronts of one row each.
constexpr int kBlockM_bf16 = 128;
constexpr int kBlockM_f32 = 4;

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* L;
  int BH;           // B * H, the number of (batch, head) slices
  int N;            // sequence length (queries = keys)
  int d;            // head dimension
  int causal;       // 0 or 1
  float scale;      // softmax scale
  int num_m_block;  // ceil(N / kBlockM)
  hipStream_t stream;
};

// Enqueue the kernel; returns the launch's hipError_t.
hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);

}  // namespace fa2
