// Internal interface between the host API (fa2_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa2 {

// Query rows per workgroup (the pages' kBlockM).  bf16: four wavefronts of 32
// rows each.  fp32 exact mode: four wavefronts of one row each.
constexpr int kBlockM_bf16 = 128;
constexpr int kBlockM_f32 = 4;
// Keys per K/V block of the bf16 kernel.
constexpr int bf16_block_n(int d) { return d == 256 ? 32 : 64; }

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
  // Split-KV (bf16 only): num_splits > 0 writes partial results to ws_O
  // [num_splits][BH][N][d] and ws_L [num_splits][BH][N] (fp32) instead of O/L.
  int num_splits = 0;
  float* ws_O = nullptr;
  float* ws_L = nullptr;
};

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* L;
  void* dQ;
  void* dK;
  void* dV;
  float* Dvec;  // workspace: rowsum(dO * O), [BH][N]
  int BH, N, d, causal;
  float scale;
  hipStream_t stream;
};

// Enqueue the kernel; returns the launch's hipError_t.
hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
// Merge num_splits partial results (ws_O, ws_L) into O (bf16) and L.
hipError_t launch_combine_bf16(const FwdArgs& a);
// Enqueue the backward pass (three kernels) on a.stream.
hipError_t launch_bwd_bf16(const BwdArgs& a);
// Workgroups of the bf16 kernel resident at once on the current device.
hipError_t bf16_resident_workgroups(int d, int* slots);

}  // namespace fa2
