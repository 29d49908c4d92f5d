// Internal interface between the host API (fa2_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa2 {

// Query rows per workgroup (the pages' kBlockM).  16-bit types (bf16, fp16):
// four wavefronts of 32 rows each, two workgroups per CU; for d = 128 without
// splits, on a grid of at least kWideMinItems items of 256 rows, eight
// wavefronts (one workgroup per CU, both wavefronts of a SIMD in the same
// workgroup).  fp32 exact mode: four wavefronts of one row each.
constexpr int kBlockM_mfma = 128;
constexpr int kBlockM_wide = 256;
constexpr int64_t kWideMinItems = 256;
constexpr int64_t fwd_block_m(int64_t d, int64_t BH, int64_t Nq) {
  return d == 128 && BH * ((Nq + kBlockM_wide - 1) / kBlockM_wide) >= kWideMinItems
             ? kBlockM_wide
             : kBlockM_mfma;
}
constexpr int kBlockM_f32 = 4;
// Keys per K/V block of the 16-bit kernel, and the wavefronts per SIMD of its
// split form (with four-wavefront workgroups, the workgroups that stay
// resident on one CU).  Without splits, d = 256 runs two wavefronts per SIMD
// on grids of at least two items per CU (see dispatch_fwd_mfma).
constexpr int mfma_block_n(int d) { return d == 256 ? 32 : 64; }
constexpr int mfma_waves_per_simd(int d) { return d == 256 ? 1 : d == 32 ? 3 : 2; }

// Element types, with the values of fa2_dtype_t.
enum Elem { kBF16 = 0, kFP32 = 1, kFP16 = 2 };

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* L;
  int BH;           // B * H, the number of (batch, head) slices
  int Nq;           // query rows per slice (Q, O, L)
  int Nk;           // key rows per slice (K, V)
  int d;            // head dimension
  int causal;       // 0 or 1; aligned bottom-right when Nq != Nk
  float scale;      // softmax scale
  int block_m = kBlockM_mfma;  // query rows per work item (kBlockM)
  int num_m_block;  // ceil(Nq / kBlockM)
  int elem;         // Elem of Q, K, V and O
  hipStream_t stream;
  // Split-KV (16-bit types only): num_splits > 0 writes partial results to
  // ws_O [num_splits][BH][Nq][d] and ws_L [num_splits][BH][Nq] (fp32) instead
  // of O/L.
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
  float* Dvec;  // workspace: -rowsum(dO * O), [BH][bwd_rows(Nq)], then L * log2(e), same shape
  int BH, Nq, Nk, d, causal;  // causal aligned bottom-right when Nq != Nk
  float scale;
  int elem;  // Elem of Q, K, V, O, dO and the gradients (bf16 or fp16)
  hipStream_t stream;
};

// Compute units of the current device (queried once per device).
hipError_t cu_count(int* cus);

// Size of the library-owned device scratch of fa2_fwd_splitkv_noalloc (one
// copy per device), and its device address on the current device (looked up
// once per device; fa2_scratch.hip).
constexpr int64_t kScratchBytes = int64_t(32) << 20;
hipError_t scratch_address(void** ptr);

// Enqueue the kernel; returns the launch's hipError_t.
hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_fp16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
// Merge num_splits partial results (ws_O, ws_L: [num_splits][BH*Nq] rows) into
// O (a.elem: bf16, fp16 or fp32) and L.
hipError_t launch_combine(const FwdArgs& a);
// The result when there are no keys (a.Nk == 0): O = 0 and L = -inf.
hipError_t launch_fill_no_keys(const FwdArgs& a);
// Enqueue the backward pass (three kernels) on a.stream.
hipError_t launch_bwd(const BwdArgs& a);
// One query per (batch, head): the decoding kernel (d = 64, 128, 256; bf16 or
// fp16).  Plain (num_splits == 0: O and L) or partial (num_splits splits:
// ws_O, ws_L in the split-KV layout).
bool decode_supported(int d, int elem);
hipError_t launch_decode(const FwdArgs& a);
// Rows per head of the backward workspace's two arrays: Nq rounded up to the
// dK/dV kernel's 32-query step (padded rows hold D = 0 and L * log2(e) = +inf).
constexpr int64_t bwd_rows(int64_t Nq) { return (Nq + 31) / 32 * 32; }

}  // namespace fa2
