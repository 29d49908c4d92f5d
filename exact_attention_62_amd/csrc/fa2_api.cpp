// Host side of libfa2.so: argument validation, error reporting, the work
// decomposition and kernel dispatch for the FlashAttention-2 forward pass.
//
// Validation order: pure argument checks first (no HIP call at all), then the
// device and each pointer's allocation are checked through the HIP runtime,
// then the kernel is enqueued and the launch status is read back.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fa2.h"
#include "fa2_internal.h"
#include "fa2_schedule.h"

namespace {

thread_local char g_last_error[512] = "";

fa2_status_t fail(fa2_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

fa2_status_t fail_hip(hipError_t e, const char* what) {
  return fail(FA2_EHIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

int64_t elem_size(fa2_dtype_t t) { return t == FA2_FP32 ? 4 : 2; }

constexpr int64_t kMaxLen = (int64_t(1) << 31) / 256;  // per-slice offsets are 32-bit in the kernels
static_assert(fa2::kScratchBytes == (int64_t)FA2_NOALLOC_SCRATCH_BYTES, "scratch size in fa2.h");

// Checks that need no HIP call, for Nq queries over Nk keys.  On success
// fills the query block size.
fa2_status_t check_shape(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                         fa2_dtype_t dtype, int64_t* kBlockM) {
  if (dtype != FA2_BF16 && dtype != FA2_FP32 && dtype != FA2_FP16)
    return fail(FA2_ENOTSUP, "dtype %d is not FA2_BF16 (0), FA2_FP32 (1) or FA2_FP16 (2)",
                (int)dtype);
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
    return fail(FA2_EINVAL, "sizes must be >= 0 (B=%lld H=%lld Nq=%lld Nk=%lld)", (long long)B,
                (long long)H, (long long)Nq, (long long)Nk);
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256)
    return fail(FA2_ENOTSUP, "head dimension d=%lld is not one of 32, 64, 96, 128, 256",
                (long long)d);
  if (Nq > kMaxLen || Nk > kMaxLen)
    return fail(FA2_EINVAL, "sequence length %lld exceeds the supported maximum %lld",
                (long long)(Nq > Nk ? Nq : Nk), (long long)kMaxLen);
  if (B > 0 && H > (int64_t(1) << 31) / B)
    return fail(FA2_EINVAL, "B*H=%lld*%lld exceeds 2^31", (long long)B, (long long)H);
  const int64_t bm = dtype == FA2_FP32 ? fa2::kBlockM_f32 : fa2::fwd_block_m(d, B * H, Nq);
  const int64_t nmb = (Nq + bm - 1) / bm;
  if (B * H > 0 && nmb > ((int64_t(1) << 31) - 1) / (B * H))
    return fail(FA2_EINVAL, "grid of %lld x %lld workgroups exceeds 2^31 - 1", (long long)nmb,
                (long long)(B * H));
  *kBlockM = bm;
  return FA2_OK;
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

// The allocation holding [p, p + bytes) must be device memory of the current device.
fa2_status_t check_device_range(const void* p, int64_t bytes, const char* name) {
  void* base = nullptr;
  size_t size = 0;
  hipError_t e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
  if (e != hipSuccess || base == nullptr) {
    (void)hipGetLastError();
    return fail(FA2_EINVAL, "%s=%p is not a device allocation (%s)", name, p, hipGetErrorName(e));
  }
  const char* b = static_cast<const char*>(base);
  const char* q = static_cast<const char*>(p);
  if (q < b || q + bytes > b + size)
    return fail(FA2_EINVAL, "%s needs %lld bytes but its allocation ends %lld bytes after it",
                name, (long long)bytes, (long long)(b + size - q));
  return FA2_OK;
}

}  // namespace

namespace fa2 {

hipError_t cu_count(int* cus) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && (*cus = cache[dev].load(std::memory_order_relaxed)) > 0)
    return hipSuccess;
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (*cus < 1) *cus = 1;
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(*cus, std::memory_order_relaxed);
  return hipSuccess;
}

}  // namespace fa2

extern "C" {

const char* fa2_strerror(fa2_status_t s) {
  switch (s) {
    case FA2_OK: return "success";
    case FA2_EINVAL: return "invalid argument";
    case FA2_ENOTSUP: return "not supported by this build";
    case FA2_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* fa2_last_error(void) { return g_last_error; }

fa2_status_t fa2_launch_shape(int64_t B, int64_t H, int64_t N, int64_t d, fa2_dtype_t dtype,
                              int64_t* kBlockM, int64_t* num_m_block, int64_t* items) {
  g_last_error[0] = '\0';
  int64_t bm = 0;
  fa2_status_t s = check_shape(B, H, N, N, d, dtype, &bm);
  if (s != FA2_OK) return s;
  const int64_t nmb = (N + bm - 1) / bm;
  if (kBlockM) *kBlockM = bm;
  if (num_m_block) *num_m_block = nmb;
  if (items) *items = nmb * B * H;
  return FA2_OK;
}

}  // extern "C"

namespace {

// Pointer checks shared by the forward entry points: non-NULL, aligned, outputs
// disjoint from everything else (extra[i] are further buffers, e.g. a
// workspace, treated as outputs), then device residency of every range.  K and
// V are not read when Nk == 0 and are not checked then.  Fills the launch
// arguments.  Returns FA2_OK with a.BH == 0 for an empty problem (nothing to
// launch).
fa2_status_t prepare(const void* Q, const void* K, const void* V, void* O, float* L, int64_t B,
                     int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                     fa2_dtype_t dtype, void* stream, const void* ws, int64_t ws_bytes,
                     fa2::FwdArgs* a, int64_t o_elem_size = 0) {
  int64_t bm = 0;
  fa2_status_t s = check_shape(B, H, Nq, Nk, d, dtype, &bm);
  if (s != FA2_OK) return s;
  if (causal != 0 && causal != 1) return fail(FA2_EINVAL, "causal=%d must be 0 or 1", causal);
  if (!std::isfinite(scale)) return fail(FA2_EINVAL, "scale must be finite");
  a->BH = 0;
  if (B * H * Nq == 0) return FA2_OK;  // empty problem: nothing to write

  const int64_t q_bytes = B * H * Nq * d * elem_size(dtype);
  const int64_t k_bytes = B * H * Nk * d * elem_size(dtype);
  const int64_t o_bytes = B * H * Nq * d * (o_elem_size ? o_elem_size : elem_size(dtype));
  const int64_t l_bytes = B * H * Nq * 4;
  const void* ptrs[6] = {Q, K, V, O, L, ws};
  const int64_t sizes[6] = {q_bytes, k_bytes, k_bytes, o_bytes, l_bytes, ws_bytes};
  const char* names[6] = {"Q", "K", "V", "O", "L", "workspace"};
  bool used[6] = {true, Nk > 0, Nk > 0, true, true, ws != nullptr};
  for (int i = 0; i < 6; ++i) {
    if (!used[i]) continue;
    if (ptrs[i] == nullptr) return fail(FA2_EINVAL, "%s is NULL", names[i]);
    const uintptr_t align = i == 4 ? 4 : 16;
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % align != 0)
      return fail(FA2_EINVAL, "%s=%p is not %d-byte aligned", names[i], ptrs[i], (int)align);
  }
  for (int o = 3; o < 6; ++o)
    for (int i = 0; i < 6; ++i)
      if (used[o] && used[i] && i != o && overlaps(ptrs[o], sizes[o], ptrs[i], sizes[i]))
        return fail(FA2_EINVAL, "%s overlaps %s", names[o], names[i]);

  // From here on the HIP runtime is involved.
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail_hip(e, "hipGetDevice");
  }
  for (int i = 0; i < 6; ++i) {
    if (!used[i]) continue;
    s = check_device_range(ptrs[i], sizes[i], names[i]);
    if (s != FA2_OK) return s;
  }
  a->Q = Q;
  a->K = K;
  a->V = V;
  a->O = O;
  a->L = L;
  a->BH = static_cast<int>(B * H);
  a->Nq = static_cast<int>(Nq);
  a->Nk = static_cast<int>(Nk);
  a->d = static_cast<int>(d);
  a->causal = causal;
  a->scale = scale;
  a->block_m = static_cast<int>(bm);
  a->num_m_block = static_cast<int>((Nq + bm - 1) / bm);
  a->elem = static_cast<int>(dtype);
  a->stream = static_cast<hipStream_t>(stream);
  return FA2_OK;
}

hipError_t launch_fwd(const fa2::FwdArgs& a) {
  if (a.Nk == 0) return fa2::launch_fill_no_keys(a);  // every row's sum is empty
  // One query row per head (decoding): the row sees every key, and the pass is
  // bound by HBM; it has a kernel of its own.
  if (a.Nq == 1 && fa2::decode_supported(a.d, a.elem)) return fa2::launch_decode(a);
  switch (a.elem) {
    case fa2::kBF16: return fa2::launch_fwd_bf16(a);
    case fa2::kFP16: return fa2::launch_fwd_fp16(a);
    case fa2::kFP32: return fa2::launch_fwd_f32(a);
  }
  return hipErrorInvalidValue;
}

// The pages' rule (page "Flash Attention V2原理解读", the thread-block grid
// section): for each candidate number of splits compute the utilisation of
// the GPU, take the highest, and choose the smallest candidate reaching 0.95
// of it.  Utilisation of n work units on `slots` concurrent workgroups: the
// busy fraction of the last round, (n / slots) / ceil(n / slots).
int choose_num_splits(int64_t items, int64_t slots, int64_t max_splits) {
  if (max_splits < 1) max_splits = 1;
  double best = 0.0;
  for (int64_t s = 1; s <= max_splits; ++s) {
    const double rounds = double(items * s) / double(slots);
    best = std::fmax(best, rounds / std::ceil(rounds));
  }
  for (int64_t s = 1; s <= max_splits; ++s) {
    const double rounds = double(items * s) / double(slots);
    if (rounds / std::ceil(rounds) >= 0.95 * best) return static_cast<int>(s);
  }
  return 1;
}

int64_t splitkv_bytes(int64_t B, int64_t H, int64_t Nq, int64_t d, int64_t splits) {
  return splits * B * H * Nq * (d + 1) * 4;  // O_s [splits][B*H][Nq][d], L_s [splits][B*H][Nq]
}

fa2_status_t check_splits(int64_t B, int64_t H, int64_t Nq, int num_splits) {
  if (num_splits < 1 || num_splits > FA2_MAX_SPLITS)
    return fail(FA2_EINVAL, "num_splits=%d is not in 1..%d", num_splits, FA2_MAX_SPLITS);
  const int64_t nmb = (Nq + fa2::kBlockM_mfma - 1) / fa2::kBlockM_mfma;
  if (B * H * Nq > 0 && (nmb * num_splits > ((int64_t(1) << 31) - 1) / (B * H) ||
                         Nq * num_splits > ((int64_t(1) << 31) - 1) / (B * H)))
    return fail(FA2_EINVAL, "B*H=%lld with Nq=%lld and %d splits exceeds 2^31 - 1 items or rows",
                (long long)(B * H), (long long)Nq, num_splits);
  return FA2_OK;
}

fa2_status_t heuristic_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                              int* num_splits) {
  int cus = 0;
  const hipError_t e = fa2::cu_count(&cus);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail_hip(e, "device query");
  }
  // Workgroups of the 16-bit kernel resident at once: kWavesPerSimd per CU.
  const int64_t slots = int64_t(cus) * fa2::mfma_waves_per_simd(static_cast<int>(d));
  const int64_t bn = fa2::mfma_block_n(static_cast<int>(d));
  const int64_t nmb = (Nq + fa2::kBlockM_mfma - 1) / fa2::kBlockM_mfma;
  const int64_t kv_blocks = (Nk + bn - 1) / bn;
  const int64_t max_splits = kv_blocks < FA2_MAX_SPLITS ? kv_blocks : FA2_MAX_SPLITS;
  *num_splits = choose_num_splits(nmb * B * H, slots, max_splits);
  return FA2_OK;
}

// The split kernel always runs four wavefronts (kBlockM_mfma query rows) per
// workgroup: it exists for grids too small to fill the chip.
void use_split_blocks(fa2::FwdArgs* a) {
  a->block_m = fa2::kBlockM_mfma;
  a->num_m_block = (a->Nq + fa2::kBlockM_mfma - 1) / fa2::kBlockM_mfma;
}

fa2_status_t fwd_common(const void* Q, const void* K, const void* V, void* O, float* L,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                        float scale, fa2_dtype_t dtype, void* stream) {
  fa2::FwdArgs a;
  fa2_status_t s =
      prepare(Q, K, V, O, L, B, H, Nq, Nk, d, causal, scale, dtype, stream, nullptr, 0, &a);
  if (s != FA2_OK || a.BH == 0) return s;
  (void)hipGetLastError();  // clear a stale error so the status below is this launch's
  hipError_t e = launch_fwd(a);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  return FA2_OK;
}

// fa2_fwd_splitkv with the partial results in the caller's workspace, or
// (library_scratch) in the library's own device scratch, whose size bounds
// the problem.  Neither path allocates device memory.
fa2_status_t splitkv_common(const void* Q, const void* K, const void* V, void* O, float* L,
                            int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                            float scale, fa2_dtype_t dtype, int num_splits, void* workspace,
                            size_t workspace_bytes, void* stream, bool library_scratch) {
  if (dtype == FA2_FP32)
    return fail(FA2_ENOTSUP, "split-KV is implemented for FA2_BF16 and FA2_FP16 only");
  int64_t bm = 0;
  fa2_status_t s = check_shape(B, H, Nq, Nk, d, dtype, &bm);
  if (s != FA2_OK) return s;
  if (num_splits < 0) return fail(FA2_EINVAL, "num_splits=%d must be >= 0", num_splits);
  if (B * H * Nq == 0) return FA2_OK;
  if (num_splits == 0) {
    s = heuristic_splits(B, H, Nq, Nk, d, &num_splits);
    if (s != FA2_OK) return s;
  }
  s = check_splits(B, H, Nq, num_splits);
  if (s != FA2_OK) return s;
  const int64_t need = splitkv_bytes(B, H, Nq, d, num_splits);
  if (library_scratch) {
    if (need > fa2::kScratchBytes)
      return fail(FA2_EINVAL,
                  "the partial results need %lld bytes (num_splits * B*H*Nq * (d + 1) * 4), "
                  "more than the library scratch of %lld bytes",
                  (long long)need, (long long)fa2::kScratchBytes);
  } else {
    if (workspace == nullptr) return fail(FA2_EINVAL, "workspace is NULL");
    if (static_cast<int64_t>(workspace_bytes) < need)
      return fail(FA2_EINVAL, "workspace of %llu bytes is smaller than the %lld bytes needed",
                  (unsigned long long)workspace_bytes, (long long)need);
  }
  fa2::FwdArgs a;
  s = prepare(Q, K, V, O, L, B, H, Nq, Nk, d, causal, scale, dtype, stream,
              library_scratch ? nullptr : workspace, library_scratch ? 0 : need, &a);
  if (s != FA2_OK) return s;
  if (library_scratch) {
    // The library's array on this device (its address looked up once per device).
    hipError_t e = fa2::scratch_address(&workspace);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail_hip(e, "scratch address lookup");
    }
  }
  a.num_splits = num_splits;
  use_split_blocks(&a);
  a.ws_O = static_cast<float*>(workspace);
  a.ws_L = a.ws_O + static_cast<size_t>(num_splits) * B * H * Nq * d;
  (void)hipGetLastError();
  hipError_t e = launch_fwd(a);
  if (e == hipSuccess && a.Nk > 0) e = fa2::launch_combine(a);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  return FA2_OK;
}

}  // namespace

extern "C" {

fa2_status_t fa2_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int64_t B,
                     int64_t H, int64_t N, int64_t d, int causal, float scale, fa2_dtype_t dtype,
                     void* stream) {
  g_last_error[0] = '\0';
  return fwd_common(Q, K, V, O, L, B, H, N, N, d, causal, scale, dtype, stream);
}

fa2_status_t fa2_fwd_cross(const void* Q, const void* K, const void* V, void* O, float* L,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                           float scale, fa2_dtype_t dtype, void* stream) {
  g_last_error[0] = '\0';
  return fwd_common(Q, K, V, O, L, B, H, Nq, Nk, d, causal, scale, dtype, stream);
}

fa2_status_t fa2_splitkv_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                        int num_splits, size_t* bytes) {
  g_last_error[0] = '\0';
  int64_t bm = 0;
  fa2_status_t s = check_shape(B, H, Nq, Nk, d, FA2_BF16, &bm);
  if (s != FA2_OK) return s;
  s = check_splits(B, H, Nq, num_splits);
  if (s != FA2_OK) return s;
  if (!bytes) return fail(FA2_EINVAL, "bytes is NULL");
  *bytes = static_cast<size_t>(splitkv_bytes(B, H, Nq, d, num_splits));
  return FA2_OK;
}

fa2_status_t fa2_num_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                            int* num_splits) {
  g_last_error[0] = '\0';
  int64_t bm = 0;
  fa2_status_t s = check_shape(B, H, Nq, Nk, d, FA2_BF16, &bm);
  if (s != FA2_OK) return s;
  if (!num_splits) return fail(FA2_EINVAL, "num_splits is NULL");
  return heuristic_splits(B, H, Nq, Nk, d, num_splits);
}

fa2_status_t fa2_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* L,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                             float scale, fa2_dtype_t dtype, int num_splits, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  return splitkv_common(Q, K, V, O, L, B, H, Nq, Nk, d, causal, scale, dtype, num_splits,
                        workspace, workspace_bytes, stream, /*library_scratch=*/false);
}

fa2_status_t fa2_fwd_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O,
                                     float* L, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                     int64_t d, int causal, float scale, fa2_dtype_t dtype,
                                     int num_splits, void* stream) {
  g_last_error[0] = '\0';
  return splitkv_common(Q, K, V, O, L, B, H, Nq, Nk, d, causal, scale, dtype, num_splits,
                        nullptr, 0, stream, /*library_scratch=*/true);
}

fa2_status_t fa2_fwd_partial(const void* Q, const void* K, const void* V, float* O_part,
                             float* L_part, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                             int64_t d, int causal, float scale, fa2_dtype_t dtype, void* stream) {
  g_last_error[0] = '\0';
  if (dtype == FA2_FP32)
    return fail(FA2_ENOTSUP, "partial results are implemented for FA2_BF16 and FA2_FP16 only");
  fa2::FwdArgs a;
  fa2_status_t s = prepare(Q, K, V, O_part, L_part, B, H, Nq, Nk, d, causal, scale, dtype, stream,
                           nullptr, 0, &a, /*o_elem_size=*/4);
  if (s != FA2_OK || a.BH == 0) return s;
  (void)hipGetLastError();
  hipError_t e;
  if (Nk == 0) {  // no key: O_part = 0, L_part = -inf, written as float32
    a.elem = fa2::kFP32;
    e = fa2::launch_fill_no_keys(a);
  } else {
    // The split kernel with one split writes exactly the float32 partial result.
    a.num_splits = 1;
    use_split_blocks(&a);
    a.ws_O = O_part;
    a.ws_L = L_part;
    e = launch_fwd(a);
  }
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  return FA2_OK;
}

fa2_status_t fa2_merge(const float* O_parts, const float* L_parts, int num_parts, void* O,
                       float* L, int64_t rows, int64_t d, fa2_dtype_t dtype, void* stream) {
  g_last_error[0] = '\0';
  if (dtype != FA2_BF16 && dtype != FA2_FP32 && dtype != FA2_FP16)
    return fail(FA2_ENOTSUP, "dtype %d is not FA2_BF16 (0), FA2_FP32 (1) or FA2_FP16 (2)",
                (int)dtype);
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256)
    return fail(FA2_ENOTSUP, "head dimension d=%lld is not one of 32, 64, 96, 128, 256",
                (long long)d);
  if (rows < 0) return fail(FA2_EINVAL, "rows=%lld must be >= 0", (long long)rows);
  if (num_parts < 1 || num_parts > FA2_MAX_SPLITS)
    return fail(FA2_EINVAL, "num_parts=%d is not in 1..%d", num_parts, FA2_MAX_SPLITS);
  if (rows > ((int64_t(1) << 31) - 1) / num_parts)
    return fail(FA2_EINVAL, "rows=%lld with %d parts exceeds 2^31 - 1 rows", (long long)rows,
                num_parts);
  if (rows == 0) return FA2_OK;
  const int64_t op = int64_t(num_parts) * rows * d * 4, lp = int64_t(num_parts) * rows * 4;
  const int64_t ob = rows * d * elem_size(dtype), lb = rows * 4;
  constexpr int n = 4;
  const void* ptrs[n] = {O_parts, L_parts, O, L};
  const int64_t sizes[n] = {op, lp, ob, lb};
  const char* names[n] = {"O_parts", "L_parts", "O", "L"};
  for (int i = 0; i < n; ++i) {
    if (ptrs[i] == nullptr) return fail(FA2_EINVAL, "%s is NULL", names[i]);
    const uintptr_t align = (i == 1 || i == 3) ? 4 : 16;
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % align != 0)
      return fail(FA2_EINVAL, "%s=%p is not %d-byte aligned", names[i], ptrs[i], (int)align);
  }
  for (int o = 2; o < n; ++o)
    for (int i = 0; i < n; ++i)
      if (i != o && overlaps(ptrs[o], sizes[o], ptrs[i], sizes[i]))
        return fail(FA2_EINVAL, "%s overlaps %s", names[o], names[i]);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail_hip(e, "hipGetDevice");
  }
  for (int i = 0; i < n; ++i) {
    fa2_status_t s = check_device_range(ptrs[i], sizes[i], names[i]);
    if (s != FA2_OK) return s;
  }
  fa2::FwdArgs a;
  a.Q = a.K = a.V = nullptr;
  a.O = O;
  a.L = L;
  a.BH = 1;  // the merge sees `rows` independent rows
  a.Nq = static_cast<int>(rows);
  a.Nk = 0;
  a.d = static_cast<int>(d);
  a.causal = 0;
  a.scale = 1.f;
  a.num_m_block = 0;
  a.elem = static_cast<int>(dtype);
  a.stream = static_cast<hipStream_t>(stream);
  a.num_splits = num_parts;
  a.ws_O = const_cast<float*>(O_parts);
  a.ws_L = const_cast<float*>(L_parts);
  (void)hipGetLastError();
  e = fa2::launch_combine(a);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  return FA2_OK;
}

fa2_status_t fa2_schedule_map(int64_t items, int64_t grid, int32_t* visits, int32_t* workgroup,
                              int32_t* position) {
  g_last_error[0] = '\0';
  if (items < 1 || items > INT32_MAX || grid < 1 || grid > INT32_MAX)
    return fail(FA2_EINVAL, "items=%lld and grid=%lld must be in 1..2^31-1", (long long)items,
                (long long)grid);
  if (!visits) return fail(FA2_EINVAL, "visits is NULL");
  for (int64_t i = 0; i < items; ++i) visits[i] = 0;
  for (int g = 0; g < static_cast<int>(grid); ++g) {
    const fa2::sched::Walk w = fa2::sched::walk_of(static_cast<int>(items), static_cast<int>(grid), g);
    for (int k = 0;; ++k) {
      const int it = fa2::sched::item_of(w, k);
      if (it < 0) break;
      if (it >= items) return fail(FA2_EINVAL, "workgroup %d step %d maps outside the items", g, k);
      ++visits[it];
      if (workgroup) workgroup[it] = g;
      if (position) position[it] = k;
    }
  }
  return FA2_OK;
}

fa2_status_t fa2_schedule_blocks(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                 fa2_dtype_t dtype, int causal, int num_splits, int64_t grid,
                                 int64_t* blocks, int64_t* items) {
  g_last_error[0] = '\0';
  if (dtype == FA2_FP32)
    return fail(FA2_ENOTSUP, "the float32 kernel launches one workgroup per item (no schedule)");
  int64_t bm = 0;
  fa2_status_t s = check_shape(B, H, Nq, Nk, d, dtype, &bm);
  if (s != FA2_OK) return s;
  if (causal != 0 && causal != 1) return fail(FA2_EINVAL, "causal=%d must be 0 or 1", causal);
  const bool split = num_splits > 0;
  if (split) {
    s = check_splits(B, H, Nq, num_splits);
    if (s != FA2_OK) return s;
    bm = fa2::kBlockM_mfma;  // the split kernel's query blocks
  } else if (num_splits < 0) {
    return fail(FA2_EINVAL, "num_splits=%d must be >= 0", num_splits);
  }
  if (Nk < 1 || B * H * Nq < 1) return fail(FA2_EINVAL, "the schedule needs Nk >= 1 and B*H*Nq >= 1");
  if (grid < 1 || grid > INT32_MAX) return fail(FA2_EINVAL, "grid=%lld must be >= 1", (long long)grid);
  if (!blocks || !items) return fail(FA2_EINVAL, "blocks and items must not be NULL");
  const int bn = fa2::mfma_block_n(static_cast<int>(d));
  const int nmb = static_cast<int>((Nq + bm - 1) / bm);
  const int nkb = static_cast<int>((Nk + bn - 1) / bn);
  const int splits = split ? num_splits : 1;
  const int64_t total = B * H * nmb * splits;
  if (total > INT32_MAX) return fail(FA2_EINVAL, "%lld items exceed 2^31 - 1", (long long)total);
  *items = total;
  for (int g = 0; g < static_cast<int>(grid); ++g) {
    const fa2::sched::Walk w = fa2::sched::walk_of(static_cast<int>(total), static_cast<int>(grid), g);
    int64_t sum = 0;
    for (int k = 0;; ++k) {
      const int it = fa2::sched::item_of(w, k);
      if (it < 0) break;
      const fa2::sched::Item item = fa2::sched::decode(it, nmb, splits, causal != 0, split);
      const int jt = fa2::sched::blocks_of(item.m, static_cast<int>(Nq), static_cast<int>(Nk - Nq),
                                           nkb, static_cast<int>(bm), bn, causal != 0, split);
      const fa2::sched::Range r = fa2::sched::range_of(jt, item.split, splits, split);
      sum += r.end - r.beg;
    }
    blocks[g] = sum;
  }
  return FA2_OK;
}

fa2_status_t fa2_bwd_block_map(int64_t G, int32_t* logical) {
  g_last_error[0] = '\0';
  if (G < 1 || G > INT32_MAX) return fail(FA2_EINVAL, "G=%lld must be in 1..2^31-1", (long long)G);
  if (!logical) return fail(FA2_EINVAL, "logical is NULL");
  for (int64_t id = 0; id < G; ++id)
    logical[id] = fa2::sched::xcd_block(static_cast<int>(id), static_cast<int>(G));
  return FA2_OK;
}

fa2_status_t fa2_bwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, size_t* bytes) {
  g_last_error[0] = '\0';
  int64_t bm = 0;
  fa2_status_t s = check_shape(B, H, N, N, d, FA2_BF16, &bm);
  if (s != FA2_OK) return s;
  if (!bytes) return fail(FA2_EINVAL, "bytes is NULL");
  // -D = -rowsum(dO * O) and L * log2(e), float32 per row, rows padded per head
  *bytes = static_cast<size_t>(B * H * fa2::bwd_rows(N) * 8);
  return FA2_OK;
}

}  // extern "C"

namespace {

// Shared by fa2_bwd and fa2_bwd_cross: argument checks (none of which needs a
// HIP call), pointer and device checks, then the three kernels.  Arrays of
// zero size (no queries, or no keys) may be NULL and are not checked.
fa2_status_t bwd_common(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* L, void* dQ, void* dK, void* dV, int64_t B,
                        int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                        fa2_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != FA2_BF16 && dtype != FA2_FP16)
    return fail(FA2_ENOTSUP,
                "the backward pass is implemented for FA2_BF16 and FA2_FP16 only (dtype %d)",
                (int)dtype);
  int64_t bm = 0;
  fa2_status_t s = check_shape(B, H, Nq, Nk, d, dtype, &bm);
  if (s != FA2_OK) return s;
  if (causal != 0 && causal != 1) return fail(FA2_EINVAL, "causal=%d must be 0 or 1", causal);
  if (!std::isfinite(scale)) return fail(FA2_EINVAL, "scale must be finite");
  if (B * H * (Nq + Nk) == 0) return FA2_OK;  // no element of dQ, dK or dV

  const int64_t qb = B * H * Nq * d * 2, kb = B * H * Nk * d * 2, lb = B * H * Nq * 4;
  const int64_t wb = B * H * fa2::bwd_rows(Nq) * 8;
  constexpr int n = 10;
  const void* ptrs[n] = {Q, K, V, O, dO, L, dQ, dK, dV, workspace};
  const int64_t sizes[n] = {qb, kb, kb, qb, qb, lb, qb, kb, kb, wb};
  const char* names[n] = {"Q", "K", "V", "O", "dO", "L", "dQ", "dK", "dV", "workspace"};
  for (int i = 0; i < n; ++i) {
    if (sizes[i] == 0) continue;
    if (ptrs[i] == nullptr) return fail(FA2_EINVAL, "%s is NULL", names[i]);
    const uintptr_t align = (i == 5 || i == 9) ? 4 : 16;
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % align != 0)
      return fail(FA2_EINVAL, "%s=%p is not %d-byte aligned", names[i], ptrs[i], (int)align);
  }
  if (static_cast<int64_t>(workspace_bytes) < wb)
    return fail(FA2_EINVAL, "workspace of %llu bytes is smaller than the %lld bytes needed",
                (unsigned long long)workspace_bytes, (long long)wb);
  for (int o = 6; o < n; ++o)  // outputs and workspace: disjoint from everything else
    for (int i = 0; i < n; ++i)
      if (i != o && sizes[o] > 0 && sizes[i] > 0 &&
          overlaps(ptrs[o], sizes[o], ptrs[i], sizes[i]))
        return fail(FA2_EINVAL, "%s overlaps %s", names[o], names[i]);

  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail_hip(e, "hipGetDevice");
  }
  for (int i = 0; i < n; ++i) {
    if (sizes[i] == 0) continue;
    s = check_device_range(ptrs[i], sizes[i], names[i]);
    if (s != FA2_OK) return s;
  }
  fa2::BwdArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.dO = dO;
  a.L = L;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.Dvec = static_cast<float*>(workspace);
  a.BH = static_cast<int>(B * H);
  a.Nq = static_cast<int>(Nq);
  a.Nk = static_cast<int>(Nk);
  a.d = static_cast<int>(d);
  a.causal = causal;
  a.scale = scale;
  a.elem = static_cast<int>(dtype);
  a.stream = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  e = fa2::launch_bwd(a);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  return FA2_OK;
}

}  // namespace

extern "C" {

fa2_status_t fa2_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* L, void* dQ, void* dK, void* dV, int64_t B, int64_t H,
                     int64_t N, int64_t d, int causal, float scale, fa2_dtype_t dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  return bwd_common(Q, K, V, O, dO, L, dQ, dK, dV, B, H, N, N, d, causal, scale, dtype, workspace,
                    workspace_bytes, stream);
}

fa2_status_t fa2_bwd_cross(const void* Q, const void* K, const void* V, const void* O,
                           const void* dO, const float* L, void* dQ, void* dK, void* dV,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                           float scale, fa2_dtype_t dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  return bwd_common(Q, K, V, O, dO, L, dQ, dK, dV, B, H, Nq, Nk, d, causal, scale, dtype,
                    workspace, workspace_bytes, stream);
}

}  // extern "C"
