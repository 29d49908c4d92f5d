// Host side of libfa2.so: argument validation, error reporting, the work
// decomposition and kernel dispatch for the FlashAttention-2 forward pass.
//
// Validation order: pure argument checks first (no HIP call at all), then the
// device and each pointer's allocation are checked through the HIP runtime,
// then the kernel is enqueued and the launch status is read back.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fa2.h"
#include "fa2_internal.h"

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

int64_t elem_size(fa2_dtype_t t) { return t == FA2_BF16 ? 2 : 4; }

// Checks that need no HIP call.  On success fills the element counts.
fa2_status_t check_shape(int64_t B, int64_t H, int64_t N, int64_t d, fa2_dtype_t dtype,
                         int64_t* kBlockM) {
  if (dtype != FA2_BF16 && dtype != FA2_FP32)
    return fail(FA2_ENOTSUP, "dtype %d is not FA2_BF16 (0) or FA2_FP32 (1)", (int)dtype);
  if (B < 0 || H < 0 || N < 0)
    return fail(FA2_EINVAL, "sizes must be >= 0 (B=%lld H=%lld N=%lld)", (long long)B,
                (long long)H, (long long)N);
  if (d != 64 && d != 128 && d != 256)
    return fail(FA2_ENOTSUP, "head dimension d=%lld is not one of 64, 128, 256", (long long)d);
  // Per-slice offsets are 32-bit inside the kernels; slice counts and the grid too.
  if (N > (int64_t(1) << 31) / 256)
    return fail(FA2_EINVAL, "N=%lld exceeds the supported maximum %lld", (long long)N,
                (long long)((int64_t(1) << 31) / 256));
  if (B > 0 && H > (int64_t(1) << 31) / B)
    return fail(FA2_EINVAL, "B*H=%lld*%lld exceeds 2^31", (long long)B, (long long)H);
  const int64_t bm = dtype == FA2_BF16 ? fa2::kBlockM_bf16 : fa2::kBlockM_f32;
  const int64_t nmb = (N + bm - 1) / bm;
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
  fa2_status_t s = check_shape(B, H, N, d, dtype, &bm);
  if (s != FA2_OK) return s;
  const int64_t nmb = (N + bm - 1) / bm;
  if (kBlockM) *kBlockM = bm;
  if (num_m_block) *num_m_block = nmb;
  if (items) *items = nmb * B * H;
  return FA2_OK;
}

fa2_status_t fa2_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int64_t B,
                     int64_t H, int64_t N, int64_t d, int causal, float scale, fa2_dtype_t dtype,
                     void* stream) {
  g_last_error[0] = '\0';
  int64_t bm = 0;
  fa2_status_t s = check_shape(B, H, N, d, dtype, &bm);
  if (s != FA2_OK) return s;
  if (causal != 0 && causal != 1) return fail(FA2_EINVAL, "causal=%d must be 0 or 1", causal);
  if (!std::isfinite(scale)) return fail(FA2_EINVAL, "scale must be finite");
  if (B * H * N == 0) return FA2_OK;  // empty problem: nothing to read or write

  const int64_t tensor_bytes = B * H * N * d * elem_size(dtype);
  const int64_t l_bytes = B * H * N * 4;
  const void* ptrs[5] = {Q, K, V, O, L};
  const char* names[5] = {"Q", "K", "V", "O", "L"};
  for (int i = 0; i < 5; ++i) {
    if (ptrs[i] == nullptr) return fail(FA2_EINVAL, "%s is NULL", names[i]);
    const uintptr_t align = i == 4 ? 4 : 16;
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % align != 0)
      return fail(FA2_EINVAL, "%s=%p is not %d-byte aligned", names[i], ptrs[i], (int)align);
  }
  for (int o = 3; o < 5; ++o) {
    const int64_t no = o == 4 ? l_bytes : tensor_bytes;
    for (int i = 0; i < 5; ++i) {
      if (i == o) continue;
      const int64_t ni = i == 4 ? l_bytes : tensor_bytes;
      if (overlaps(ptrs[o], no, ptrs[i], ni))
        return fail(FA2_EINVAL, "output %s overlaps %s", names[o], names[i]);
    }
  }

  // From here on the HIP runtime is involved.
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail_hip(e, "hipGetDevice");
  }
  for (int i = 0; i < 5; ++i) {
    s = check_device_range(ptrs[i], i == 4 ? l_bytes : tensor_bytes, names[i]);
    if (s != FA2_OK) return s;
  }

  fa2::FwdArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.L = L;
  a.BH = static_cast<int>(B * H);
  a.N = static_cast<int>(N);
  a.d = static_cast<int>(d);
  a.causal = causal;
  a.scale = scale;
  a.num_m_block = static_cast<int>((N + bm - 1) / bm);
  a.stream = static_cast<hipStream_t>(stream);

  (void)hipGetLastError();  // clear a stale error so the status below is this launch's
  e = dtype == FA2_BF16 ? fa2::launch_fwd_bf16(a) : fa2::launch_fwd_f32(a);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail_hip(e, "kernel launch");
  return FA2_OK;
}

}  // extern "C"
