// extern "C" entry points of libcce: argument validation (host only, before any
// HIP call), then the call's kernel launches (one, or two for the transposed
// convolution and the wide-row 16 -> 64 Conv3d).  No allocation, no
// synchronisation (unless CCE_DEBUG is set) and no mutable global state beyond
// per-device caches of device properties and of each kernel instance's launch
// set-up.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>

#include "cce.h"
#include "cce_internal.hpp"

namespace cce {

namespace {
constexpr int kMaxDevices = 64;
// Cached per device: CU count and LDS bytes per workgroup (0 = not yet read).
std::atomic<int> g_cus[kMaxDevices];
std::atomic<long long> g_lds[kMaxDevices];
}  // namespace

int current_device_info(DeviceInfo *info) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CCE_ERR_LAUNCH;
  info->device = dev;
  if (dev >= 0 && dev < kMaxDevices) {
    const int cus = g_cus[dev].load(std::memory_order_relaxed);
    const long long lds = g_lds[dev].load(std::memory_order_relaxed);
    if (cus > 0 && lds > 0) {
      info->num_cus = cus;
      info->lds_per_block = (size_t)lds;
      return CCE_OK;
    }
  }
  int cus = 0, lds = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      cus < 1 || lds < 1)
    return CCE_ERR_LAUNCH;
  info->num_cus = cus;
  info->lds_per_block = (size_t)lds;
  if (dev >= 0 && dev < kMaxDevices) {
    g_cus[dev].store(cus, std::memory_order_relaxed);
    g_lds[dev].store(lds, std::memory_order_relaxed);
  }
  return CCE_OK;
}

bool debug_sync() {
  static std::atomic<int> state{-1};  // -1 = not read yet
  int v = state.load(std::memory_order_relaxed);
  if (v < 0) {
    const char *e = getenv("CCE_DEBUG");
    v = (e && e[0] && !(e[0] == '0' && e[1] == 0)) ? 1 : 0;
    state.store(v, std::memory_order_relaxed);
  }
  return v != 0;
}

}  // namespace cce

static bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
static bool is_finite_f(float v) { return isfinite(v); }

extern "C" {

const char *cce_status_string(int status) {
  switch (status) {
    case CCE_OK: return "success";
    case CCE_ERR_NULL: return "a required pointer is NULL";
    case CCE_ERR_SHAPE: return "a size is non-positive or the output would be empty";
    case CCE_ERR_UNSUPPORTED: return "shape or parameter outside the supported set";
    case CCE_ERR_ALIGN: return "a tensor pointer is not 4-byte aligned";
    case CCE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case CCE_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
    case CCE_ERR_TOO_LARGE: return "problem too large for 32-bit index arithmetic";
    case CCE_ERR_SCRATCH_LIMIT:
      return "the call needs more than the library's static scratch (CCE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int cce_version(void) { return 104; }

// Layer shapes the Conv2d kernel is instantiated for (see the header).
static bool conv2d_layer_supported(int C_in, int C_out, int k) {
  const bool ci = C_in == 4 || C_in == 8 || C_in == 16;
  const bool co = C_out == 16 || C_out == 32 || C_out == 64;
  const bool ks = k == 1 || k == 3 || (k == 5 && C_in <= 8);
  return ci && co && ks;
}

int conv2d_relu_hswish(const float *x, const float *w, const float *b, float *y, int N, int C_in,
                       int H, int W, int C_out, int k, void *stream) {
  if (!x || !w || !y) return CCE_ERR_NULL;
  if (N < 1 || C_in < 1 || C_out < 1 || k < 1 || H < k || W < k) return CCE_ERR_SHAPE;
  if (!conv2d_layer_supported(C_in, C_out, k)) return CCE_ERR_UNSUPPORTED;
  if (!aligned4(x) || !aligned4(w) || !aligned4(y) || (b && !aligned4(b))) return CCE_ERR_ALIGN;
  const long long P = (long long)(H - k + 1) * (W - k + 1);
  if ((long long)N * P >= (1LL << 31) || (long long)N * H >= (1LL << 31) ||
      (long long)C_in * H * W >= (1LL << 31) || (long long)C_out * P >= (1LL << 31) ||
      (long long)N * C_in * H * W >= (1LL << 40))
    return CCE_ERR_TOO_LARGE;
  return cce::launch_conv2d_relu_hswish(x, w, b, y, N, C_in, H, W, C_out, k, (hipStream_t)stream);
}

int conv3d_lrelu_add_clamp_gelu(const float *x, const float *w, const float *b, const float *s,
                                float *y, int N, int C_in, int D, int H, int W, int C_out, int k,
                                float negative_slope, float clamp_lo, float clamp_hi,
                                void *stream) {
  if (!x || !w || !s || !y) return CCE_ERR_NULL;
  if (N < 1 || C_in < 1 || C_out < 1 || k < 1 || D < k || H < k || W < k) return CCE_ERR_SHAPE;
  const bool ci = C_in == 4 || C_in == 8 || C_in == 16, co = C_out == 16 || C_out == 32 || C_out == 64;
  if (!ci || !co || (k != 3 && k != 1)) return CCE_ERR_UNSUPPORTED;
  if (!is_finite_f(negative_slope) || !is_finite_f(clamp_lo) || !is_finite_f(clamp_hi) || clamp_lo > clamp_hi)
    return CCE_ERR_UNSUPPORTED;
  if (!aligned4(x) || !aligned4(w) || !aligned4(y) || !aligned4(s) || (b && !aligned4(b)))
    return CCE_ERR_ALIGN;
  const long long Do = D - k + 1, Ho = H - k + 1, Wo = W - k + 1;
  const long long outs = (long long)N * C_out * Do * Ho * Wo;
  if (outs >= (1LL << 31) || (long long)N * Do * Ho >= (1LL << 31)) return CCE_ERR_TOO_LARGE;
  return cce::launch_conv3d_lrelu_add_clamp_gelu(x, w, b, s, y, N, C_in, D, H, W, C_out, k,
                                                 negative_slope, clamp_lo, clamp_hi,
                                                 (hipStream_t)stream);
}

static int convT_check_shape(int N, int C_in, int H, int W, int C_out, int k, int stride, int pad,
                             int pool_k, int pool_s) {
  if (N < 1 || C_in < 1 || C_out < 1 || k < 1 || H < 1 || W < 1 || stride < 1 || pad < 0 ||
      pool_k < 1 || pool_s < 1)
    return CCE_ERR_SHAPE;
  const long long Ho = (long long)(H - 1) * stride - 2LL * pad + k;
  const long long Wo = (long long)(W - 1) * stride - 2LL * pad + k;
  if (Ho < pool_k || Wo < pool_k) return CCE_ERR_SHAPE;
  if (!cce::convT_layer_supported(C_in, C_out) || k != 3 || stride != 1 || pad != 1 || pool_k != 2 ||
      pool_s != 2)
    return CCE_ERR_UNSUPPORTED;
  if ((long long)N * C_in * H * W >= (1LL << 31)) return CCE_ERR_TOO_LARGE;
  return CCE_OK;
}

size_t convT2d_pool_htanh_mean_tanh_workspace_bytes(int N, int C_in, int H, int W, int C_out,
                                                    int k, int stride, int pad, int pool_k,
                                                    int pool_s) {
  if (convT_check_shape(N, C_in, H, W, C_out, k, stride, pad, pool_k, pool_s) != CCE_OK) return 0;
  return cce::convT_workspace_bytes(N, C_in, H, W, C_out);
}

int convT2d_pool_htanh_mean_tanh(const float *x, const float *w, const float *b, float *y, int N,
                                 int C_in, int H, int W, int C_out, int k, int stride, int pad,
                                 int pool_k, int pool_s, float htanh_lo, float htanh_hi,
                                 void *workspace, size_t workspace_bytes, void *stream) {
  if (!x || !w || !y) return CCE_ERR_NULL;
  const int st = convT_check_shape(N, C_in, H, W, C_out, k, stride, pad, pool_k, pool_s);
  if (st != CCE_OK) return st;
  if (!is_finite_f(htanh_lo) || !is_finite_f(htanh_hi) || htanh_lo > htanh_hi) return CCE_ERR_UNSUPPORTED;
  if (!aligned4(x) || !aligned4(w) || !aligned4(y) || (b && !aligned4(b))) return CCE_ERR_ALIGN;
  if (!workspace || ((uintptr_t)workspace & 255u) != 0 ||
      workspace_bytes < cce::convT_workspace_bytes(N, C_in, H, W, C_out))
    return CCE_ERR_WORKSPACE;
  return cce::launch_convT2d_pool_htanh_mean_tanh(x, w, b, y, N, C_in, H, W, C_out, htanh_lo,
                                                  htanh_hi, workspace, (hipStream_t)stream);
}

int convT2d_pool_htanh_mean_tanh_noalloc(const float *x, const float *w, const float *b, float *y,
                                         int N, int C_in, int H, int W, int C_out, int k, int stride,
                                         int pad, int pool_k, int pool_s, float htanh_lo,
                                         float htanh_hi, void *stream) {
  if (!x || !w || !y) return CCE_ERR_NULL;
  const int st = convT_check_shape(N, C_in, H, W, C_out, k, stride, pad, pool_k, pool_s);
  if (st != CCE_OK) return st;
  if (!is_finite_f(htanh_lo) || !is_finite_f(htanh_hi) || htanh_lo > htanh_hi) return CCE_ERR_UNSUPPORTED;
  if (!aligned4(x) || !aligned4(w) || !aligned4(y) || (b && !aligned4(b))) return CCE_ERR_ALIGN;
  return cce::launch_convT2d_pool_htanh_mean_tanh_noalloc(x, w, b, y, N, C_in, H, W, C_out, htanh_lo,
                                                          htanh_hi, (hipStream_t)stream);
}

int pool_htanh_mean_tanh(const float *z, float *y, int N, int C, int H, int W, int pool_k,
                         int pool_s, float htanh_lo, float htanh_hi, void *stream) {
  if (!z || !y) return CCE_ERR_NULL;
  if (N < 1 || C < 1 || H < 1 || W < 1 || pool_k < 1 || pool_s < 1) return CCE_ERR_SHAPE;
  if (H < pool_k || W < pool_k) return CCE_ERR_SHAPE;
  if (!is_finite_f(htanh_lo) || !is_finite_f(htanh_hi) || htanh_lo > htanh_hi) return CCE_ERR_UNSUPPORTED;
  if (!aligned4(z) || !aligned4(y)) return CCE_ERR_ALIGN;
  if ((long long)N * C >= (1LL << 31) || (long long)H * W >= (1LL << 31)) return CCE_ERR_TOO_LARGE;
  return cce::launch_pool_htanh_mean_tanh(z, y, N, C, H, W, pool_k, pool_s, htanh_lo, htanh_hi,
                                          (hipStream_t)stream);
}

int lrelu_add_clamp_gelu(const float *z, const float *s, float *y, int N, int C, long long S,
                         float negative_slope, float clamp_lo, float clamp_hi, void *stream) {
  if (!z || !s || !y) return CCE_ERR_NULL;
  if (N < 1 || C < 1 || S < 1) return CCE_ERR_SHAPE;
  if (!is_finite_f(negative_slope) || !is_finite_f(clamp_lo) || !is_finite_f(clamp_hi) ||
      clamp_lo > clamp_hi)
    return CCE_ERR_UNSUPPORTED;
  if (!aligned4(z) || !aligned4(s) || !aligned4(y)) return CCE_ERR_ALIGN;
  if ((long long)N * C >= (1LL << 31) || S >= (1LL << 40)) return CCE_ERR_TOO_LARGE;
  return cce::launch_lrelu_add_clamp_gelu(z, s, y, N, C, S, negative_slope, clamp_lo, clamp_hi,
                                          (hipStream_t)stream);
}

}  // extern "C"
