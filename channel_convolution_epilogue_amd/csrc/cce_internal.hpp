// Internal launch entry points of libcce (host side).  The extern "C" API in
// cce_api.cpp validates every argument and then calls these; they pick the
// kernel instance, grid and LDS size and enqueue one launch on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdio.h>

#include <atomic>

#include "cce.h"

namespace cce {

// Properties of the current device that size the persistent grids.
struct DeviceInfo {
  int device;
  int num_cus;
  size_t lds_per_block;
};
int current_device_info(DeviceInfo *info);  // CCE_OK or CCE_ERR_LAUNCH

// Conv2d (page layer 3x3, 8 -> 64) + ReLU + HardSwish.  Arguments already validated.
int launch_conv2d_relu_hswish(const float *x, const float *w, const float *b, float *y, int N,
                              int C_in, int H, int W, int C_out, int k, hipStream_t stream);

// 1 x 1 Conv2d over `rows` x W pixels + LeakyReLU + add + clamp + GELU: the
// 1 x 1 x 1 Conv3d layers (rows = D * H), on the Conv2d strip kernel.
int launch_pointwise_lrelu_add_clamp_gelu(const float *x, const float *w, const float *b,
                                          const float *s, float *y, int N, int C_in, int rows,
                                          int W, int C_out, float slope, float lo, float hi,
                                          hipStream_t stream);

// Conv3d k^3 (page layer 3^3, 8 -> 64) + LeakyReLU + add + clamp + GELU.  Validated.
int launch_conv3d_lrelu_add_clamp_gelu(const float *x, const float *w, const float *b,
                                       const float *s, float *y, int N, int C_in, int D, int H,
                                       int W, int C_out, int k, float slope, float lo, float hi,
                                       hipStream_t stream);

// ConvTranspose2d 3x3 s1 p1 (C_in % 8 == 0, C_out in {16, 32, 64}) + MaxPool
// 2x2 + Hardtanh + mean + tanh.
bool convT_layer_supported(int C_in, int C_out);
size_t convT_workspace_bytes(int N, int C_in, int H, int W, int C_out);
int launch_convT2d_pool_htanh_mean_tanh(const float *x, const float *w, const float *b, float *y,
                                        int N, int C_in, int H, int W, int C_out, float lo, float hi,
                                        void *workspace, hipStream_t stream);
// The same with the library's static per-device scratch as the workspace
// (CCE_ERR_SCRATCH_LIMIT when the call needs more than it holds).
int launch_convT2d_pool_htanh_mean_tanh_noalloc(const float *x, const float *w, const float *b,
                                                float *y, int N, int C_in, int H, int W, int C_out,
                                                float lo, float hi, hipStream_t stream);

// Epilogue-only operators over a precomputed convolution output.
int launch_pool_htanh_mean_tanh(const float *z, float *y, int N, int C, int H, int W, int pool_k,
                                int pool_s, float lo, float hi, hipStream_t stream);
int launch_lrelu_add_clamp_gelu(const float *z, const float *s, float *y, int N, int C, long long S,
                                float slope, float lo, float hi, hipStream_t stream);

// Launch set-up of one kernel instance, cached per device: its dynamic-LDS
// limit is raised once to the device's maximum (so that no call ever lowers
// it under another thread's launch), and its workgroups per CU are queried
// for the launch's LDS size and re-queried only when that size changes.  The
// runtime calls cost microseconds of host time, which small launches would
// otherwise pay on every call.  One cache per kernel instance; each entry
// packs the LDS size and the workgroups per CU into one atomic word, so
// concurrent callers at worst repeat a query.
constexpr int kLaunchCacheDevices = 64;
struct LaunchCache {
  std::atomic<int> raised[kLaunchCacheDevices];       // 1 once the LDS limit is raised
  std::atomic<long long> entry[kLaunchCacheDevices];  // (lds_bytes << 8) | per_cu, 0 = unset
};

// Workgroups of `threads` threads and `lds_bytes` of dynamic LDS that fit on
// one CU of the current device (at least 1), or -1 when the runtime refuses
// the set-up.
inline int launch_setup(const void *kern, LaunchCache &cache, int device, size_t lds_bytes,
                        int threads) {
  const bool cached = device >= 0 && device < kLaunchCacheDevices;
  if (cached) {
    const long long e = cache.entry[device].load(std::memory_order_relaxed);
    if (e != 0 && (e >> 8) == (long long)lds_bytes) return (int)(e & 255);
  }
  if (!cached || cache.raised[device].load(std::memory_order_acquire) == 0) {
    DeviceInfo dev;
    if (current_device_info(&dev) != CCE_OK || lds_bytes > dev.lds_per_block ||
        hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)dev.lds_per_block) != hipSuccess)
      return -1;
    if (cached) cache.raised[device].store(1, std::memory_order_release);
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds_bytes) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (per_cu > 255) per_cu = 255;
  if (cached)
    cache.entry[device].store(((long long)lds_bytes << 8) | per_cu, std::memory_order_relaxed);
  return per_cu;
}

// True when the environment variable CCE_DEBUG was set to a non-empty value
// other than "0" when the library first looked (read once per process).
bool debug_sync();

// Map the runtime's last error after a launch onto a cce_status.  Under
// CCE_DEBUG every launch is also followed by a synchronisation of its
// stream, so that a kernel that faults is reported by the call that
// launched it (on stderr, naming `what`) and the call returns
// CCE_ERR_LAUNCH.  That synchronisation makes calls blocking and is not
// allowed under HIP graph capture: CCE_DEBUG is for debugging only.
inline int launch_status(hipStream_t stream, const char *what) {
  hipError_t e = hipGetLastError();
  const bool debug = debug_sync();
  if (e == hipSuccess && debug) e = hipStreamSynchronize(stream);
  if (e == hipSuccess) return CCE_OK;
  if (debug) fprintf(stderr, "libcce: %s: %s\n", what, hipGetErrorString(e));
  return CCE_ERR_LAUNCH;
}

}  // namespace cce
