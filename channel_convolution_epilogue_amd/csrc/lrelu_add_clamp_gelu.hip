// Epilogue-only form of the Conv3d model over a precomputed conv output
// z[N][C][S] (S = spatial elements per channel):
//   y = GELU(clamp(LeakyReLU(z, slope) + s[c], lo, hi))   (exact GELU)
// This is the elementwise fallback POPCORNBENCH Kimi-K2.6 l2_p90 sketches
// (one fused kernel after a library Conv3d); here it is the HBM read+write
// bound companion of the fully fused operator.
//
// Design: a 1-D grid of workgroups, each owning a 4096-element chunk of one
// (n, c) plane, so the channel offset s[c] is one value per workgroup.  With S
// a multiple of 4 every thread moves four 16-byte quads (loads issued first);
// otherwise single floats.  The arithmetic is the same device function the
// fused Conv3d kernel applies to its accumulators.
#include "cce_device.hpp"
#include "cce_internal.hpp"

namespace cce {
namespace {

constexpr int THREADS = 256;
constexpr int QPT = 4;                       // quads per thread
constexpr int CHUNK = THREADS * QPT * 4;     // elements per workgroup

// z and y may be the same buffer (in place): every element is read and then
// written by the same thread, so they are not declared __restrict__.
struct EltArgs {
  const float *z;
  const float *__restrict__ s;
  float *y;
  long long S;
  int C, chunks;  // chunks per plane
  FastDiv divChunks;
  float slope, lo, hi;
};

template <bool VEC, bool SERIES>
__global__ __launch_bounds__(THREADS) void lrelu_add_clamp_gelu_kernel(EltArgs a) {
  const int plane = fdiv(blockIdx.x, a.divChunks);
  const int chunk = blockIdx.x - plane * a.chunks;
  const int c = plane % a.C;
  const float sadd = a.s[c];
  const size_t base = (size_t)plane * a.S + (size_t)chunk * CHUNK;
  const long long left = a.S - (long long)chunk * CHUNK;  // elements of this plane from base
  const int n_here = left < CHUNK ? (int)left : CHUNK;
  const float *zp = a.z + base;
  float *yp = a.y + base;
  if (VEC) {
    // S % 4 == 0: every quad lies in one plane and is 16-byte aligned.
    v4f v[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int e = 4 * (threadIdx.x + k * THREADS);
      if (e < n_here) v[k] = *reinterpret_cast<const v4f *>(zp + e);
    }
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int e = 4 * (threadIdx.x + k * THREADS);
      if (e < n_here) {
        v4f r = v[k];
        r.x = lrelu_add_clamp_gelu_value<SERIES>(r.x, sadd, a.slope, a.lo, a.hi);
        r.y = lrelu_add_clamp_gelu_value<SERIES>(r.y, sadd, a.slope, a.lo, a.hi);
        r.z = lrelu_add_clamp_gelu_value<SERIES>(r.z, sadd, a.slope, a.lo, a.hi);
        r.w = lrelu_add_clamp_gelu_value<SERIES>(r.w, sadd, a.slope, a.lo, a.hi);
        store4(yp + e, r);
      }
    }
  } else {
    for (int e = threadIdx.x; e < n_here; e += THREADS)
      yp[e] = lrelu_add_clamp_gelu_value<SERIES>(zp[e], sadd, a.slope, a.lo, a.hi);
  }
}

template <bool VEC>
void launch_vec(const EltArgs &a, unsigned grid, hipStream_t stream) {
  if (a.lo >= -1.0f && a.hi <= 1.0f)
    hipLaunchKernelGGL((lrelu_add_clamp_gelu_kernel<VEC, true>), dim3(grid), dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((lrelu_add_clamp_gelu_kernel<VEC, false>), dim3(grid), dim3(THREADS), 0, stream, a);
}

}  // namespace

int launch_lrelu_add_clamp_gelu(const float *z, const float *s, float *y, int N, int C, long long S,
                                float slope, float lo, float hi, hipStream_t stream) {
  EltArgs a;
  a.z = z;
  a.s = s;
  a.y = y;
  a.S = S;
  a.C = C;
  const long long chunks = (S + CHUNK - 1) / CHUNK;
  const long long grid = (long long)N * C * chunks;
  if (grid >= (1LL << 31)) return CCE_ERR_TOO_LARGE;
  a.chunks = (int)chunks;
  a.divChunks = make_fastdiv((uint32_t)chunks);
  a.slope = slope;
  a.lo = lo;
  a.hi = hi;
  const bool vec = (S % 4 == 0) && ((uintptr_t)z % 16 == 0) && ((uintptr_t)y % 16 == 0);
  if (vec)
    launch_vec<true>(a, (unsigned)grid, stream);
  else
    launch_vec<false>(a, (unsigned)grid, stream);
  return launch_status();
}

}  // namespace cce
