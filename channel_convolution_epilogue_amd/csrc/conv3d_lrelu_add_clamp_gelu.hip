// Conv3d 3x3x3, 8 -> 64 channels, stride 1, padding 0, + bias -> LeakyReLU ->
// + s[channel] -> clamp -> exact GELU, fused in one gfx950 kernel
// (POPCORNBENCH Kimi-K2.6 l2_p90: Conv3d followed by LeakyReLU(0.2), the
// learnable [C_out,1,1,1] sum_tensor, clamp to [-1, 1] and GELU with
// approximate=False).
//
// Design:
//  * Implicit GEMM on the fp32 matrix cores: M = output voxels, N = output
//    channels, K = 8 channels x 27 taps = 216.  A tile is one output depth
//    plane d of one image and TR consecutive output rows (all columns); its
//    input -- 8 channels x 3 depth planes x (TR + 2) rows x W -- is staged in
//    LDS once.  Voxels inside the tile are numbered flat (row-major), so a
//    lane's four result voxels are consecutive in memory.
//  * Each wave owns 32 of the 64 output channels; the matching 216 x 32
//    weight slice lives in 108 VGPRs per lane for the whole (persistent)
//    workgroup.  Two waves share a channel half and split the tile's
//    16-voxel blocks.  Per K-step a lane reads one A value from LDS at a
//    lane-independent step offset (lane group g = channel within a group of 4).
//  * The epilogue (bias as accumulator init, LeakyReLU, add, clamp, GELU with
//    erf) runs in registers; only the final value is stored.
#include "cce_device.hpp"
#include "cce_internal.hpp"

namespace cce {
namespace {

constexpr int CI = 8, CO = 64, KS = 3, TAPS = KS * KS * KS;
constexpr int KSTEPS = (CI / 4) * TAPS;  // 54 steps of 4 taps
constexpr int NTW = 2;                   // 16-channel blocks per wave (32 channels)
constexpr int WAVES = 4, THREADS = 64 * WAVES;
constexpr int MT_BATCH = 2;

struct Conv3dArgs {
  const float *__restrict__ x;
  const float *__restrict__ w;
  const float *__restrict__ b;
  const float *__restrict__ s;
  float *__restrict__ y;
  int D, H, W, Do, Ho, Wo;
  int TR;           // output rows per tile
  int rowtiles;     // ceil(Ho / TR)
  int ntiles;       // N * Do * rowtiles
  int chstride;     // floats between channel blocks in LDS
  int planestride;  // floats between depth planes in LDS, (TR + 2) * W
  float slope, lo, hi;
};

__device__ __forceinline__ float epilogue(float v, float s, float slope, float lo, float hi) {
  float t = v >= 0.0f ? v : slope * v;
  t = clampf(t + s, lo, hi);
  return 0.5f * t * (1.0f + erff(t * 0.70710678118654752f));
}

template <bool VLOAD, bool VSTORE>
__global__ __launch_bounds__(THREADS) void conv3d_lrelu_add_clamp_gelu_kernel(Conv3dArgs a) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int half = wave & 1;  // which 32 output channels
  const int mg = wave >> 1;   // which interleaved set of 16-voxel blocks

  float wr[KSTEPS][NTW];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int o = 32 * half + 16 * nt + col, ci = 4 * (s / TAPS) + g;
      wr[s][nt] = a.w[(o * CI + ci) * TAPS + (s % TAPS)];
    }
  float bias[NTW], sadd[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int o = 32 * half + 16 * nt + col;
    bias[nt] = a.b ? a.b[o] : 0.0f;
    sadd[nt] = a.s[o];
  }
  const size_t vol = (size_t)a.Do * a.Ho * a.Wo;  // output voxels per (n, channel)

  const int t_begin = (int)(((long long)blockIdx.x * a.ntiles) / gridDim.x);
  const int t_end = (int)(((long long)(blockIdx.x + 1) * a.ntiles) / gridDim.x);

  for (int t = t_begin; t < t_end; ++t) {
    const int rt = t % a.rowtiles, nd = t / a.rowtiles;
    const int d = nd % a.Do, n = nd / a.Do;
    const int h0 = rt * a.TR;
    const int rows = min(a.TR, a.Ho - h0);
    const int V = rows * a.Wo;  // voxels in this tile
    const int MTT = (V + 15) >> 4;
    const int rows_in = rows + (KS - 1);

    __syncthreads();
    {
      const int cw = VLOAD ? (a.W >> 2) : a.W;
      const int tpr = cw < THREADS ? cw : THREADS;
      const int rpp = THREADS / tpr;
      const int my_row = tid / tpr, my_col = tid - my_row * tpr;
      const int nrows = CI * KS * rows_in;
      if (my_row < rpp) {
        for (int ri = my_row; ri < nrows; ri += rpp) {
          const int rr = ri % rows_in, pk = ri / rows_in, kd = pk % KS, ci = pk / KS;
          const float *src =
              a.x + ((((size_t)n * CI + ci) * a.D + (d + kd)) * a.H + (h0 + rr)) * a.W;
          float *dst = lds + ci * a.chstride + kd * a.planestride + rr * a.W;
          if (VLOAD) {
            for (int c = my_col; c < cw; c += tpr)
              *reinterpret_cast<v4f *>(dst + 4 * c) = *reinterpret_cast<const v4f *>(src + 4 * c);
          } else {
            for (int c = my_col; c < cw; c += tpr) dst[c] = src[c];
          }
        }
      }
    }
    __syncthreads();

    float *ybase = a.y + ((size_t)n * CO) * vol + (size_t)d * a.Ho * a.Wo + (size_t)h0 * a.Wo;

#pragma unroll 1
    for (int mb = mg * MT_BATCH; mb < MTT; mb += 2 * MT_BATCH) {
      int base[MT_BATCH];
#pragma unroll
      for (int j = 0; j < MT_BATCH; ++j) {
        const int v = min(16 * (mb + j) + col, V - 1);
        const int hl = v / a.Wo, w = v - hl * a.Wo;
        base[j] = g * a.chstride + hl * a.W + w;
      }
      v4f acc[MT_BATCH][NTW];
#pragma unroll
      for (int j = 0; j < MT_BATCH; ++j)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) acc[j][nt] = splat4(bias[nt]);

#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int tt = s % TAPS, kd = tt / 9, kh = (tt / 3) % 3, kw = tt % 3;
        const int off = (s / TAPS) * 4 * a.chstride + kd * a.planestride + kh * a.W + kw;
        float av[MT_BATCH];
#pragma unroll
        for (int j = 0; j < MT_BATCH; ++j) av[j] = lds[base[j] + off];
#pragma unroll
        for (int j = 0; j < MT_BATCH; ++j)
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) acc[j][nt] = mfma16x16x4(av[j], wr[s][nt], acc[j][nt]);
      }

#pragma unroll
      for (int j = 0; j < MT_BATCH; ++j) {
        const int v0 = 16 * (mb + j) + 4 * g;
        if (v0 >= V) continue;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const int o = 32 * half + 16 * nt + col;
          float *dst = ybase + (size_t)o * vol + v0;
          v4f r = acc[j][nt];
          r.x = epilogue(r.x, sadd[nt], a.slope, a.lo, a.hi);
          r.y = epilogue(r.y, sadd[nt], a.slope, a.lo, a.hi);
          r.z = epilogue(r.z, sadd[nt], a.slope, a.lo, a.hi);
          r.w = epilogue(r.w, sadd[nt], a.slope, a.lo, a.hi);
          if (VSTORE && v0 + 3 < V) {
            store4(dst, r);
          } else {
            dst[0] = r.x;
            if (v0 + 1 < V) dst[1] = r.y;
            if (v0 + 2 < V) dst[2] = r.z;
            if (v0 + 3 < V) dst[3] = r.w;
          }
        }
      }
    }
  }
}

template <bool VL, bool VS>
int launch_instance(const Conv3dArgs &a, size_t lds_bytes, const DeviceInfo &dev,
                    hipStream_t stream) {
  auto kern = conv3d_lrelu_add_clamp_gelu_kernel<VL, VS>;
  if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)lds_bytes) != hipSuccess)
    return CCE_ERR_LAUNCH;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, THREADS, lds_bytes) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int grid = dev.num_cus * per_cu;
  if (grid > a.ntiles) grid = a.ntiles;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(THREADS), lds_bytes, stream, a);
  return launch_status();
}

}  // namespace

int launch_conv3d_lrelu_add_clamp_gelu(const float *x, const float *w, const float *b,
                                       const float *s, float *y, int N, int D, int H, int W,
                                       float slope, float lo, float hi, hipStream_t stream) {
  DeviceInfo dev;
  if (current_device_info(&dev) != CCE_OK) return CCE_ERR_LAUNCH;
  Conv3dArgs a;
  a.x = x;
  a.w = w;
  a.b = b;
  a.s = s;
  a.y = y;
  a.D = D;
  a.H = H;
  a.W = W;
  a.Do = D - 2;
  a.Ho = H - 2;
  a.Wo = W - 2;
  a.slope = slope;
  a.lo = lo;
  a.hi = hi;
  // Largest row count per tile (8, 4, 2 or 1) whose input slab fits in LDS.
  size_t lds_bytes = 0;
  a.TR = 0;
  for (int tr = 8; tr >= 1; tr /= 2) {
    const int plane = (tr + 2) * W;
    const int cs = KS * plane + ((16 - (KS * plane) % 64) + 64) % 64;
    const size_t bytes = (size_t)CI * cs * sizeof(float);
    if (bytes <= dev.lds_per_block) {
      a.TR = tr;
      a.planestride = plane;
      a.chstride = cs;
      lds_bytes = bytes;
      break;
    }
  }
  if (a.TR == 0) return CCE_ERR_UNSUPPORTED;
  a.rowtiles = (a.Ho + a.TR - 1) / a.TR;
  const long long nt = (long long)N * a.Do * a.rowtiles;
  if (nt >= (1LL << 31)) return CCE_ERR_TOO_LARGE;
  a.ntiles = (int)nt;

  const bool vl = (W % 4 == 0) && ((uintptr_t)x % 16 == 0);
  const bool vs = ((a.Ho * a.Wo) % 4 == 0) && ((a.TR * a.Wo) % 4 == 0) && ((uintptr_t)y % 16 == 0);
  if (vl) return vs ? launch_instance<true, true>(a, lds_bytes, dev, stream)
                    : launch_instance<true, false>(a, lds_bytes, dev, stream);
  return vs ? launch_instance<false, true>(a, lds_bytes, dev, stream)
            : launch_instance<false, false>(a, lds_bytes, dev, stream);
}

}  // namespace cce
