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
//  * Each of the 8 waves owns 16 of the 64 output channels; the matching
//    216 x 16 weight slice lives in 54 VGPRs per lane for the whole
//    (persistent) workgroup, which keeps 4 waves per SIMD resident.  The
//    four waves of a channel split the tile's 16-voxel blocks two ways.  Per
//    K-step a lane reads one A value from LDS at a lane-independent step
//    offset (lane group g = input channel within a group of 4).
//  * The epilogue (bias as accumulator init, LeakyReLU, add, clamp, GELU with
//    erf) runs in registers; only the final value is stored.
#include "cce_device.hpp"
#include "cce_internal.hpp"

namespace cce {
namespace {

constexpr int CI = 8, CO = 64, KS = 3, TAPS = KS * KS * KS;
constexpr int KSTEPS = (CI / 4) * TAPS;  // 54 steps of 4 taps
constexpr int CG = 4;                    // channel groups of 16: wave w owns channels 16 (w % 4) ..
constexpr int MG = 2;                    // voxel groups: wave w takes 16-voxel blocks w / 4, + 2, ...
constexpr int WAVES = CG * MG, THREADS = 64 * WAVES;
constexpr int MT_BATCH = 2;
constexpr int kPrefetchPasses = 3;  // one plane: 8 ch x 10 rows of 64 floats, 32 rows per pass

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
  FastDiv divDo, divRowtiles, divWo;
};

// One tile: output depth plane d of image n, output rows h0 .. h0 + rows - 1.
// Tiles are numbered with d fastest, so a run of consecutive tiles walks down
// the depth axis of one row block and each step needs one new input plane.
struct Tile3 {
  int n, d, h0, rows;
};

// One input depth plane dd of a row block: staged row `row` = rr * 8 + ci
// <-> x[n][ci][dd][h0 + rr][:], stored in LDS ring slot dd % 3.
struct PlaneSrc {
  const float *x;
  int D, H, W, n, dd, h0;
  __device__ __forceinline__ const float *operator()(int row) const {
    const int ci = row & (CI - 1), rr = row >> 3;
    return x + ((((size_t)n * CI + ci) * D + dd) * H + (h0 + rr)) * W;
  }
};
struct PlaneDst {
  float *lds;
  int chstride, slot_off, W;
  __device__ __forceinline__ float *operator()(int row) const {
    return lds + (row & (CI - 1)) * chstride + slot_off + (row >> 3) * W;
  }
};

template <bool VLOAD, bool VSTORE, bool SERIES, int KPRE>
__global__ __launch_bounds__(THREADS, 4) void conv3d_lrelu_add_clamp_gelu_kernel(Conv3dArgs a) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int o = 16 * (wave % CG) + col;  // this lane's output channel
  const int mg = wave / CG;              // which interleaved set of 16-voxel blocks

  // B operand of every K-step for this wave's 16 channels (54 VGPRs).
  float wr[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) wr[s] = a.w[(o * CI + 4 * (s / TAPS) + g) * TAPS + (s % TAPS)];
  const float bias = a.b ? a.b[o] : 0.0f;
  const float sadd = a.s[o];
  const size_t vol = (size_t)a.Do * a.Ho * a.Wo;  // output voxels per (n, channel)

  const int t_begin = (int)(((long long)blockIdx.x * a.ntiles) / gridDim.x);
  const int t_end = (int)(((long long)(blockIdx.x + 1) * a.ntiles) / gridDim.x);
  if (t_begin >= t_end) return;

  auto tile_of = [&](int t) {
    Tile3 tl;
    const int q = fdiv(t, a.divDo);
    tl.d = t - q * a.Do;
    tl.n = fdiv(q, a.divRowtiles);
    const int rt = q - tl.n * a.rowtiles;
    tl.h0 = rt * a.TR;
    tl.rows = min(a.TR, a.Ho - tl.h0);
    return tl;
  };
  auto src_of = [&](const Tile3 &tl, int dd) {
    return PlaneSrc{a.x, a.D, a.H, a.W, tl.n, dd, tl.h0};
  };
  auto dst_of = [&](const Tile3 &, int dd) {
    return PlaneDst{lds, a.chstride, (dd % KS) * a.planestride, a.W};
  };
  auto nrows = [&](const Tile3 &tl) { return CI * (tl.rows + (KS - 1)); };

  // Registers carry one input plane ahead: plane d + 3 while tile d computes,
  // or the first plane of a new row block (its other two are copied directly).
  RowStage<KPRE, VLOAD, THREADS> stage;
  stage.init(a.W, tid);
  Tile3 cur = tile_of(t_begin);
  stage.load(nrows(cur), src_of(cur, cur.d));
  stage.store(nrows(cur), src_of(cur, cur.d), dst_of(cur, cur.d));
  stage.load(nrows(cur), src_of(cur, cur.d + 1));
  stage.store(nrows(cur), src_of(cur, cur.d + 1), dst_of(cur, cur.d + 1));
  stage.load(nrows(cur), src_of(cur, cur.d + 2));
  stage.store(nrows(cur), src_of(cur, cur.d + 2), dst_of(cur, cur.d + 2));
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const bool more = t + 1 < t_end;
    Tile3 nxt = cur;
    bool fresh = false;  // next tile starts a new row block (needs three planes)
    if (more) {
      nxt = tile_of(t + 1);
      fresh = nxt.d == 0;
      stage.load(nrows(nxt), src_of(nxt, fresh ? 0 : nxt.d + 2));
    }
    const int V = cur.rows * a.Wo;  // voxels in this tile
    const int MTT = (V + 15) >> 4;
    float *ybase = a.y + ((size_t)cur.n * CO) * vol + (size_t)cur.d * a.Ho * a.Wo +
                   (size_t)cur.h0 * a.Wo;
    // LDS offsets of input planes d, d + 1, d + 2 in the ring.
    const int so0 = (cur.d % KS) * a.planestride;
    const int so1 = ((cur.d + 1) % KS) * a.planestride;
    const int so2 = ((cur.d + 2) % KS) * a.planestride;

#pragma unroll 1
    for (int mb = mg * MT_BATCH; mb < MTT; mb += MG * MT_BATCH) {
      int base[MT_BATCH][KS];
#pragma unroll
      for (int j = 0; j < MT_BATCH; ++j) {
        const int v = min(16 * (mb + j) + col, V - 1);
        const int hl = fdiv(v, a.divWo), w = v - hl * a.Wo;
        const int b0 = g * a.chstride + hl * a.W + w;
        base[j][0] = b0 + so0;
        base[j][1] = b0 + so1;
        base[j][2] = b0 + so2;
      }
      v4f acc[MT_BATCH];
#pragma unroll
      for (int j = 0; j < MT_BATCH; ++j) acc[j] = splat4(bias);

#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int tt = s % TAPS, kd = tt / 9, kh = (tt / 3) % 3, kw = tt % 3;
        const int off = (s / TAPS) * 4 * a.chstride + kh * a.W + kw;
        float av[MT_BATCH];
#pragma unroll
        for (int j = 0; j < MT_BATCH; ++j) av[j] = lds[base[j][kd] + off];
#pragma unroll
        for (int j = 0; j < MT_BATCH; ++j) acc[j] = mfma16x16x4(av[j], wr[s], acc[j]);
      }

#pragma unroll
      for (int j = 0; j < MT_BATCH; ++j) {
        const int v0 = 16 * (mb + j) + 4 * g;
        if (v0 >= V) continue;
        float *dst = ybase + (size_t)o * vol + v0;
        v4f r = acc[j];
        r.x = lrelu_add_clamp_gelu_value<SERIES>(r.x, sadd, a.slope, a.lo, a.hi);
        r.y = lrelu_add_clamp_gelu_value<SERIES>(r.y, sadd, a.slope, a.lo, a.hi);
        r.z = lrelu_add_clamp_gelu_value<SERIES>(r.z, sadd, a.slope, a.lo, a.hi);
        r.w = lrelu_add_clamp_gelu_value<SERIES>(r.w, sadd, a.slope, a.lo, a.hi);
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

    if (more) {
      __syncthreads();  // every wave is done reading plane d (its slot is reused)
      if (fresh) {
        stage.store(nrows(nxt), src_of(nxt, 0), dst_of(nxt, 0));
        stage.load(nrows(nxt), src_of(nxt, 1));
        stage.store(nrows(nxt), src_of(nxt, 1), dst_of(nxt, 1));
        stage.load(nrows(nxt), src_of(nxt, 2));
        stage.store(nrows(nxt), src_of(nxt, 2), dst_of(nxt, 2));
      } else {
        stage.store(nrows(nxt), src_of(nxt, nxt.d + 2), dst_of(nxt, nxt.d + 2));
      }
      __syncthreads();
      cur = nxt;
    }
  }
}

template <bool VL, bool VS, bool SER>
int launch_instance(const Conv3dArgs &a, size_t lds_bytes, const DeviceInfo &dev,
                    hipStream_t stream) {
  auto kern = conv3d_lrelu_add_clamp_gelu_kernel<VL, VS, SER, kPrefetchPasses>;
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

template <bool VL, bool VS>
int launch_series(const Conv3dArgs &a, size_t lds_bytes, const DeviceInfo &dev,
                  hipStream_t stream) {
  const bool series = a.lo >= -1.0f && a.hi <= 1.0f;
  return series ? launch_instance<VL, VS, true>(a, lds_bytes, dev, stream)
                : launch_instance<VL, VS, false>(a, lds_bytes, dev, stream);
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
  a.divDo = make_fastdiv((uint32_t)a.Do);
  a.divRowtiles = make_fastdiv((uint32_t)a.rowtiles);
  a.divWo = make_fastdiv((uint32_t)a.Wo);

  const bool vl = (W % 4 == 0) && ((uintptr_t)x % 16 == 0);
  const bool vs = ((a.Ho * a.Wo) % 4 == 0) && ((a.TR * a.Wo) % 4 == 0) && ((uintptr_t)y % 16 == 0);
  if (vl) return vs ? launch_series<true, true>(a, lds_bytes, dev, stream)
                    : launch_series<true, false>(a, lds_bytes, dev, stream);
  return vs ? launch_series<false, true>(a, lds_bytes, dev, stream)
            : launch_series<false, false>(a, lds_bytes, dev, stream);
}

}  // namespace cce
