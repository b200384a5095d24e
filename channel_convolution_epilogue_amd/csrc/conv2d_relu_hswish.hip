// Conv2d 3x3, 8 -> 64 channels, stride 1, padding 0, + bias -> ReLU -> HardSwish,
// fused in one gfx950 kernel (POPCORNBENCH Kimi-K2.6 l2_p57: its model is
// Conv2d(8, 64, 3) followed by ReLU and HardSwish x * clamp((x + 3) / 6, 0, 1)).
//
// Design (MI355X-first, not the page's one-thread-per-output CUDA tiling):
//  * Implicit GEMM on the fp32 matrix cores: M = output pixels, N = the 64
//    output channels, K = 8 channels x 9 taps = 72.  Packed fp32 VALU math is
//    not used, so the matrix cores are the only units that reach the fp32
//    peak; the contraction is dense enough (72 x 64 per pixel) to feed them.
//  * Output pixels are numbered flat over (n, h, w) and cut into tiles of
//    256.  A flat numbering keeps every lane's four result pixels 16-byte
//    aligned even though the 126-wide rows are not, so results leave as
//    16-byte stores, and no tile is ragged except the last one.
//  * A tile's input rows (all 8 channels, full width) are staged in LDS;
//    each 16-pixel block reads one A value per lane per K-step from LDS.  The
//    K order puts the four lane groups on four input channels and one
//    (channel half, kh, kw) per step, so the step's LDS offset is the same for
//    all lanes.  The 72 x 64 weight sits in LDS in B-operand order: one
//    16-byte read per K-step serves all four 16-channel blocks.
//  * Workgroups of 8 waves are persistent (4 waves per SIMD) and take tiles
//    round-robin, remapped so each XCD runs consecutive tiles; the next
//    tile's input rows are loaded into registers during the current tile's
//    MFMAs.  The waves' 16-pixel blocks interleave, so a workgroup writes
//    one contiguous run of every channel plane per round.
//  * Bias is the accumulator's initial value; ReLU and HardSwish are applied
//    in registers before the store: the conv result never reaches memory.
#include "cce_device.hpp"
#include "cce_internal.hpp"

namespace cce {
namespace {

constexpr int CI = 8, CO = 64, KS = 3, TAPS = KS * KS;
constexpr int KSTEPS = (CI / 4) * TAPS;  // 18 steps of 4 taps
constexpr int NT = CO / 16;              // 4 channel blocks of 16
constexpr int WAVES = 8, THREADS = 64 * WAVES;
constexpr int MT_BATCH = 2;              // 16-pixel blocks in flight per wave
constexpr int WS_FLOATS = KSTEPS * 64 * NT;  // weights in LDS, B-operand order (18 KB)
constexpr int kPrefetchPasses = 4;       // a 256-pixel tile of 128-wide rows stages <= 64 rows, 16 per pass

struct Conv2dArgs {
  const float *__restrict__ x;
  const float *__restrict__ w;
  const float *__restrict__ b;
  float *__restrict__ y;
  int H, W, Wo;
  int P;         // output pixels per image plane, (H-2)*(W-2)
  int Q;         // output pixels over the batch, N*P
  int ntiles;    // ceil(Q / tile)
  int chstride;  // floats between channel planes in LDS
  FastDiv divP, divWo, divH;
};

// HardSwish(ReLU(v)) = r * clamp((r + 3) / 6, 0, 1) with r = max(v, 0).  For
// v >= 0 the gate (v + 3) / 6 is at least 0.5, and for v < 0 the result is 0
// whatever the gate, so the gate can be taken from v itself, clamped to
// [0.5, 1], and the ReLU applied to the (positive-gated) product:
// max(v * gate, 0) = max(v, 0) * gate.  Four operations.
__device__ __forceinline__ float relu_hswish(float v) {
  const float gate = __builtin_amdgcn_fmed3f(fmaf(v, 1.0f / 6.0f, 0.5f), 0.5f, 1.0f);
  return fmaxf(v * gate, 0.0f);
}

// Input rows of one tile: flat output pixels [q0, q0 + TILE) need input rows
// r = n * H + h from r_first to r_first + R - 1 of all 8 channels.
struct TileRows {
  int q0, r_first, R;
};

// Staged row `row` = rr * 8 + ci  <->  input row r_first + rr of channel ci.
struct Conv2dSrc {
  const float *x;
  int H, W, r_first;
  FastDiv divH;
  __device__ __forceinline__ const float *operator()(int row) const {
    const int ci = row & (CI - 1), rr = row >> 3;
    const int r = r_first + rr, n = fdiv(r, divH), hh = r - n * H;
    return x + (((size_t)n * CI + ci) * H + hh) * W;
  }
};
struct Conv2dDst {
  float *lds;
  int chstride, W;
  __device__ __forceinline__ float *operator()(int row) const {
    return lds + (row & (CI - 1)) * chstride + (row >> 3) * W;
  }
};

// MT_WAVE: 16-pixel blocks per wave per tile (tile = 16 * MT_WAVE * WAVES pixels).
// VLOAD: W % 4 == 0 and x 16-byte aligned (16-byte row loads).
// VSTORE: P % 4 == 0 and y 16-byte aligned (16-byte result stores).
// KPRE: staged row passes held in registers while the previous tile computes.
template <int MT_WAVE, bool VLOAD, bool VSTORE, int KPRE>
__global__ __launch_bounds__(THREADS, 4) void conv2d_relu_hswish_kernel(Conv2dArgs a) {
  constexpr int TILE = 16 * MT_WAVE * WAVES;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  float *ws = lds;              // weights in B-operand order, WS_FLOATS
  float *xs = lds + WS_FLOATS;  // input rows, 8 channel planes of chstride floats
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;

  // B operand of K-step s = (half, kh, kw) for all four 16-channel blocks:
  // ws[s][lane][nt] = w[16 nt + lane % 16][4 half + lane / 16][kh][kw].
  for (int e = tid; e < WS_FLOATS; e += THREADS) {
    const int nt = e & 3, ln = (e >> 2) & 63, st = e >> 8;
    const int o = 16 * nt + (ln & 15), ci = 4 * (st / TAPS) + (ln >> 4);
    ws[e] = a.w[(o * CI + ci) * TAPS + (st % TAPS)];
  }
  float bias[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) bias[nt] = a.b ? a.b[16 * nt + col] : 0.0f;

  // Tiles are dealt round-robin, so the workgroups running at any moment
  // write neighbouring stretches of the same output channel planes.  The
  // hardware hands workgroups to the 8 XCDs in turn (b -> XCD b % 8); the
  // remap gives each XCD a contiguous block of each round's tiles, so one
  // L2 collects long runs of every plane.  (gridDim.x is a multiple of 8.)
  const int per_xcd = gridDim.x >> 3;
  const int t_begin = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3), t_step = gridDim.x;
  if (t_begin >= a.ntiles) return;

  auto rows_of = [&](int t) {
    TileRows tr;
    tr.q0 = t * TILE;
    const int qlast = min(tr.q0 + TILE, a.Q) - 1;
    const int n0 = fdiv(tr.q0, a.divP), n1 = fdiv(qlast, a.divP);
    tr.r_first = n0 * a.H + fdiv(tr.q0 - n0 * a.P, a.divWo);
    tr.R = n1 * a.H + fdiv(qlast - n1 * a.P, a.divWo) + (KS - 1) - tr.r_first + 1;
    return tr;
  };
  auto src_of = [&](const TileRows &tr) { return Conv2dSrc{a.x, a.H, a.W, tr.r_first, a.divH}; };
  auto dst_of = [&](const TileRows &) { return Conv2dDst{xs, a.chstride, a.W}; };

  RowStage<KPRE, VLOAD, THREADS> stage;
  stage.init(a.W, tid);
  TileRows cur = rows_of(t_begin);
  stage.load(CI * cur.R, src_of(cur));
  stage.store(CI * cur.R, src_of(cur), dst_of(cur));
  __syncthreads();

  for (int t = t_begin; t < a.ntiles; t += t_step) {
    const bool more = t + t_step < a.ntiles;
    TileRows nxt = cur;
    if (more) {
      nxt = rows_of(t + t_step);
      stage.load(CI * nxt.R, src_of(nxt));  // in flight during this tile's MFMAs
    }
    const int q0 = cur.q0, r_first = cur.r_first;

#pragma unroll 1
    for (int mb = 0; mb < MT_WAVE; mb += MT_BATCH) {
      // Compiler-only fence: keeps the per-step weight reads inside the loop
      // instead of hoisting all 18 of them (72 VGPRs) out of it.
      asm volatile("" ::: "memory");
      // The waves' blocks interleave: together they cover one contiguous run
      // of 16 * MT_BATCH * WAVES pixels per round.
      const int blk0 = (mb / MT_BATCH * WAVES + wave) * MT_BATCH;
      int base[MT_BATCH];
#pragma unroll
      for (int j = 0; j < MT_BATCH; ++j) {
        int q = q0 + 16 * (blk0 + j) + col;
        q = min(q, a.Q - 1);  // lanes past the end read a valid pixel; their results are dropped
        const int n = fdiv(q, a.divP), p = q - n * a.P, h = fdiv(p, a.divWo), w = p - h * a.Wo;
        base[j] = g * a.chstride + (n * a.H + h - r_first) * a.W + w;
      }
      v4f acc[MT_BATCH][NT];
#pragma unroll
      for (int j = 0; j < MT_BATCH; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[j][nt] = splat4(bias[nt]);

#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int tap = s % TAPS;
        const int off = (s / TAPS) * 4 * a.chstride + (tap / KS) * a.W + (tap % KS);
        const v4f bv = *reinterpret_cast<const v4f *>(&ws[(s * 64 + lane) * NT]);
        float av[MT_BATCH];
#pragma unroll
        for (int j = 0; j < MT_BATCH; ++j) av[j] = xs[base[j] + off];
#pragma unroll
        for (int j = 0; j < MT_BATCH; ++j) {
          acc[j][0] = mfma16x16x4(av[j], bv.x, acc[j][0]);
          acc[j][1] = mfma16x16x4(av[j], bv.y, acc[j][1]);
          acc[j][2] = mfma16x16x4(av[j], bv.z, acc[j][2]);
          acc[j][3] = mfma16x16x4(av[j], bv.w, acc[j][3]);
        }
      }

#pragma unroll
      for (int j = 0; j < MT_BATCH; ++j) {
        const int qq = q0 + 16 * (blk0 + j) + 4 * g;  // this lane's first pixel
        if (qq >= a.Q) continue;
        if (VSTORE) {
          // P % 4 == 0 and Q % 4 == 0: the four pixels are in one plane and all valid.
          const int n = fdiv(qq, a.divP), p = qq - n * a.P;
          float *dst = a.y + (size_t)n * CO * a.P + p;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            v4f v = acc[j][nt];
            v.x = relu_hswish(v.x);
            v.y = relu_hswish(v.y);
            v.z = relu_hswish(v.z);
            v.w = relu_hswish(v.w);
            store4(dst + (size_t)(16 * nt + col) * a.P, v);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int qr = qq + r;
            if (qr >= a.Q) break;
            const int n = fdiv(qr, a.divP), p = qr - n * a.P;
            float *dst = a.y + (size_t)n * CO * a.P + p;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              dst[(size_t)(16 * nt + col) * a.P] = relu_hswish(acc[j][nt][r]);
          }
        }
      }
    }

    if (more) {
      __syncthreads();  // every wave is done reading this tile's rows
      stage.store(CI * nxt.R, src_of(nxt), dst_of(nxt));
      __syncthreads();
      cur = nxt;
    }
  }
}

template <int MT_WAVE, bool VL, bool VS>
int launch_instance(const Conv2dArgs &a, int R_max, hipStream_t stream) {
  constexpr int TILE = 16 * MT_WAVE * WAVES;
  (void)TILE;
  DeviceInfo dev;
  if (current_device_info(&dev) != CCE_OK) return CCE_ERR_LAUNCH;
  const size_t lds_bytes = ((size_t)WS_FLOATS + (size_t)CI * a.chstride) * sizeof(float);
  (void)R_max;
  if (lds_bytes > dev.lds_per_block) return CCE_ERR_UNSUPPORTED;
  auto kern = conv2d_relu_hswish_kernel<MT_WAVE, VL, VS, kPrefetchPasses>;
  if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)lds_bytes) != hipSuccess)
    return CCE_ERR_LAUNCH;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, THREADS, lds_bytes) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int grid = dev.num_cus * per_cu;
  if (grid > a.ntiles) grid = a.ntiles;
  grid = (grid + 7) & ~7;  // the XCD remap needs a multiple of 8; surplus workgroups exit
  hipLaunchKernelGGL(kern, dim3(grid), dim3(THREADS), lds_bytes, stream, a);
  return launch_status();
}

}  // namespace

int launch_conv2d_relu_hswish(const float *x, const float *w, const float *b, float *y, int N,
                              int H, int W, hipStream_t stream) {
  Conv2dArgs a;
  a.x = x;
  a.w = w;
  a.b = b;
  a.y = y;
  a.H = H;
  a.W = W;
  a.Wo = W - (KS - 1);
  const int Ho = H - (KS - 1);
  a.P = Ho * a.Wo;
  a.Q = N * a.P;
  a.divP = make_fastdiv((uint32_t)a.P);
  a.divWo = make_fastdiv((uint32_t)a.Wo);
  a.divH = make_fastdiv((uint32_t)H);

  DeviceInfo dev;
  if (current_device_info(&dev) != CCE_OK) return CCE_ERR_LAUNCH;
  // Tiles of 256 pixels (8 waves x 2 blocks of 16).  Measured on MI355X at
  // N = 128: 256-pixel tiles 0.222 ms, 512: 0.227 ms, 1024: 0.234 ms -- with
  // round-robin tiles, smaller tiles keep the concurrently written stretches
  // of each output plane closer together.
  const int tile = 256;
  a.ntiles = (a.Q + tile - 1) / tile;

  // Upper bound on the input rows one tile touches: output rows spanned plus
  // (k - 1) halo rows for every image the tile reaches into.
  const int rows_spanned = (tile - 1 + a.Wo - 1) / a.Wo + 1;
  const int images_spanned = (tile - 1 + a.P - 1) / a.P + 1;
  int R_max = rows_spanned + (KS - 1) * images_spanned;
  if (R_max > N * H) R_max = N * H;
  // Channel planes padded so the four lane groups (four channels) of a read
  // start 16 banks apart.
  int plane = R_max * W;
  a.chstride = plane + ((16 - plane % 64) + 64) % 64;

  const bool vl = (W % 4 == 0) && ((uintptr_t)x % 16 == 0);
  const bool vs = (a.P % 4 == 0) && ((uintptr_t)y % 16 == 0);
  if (vl) return vs ? launch_instance<2, true, true>(a, R_max, stream)
                    : launch_instance<2, true, false>(a, R_max, stream);
  return vs ? launch_instance<2, false, true>(a, R_max, stream)
            : launch_instance<2, false, false>(a, R_max, stream);
}

}  // namespace cce
