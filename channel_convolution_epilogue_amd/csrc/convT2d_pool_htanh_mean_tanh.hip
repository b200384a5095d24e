// ConvTranspose2d 3x3, stride 1, padding 1, 64 -> 64 channels, + bias ->
// MaxPool2d(2, 2) -> Hardtanh[lo, hi] -> mean over (H, W) -> tanh, fused in one
// gfx950 kernel (POPCORNBENCH Kimi-K2.6 l2_p10).  The 64 x H x W conv result
// and the pooled map never reach memory; each workgroup leaves 64 partial
// sums and the last workgroup of an image writes y[n, 0..63].
//
// Algebra (l2_p10's derivation of the stride-1 transposed conv): with
// padding 1, output pixel (h, w) gathers x[i, h + 1 - kh, w + 1 - kw] *
// W[i, o, kh, kw]; substituting kh' = 2 - kh turns it into a correlation
//   z[o, h, w] = b[o] + sum_{i, kh', kw'} x[i, h - 1 + kh', w - 1 + kw'] * W[i, o, 2 - kh', 2 - kw']
// with the kernel flipped and its channel axes swapped.  The flip and swap
// are applied when the weight is staged into LDS.
//
// Design:
//  * Implicit GEMM on the fp32 matrix cores: M = conv-output pixels, N = 64
//    output channels, K = 64 channels x 9 taps = 576.  A tile is 16 x 32
//    conv pixels (8 x 16 pooling windows) of one image; K is walked in 8
//    chunks of 8 input channels whose input halo tile (18 x 34) and weight
//    slice (8 x 9 x 64) are staged in LDS.
//  * The M order puts the four pixels of one 2 x 2 pooling window on four
//    consecutive M rows, which the matrix core returns in one lane's four
//    accumulator registers: the max-pool is three in-lane max operations.
//  * Bias is added after the max (rounding is monotone, so max(z) + b equals
//    max(z + b) exactly), then Hardtanh, then the window sums are reduced
//    lane -> wave (cross-lane shuffles) -> workgroup (LDS).
//  * Each workgroup stores its 64 partial sums and bumps a per-image counter
//    (agent-scope acquire/release); the workgroup that completes an image
//    adds that image's partials in a fixed order, applies mean and tanh, and
//    resets the counter.  The result is deterministic.
#include "cce_device.hpp"
#include "cce_internal.hpp"

namespace cce {
namespace {

constexpr int CI = 64, CO = 64, NT = CO / 16;
constexpr int WAVES = 4, THREADS = 64 * WAVES;
constexpr int TH = 16, TW = 32;             // conv-output pixels per tile
constexpr int PTH = TH / 2, PTW = TW / 2;   // pooling windows per tile
constexpr int CC = 8, NCHUNK = CI / CC;     // input channels per K chunk
constexpr int XR = TH + 2, XC = TW + 2;     // input halo tile rows / cols
constexpr int XRS = 40;                     // LDS row stride: 8 (mod 64) banks between rows
constexpr int XCS = XR * XRS;               // 720 = 16 (mod 64): lane groups 16 banks apart
constexpr int XOFF = 3;                     // LDS column of input column w0 - 1
constexpr int XS_FLOATS = CC * XCS;
constexpr int WS_FLOATS = (CC / 4) * 9 * 64 * NT;
constexpr int MT = 8;                       // 16-pixel blocks per wave

static_assert(XOFF + XC <= XRS, "halo row fits the LDS row");

struct ConvTArgs {
  const float *__restrict__ x;
  const float *__restrict__ w;
  const float *__restrict__ b;
  float *__restrict__ y;
  unsigned *tickets;  // [N] per-image completion counters (zero between calls)
  float *partials;    // [N][tiles_per_image][64]
  int H, W, PH, PW;
  int tiles_x, tiles_per_image;
  float lo, hi, inv_count;
};

__global__ __launch_bounds__(THREADS) void convT2d_pool_htanh_mean_tanh_kernel(ConvTArgs a) {
  __shared__ __attribute__((aligned(16))) float xs[XS_FLOATS];
  __shared__ __attribute__((aligned(16))) float ws[WS_FLOATS];
  __shared__ float red[WAVES][64];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int n = blockIdx.x / a.tiles_per_image;
  const int ti = blockIdx.x - n * a.tiles_per_image;
  const int ty = ti / a.tiles_x, tx = ti - ty * a.tiles_x;
  const int h0 = ty * TH, w0 = tx * TW;

  // A-operand lane: M row m = col -> pooling window col/4 of the block, pixel
  // (dh, dw) = ((col & 3) >> 1, col & 1) inside it; lane group g = channel.
  const int wi = col >> 2, dh = (col & 3) >> 1, dw = col & 1;
  const int abase = g * XCS + (4 * wave + dh) * XRS + XOFF + 2 * wi + dw;

  v4f acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = splat4(0.0f);

#pragma unroll 1
  for (int c = 0; c < NCHUNK; ++c) {
    __syncthreads();  // previous chunk's LDS reads are done
    // Input halo tile of channels 8c..8c+7, zero outside the image (padding 1).
    for (int idx = tid; idx < CC * XR * XC; idx += THREADS) {
      const int cl = idx / (XR * XC), rem = idx - cl * (XR * XC);
      const int rr = rem / XC, cc = rem - rr * XC;
      const int h = h0 - 1 + rr, wc = w0 - 1 + cc;
      float v = 0.0f;
      if (h >= 0 && h < a.H && wc >= 0 && wc < a.W)
        v = a.x[(((size_t)n * CI + CC * c + cl) * a.H + h) * a.W + wc];
      xs[cl * XCS + rr * XRS + XOFF + cc] = v;
    }
    // Weight slice, flipped and swapped into B-operand order:
    // ws[cb][tap'][lane][nt] = W[8c + 4cb + lane/16][16nt + lane%16][2-kh'][2-kw'].
    for (int e = tid; e < CC * CO * 9; e += THREADS) {
      const int cl = e / (CO * 9), rem = e - cl * (CO * 9);
      const int o = rem / 9, t = rem - o * 9;
      const int tapf = 8 - t;  // (2 - kh) * 3 + (2 - kw)
      const int ln = 16 * (cl & 3) + (o & 15);
      ws[(((cl >> 2) * 9 + tapf) * 64 + ln) * NT + (o >> 4)] = a.w[((size_t)(CC * c + cl) * CO + o) * 9 + t];
    }
    __syncthreads();

#pragma unroll
    for (int cb = 0; cb < CC / 4; ++cb) {
#pragma unroll
      for (int tap = 0; tap < 9; ++tap) {
        const int kh = tap / 3, kw = tap % 3;
        const v4f bv = *reinterpret_cast<const v4f *>(&ws[((cb * 9 + tap) * 64 + lane) * NT]);
        float av[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          av[mt] = xs[abase + cb * 4 * XCS + (2 * (mt >> 2) + kh) * XRS + 8 * (mt & 3) + kw];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt][0] = mfma16x16x4(av[mt], bv.x, acc[mt][0]);
          acc[mt][1] = mfma16x16x4(av[mt], bv.y, acc[mt][1]);
          acc[mt][2] = mfma16x16x4(av[mt], bv.z, acc[mt][2]);
          acc[mt][3] = mfma16x16x4(av[mt], bv.w, acc[mt][3]);
        }
      }
    }
  }

  // Epilogue: lane holds, per block and channel block, the 4 pixels of pooling
  // window (ph, pw) = (ph0 + 2 wave + mt/4, pw0 + 4 (mt%4) + g), channel 16 nt + col.
  float bias[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) bias[nt] = a.b ? a.b[16 * nt + col] : 0.0f;
  float sum[NT] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int ph0 = ty * PTH, pw0 = tx * PTW;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int ph = ph0 + 2 * wave + (mt >> 2), pw = pw0 + 4 * (mt & 3) + g;
    const bool valid = ph < a.PH && pw < a.PW;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const v4f v = acc[mt][nt];
      const float m = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
      const float q = clampf(m + bias[nt], a.lo, a.hi);
      sum[nt] += valid ? q : 0.0f;
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    sum[nt] += __shfl_xor(sum[nt], 16);
    sum[nt] += __shfl_xor(sum[nt], 32);
  }
  if (g == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) red[wave][16 * nt + col] = sum[nt];
  }
  __syncthreads();
  if (tid < 64) {
    const float tot = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    __hip_atomic_store(&a.partials[((size_t)n * a.tiles_per_image + ti) * 64 + tid], tot,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const unsigned done = __hip_atomic_fetch_add(&a.tickets[n], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (done == (unsigned)a.tiles_per_image - 1u);
  }
  __syncthreads();
  if (!last_flag) return;

  // Last workgroup of image n: all partials of the image are visible.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  {
    const int o = tid & 63, part = tid >> 6;
    const float *pp = a.partials + (size_t)n * a.tiles_per_image * 64 + o;
    float s = 0.0f;
    for (int t = part; t < a.tiles_per_image; t += WAVES)
      s += __hip_atomic_load(pp + (size_t)t * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    red[part][o] = s;
  }
  __syncthreads();
  if (tid < 64) {
    const float tot = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    a.y[(size_t)n * CO + tid] = tanhf(tot * a.inv_count);
  }
  if (tid == 0)
    __hip_atomic_store(&a.tickets[n], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr size_t kTicketAlign = 256;

void convT_tiles(int H, int W, int *tiles_x, int *tiles_per_image) {
  const int PH = H / 2, PW = W / 2;
  *tiles_x = (PW + PTW - 1) / PTW;
  *tiles_per_image = ((PH + PTH - 1) / PTH) * *tiles_x;
}

}  // namespace

size_t convT_workspace_bytes(int N, int H, int W) {
  int tx, tpi;
  convT_tiles(H, W, &tx, &tpi);
  const size_t tick = ((size_t)N * sizeof(unsigned) + kTicketAlign - 1) / kTicketAlign * kTicketAlign;
  return tick + (size_t)N * tpi * 64 * sizeof(float);
}

int launch_convT2d_pool_htanh_mean_tanh(const float *x, const float *w, const float *b, float *y,
                                        int N, int H, int W, float lo, float hi, void *workspace,
                                        hipStream_t stream) {
  ConvTArgs a;
  a.x = x;
  a.w = w;
  a.b = b;
  a.y = y;
  a.H = H;
  a.W = W;
  a.PH = H / 2;  // conv output is H x W at stride 1, padding 1; floor pooling
  a.PW = W / 2;
  convT_tiles(H, W, &a.tiles_x, &a.tiles_per_image);
  a.lo = lo;
  a.hi = hi;
  a.inv_count = (float)(1.0 / ((double)a.PH * (double)a.PW));
  const size_t tick = ((size_t)N * sizeof(unsigned) + kTicketAlign - 1) / kTicketAlign * kTicketAlign;
  a.tickets = reinterpret_cast<unsigned *>(workspace);
  a.partials = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + tick);
  const long long grid = (long long)N * a.tiles_per_image;
  if (grid >= (1LL << 31)) return CCE_ERR_TOO_LARGE;
  hipLaunchKernelGGL(convT2d_pool_htanh_mean_tanh_kernel, dim3((unsigned)grid), dim3(THREADS), 0,
                     stream, a);
  return launch_status();
}

}  // namespace cce
