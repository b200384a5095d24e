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
  const float *wprep; // prepared weight, NCHUNK x WS_FLOATS
  int H, W, PH, PW;
  int tiles_x, tiles_per_image;
  float lo, hi, inv_count;
};

// Per-chunk staging in 16-byte units.  The weight slice of chunk c is
// contiguous in the prepared layout; the input tile's 32 interior columns of
// each (channel, row) are four-aligned in the image (w0 % 32 == 0, W % 4 == 0)
// and land on four-aligned LDS columns (XOFF + 1 = 4); the two halo columns
// are single floats.
constexpr int W4_PER_CHUNK = WS_FLOATS / 4;                        // 1152
constexpr int W4_PT = (W4_PER_CHUNK + THREADS - 1) / THREADS;      // 5
constexpr int XQ = TW / 4;                                         // 8 float4 per row
constexpr int X4_PER_CHUNK = CC * XR * XQ;                         // 1152
constexpr int X4_PT = (X4_PER_CHUNK + THREADS - 1) / THREADS;      // 5
constexpr int XH_PER_CHUNK = CC * XR * 2;                          // 288 halo floats
constexpr int XH_PT = (XH_PER_CHUNK + THREADS - 1) / THREADS;      // 2
static_assert(XOFF + 1 == 4, "interior columns start 16-byte aligned in LDS");

struct ChunkRegs {
  v4f w4[W4_PT];
  v4f x4[X4_PT];
  float xh[XH_PT];
};

// Global -> registers for channel chunk c (issued a whole chunk ahead of use).
// VEC: W % 4 == 0 and x 16-byte aligned, so each interior quad is one aligned
// 16-byte load that is either wholly inside the row or wholly past its end.
template <bool VEC>
__device__ __forceinline__ void load_chunk(const ConvTArgs &a, int n, int c, int h0, int w0, int tid,
                                           ChunkRegs &r) {
  const v4f *wsrc = reinterpret_cast<const v4f *>(a.wprep) + (size_t)c * W4_PER_CHUNK;
#pragma unroll
  for (int j = 0; j < W4_PT; ++j) {
    const int i = tid + j * THREADS;
    if (i < W4_PER_CHUNK) r.w4[j] = wsrc[i];
  }
  const float *xc = a.x + ((size_t)n * CI + CC * c) * a.H * a.W;
#pragma unroll
  for (int j = 0; j < X4_PT; ++j) {
    const int i = tid + j * THREADS;
    v4f v = splat4(0.0f);
    if (i < X4_PER_CHUNK) {
      const int row = i / XQ, q = i - row * XQ;  // row = cl * XR + rr
      const int cl = row / XR, rr = row - cl * XR;
      const int h = h0 - 1 + rr, wc = w0 + 4 * q;
      if (h >= 0 && h < a.H) {
        const float *src = xc + ((size_t)cl * a.H + h) * a.W + wc;
        if (VEC) {
          if (wc < a.W) v = *reinterpret_cast<const v4f *>(src);
        } else {
          if (wc < a.W) v.x = src[0];
          if (wc + 1 < a.W) v.y = src[1];
          if (wc + 2 < a.W) v.z = src[2];
          if (wc + 3 < a.W) v.w = src[3];
        }
      }
    }
    r.x4[j] = v;
  }
#pragma unroll
  for (int j = 0; j < XH_PT; ++j) {
    const int i = tid + j * THREADS;
    float v = 0.0f;
    if (i < XH_PER_CHUNK) {
      const int row = i >> 1, side = i & 1;
      const int cl = row / XR, rr = row - cl * XR;
      const int h = h0 - 1 + rr, wc = side ? w0 + TW : w0 - 1;
      if (h >= 0 && h < a.H && wc >= 0 && wc < a.W) v = xc[((size_t)cl * a.H + h) * a.W + wc];
    }
    r.xh[j] = v;
  }
}

// Registers -> LDS.
__device__ __forceinline__ void store_chunk(float *xs, float *ws, int tid, const ChunkRegs &r) {
#pragma unroll
  for (int j = 0; j < W4_PT; ++j) {
    const int i = tid + j * THREADS;
    if (i < W4_PER_CHUNK) reinterpret_cast<v4f *>(ws)[i] = r.w4[j];
  }
#pragma unroll
  for (int j = 0; j < X4_PT; ++j) {
    const int i = tid + j * THREADS;
    if (i < X4_PER_CHUNK) {
      const int row = i / XQ, q = i - row * XQ;
      const int cl = row / XR, rr = row - cl * XR;
      *reinterpret_cast<v4f *>(&xs[cl * XCS + rr * XRS + XOFF + 1 + 4 * q]) = r.x4[j];
    }
  }
#pragma unroll
  for (int j = 0; j < XH_PT; ++j) {
    const int i = tid + j * THREADS;
    if (i < XH_PER_CHUNK) {
      const int row = i >> 1, side = i & 1;
      const int cl = row / XR, rr = row - cl * XR;
      xs[cl * XCS + rr * XRS + (side ? XOFF + 1 + TW : XOFF)] = r.xh[j];
    }
  }
}

// Weight preparation (once per call, 36,864 floats): the flipped, channel-
// swapped kernel in exactly the LDS B-operand order of every chunk,
//   wprep[c][cb][tap'][lane][nt] = W[8c + 4cb + lane/16][16nt + lane%16][8 - tap'],
// where tap' = 3 kh' + kw' and W's tap index 3 kh + kw = 8 - tap'.
__global__ __launch_bounds__(THREADS) void convT_prepare_weight_kernel(const float *__restrict__ w,
                                                                      float *__restrict__ wprep) {
  const int p = blockIdx.x * THREADS + threadIdx.x;
  if (p >= NCHUNK * WS_FLOATS) return;
  const int nt = p & 3, lane = (p >> 2) & 63, rest = p >> 8;  // rest = (c * 2 + cb) * 9 + tap
  const int tap = rest % 9, ccb = rest / 9;                    // ccb = c * 2 + cb
  const int ci = 4 * ccb + (lane >> 4), o = 16 * nt + (lane & 15);
  wprep[p] = w[((size_t)ci * CO + o) * 9 + (8 - tap)];
}

template <bool VEC>
__global__ __launch_bounds__(THREADS, 2) void convT2d_pool_htanh_mean_tanh_kernel(ConvTArgs a) {
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

  ChunkRegs r;
  load_chunk<VEC>(a, n, 0, h0, w0, tid, r);
  store_chunk(xs, ws, tid, r);
  __syncthreads();

#pragma unroll 1
  for (int c = 0; c < NCHUNK; ++c) {
    // Next chunk's global loads are in flight while this chunk's MFMAs run.
    if (c + 1 < NCHUNK) load_chunk<VEC>(a, n, c + 1, h0, w0, tid, r);
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
    if (c + 1 < NCHUNK) {
      __syncthreads();  // every wave is done reading chunk c
      store_chunk(xs, ws, tid, r);
      __syncthreads();
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
constexpr size_t kWprepBytes = (size_t)NCHUNK * WS_FLOATS * sizeof(float);  // 147,456

void convT_tiles(int H, int W, int *tiles_x, int *tiles_per_image) {
  const int PH = H / 2, PW = W / 2;
  *tiles_x = (PW + PTW - 1) / PTW;
  *tiles_per_image = ((PH + PTH - 1) / PTH) * *tiles_x;
}

}  // namespace

// Workspace: [per-image counters, padded to 256 B][prepared weight][partials].
size_t convT_workspace_bytes(int N, int H, int W) {
  int tx, tpi;
  convT_tiles(H, W, &tx, &tpi);
  const size_t tick = ((size_t)N * sizeof(unsigned) + kTicketAlign - 1) / kTicketAlign * kTicketAlign;
  return tick + kWprepBytes + (size_t)N * tpi * 64 * sizeof(float);
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
  char *wsp = reinterpret_cast<char *>(workspace);
  float *wprep = reinterpret_cast<float *>(wsp + tick);
  a.tickets = reinterpret_cast<unsigned *>(wsp);
  a.wprep = wprep;
  a.partials = reinterpret_cast<float *>(wsp + tick + kWprepBytes);
  const long long grid = (long long)N * a.tiles_per_image;
  if (grid >= (1LL << 31)) return CCE_ERR_TOO_LARGE;
  hipLaunchKernelGGL(convT_prepare_weight_kernel, dim3(NCHUNK * WS_FLOATS / THREADS), dim3(THREADS),
                     0, stream, w, wprep);
  if (launch_status() != CCE_OK) return CCE_ERR_LAUNCH;
  const bool vec = (W % 4 == 0) && ((uintptr_t)x % 16 == 0);
  if (vec)
    hipLaunchKernelGGL(convT2d_pool_htanh_mean_tanh_kernel<true>, dim3((unsigned)grid), dim3(THREADS),
                       0, stream, a);
  else
    hipLaunchKernelGGL(convT2d_pool_htanh_mean_tanh_kernel<false>, dim3((unsigned)grid),
                       dim3(THREADS), 0, stream, a);
  return launch_status();
}

}  // namespace cce
