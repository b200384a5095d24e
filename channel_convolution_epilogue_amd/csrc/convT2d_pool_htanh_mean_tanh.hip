// ConvTranspose2d 3x3, stride 1, padding 1, C_in -> C_out channels, + bias ->
// MaxPool2d(2, 2) -> Hardtanh[lo, hi] -> mean over (H, W) -> tanh, fused in one
// gfx950 kernel (POPCORNBENCH Kimi-K2.6 l2_p10, whose layer is 64 -> 64).  The
// C_out x H x W conv result and the pooled map never reach memory; each
// workgroup leaves C_out partial sums and the last workgroup of an image
// writes y[n, 0..C_out-1].
//
// Algebra (l2_p10's derivation of the stride-1 transposed conv): with
// padding 1, output pixel (h, w) gathers x[i, h + 1 - kh, w + 1 - kw] *
// W[i, o, kh, kw]; substituting kh' = 2 - kh turns it into a correlation
//   z[o, h, w] = b[o] + sum_{i, kh', kw'} x[i, h - 1 + kh', w - 1 + kw'] * W[i, o, 2 - kh', 2 - kw']
// with the kernel flipped and its channel axes swapped.  The flip and swap
// are applied when the weight is staged into LDS.
//
// Design:
//  * Implicit GEMM on the fp32 matrix cores: M = conv-output pixels, N =
//    C_out output channels (16, 32 or 64: one to four 16-column MFMA
//    blocks), K = C_in channels x 9 taps (576 for the page's layer).  A tile
//    is 16 x 32 conv pixels (8 x 16 pooling windows) of one image for 64 or
//    32 output channels (32 x 32 for 16); K is walked in
//    C_in / 8 chunks of 8 input channels whose input halo tile (18 x 34 for
//    64 channels) and weight slice (8 x 9 x C_out) are staged in LDS.
//  * The M order puts the four pixels of one 2 x 2 pooling window on four
//    consecutive M rows, which the matrix core returns in one lane's four
//    accumulator registers: the max-pool is three in-lane max operations.
//  * Bias is added after the max (rounding is monotone, so max(z) + b equals
//    max(z + b) exactly), then Hardtanh, then the window sums are reduced
//    lane -> wave (cross-lane shuffles) -> workgroup (LDS).
//  * Each workgroup stores its 64 partial sums and bumps a per-image counter
//    (an agent-scope release); the workgroup that completes an image
//    acquires, adds that image's partials in a fixed order and applies mean
//    and tanh.
//    The result is deterministic.  A small kernel launched just before the
//    main one zeroes the counters and writes the prepared weight.
//  * XCD-aware tile order: each of the 8 XCDs takes one contiguous range of
//    tiles, so the tiles that share halo rows and columns, and the weight
//    chunks every tile reads, meet in the same L2.  Measured on MI355X at
//    N = 16: HBM reads fall from 2.78x to 1.03x the input's size, and the
//    kernel takes 0.573 instead of 0.588 ms (bit-identical results).
#include "cce_device.hpp"
#include "cce_internal.hpp"

// Scratch of convT2d_pool_htanh_mean_tanh_noalloc, the entry point for
// callers that cannot allocate device memory: what the workspace holds for
// the other entry point (counters, prepared weight, partial sums), in a
// file-scope device array.  Each GPU the library runs on holds its own copy
// until the process ends; host code uses the per-device address that
// hipGetSymbolAddress returns, never this name.
static __device__ __align__(256) unsigned char scratch[CCE_NOALLOC_SCRATCH_BYTES];

namespace cce {
namespace {

constexpr int WAVES = 4, THREADS = 64 * WAVES;
constexpr int TW = 32;                      // conv-output columns per tile
constexpr int PTW = TW / 2;                 // pooling-window columns per tile
constexpr int CC = 8;                       // input channels per K chunk
constexpr int XC = TW + 2;                  // input halo tile columns
constexpr int XRS = 40;                     // LDS row stride: 8 (mod 64) banks between rows
constexpr int XOFF = 3;                     // LDS column of input column w0 - 1

static_assert(XOFF + XC <= XRS, "halo row fits the LDS row");

// Geometry per output-channel count: NT 16-column MFMA blocks; every wave
// computes MT 16-pixel blocks, RP = MT / 4 row pairs of the tile's 32
// columns, so a tile has TH = 8 RP rows.  With 64 channels (NT = 4) 8 blocks
// per wave fill 128 accumulator registers (16 x 32 tiles); 16 channels take
// 16 blocks per wave (32 x 32 tiles), so that each staged chunk and each
// barrier carry more MFMAs.  32 channels keep 16 x 32 tiles: 16 blocks
// spill (the 34-row halo chunk's staging registers on top of 128
// accumulators), and 24 x 32 tiles leave a partial tile row on 2^k-row images
// and an uneven last round (1408 tiles for 512 workgroup slots at N = 16,
// 256 x 256): 0.1856 -> 0.1805 ms there, 0.0605 -> 0.0469 ms at 128 x 128.
// The weight slice of one K chunk holds (CC / 4) x 9 x 64 lanes x NT floats.
template <int CO_>
struct OutCh {
  static constexpr int CO = CO_, NT = CO / 16;
  static constexpr int MT = NT == 1 ? 16 : 8, RP = MT / 4;
  static constexpr int TH = 2 * RP * WAVES, PTH = TH / 2;  // conv-output / pooled rows per tile
  static constexpr int XR = TH + 2;                      // input halo tile rows
  static constexpr int XCS = XR * XRS;  // 16 (mod 64): the lane groups' channels 16 banks apart
  static constexpr int XS_FLOATS = CC * XCS;
  static constexpr int WS_FLOATS = (CC / 4) * 9 * 64 * NT;
  static constexpr int W4_PER_CHUNK = WS_FLOATS / 4;
  static constexpr int W4_PT = (W4_PER_CHUNK + THREADS - 1) / THREADS;
  // Per-chunk input staging in 16-byte units (interior) and single floats (halo columns).
  static constexpr int XQ = TW / 4;                                  // 8 float4 per row
  static constexpr int X4_PER_CHUNK = CC * XR * XQ;
  static constexpr int X4_PT = (X4_PER_CHUNK + THREADS - 1) / THREADS;
  static constexpr int XH_PER_CHUNK = CC * XR * 2;
  static constexpr int XH_PT = (XH_PER_CHUNK + THREADS - 1) / THREADS;
  static_assert(CO == 16 || CO == 32 || CO == 64, "C_out is 16, 32 or 64");
  static_assert(XCS % 64 == 16, "lane groups' channel planes 16 banks apart");
};

struct ConvTArgs {
  const float *__restrict__ x;
  const float *__restrict__ w;
  const float *__restrict__ b;
  float *__restrict__ y;
  unsigned *tickets;  // [N] per-image completion counters (zeroed per call)
  float *partials;    // [N][tiles_per_image][C_out]
  const float *wprep; // prepared weight, nchunk x WS_FLOATS
  int C_in, nchunk;   // nchunk = C_in / CC
  int H, W, PH, PW;
  int tiles_x, tiles_per_image;
  float lo, hi, inv_count;
};

// Per-chunk staging in 16-byte units.  The weight slice of chunk c is
// contiguous in the prepared layout; the input tile's 32 interior columns of
// each (channel, row) are four-aligned in the image (w0 % 32 == 0, W % 4 == 0)
// and land on four-aligned LDS columns (XOFF + 1 = 4); the two halo columns
// are single floats.
static_assert(XOFF + 1 == 4, "interior columns start 16-byte aligned in LDS");

template <class OC>
struct ChunkRegs {
  v4f w4[OC::W4_PT];
  v4f x4[OC::X4_PT];
  float xh[OC::XH_PT];
};

// Global -> registers for channel chunk c (issued a whole chunk ahead of use).
// VEC: W % 4 == 0 and x 16-byte aligned, so each interior quad is one aligned
// 16-byte load that is either wholly inside the row or wholly past its end.
template <class OC, bool VEC>
__device__ __forceinline__ void load_chunk(const ConvTArgs &a, int n, int c, int h0, int w0, int tid,
                                           ChunkRegs<OC> &r) {
  const v4f *wsrc = reinterpret_cast<const v4f *>(a.wprep) + (size_t)c * OC::W4_PER_CHUNK;
#pragma unroll
  for (int j = 0; j < OC::W4_PT; ++j) {
    const int i = tid + j * THREADS;
    if (i < OC::W4_PER_CHUNK) r.w4[j] = wsrc[i];
  }
  const float *xc = a.x + ((size_t)n * a.C_in + CC * c) * a.H * a.W;
#pragma unroll
  for (int j = 0; j < OC::X4_PT; ++j) {
    const int i = tid + j * THREADS;
    v4f v = splat4(0.0f);
    if (i < OC::X4_PER_CHUNK) {
      const int row = i / OC::XQ, q = i - row * OC::XQ;  // row = cl * OC::XR + rr
      const int cl = row / OC::XR, rr = row - cl * OC::XR;
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
  for (int j = 0; j < OC::XH_PT; ++j) {
    const int i = tid + j * THREADS;
    float v = 0.0f;
    if (i < OC::XH_PER_CHUNK) {
      const int row = i >> 1, side = i & 1;
      const int cl = row / OC::XR, rr = row - cl * OC::XR;
      const int h = h0 - 1 + rr, wc = side ? w0 + TW : w0 - 1;
      if (h >= 0 && h < a.H && wc >= 0 && wc < a.W) v = xc[((size_t)cl * a.H + h) * a.W + wc];
    }
    r.xh[j] = v;
  }
}

// Registers -> LDS.
template <class OC>
__device__ __forceinline__ void store_chunk(float *xs, float *ws, int tid, const ChunkRegs<OC> &r) {
#pragma unroll
  for (int j = 0; j < OC::W4_PT; ++j) {
    const int i = tid + j * THREADS;
    if (i < OC::W4_PER_CHUNK) reinterpret_cast<v4f *>(ws)[i] = r.w4[j];
  }
#pragma unroll
  for (int j = 0; j < OC::X4_PT; ++j) {
    const int i = tid + j * THREADS;
    if (i < OC::X4_PER_CHUNK) {
      const int row = i / OC::XQ, q = i - row * OC::XQ;
      const int cl = row / OC::XR, rr = row - cl * OC::XR;
      *reinterpret_cast<v4f *>(&xs[cl * OC::XCS + rr * XRS + XOFF + 1 + 4 * q]) = r.x4[j];
    }
  }
#pragma unroll
  for (int j = 0; j < OC::XH_PT; ++j) {
    const int i = tid + j * THREADS;
    if (i < OC::XH_PER_CHUNK) {
      const int row = i >> 1, side = i & 1;
      const int cl = row / OC::XR, rr = row - cl * OC::XR;
      xs[cl * OC::XCS + rr * XRS + (side ? XOFF + 1 + TW : XOFF)] = r.xh[j];
    }
  }
}

// Per-call preparation of the workspace, launched on the same stream just
// before the main kernel:
//  * the flipped, channel-swapped kernel (C_in x C_out x 9 floats) in exactly
//    the LDS B-operand order of every chunk,
//      wprep[c][cb][tap'][lane][nt] = W[8c + 4cb + lane/16][16nt + lane%16][8 - tap'],
//    where tap' = 3 kh' + kw' and W's tap index 3 kh + kw = 8 - tap';
//  * the N per-image completion counters set to zero.
// Every workspace byte the main kernel reads is thus written by this call
// (the per-tile partials by the main kernel itself before they are read),
// so the workspace needs no initial contents, and a workspace last used by a
// call of another shape -- whose prepared weight may cover this call's
// counters -- is as good as a fresh one.
template <class OC>
__global__ __launch_bounds__(THREADS) void convT_prepare_weight_kernel(const float *__restrict__ w,
                                                                      float *__restrict__ wprep,
                                                                      int total, unsigned *tickets,
                                                                      int N) {
  const int p = blockIdx.x * THREADS + threadIdx.x;
  if (p < N) tickets[p] = 0u;
  if (p >= total) return;
  const int nt = p % OC::NT, lane = (p / OC::NT) & 63, rest = p / (OC::NT * 64);
  const int tap = rest % 9, ccb = rest / 9;  // rest = (c * 2 + cb) * 9 + tap, ccb = c * 2 + cb
  const int ci = 4 * ccb + (lane >> 4), o = 16 * nt + (lane & 15);
  wprep[p] = w[((size_t)ci * OC::CO + o) * 9 + (8 - tap)];
}

// NCH > 0: a compile-time chunk count (the page's 64-channel layer, NCH = 8);
// with the runtime count the compiler schedules the chunk loop's LDS reads
// later and the kernel runs 5 % slower.
template <class OC, bool VEC, int NCH>
__global__ __launch_bounds__(THREADS, 2) void convT2d_pool_htanh_mean_tanh_kernel(ConvTArgs a) {
  const int nchunk = NCH > 0 ? NCH : a.nchunk;
  constexpr int CO = OC::CO, NT = OC::NT, MT = OC::MT, RP = OC::RP, XCS = OC::XCS;
  __shared__ __attribute__((aligned(16))) float xs[OC::XS_FLOATS];
  __shared__ __attribute__((aligned(16))) float ws[OC::WS_FLOATS];
  __shared__ float red[THREADS];  // [WAVES][CO], then [THREADS / CO][CO]
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  // XCD-aware tile order: the hardware hands workgroup b to XCD b % 8; each
  // XCD takes one contiguous range of tiles, so neighbouring tiles (which
  // share halo rows and columns) and the weight slices they all read meet
  // in the same L2.  grid = 8 q + r; XCD j takes r > j ? q + 1 : q tiles.
  const int G = gridDim.x, q = G >> 3, rr = G & 7, xcd = blockIdx.x & 7;
  const int tile = xcd * q + min(xcd, rr) + (int)(blockIdx.x >> 3);
  const int n = tile / a.tiles_per_image;
  const int ti = tile - n * a.tiles_per_image;
  const int ty = ti / a.tiles_x, tx = ti - ty * a.tiles_x;
  const int h0 = ty * OC::TH, w0 = tx * TW;

  // A-operand lane: M row m = col -> pooling window col/4 of the block, pixel
  // (dh, dw) = ((col & 3) >> 1, col & 1) inside it; lane group g = channel.
  // Wave w covers the tile's rows 2 RP w .. 2 RP w + 2 RP - 1; block mt its
  // row pair mt / 4 and columns 8 (mt % 4) .. + 7.
  const int wi = col >> 2, dh = (col & 3) >> 1, dw = col & 1;
  const int abase = g * XCS + (2 * RP * wave + dh) * XRS + XOFF + 2 * wi + dw;

  v4f acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = splat4(0.0f);

  ChunkRegs<OC> r;
  load_chunk<OC, VEC>(a, n, 0, h0, w0, tid, r);
  store_chunk(xs, ws, tid, r);
  __syncthreads();

#pragma unroll 1
  for (int c = 0; c < nchunk; ++c) {
    // Next chunk's global loads are in flight while this chunk's MFMAs run.
    if (c + 1 < nchunk) load_chunk<OC, VEC>(a, n, c + 1, h0, w0, tid, r);
#pragma unroll
    for (int cb = 0; cb < CC / 4; ++cb) {
#pragma unroll
      for (int tap = 0; tap < 9; ++tap) {
        const int kh = tap / 3, kw = tap % 3;
        float bv[NT];
        load_b<NT>(bv, &ws[((cb * 9 + tap) * 64 + lane) * NT]);
        float av[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          av[mt] = xs[abase + cb * 4 * XCS + (2 * (mt >> 2) + kh) * XRS + 8 * (mt & 3) + kw];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16x16x4(av[mt], bv[nt], acc[mt][nt]);
      }
    }
    if (c + 1 < nchunk) {
      __syncthreads();  // every wave is done reading chunk c
      store_chunk(xs, ws, tid, r);
      __syncthreads();
    }
  }

  // Epilogue: lane holds, per block and channel block, the 4 pixels of pooling
  // window (ph, pw) = (ph0 + RP wave + mt/4, pw0 + 4 (mt%4) + g), channel 16 nt + col.
  float bias[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) bias[nt] = a.b ? a.b[16 * nt + col] : 0.0f;
  float sum[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) sum[nt] = 0.0f;
  const int ph0 = ty * OC::PTH, pw0 = tx * PTW;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int ph = ph0 + RP * wave + (mt >> 2), pw = pw0 + 4 * (mt & 3) + g;
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
    for (int nt = 0; nt < NT; ++nt) red[wave * CO + 16 * nt + col] = sum[nt];
  }
  __syncthreads();
  if (tid < CO) {
    const float tot = ((red[tid] + red[CO + tid]) + red[2 * CO + tid]) + red[3 * CO + tid];
    __hip_atomic_store(&a.partials[((size_t)n * a.tiles_per_image + ti) * CO + tid], tot,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  // The counter update releases this workgroup's partials (its stores, all
  // from wave 0, come before it in program order, the other waves' work
  // through the barrier above); only the workgroup that completes the image
  // acquires, below.  (An acquire on every update, or a separate fence before
  // it, costs 2 % of the page's layer at N = 128: each one writes back or
  // invalidates this XCD's L2.)
  if (tid == 0) {
    const unsigned done = __hip_atomic_fetch_add(&a.tickets[n], 1u, __ATOMIC_RELEASE,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (done == (unsigned)a.tiles_per_image - 1u);
    // The update that completes the image read every other workgroup's
    // (they form one release sequence): acquire them before the barrier
    // hands the result to the other threads.
    if (last_flag) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!last_flag) return;

  // Last workgroup of image n: all partials of the image are visible.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  constexpr int PARTS = THREADS / CO;  // threads per output channel
  {
    const int o = tid % CO, part = tid / CO;
    const float *pp = a.partials + (size_t)n * a.tiles_per_image * CO + o;
    float s = 0.0f;
    for (int t = part; t < a.tiles_per_image; t += PARTS)
      s += __hip_atomic_load(pp + (size_t)t * CO, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    red[part * CO + o] = s;
  }
  __syncthreads();
  if (tid < CO) {
    float tot = 0.0f;
#pragma unroll
    for (int part = 0; part < PARTS; ++part) tot += red[part * CO + tid];
    a.y[(size_t)n * CO + tid] = tanhf(tot * a.inv_count);
  }
}

constexpr size_t kTicketAlign = 256;

// Tiles of a layer: 16 pooling-window columns by OutCh<C_out>::PTH rows (8
// for 64 or 32 output channels, 16 for 16).
void convT_tiles(int H, int W, int C_out, int *tiles_x, int *tiles_per_image) {
  const int PH = H / 2, PW = W / 2;
  const int pth = C_out == 64 ? OutCh<64>::PTH : C_out == 32 ? OutCh<32>::PTH : OutCh<16>::PTH;
  *tiles_x = (PW + PTW - 1) / PTW;
  *tiles_per_image = ((PH + pth - 1) / pth) * *tiles_x;
}


size_t ticket_bytes(int N) {
  return ((size_t)N * sizeof(unsigned) + kTicketAlign - 1) / kTicketAlign * kTicketAlign;
}

// C_in * C_out * 9 floats; a multiple of 256 bytes for every supported shape
// (C_in % 8 == 0, C_out % 16 == 0), so the partials stay 256-byte aligned.
size_t wprep_bytes(int C_in, int C_out) { return (size_t)C_in * C_out * 9 * sizeof(float); }

template <class OC, int NCH>
int launch_for(ConvTArgs a, const float *w, float *wprep, int N, long long grid, hipStream_t stream) {
  const int total = a.C_in * OC::CO * 9;
  const int prep_items = total > N ? total : N;
  hipLaunchKernelGGL(convT_prepare_weight_kernel<OC>, dim3((prep_items + THREADS - 1) / THREADS),
                     dim3(THREADS), 0, stream, w, wprep, total, a.tickets, N);
  if (launch_status(stream, "convT_prepare_weight_kernel") != CCE_OK) return CCE_ERR_LAUNCH;
  const bool vec = (a.W % 4 == 0) && ((uintptr_t)a.x % 16 == 0);
  if (vec)
    hipLaunchKernelGGL((convT2d_pool_htanh_mean_tanh_kernel<OC, true, NCH>), dim3((unsigned)grid),
                       dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((convT2d_pool_htanh_mean_tanh_kernel<OC, false, NCH>), dim3((unsigned)grid),
                       dim3(THREADS), 0, stream, a);
  return launch_status(stream, "convT2d_pool_htanh_mean_tanh_kernel");
}

}  // namespace

bool convT_layer_supported(int C_in, int C_out) {
  return C_in >= CC && C_in <= 512 && C_in % CC == 0 && (C_out == 16 || C_out == 32 || C_out == 64);
}

// Workspace: [per-image counters, padded to 256 B][prepared weight][partials].
size_t convT_workspace_bytes(int N, int C_in, int H, int W, int C_out) {
  int tx, tpi;
  convT_tiles(H, W, C_out, &tx, &tpi);
  return ticket_bytes(N) + wprep_bytes(C_in, C_out) + (size_t)N * tpi * C_out * sizeof(float);
}

int launch_convT2d_pool_htanh_mean_tanh(const float *x, const float *w, const float *b, float *y,
                                        int N, int C_in, int H, int W, int C_out, float lo, float hi,
                                        void *workspace, hipStream_t stream) {
  if (!convT_layer_supported(C_in, C_out)) return CCE_ERR_UNSUPPORTED;
  ConvTArgs a;
  a.x = x;
  a.w = w;
  a.b = b;
  a.y = y;
  a.C_in = C_in;
  a.nchunk = C_in / CC;
  a.H = H;
  a.W = W;
  a.PH = H / 2;  // conv output is H x W at stride 1, padding 1; floor pooling
  a.PW = W / 2;
  convT_tiles(H, W, C_out, &a.tiles_x, &a.tiles_per_image);
  a.lo = lo;
  a.hi = hi;
  a.inv_count = (float)(1.0 / ((double)a.PH * (double)a.PW));
  char *wsp = reinterpret_cast<char *>(workspace);
  float *wprep = reinterpret_cast<float *>(wsp + ticket_bytes(N));
  a.tickets = reinterpret_cast<unsigned *>(wsp);
  a.wprep = wprep;
  a.partials = reinterpret_cast<float *>(wsp + ticket_bytes(N) + wprep_bytes(C_in, C_out));
  const long long grid = (long long)N * a.tiles_per_image;
  if (grid >= (1LL << 31)) return CCE_ERR_TOO_LARGE;
  switch (C_out) {
    case 16: return launch_for<OutCh<16>, 0>(a, w, wprep, N, grid, stream);
    case 32: return launch_for<OutCh<32>, 0>(a, w, wprep, N, grid, stream);
    default:
      if (C_in == 64) return launch_for<OutCh<64>, 64 / CC>(a, w, wprep, N, grid, stream);
      return launch_for<OutCh<64>, 0>(a, w, wprep, N, grid, stream);
  }
}

namespace {
// Device address of `scratch`, per device (null until the first call there).
std::atomic<void *> g_scratch[kLaunchCacheDevices];
}  // namespace

int launch_convT2d_pool_htanh_mean_tanh_noalloc(const float *x, const float *w, const float *b,
                                                float *y, int N, int C_in, int H, int W, int C_out,
                                                float lo, float hi, hipStream_t stream) {
  if (convT_workspace_bytes(N, C_in, H, W, C_out) > (size_t)CCE_NOALLOC_SCRATCH_BYTES)
    return CCE_ERR_SCRATCH_LIMIT;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CCE_ERR_LAUNCH;
  const bool cached = dev >= 0 && dev < kLaunchCacheDevices;
  void *ptr = cached ? g_scratch[dev].load(std::memory_order_acquire) : nullptr;
  if (!ptr) {
    // Once per device, with that device current: the array's address on it.
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return CCE_ERR_LAUNCH;
    if (cached) g_scratch[dev].store(ptr, std::memory_order_release);
  }
  return launch_convT2d_pool_htanh_mean_tanh(x, w, b, y, N, C_in, H, W, C_out, lo, hi, ptr, stream);
}

}  // namespace cce
