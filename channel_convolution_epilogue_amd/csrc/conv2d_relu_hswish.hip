// Conv2d 3x3, 8 -> 64 channels, stride 1, padding 0, + bias -> ReLU -> HardSwish,
// fused in one gfx950 kernel (POPCORNBENCH Kimi-K2.6 l2_p57: its model is
// Conv2d(8, 64, 3) followed by ReLU and HardSwish x * clamp((x + 3) / 6, 0, 1)).
//
// Design (MI355X-first, not the page's one-thread-per-output CUDA tiling):
//  * Implicit GEMM on the fp32 matrix cores: M = output pixels, N = the 64
//    output channels, K = 8 channels x 9 taps = 72.  Packed fp32 VALU math is
//    not used, so the matrix cores are the only units that reach the fp32
//    peak; the contraction is dense enough (72 x 64 per pixel) to feed them.
//  * The unit of work is one wave's strip: 16 output columns of one output
//    row of one image, all 64 channels (one 16-pixel MFMA block per channel
//    block); layers with 16 or 32 output channels take two rows per strip.  Each wave stages its strip's input window (8 channels x 3 rows
//    x 24 columns) in a slice of LDS of its own, so no wave ever waits for
//    another's data.  The next strip's window is loaded into registers while
//    the current strip's MFMAs run, and written to the wave's slice after
//    them.
//  * Strips are dealt in rounds, strip index fastest: in one round the 16
//    waves of a workgroup take 16 consecutive strips, i.e. whole rows of the
//    output (8 strips cover 126 columns), and write 2 full rows of every
//    channel plane.  One barrier per round keeps the waves in step, so that
//    the 64-byte pieces that neighbouring waves write into one 128-byte line
//    reach the L2 together.  Measured on MI355X: without it, partly written
//    lines are evicted and rewritten, which costs 1.6x more HBM traffic and
//    makes the kernel 1.6x slower.  Consecutive workgroups take consecutive
//    rounds, and the blockIdx remap gives each XCD a contiguous block.
//  * Results leave as 16-byte stores.  A row's strips are shifted left by
//    (row offset mod 4) columns so that every lane's four pixels start on a
//    16-byte boundary even when the row length is not a multiple of four;
//    pixels that fall outside the row are masked.
//  * Window loads and result stores are raw buffer accesses over one image,
//    with 32-bit lane offsets: a position outside the image gets an offset
//    past the buffer's end, which loads zeros (or drops the store), so no
//    lane branches and the per-strip address arithmetic is a few adds.  On
//    gfx950 fp32 MFMAs and plain VALU instructions share one datapath, so
//    this arithmetic is matrix-core time: the checked global loads and
//    stores they replace cost 5-7 % of the kernel.
//  * The K order puts the four lane groups on four input channels and one
//    (channel half, kh, kw) per step, so the step's LDS offset is the same for
//    all lanes.  The 72 x 64 weight sits in LDS in B-operand order: one
//    16-byte read per K-step serves all four 16-channel blocks.
//  * Bias is the accumulator's initial value; ReLU and HardSwish are applied
//    in registers before the store: the conv result never reaches memory.
//  * The same kernel, with the Conv3d operator's epilogue (LeakyReLU, + s[c],
//    clamp, GELU) as a template parameter, runs the 1 x 1 x 1 Conv3d layers:
//    a pointwise Conv3d over D x H x W is a 1 x 1 Conv2d over D * H rows.
#include "cce_device.hpp"
#include "cce_internal.hpp"

namespace cce {
namespace {

constexpr int WAVES = 16, THREADS = 64 * WAVES;  // one workgroup per CU, 4 waves per SIMD

// Geometry of one wave's strip and of the layer: RB output rows by CB blocks
// of 16 columns, for CI input channels (a multiple of 4: one per lane group
// per K-step), CO output channels (16 per MFMA block, at most 64) and k x k
// kernels.  The staged window spans columns [c0 - 4, c0 + 16 CB + 4 +
// pad(k - 1)) (quad-aligned, wide enough for the 0..3 column shift and the
// k - 1 halo) and RB + k - 1 rows.  Its channel planes are CS floats apart,
// CS = 16 or 48 mod 64, so the four lane groups of an A read (four channels)
// start on four different quarters of the 64 LDS banks.
constexpr int chan_stride(int need) {
  int c = need;
  while (c % 64 != 16 && c % 64 != 48) ++c;
  return c;
}
template <int RB_, int CB_, int CI_, int CO_, int KS_>
struct StripGeo {
  static constexpr int RB = RB_, CB = CB_, MT = RB * CB;
  static constexpr int CI = CI_, CO = CO_, KS = KS_, TAPS = KS * KS;
  static constexpr int KSTEPS = (CI / 4) * TAPS;  // K-steps of 4 taps
  static constexpr int NT = CO / 16;              // 16-channel MFMA blocks
  static constexpr int WS_FLOATS = KSTEPS * 64 * NT;  // weights in LDS, B-operand order
  static constexpr int SW = 16 * CB;              // output columns per strip
  static constexpr int XW = SW + 4 + ((KS - 1 + 3) & ~3);  // staged columns per row
  static constexpr int XQ = XW / 4;               // 16-byte quads per staged row
  static constexpr int ROWS = RB + KS - 1;        // staged rows
  static constexpr int CS = chan_stride(ROWS * XW);
  static constexpr int WIN = CI * CS;             // floats per wave window
  static_assert(CI % 4 == 0 && CO % 16 == 0 && NT >= 1 && NT <= 4 && KS % 2 == 1, "layer shape");
};

struct Conv2dArgs {
  const float *__restrict__ x;
  const float *__restrict__ w;
  const float *__restrict__ b;
  float *__restrict__ y;
  int H, W, Ho, Wo;
  int P;       // output pixels per plane, Ho * Wo
  int S;       // strips per row group, ceil((Wo + largest shift) / strip width)
  int G;       // row groups per image, ceil(Ho / rows per strip)
  int items;   // strips in the whole problem, N * G * S
  FastDiv divS, divG;
  // Epilogue of the pointwise Conv3d layers that run on this kernel:
  // GELU(clamp(LeakyReLU(v, slope) + s[o], lo, hi)).  Unused by HardSwish.
  const float *__restrict__ s;
  float slope, lo, hi;
};

// Epilogue applied in registers before the store: the page's ReLU ->
// HardSwish, or (for 1 x 1 x 1 Conv3d layers, which are 1 x 1 Conv2d layers
// over D * H rows) LeakyReLU -> + s[o] -> clamp -> GELU, with the fitted
// polynomial when the clamp bounds lie in [-1, 1] and erff otherwise.
enum Epilogue { kReluHswish = 0, kGeluSeries = 1, kGeluErf = 2 };

// HardSwish(ReLU(v)) = r * clamp((r + 3) / 6, 0, 1) with r = max(v, 0).  For
// v >= 0 the gate (v + 3) / 6 is at least 0.5, and for v < 0 the result is 0
// whatever the (non-negative) gate, so the gate can be taken from v itself,
// clamped to [0, 1] -- the clamp modifier of the fma, free -- and the ReLU
// applied to the product: max(v * gate, 0) = max(v, 0) * gate.  Three
// instructions.  (On gfx950 fp32 MFMAs and plain VALU instructions share one
// datapath, so every epilogue instruction costs matrix-core time.)
__device__ __forceinline__ float relu_hswish(float v) {
  const float gate = __builtin_amdgcn_fmed3f(fmaf(v, 1.0f / 6.0f, 0.5f), 0.0f, 1.0f);
  return fmaxf(v * gate, 0.0f);
}

struct Strip {
  int n, r0, c0;
};

// VLOAD: W % 4 == 0 and x 16-byte aligned (16-byte window loads).
// VSTORE: P % 4 == 0 and y 16-byte aligned (16-byte result stores).
// EPI: an Epilogue.
template <class GEO, bool VLOAD, bool VSTORE, int EPI>
__global__ __launch_bounds__(THREADS, 4) void conv2d_relu_hswish_kernel(Conv2dArgs a) {
  constexpr int RB = GEO::RB, CB = GEO::CB, MT = GEO::MT, SW = GEO::SW, XW = GEO::XW,
                XQ = GEO::XQ, ROWS = GEO::ROWS, CS = GEO::CS, WIN = GEO::WIN;
  constexpr int CI = GEO::CI, CO = GEO::CO, KS = GEO::KS, TAPS = GEO::TAPS, KSTEPS = GEO::KSTEPS,
                NT = GEO::NT, WS_FLOATS = GEO::WS_FLOATS;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  float *ws = lds;                                  // weights, WS_FLOATS
  float *win = lds + WS_FLOATS + (threadIdx.x >> 6) * WIN;  // this wave's window
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;

  // The hardware hands workgroups to the 8 XCDs in turn (b -> XCD b % 8); the
  // remap gives each XCD a contiguous block of each round's strips, so one L2
  // collects long runs of every output plane.  (gridDim.x is a multiple of 8.)
  const int per_xcd = gridDim.x >> 3;
  const int wg = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int step = gridDim.x * WAVES;
  // The strip index is the same for every lane of the wave: keep it scalar.
  // Rounds are workgroup-uniform: round k gives wave w strip
  // wg * WAVES + k * step + w, and a wave whose strip is past the end idles
  // through the round, so every wave meets the same barriers.
  // A surplus workgroup (the grid is rounded up to a multiple of 8) leaves
  // after the prologue's loads, so that no branch splits the kernel-argument
  // reads in two.
  int first = wg * WAVES;
  int item = __builtin_amdgcn_readfirstlane(first + wave);
  bool valid = item < a.items;
  if (!valid) item = a.items - 1;

  auto decode = [&](int i) {
    const int t = fdiv(i, a.divS), k = i - t * a.S;
    const int n = fdiv(t, a.divG), rg = t - n * a.G;
    return Strip{n, rg * RB, k * SW};
  };

  // Window staging.  Element e of a window is (channel, row, column) with the
  // column fastest; VLOAD moves quads, otherwise single floats.  Positions
  // outside the image (left of column 0, right of W - 1, below row H - 1)
  // are staged as zeros; only masked outputs read them.
  constexpr int UNITS = VLOAD ? CI * ROWS * XQ : CI * ROWS * XW;
  constexpr int PER_LANE = (UNITS + 63) / 64;
  v4f pre[VLOAD ? PER_LANE : 1];
  float pres[VLOAD ? 1 : PER_LANE];
  // One image is less than 2^31 floats, so in-image offsets are 32-bit.
  // VLOAD: buffer loads over one image (less than 2^31 bytes), with
  // positions outside it given the out-of-range offset, which loads zeros.
  // Per lane and quad f: the staged row, the column offset from c0 and the
  // byte offset within the image relative to (row r0, column c0).
  int lrow[VLOAD ? PER_LANE : 1], ldc[VLOAD ? PER_LANE : 1], lofs[VLOAD ? PER_LANE : 1];
#pragma unroll
  for (int f = 0; f < (VLOAD ? PER_LANE : 1); ++f) {
    // Lanes past the window's last quad repeat quad e % UNITS (same data to
    // the same LDS address), so every lane loads and stores unconditionally.
    const int e = (lane + 64 * f) % UNITS;
    const int cq = e % XQ, rc = e / XQ, row = rc % ROWS, ch = rc / ROWS;
    lrow[f] = row;
    ldc[f] = 4 * cq - 4;
    lofs[f] = ((ch * a.H + row) * a.W + 4 * cq - 4) * 4;
  }
  auto load = [&](const Strip &s) {
    if constexpr (VLOAD) {
      const auto rx = buffer_rsrc(a.x + (size_t)s.n * CI * a.H * a.W, (uint32_t)(CI * a.H * a.W) * 4u);
      const int uni = (s.r0 * a.W + s.c0) * 4, rows_left = a.H - s.r0;
#pragma unroll
      for (int f = 0; f < PER_LANE; ++f) {
        const bool ok = lrow[f] < rows_left && (unsigned)(s.c0 + ldc[f]) < (unsigned)a.W;
        pre[f] = buffer_load4(rx, ok ? (uint32_t)(lofs[f] + uni) : kBufferOOB, 0u);
      }
      return;
    }
    const float *xs = a.x + (size_t)s.n * CI * a.H * a.W + s.r0 * a.W + s.c0;
#pragma unroll
    for (int f = 0; f < PER_LANE; ++f) {
      const int e = lane + 64 * f;
      if (e < UNITS) {
        const int per_row = VLOAD ? XQ : XW;
        const int cq = e % per_row, rc = e / per_row, row = rc % ROWS, ch = rc / ROWS;
        const int dc = (VLOAD ? 4 * cq : cq) - 4;
        const bool ok = s.r0 + row < a.H && s.c0 + dc >= 0 && s.c0 + dc < a.W;
        const float *p = xs + (ok ? (ch * a.H + row) * a.W + dc : 0);
        if (VLOAD)
          pre[f] = ok ? *reinterpret_cast<const v4f *>(p) : splat4(0.0f);
        else
          pres[f] = ok ? *p : 0.0f;
      }
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int f = 0; f < PER_LANE; ++f) {
      const int e = VLOAD ? (lane + 64 * f) % UNITS : lane + 64 * f;
      if (e < UNITS) {
        const int per_row = VLOAD ? XQ : XW;
        const int cq = e % per_row, rc = e / per_row, row = rc % ROWS, ch = rc / ROWS;
        float *d = win + ch * CS + row * XW + (VLOAD ? 4 * cq : cq);
        if (VLOAD)
          *reinterpret_cast<v4f *>(d) = pre[f];
        else
          *d = pres[f];
      }
    }
  };

  // Prologue: the first window, the weight and the bias are all requested
  // before any of them is waited for, so the workgroup waits for one memory
  // latency before its first MFMA, not one per staging pass.
  Strip cur = decode(item);
  load(cur);
  // B operand of K-step s = (channel quad, kh, kw) for all NT 16-channel blocks.
  WeightStageB<CI, CO, TAPS, THREADS> wstage;
  wstage.load(a.w, tid);
  float bias[NT];
  // The GELU epilogue works on halved values (weights, bias and s staged at
  // half scale, exactly): bit-identical, one multiplication fewer per output.
  constexpr float kScale = EPI == kReluHswish ? 1.0f : 0.5f;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) bias[nt] = a.b ? kScale * a.b[16 * nt + col] : 0.0f;
  float sadd[NT];  // per-channel term of the GELU epilogue
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) sadd[nt] = EPI == kReluHswish ? 0.0f : kScale * a.s[16 * nt + col];
  const float lo_half = kScale * a.lo, hi_half = kScale * a.hi;
  // The first K-step's MFMAs start from the bias (as their C operand), so
  // the accumulators need no initialising copies.
  v4f bias4[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) bias4[nt] = splat4(bias[nt]);
  // Byte offset of this lane's result quad within channel block 0's planes,
  // relative to a strip's first output pixel.
  const int sofs = VSTORE ? (col * a.P + 4 * g) * 4 : 0;
  if (first >= a.items) return;  // workgroup-uniform
  wstage.place(ws, a.w, tid, kScale);
  put();
  __syncthreads();  // weights in place; from here on only the per-round barrier

  for (;;) {
    const bool more = first + step < a.items;  // workgroup-uniform
    int next = __builtin_amdgcn_readfirstlane(first + step + wave);
    const bool next_valid = next < a.items;
    if (!next_valid) next = a.items - 1;
    // The last strip reloads itself: loads and LDS writes stay unconditional,
    // so the compiler's wait counts never hold a later load behind a store.
    const Strip nxt = more ? decode(next) : cur;
    load(nxt);  // in flight during this strip's MFMAs
    // Keep the loads here: the scheduler would otherwise sink them to their
    // use after the MFMAs.
    __builtin_amdgcn_sched_barrier(0);

    // Block (jr, jc) covers output row r0 + jr, columns
    // [c0 + 16 jc - sh, c0 + 16 jc - sh + 16) with sh = (row offset) mod 4, so
    // its stores are 16-byte aligned.
    int sh[RB], base[MT];
#pragma unroll
    for (int jr = 0; jr < RB; ++jr) {
      const int r = cur.r0 + jr;
      sh[jr] = VSTORE ? (((r & 3) * (a.Wo & 3)) & 3) : 0;
#pragma unroll
      for (int jc = 0; jc < CB; ++jc) base[jr * CB + jc] = g * CS + jr * XW + 16 * jc + col + 4 - sh[jr];
    }
    v4f acc[MT][NT];

#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int tap = s % TAPS;
      const int off = (s / TAPS) * 4 * CS + (tap / KS) * XW + (tap % KS);
      float bv[NT];
      load_b<NT>(bv, &ws[(s * 64 + lane) * NT]);
      float av[MT];
#pragma unroll
      for (int j = 0; j < MT; ++j) av[j] = win[base[j] + off];
#pragma unroll
      for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[j][nt] = mfma16x16x4(av[j], bv[nt], s == 0 ? bias4[nt] : acc[j][nt]);
    }

    // The window has been read (the MFMAs above consumed every value), so the
    // next strip's window may overwrite it; this wave's LDS operations run in
    // program order.  The scheduling barrier keeps the LDS writes, and their
    // wait for the window loads, after the MFMAs (with a short K-loop the
    // scheduler would hoist them above, exposing the loads' latency).
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    put();

    auto epilogue = [&](float v, int nt) {
      if constexpr (EPI == kReluHswish)
        return relu_hswish(v);
      else
        return lrelu_add_clamp_gelu_half<EPI == kGeluSeries>(v, sadd[nt], a.slope, lo_half, hi_half);
    };
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[j][nt].x = epilogue(acc[j][nt].x, nt);
        acc[j][nt].y = epilogue(acc[j][nt].y, nt);
        acc[j][nt].z = epilogue(acc[j][nt].z, nt);
        acc[j][nt].w = epilogue(acc[j][nt].w, nt);
      }

    if constexpr (VSTORE) {
      // Buffer stores over one image's output (less than 2^31 bytes), at the
      // lane's byte offset in channel block 0 plus block nt's plane offset.
      // A lane quad that crosses a row
      // end or start stores its in-row pixels one by one; the others get the
      // out-of-range offset, which drops their stores.
      const auto ry = buffer_rsrc(a.y + (size_t)cur.n * CO * a.P, (uint32_t)(CO * a.P) * 4u);
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int jr = j / CB, jc = j % CB, r = cur.r0 + jr;
        if (r >= a.Ho || !valid) break;
        const int c = cur.c0 + 16 * jc - sh[jr];  // the block's first output column
        const int cb = c + 4 * g;                 // this lane's
        const uint32_t voff = (uint32_t)(sofs + (r * a.Wo + c) * 4);
        if (cb >= 0 && cb + 3 < a.Wo) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) buffer_store4(ry, acc[j][nt], voff + (uint32_t)(16 * nt * a.P) * 4u);
        } else {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool in_row = cb + e >= 0 && cb + e < a.Wo;
              buffer_store1(ry, acc[j][nt][e], in_row ? voff + (uint32_t)(16 * nt * a.P + e) * 4u : kBufferOOB);
            }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const int jr = j / CB, jc = j % CB, r = cur.r0 + jr;
        if (r >= a.Ho || !valid) break;
        const int cb = cur.c0 + 16 * jc + 4 * g;  // this lane's first output column
        float *dst = a.y + (size_t)cur.n * CO * a.P + (size_t)r * a.Wo + cb;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float *d = dst + (size_t)(16 * nt + col) * a.P;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (cb + e < a.Wo) d[e] = acc[j][nt][e];
        }
      }
    }

    if (!more) break;
    __syncthreads();  // the workgroup's waves start the next round together
    cur = nxt;
    item = next;
    valid = next_valid;
    first += step;
  }
}

template <class GEO, bool VL, bool VS, int EPI>
int launch_instance(const Conv2dArgs &a, hipStream_t stream) {
  DeviceInfo dev;
  if (current_device_info(&dev) != CCE_OK) return CCE_ERR_LAUNCH;
  const size_t lds_bytes = ((size_t)GEO::WS_FLOATS + (size_t)WAVES * GEO::WIN) * sizeof(float);
  if (lds_bytes > dev.lds_per_block) return CCE_ERR_UNSUPPORTED;
  auto kern = conv2d_relu_hswish_kernel<GEO, VL, VS, EPI>;
  static LaunchCache cache;
  const int per_cu = launch_setup((const void *)kern, cache, dev.device, lds_bytes, THREADS);
  if (per_cu < 0) return CCE_ERR_LAUNCH;
  int grid = dev.num_cus * per_cu;
  const int needed = (a.items + WAVES - 1) / WAVES;
  if (grid > needed) grid = needed;
  grid = (grid + 7) & ~7;  // the XCD remap needs a multiple of 8; surplus waves exit
  hipLaunchKernelGGL(kern, dim3(grid), dim3(THREADS), lds_bytes, stream, a);
  return launch_status(stream, "conv2d_relu_hswish_kernel");
}

// Strip decomposition of one layer shape and its launch: 16-byte window
// loads when W % 4 == 0 and x is 16-byte aligned, 16-byte stores when
// Ho * Wo % 4 == 0 and y is 16-byte aligned, scalar ones otherwise.
// Epilogue parameters of the GELU form (ignored by HardSwish).
struct EpiParams {
  const float *s = nullptr;
  float slope = 0.0f, lo = 0.0f, hi = 0.0f;
};

// GEO serves the 16-byte window loads, GEO_S the scalar ones (a taller
// strip's scalar window prefetch can spill where its 16-byte one does not).
template <class GEO, int EPI = kReluHswish, class GEO_S = GEO>
int launch_layer(const float *x, const float *w, const float *b, float *y, int N, int H, int W,
                 hipStream_t stream, const EpiParams &ep = EpiParams()) {
  static_assert(GEO::CI == GEO_S::CI && GEO::CO == GEO_S::CO && GEO::KS == GEO_S::KS, "one layer shape");
  Conv2dArgs a;
  a.x = x;
  a.w = w;
  a.b = b;
  a.y = y;
  a.s = ep.s;
  a.slope = ep.slope;
  a.lo = ep.lo;
  a.hi = ep.hi;
  a.H = H;
  a.W = W;
  a.Ho = H - (GEO::KS - 1);
  a.Wo = W - (GEO::KS - 1);
  a.P = a.Ho * a.Wo;

  // The 16-byte paths address one image through 32-bit buffer offsets.
  const bool vl = (W % 4 == 0) && ((uintptr_t)x % 16 == 0) && (long long)GEO::CI * H * W * 4 < (1LL << 31);
  const bool vs = (a.P % 4 == 0) && ((uintptr_t)y % 16 == 0) && (long long)GEO::CO * a.P * 4 < (1LL << 31);
  // Largest left shift any row's strips take (0 when stores are scalar).
  int sh_max = 0;
  if (vs)
    for (int r = 0; r < 4 && r < a.Ho; ++r) {
      const int sh = (r * (a.Wo & 3)) & 3;
      if (sh > sh_max) sh_max = sh;
    }
  auto strips = [&](int sw, int rb) {
    a.S = (a.Wo + sh_max + sw - 1) / sw;
    a.G = (a.Ho + rb - 1) / rb;
    const long long items = (long long)N * a.G * a.S;
    if (items >= (1LL << 31) - (1LL << 24)) return false;
    a.items = (int)items;
    a.divS = make_fastdiv((uint32_t)a.S);
    a.divG = make_fastdiv((uint32_t)a.G);
    return true;
  };

  if (vl) {
    if (!strips(GEO::SW, GEO::RB)) return CCE_ERR_TOO_LARGE;
    return vs ? launch_instance<GEO, true, true, EPI>(a, stream) : launch_instance<GEO, true, false, EPI>(a, stream);
  }
  if (!strips(GEO_S::SW, GEO_S::RB)) return CCE_ERR_TOO_LARGE;
  return vs ? launch_instance<GEO_S, false, true, EPI>(a, stream)
            : launch_instance<GEO_S, false, false, EPI>(a, stream);
}

}  // namespace

int launch_conv2d_relu_hswish(const float *x, const float *w, const float *b, float *y, int N,
                              int C_in, int H, int W, int C_out, int k, hipStream_t stream) {
  // The page's layer, 8 -> 64 channels, 3 x 3: strips of 1 row x 16 columns.
  // Measured on MI355X with 16-wave workgroups (ms):
  // 1 x 16: 0.194 at N = 128 and 0.0184 at N = 8 (two rounds per workgroup,
  // so the first round's stores overlap the second round's MFMAs); 2 x 16:
  // 0.196 and 0.0197.  With 8-wave workgroups 2 x 16 was best (0.199), 1 x 32
  // 0.211, 3 x 16 0.294 (spills).
  if (C_in == 8 && C_out == 64 && k == 3)
    return launch_layer<StripGeo<1, 1, 8, 64, 3>>(x, w, b, y, N, H, W, stream);
  // Other layer shapes whose weights and 16 wave windows fit in LDS: C_in of
  // 4, 8 or 16, C_out of 16, 32 or 64, 1 x 1, 3 x 3 or 5 x 5 kernels (5 x 5
  // up to 8 input channels).  The 16-byte paths matter as much here: with
  // scalar loads the 16-channel and 5 x 5 windows (15-18 floats per lane in
  // flight) spill, and 16 -> 64, 3 x 3 ran at 0.31 instead of 0.69 of peak.
  // With 16 or 32 output channels a 1 x 16 strip carries only 1 or 2 MFMAs
  // per K-step against the same window staging, addressing and barrier:
  // their 16-byte instances take 2 x 16 strips (N = 32, 128 x 128: 8 -> 16,
  // 3 x 3 0.0176 -> 0.0167 ms, 16 -> 32 0.0482 -> 0.0463, 8 -> 16, 5 x 5
  // 0.0382 -> 0.0345, 4 -> 16, 1 x 1 0.0100 -> 0.0092).  With 64 channels
  // 2 x 16 strips gained nothing; their scalar instances spill.
#define CCE_CONV2D_LAYER(CI, CO, KS)                                                        \
  if (C_in == CI && C_out == CO && k == KS)                                                \
    return launch_layer<StripGeo<CO <= 32 ? 2 : 1, 1, CI, CO, KS>, kReluHswish,              \
                        StripGeo<1, 1, CI, CO, KS>>(x, w, b, y, N, H, W, stream);
#define CCE_CONV2D_LAYERS_CO(CI, KS) \
  CCE_CONV2D_LAYER(CI, 16, KS) CCE_CONV2D_LAYER(CI, 32, KS) CCE_CONV2D_LAYER(CI, 64, KS)
  CCE_CONV2D_LAYERS_CO(4, 1) CCE_CONV2D_LAYERS_CO(8, 1) CCE_CONV2D_LAYERS_CO(16, 1)
  CCE_CONV2D_LAYERS_CO(4, 3) CCE_CONV2D_LAYER(8, 16, 3) CCE_CONV2D_LAYER(8, 32, 3)
  CCE_CONV2D_LAYERS_CO(16, 3)
  CCE_CONV2D_LAYERS_CO(4, 5) CCE_CONV2D_LAYERS_CO(8, 5)
#undef CCE_CONV2D_LAYERS_CO
#undef CCE_CONV2D_LAYER
  return CCE_ERR_UNSUPPORTED;
}

int launch_pointwise_lrelu_add_clamp_gelu(const float *x, const float *w, const float *b,
                                          const float *s, float *y, int N, int C_in, int rows,
                                          int W, int C_out, float slope, float lo, float hi,
                                          hipStream_t stream) {
  // A 1 x 1 x 1 Conv3d over [N, C_in, D, H, W] is a 1 x 1 Conv2d over
  // [N, C_in, D * H, W]: the strip kernel with the GELU epilogue.  Measured
  // on MI355X at N = 32, 16 x 64 x 64: 0.129 ms here against 0.173 ms on the
  // Conv3d plane-ring kernel for 8 -> 64, 0.128 against 0.173 ms for
  // 16 -> 64 (that kernel's per-tile barrier and plane staging carry only two
  // K-steps of work).
  if ((long long)N * rows >= (1LL << 31) || (long long)C_in * rows * W >= (1LL << 31) ||
      (long long)C_out * rows * W >= (1LL << 31))
    return CCE_ERR_TOO_LARGE;
  EpiParams ep;
  ep.s = s;
  ep.slope = slope;
  ep.lo = lo;
  ep.hi = hi;
  const bool series = lo >= -1.0f && hi <= 1.0f;
#define CCE_POINTWISE_LAYER(CI, CO)                                                              \
  if (C_in == CI && C_out == CO)                                                                 \
    return series ? launch_layer<StripGeo<1, 1, CI, CO, 1>, kGeluSeries>(x, w, b, y, N, rows, W, stream, ep) \
                  : launch_layer<StripGeo<1, 1, CI, CO, 1>, kGeluErf>(x, w, b, y, N, rows, W, stream, ep);
#define CCE_POINTWISE_LAYERS_CO(CI) CCE_POINTWISE_LAYER(CI, 16) CCE_POINTWISE_LAYER(CI, 32) CCE_POINTWISE_LAYER(CI, 64)
  CCE_POINTWISE_LAYERS_CO(4) CCE_POINTWISE_LAYERS_CO(8) CCE_POINTWISE_LAYERS_CO(16)
#undef CCE_POINTWISE_LAYERS_CO
#undef CCE_POINTWISE_LAYER
  return CCE_ERR_UNSUPPORTED;
}

}  // namespace cce
