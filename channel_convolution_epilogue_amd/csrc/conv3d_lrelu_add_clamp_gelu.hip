// Conv3d k x k x k (the page's 3 x 3 x 3, 8 -> 64 channels, and other channel
// counts; 1 x 1 x 1 layers run on the Conv2d strip kernel, see the dispatch at
// the end), stride 1, padding 0, + bias -> LeakyReLU ->
// + s[channel] -> clamp -> exact GELU, fused in one gfx950 kernel
// (POPCORNBENCH Kimi-K2.6 l2_p90: Conv3d followed by LeakyReLU(0.2), the
// learnable [C_out,1,1,1] sum_tensor, clamp to [-1, 1] and GELU with
// approximate=False).
//
// Design:
//  * Implicit GEMM on the fp32 matrix cores: M = output voxels, N = the 64
//    output channels, K = 8 channels x 27 taps = 216 (54 K-steps of 4).
//  * A tile is one output depth plane d of a block of TR output rows and TC
//    output columns of one image (TC = the whole row when it fits).  Its
//    input -- 8 channels x 3 depth planes x (TR + 2) rows x (TC + 2) columns
//    -- comes from a ring of 4 staged input planes in LDS: a workgroup walks
//    d = 0, 1, 2, ... down one row block, so each tile needs one new plane,
//    which is loaded into registers during the tile's MFMAs and written to
//    the ring's free slot after them; one barrier per tile.
//  * The 216 x 64 weight sits in LDS in B-operand order (55 KB): one 16-byte
//    read per K-step gives a lane its B values for all four 16-channel blocks,
//    so each A value read from LDS feeds four MFMAs.  Every wave of the
//    16-wave workgroup computes one or two 16-voxel blocks x 64 channels per
//    tile pass: four or eight independent accumulator chains.
//  * Workgroups take row blocks round-robin (remapped so each XCD gets a
//    contiguous run): neighbouring row blocks of one image run at the same
//    time and write neighbouring stretches of every output plane.
//  * A tile's time is set by the busiest SIMD (a barrier ends each tile), so
//    for the page's layer the row blocks are balanced (62 rows as 7, 8, 8,
//    8, 7, 8, 8, 8), each workgroup's successive blocks rotate through an
//    image's row blocks (four rounds give every workgroup 31 rows, where
//    fixed 8-row blocks gave most of them 32 and one in eight 24), and the
//    waves take one or two 16-voxel blocks each so that the four SIMDs
//    share a tile's blocks evenly: 1.482 -> 1.456 ms, bit-identical.
//  * The epilogue (bias as accumulator init, LeakyReLU, add, clamp, GELU with
//    erf) runs in registers; only the final value is stored.
//  * The page's layer (64-float staged rows, 8-row tiles, 16-byte loads)
//    stages planes with raw buffer loads whose per-thread offsets are fixed
//    per row block, and stores whole-row tiles with buffer stores: a few adds
//    per plane and per quad instead of per-lane address arithmetic and
//    bounds checks, which on gfx950 cost matrix-core time (fp32 MFMAs and
//    VALU instructions share a SIMD's datapath).  Each wave writes the next
//    plane to LDS right after its MFMAs and before its result stores, so
//    the wait for the plane's loads is not also a wait for those stores
//    (vector-memory loads and stores share one counter).  1.53 -> 1.49 ms
//    for the page's workload, bit-identical.
#include <type_traits>

#include "cce_device.hpp"
#include "cce_internal.hpp"

namespace cce {
namespace {

constexpr int WAVES = 16, THREADS = 64 * WAVES;  // one workgroup per CU, 4 waves per SIMD

// Layer shape: CI input channels (a multiple of 4: one per lane group per
// K-step), CO output channels (16 per MFMA block, at most 64), KS x KS x KS
// kernel.  The LDS ring holds KS + 1 input planes: KS for the current tile
// and one being filled for the next.
template <int CI_, int CO_, int KS_>
struct Layer3 {
  static constexpr int CI = CI_, CO = CO_, KS = KS_, TAPS = KS * KS * KS, SLOTS = KS + 1;
  static constexpr int KSTEPS = (CI / 4) * TAPS;      // K-steps of 4 taps (54 for 8 channels, 3^3)
  static constexpr int NT = CO / 16;                  // 16-channel MFMA blocks
  static constexpr int WS_FLOATS = KSTEPS * 64 * NT;  // weights, B-operand order (55 KB for 8 -> 64)
  static_assert(CI % 4 == 0 && CO % 16 == 0 && NT >= 1 && NT <= 4, "layer shape");
};
constexpr int MT = 2;                        // 16-voxel blocks per wave per pass, at most
constexpr int kPrefetchPasses = 2;           // a plane of 8 x 10 rows of 64 floats takes 2 passes

struct Conv3dArgs {
  const float *__restrict__ x;
  const float *__restrict__ w;
  const float *__restrict__ b;
  const float *__restrict__ s;
  float *__restrict__ y;
  int D, H, W, Do, Ho, Wo;
  int TR;           // output rows per tile
  int TC;           // output columns per tile (a multiple of 4, or Wo)
  int XC;           // staged columns per row in LDS
  int rowtiles;     // ceil(Ho / TR)
  int coltiles;     // ceil(Wo / TC)
  int nblocks;      // N * rowtiles * coltiles row-column blocks
  int chstride;     // floats between channels in LDS (KS + 1 planes + padding)
  int planestride;  // floats between ring slots, (TR + 2) * XC
  int ych;          // output channels per image in y (CO, or more when a
                    // launch writes a slice of the channels)
  float slope, lo, hi;
  FastDiv divRowCol, divCol, divTC, divTClast;
};

// One staged input plane dd of a row-column block: staged row `row` =
// rr * CI + ci <-> x[n][ci][dd][h0 + rr][c0 ...], stored in ring slot dd % 4.
template <int CI>
struct PlaneSrc {
  const float *x;
  int D, H, W, n, dd, h0, c0;
  __device__ __forceinline__ const float *operator()(int row) const {
    const int ci = row % CI, rr = row / CI;
    return x + ((((size_t)n * CI + ci) * D + dd) * H + (h0 + rr)) * W + c0;
  }
};
template <int CI>
struct PlaneDst {
  float *xs;
  int chstride, slot_off, XC;
  __device__ __forceinline__ float *operator()(int row) const {
    return xs + (row % CI) * chstride + slot_off + (row / CI) * XC;
  }
};

// Plane staging with raw buffer loads (16-byte quads; the image is below
// 2^31 bytes) for planes that one thread can cover in KPRE passes of one
// quad each: the per-thread source offsets and LDS destinations are fixed
// per row block, so staging a plane costs one add per quad.  Threads past
// the plane's rows repeat a quad another thread stages (the same data to the
// same LDS place), so every load and LDS write is unconditional.
template <int CI, int KPRE, int THREADS>
struct FastPlane {
  v4f v[KPRE];
  uint32_t src[KPRE];  // byte offset in the image, less the plane's
  int dst[KPRE];       // float offset in a ring slot

  __device__ __forceinline__ void init(int nr, int len, int tid, int D, int H, int W, int h0, int c0,
                                       int chstride, int XC) {
    const int cw = len >> 2, rpp = THREADS / cw;
    const int my_row = tid / cw, my_col = tid - my_row * cw;
#pragma unroll
    for (int k = 0; k < KPRE; ++k) {
      int row = my_row + k * rpp;
      if (row >= nr) row = my_row < nr ? my_row : 0;
      const int ci = row % CI, rr = row / CI;
      src[k] = (uint32_t)((ci * D * H + h0 + rr) * W + c0 + 4 * my_col) * 4u;
      dst[k] = ci * chstride + rr * XC + 4 * my_col;
    }
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t plane_off) {
#pragma unroll
    for (int k = 0; k < KPRE; ++k) v[k] = buffer_load4(r, src[k] + plane_off, 0u);
  }
  __device__ __forceinline__ void store(float *slot) const {
#pragma unroll
    for (int k = 0; k < KPRE; ++k) *reinterpret_cast<v4f *>(slot + dst[k]) = v[k];
  }
};

// LDS floats for tiles of tr rows whose staged rows hold xc floats: ring
// slots of (tr + KS - 1) xc floats, channels 16 mod 64 floats apart so the
// four lane groups of an A read (four channels) start on four different
// quarters of the 64 LDS banks.
template <int KS>
constexpr int plane_floats(int tr, int xc) { return (tr + KS - 1) * xc; }
template <int KS>
constexpr int chan_floats(int tr, int xc) {
  return (KS + 1) * plane_floats<KS>(tr, xc) + ((16 - ((KS + 1) * plane_floats<KS>(tr, xc)) % 64) + 64) % 64;
}

// FIXED_XC / FIXED_TR: staged row length and tile rows known at compile time
// (then every per-step LDS offset is an immediate); 0 = taken from the args.
// VLOAD: W % 4 == 0 and x 16-byte aligned (16-byte plane loads).
// VSTORE: every lane's four voxels are consecutive and 16-byte aligned in y.
// SERIES: the clamp bounds lie in [-1, 1] (series GELU).
template <class L, int FIXED_XC, int FIXED_TR, bool VLOAD, bool VSTORE, bool SERIES>
__global__ __launch_bounds__(THREADS, 4) void conv3d_lrelu_add_clamp_gelu_kernel(Conv3dArgs a) {
  constexpr int CI = L::CI, CO = L::CO, KSTEPS = L::KSTEPS, NT = L::NT, WS_FLOATS = L::WS_FLOATS;
  constexpr int KS = L::KS, TAPS = L::TAPS, SLOTS = L::SLOTS;
  const int XC = FIXED_XC ? FIXED_XC : a.XC;
  const int TR = FIXED_TR ? FIXED_TR : a.TR;
  const int chstride = FIXED_XC ? chan_floats<KS>(FIXED_TR, FIXED_XC) : a.chstride;
  const int planestride = FIXED_XC ? plane_floats<KS>(FIXED_TR, FIXED_XC) : a.planestride;
  // FAST: compile-time row length with 16-byte loads -- buffer-addressed
  // plane staging and (for whole-row tiles) result stores.
  constexpr bool FAST = FIXED_XC != 0 && VLOAD;
  // BAL (FAST with 16-byte stores, whole-row tiles): balanced row tiles in
  // a rotating order.  A FAST tile has at most 32 blocks (8 rows of at most
  // XC - KS + 1 voxels, plus 3 + 3 for alignment): one pass per wave.
  constexpr bool BAL = FAST && VSTORE;
  static_assert(!FAST || FIXED_TR * (FIXED_XC - KS + 1) + 6 <= MT * 16 * WAVES, "one pass per wave");
  static_assert(!FAST || kPrefetchPasses * (THREADS / (FIXED_XC / 4)) >= CI * (FIXED_TR + KS - 1),
                "a plane fits in the prefetch passes");
  extern __shared__ __attribute__((aligned(16))) float lds[];
  float *ws = lds;              // weights, B-operand order
  float *xs = lds + WS_FLOATS;  // ring of input planes
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;

  // ws[s][lane][nt] = w[16 nt + lane % 16][4 (s / TAPS) + lane / 16][tap s % TAPS].
  // At half scale (exact): the accumulators then hold v / 2, and the
  // epilogue on halved values skips one multiplication per output.
  stage_weights_b<CI, CO, TAPS, THREADS>(ws, a.w, tid, 0.5f);
  // Bias and the added per-channel term, halved, read from LDS when needed
  // (fewer live registers): ep[c] = b[c] / 2, ep[64 + c] = s[c] / 2.
  float *ep = xs + CI * chstride;
  if (tid < CO) {
    ep[tid] = a.b ? 0.5f * a.b[tid] : 0.0f;
    ep[CO + tid] = 0.5f * a.s[tid];
  }
  const float lo_half = 0.5f * a.lo, hi_half = 0.5f * a.hi;
  // Output voxels per (n, channel); one image's output is below 2^31 floats,
  // so offsets within it are 32-bit.
  const int vol = a.Do * a.Ho * a.Wo;

  // Row-column blocks round-robin; the hardware hands workgroups to the 8
  // XCDs in turn, and the remap gives each XCD consecutive blocks.
  // (gridDim.x is a multiple of 8.)
  const int per_xcd = gridDim.x >> 3;
  const int vb = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);

  RowStage<kPrefetchPasses, VLOAD, THREADS> stage;
  FastPlane<CI, kPrefetchPasses, THREADS> fp;
  const uint32_t plane_bytes = (uint32_t)(a.H * a.W) * 4u;
  // FAST stores: this lane's byte offset in channel block 0 of an image's
  // output, relative to a tile's first voxel.
  const uint32_t sofs = (uint32_t)(((size_t)col * vol + 4 * g) * 4);
  __syncthreads();  // weights in place

  for (int rb = vb; rb < a.nblocks; rb += gridDim.x) {
    const int n = fdiv(rb, a.divRowCol), rc = rb - n * (a.rowtiles * a.coltiles);
    int rt = fdiv(rc, a.divCol), h0, rows;
    const int ct = rc - rt * a.coltiles;
    if constexpr (BAL) {
      // Row tiles of floor or ceil(Ho / rowtiles) rows, taken in an order
      // that rotates with the round (the image's first block index over the
      // grid), so that the row tiles one workgroup takes in consecutive
      // rounds are consecutive: 62 rows as 7, 8, 8, 8, 7, 8, 8, 8 give
      // every workgroup 31 rows over four rounds.
      rt = (rt + (n * a.rowtiles) / (int)gridDim.x) % a.rowtiles;
      h0 = (int)((long long)rt * a.Ho / a.rowtiles);
      rows = (int)((long long)(rt + 1) * a.Ho / a.rowtiles) - h0;
    } else {
      h0 = rt * TR;
      rows = min(TR, a.Ho - h0);
    }
    const int c0 = ct * a.TC, cols = min(a.TC, a.Wo - c0);
    const bool last_col = ct == a.coltiles - 1;
    const int nr = CI * (rows + KS - 1);                // staged rows per plane
    const int len = min(XC, a.W - c0);                // staged floats per row
    const bool contig = a.coltiles == 1;                // the tile spans whole output rows
    // BAL: the tile's voxels are [f_lo, f_hi) of the output plane, taken as
    // 16-voxel blocks from the 4-aligned s0 up to the 4-aligned e0 (so every
    // lane's quad is 16-byte aligned); the quads at either end may be partial.
    const int f_lo = h0 * a.Wo, f_hi = f_lo + rows * a.Wo;
    const int s0 = BAL ? (f_lo & ~3) : f_lo, e0 = BAL ? ((f_hi + 3) & ~3) : f_hi;
    const int V = BAL ? e0 - s0 : rows * cols, MTT = (V + 15) >> 4;  // voxels and 16-voxel blocks
    auto src_of = [&](int dd) { return PlaneSrc<CI>{a.x, a.D, a.H, a.W, n, dd, h0, c0}; };
    auto dst_of = [&](int dd) { return PlaneDst<CI>{xs, chstride, (dd % SLOTS) * planestride, XC}; };
    const size_t img = (size_t)CI * a.D * a.H * a.W;  // input floats per image
    const auto rx = buffer_rsrc(a.x + n * img, (uint32_t)(img * 4));  // used when FAST

    // Planes 0 .. KS - 1 of this block (every wave is past the previous
    // block's last barrier, so all slots are free).
    if constexpr (FAST) {
      fp.init(nr, len, tid, a.D, a.H, a.W, h0, c0, chstride, XC);
#pragma unroll 1
      for (int dd = 0; dd < KS; ++dd) {
        fp.load(rx, (uint32_t)dd * plane_bytes);
        fp.store(xs + (dd % SLOTS) * planestride);
      }
    } else {
      stage.init(len, tid);
#pragma unroll 1
      for (int dd = 0; dd < KS; ++dd) {
        stage.load(nr, src_of(dd));
        stage.store(nr, src_of(dd), dst_of(dd));
      }
    }
    __syncthreads();

#pragma unroll 1
    for (int d = 0; d < a.Do; ++d) {
      const bool more = d + KS < a.D;  // plane d + KS exists
      // Plane d + KS, in flight during this tile's MFMAs.
      // FAST: loaded and written to its slot unconditionally (the last tile
      // of a block reloads plane D - 1 into a slot no later tile of the block
      // reads), so that the compiler's wait counts see every load consumed.
      if constexpr (FAST) {
        fp.load(rx, (uint32_t)min(d + KS, a.D - 1) * plane_bytes);
      } else {
        if (more) stage.load(nr, src_of(d + KS));
      }
      int so[KS];  // ring slot offsets of planes d .. d + KS - 1
#pragma unroll
      for (int kd = 0; kd < KS; ++kd) so[kd] = ((d + kd) % SLOTS) * planestride;
      float *ytile = a.y + (size_t)n * a.ych * vol + (size_t)d * a.Ho * a.Wo;  // uniform

      // One pass: blocks mb_iv .. mb_iv + NB - 1 of the tile (NB = 1 or 2).
      // FIRST (FAST only): plane d + KS goes to slot (d + KS) % (KS + 1)
      // (last read by tile d - 1, which every wave finished before the
      // previous barrier) right after the pass's MFMAs, before any of the
      // tile's result stores, so that waiting for its loads does not also
      // wait for those stores.
      auto pass = [&](int mb_iv, auto first, auto nblk) {
        constexpr int NB = decltype(nblk)::value;
        // Compiler-only fences: the first keeps the per-step weight reads
        // inside the loop instead of hoisting all 54 of them (216 VGPRs) out
        // of it; the second hides the block index from strength reduction,
        // which would otherwise keep eight 64-bit store pointers live.
        asm volatile("" ::: "memory");
        int mb = mb_iv;
        asm volatile("" : "+v"(mb));
        int base[NB][KS];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          // Surplus lanes repeat a voxel of the tile (results not stored).
          const int v = BAL ? min(max(s0 + 16 * (mb + j) + col, f_lo), f_hi - 1) - f_lo
                            : min(16 * (mb + j) + col, V - 1);
          const int hl = fdiv(v, last_col ? a.divTClast : a.divTC), wl = v - hl * cols;
          const int b0 = g * chstride + hl * XC + wl;
#pragma unroll
          for (int kd = 0; kd < KS; ++kd) base[j][kd] = b0 + so[kd];
        }
        v4f acc[NB][NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float bias = ep[16 * nt + col];
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[j][nt] = splat4(bias);
        }

        // The A and B operands of K-step s + 1 are read from LDS while step s's
        // MFMAs run (two register slots, the read pinned before the MFMAs by a
        // scheduling barrier).  The four waves of a SIMD finish a pass in age
        // order, so each pass ends with one wave issuing alone; reading its
        // operands a step ahead keeps it from waiting on LDS at every step
        // (1.543 instead of 1.592 ms for the page's workload).
        float bq[2][NT], aq[2][NB];
        auto fetch = [&](int s, int slot) {
          const int tt = s % TAPS, kd = tt / (KS * KS), kh = (tt / KS) % KS, kw = tt % KS;
          const int off = (s / TAPS) * 4 * chstride + kh * XC + kw;
          load_b<NT>(bq[slot], &ws[(s * 64 + lane) * NT]);
#pragma unroll
          for (int j = 0; j < NB; ++j) aq[slot][j] = xs[base[j][kd] + off];
        };
        fetch(0, 0);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          if (s + 1 < KSTEPS) fetch(s + 1, (s + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              acc[j][nt] = mfma16x16x4(aq[s & 1][j], bq[s & 1][nt], acc[j][nt]);
        }

        if constexpr (FAST && decltype(first)::value) {
          asm volatile("" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
          fp.store(xs + ((d + KS) % SLOTS) * planestride);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (FAST) {
          if (VSTORE && contig) {
            // Whole-row tiles: the plane's voxel count and every lane's
            // first voxel are multiples of 4 (VSTORE), so each lane's quad is
            // 16-byte aligned; only the tile's first and last quads can be
            // partial, and store element by element (voxels outside the tile
            // get an offset past the buffer's end).
            const auto ry = buffer_rsrc(a.y + (size_t)n * a.ych * vol, (uint32_t)(CO * vol) * 4u);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              const int q0 = s0 + 16 * (mb + j) + 4 * g;  // this lane's first voxel in the plane
              if (q0 >= e0) continue;
              const bool whole = q0 >= f_lo && q0 + 4 <= f_hi;
              const uint32_t voff = sofs + (uint32_t)(d * a.Ho * a.Wo + s0 + 16 * (mb + j)) * 4u;
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) {
                const float sadd = ep[CO + 16 * nt + col];
                v4f r = acc[j][nt];
                r.x = lrelu_add_clamp_gelu_half<SERIES>(r.x, sadd, a.slope, lo_half, hi_half);
                r.y = lrelu_add_clamp_gelu_half<SERIES>(r.y, sadd, a.slope, lo_half, hi_half);
                r.z = lrelu_add_clamp_gelu_half<SERIES>(r.z, sadd, a.slope, lo_half, hi_half);
                r.w = lrelu_add_clamp_gelu_half<SERIES>(r.w, sadd, a.slope, lo_half, hi_half);
                const uint32_t o = voff + (uint32_t)(16 * nt * vol) * 4u;
                if (whole) {
                  buffer_store4(ry, r, o);
                } else {
#pragma unroll
                  for (int e = 0; e < 4; ++e)
                    buffer_store1(ry, r[e], q0 + e >= f_lo && q0 + e < f_hi ? o + 4u * e : kBufferOOB);
                }
              }
            }
            return;
          }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int v0 = 16 * (mb + j) + 4 * g;  // this lane's first voxel in the tile
          if (v0 >= V) continue;  // (inside the block loop)
          // Output offset of voxel v0 within the (n, channel, d) plane.
          int off0, run;  // run: voxels from v0 that are consecutive in memory
          if (contig) {
            off0 = h0 * a.Wo + v0;
            run = V - v0;
          } else {
            const int hl = fdiv(v0, last_col ? a.divTClast : a.divTC), wl = v0 - hl * cols;
            off0 = (h0 + hl) * a.Wo + c0 + wl;
            run = cols - wl;
          }
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const float sadd = ep[CO + 16 * nt + col];
            v4f r = acc[j][nt];
            r.x = lrelu_add_clamp_gelu_half<SERIES>(r.x, sadd, a.slope, lo_half, hi_half);
            r.y = lrelu_add_clamp_gelu_half<SERIES>(r.y, sadd, a.slope, lo_half, hi_half);
            r.z = lrelu_add_clamp_gelu_half<SERIES>(r.z, sadd, a.slope, lo_half, hi_half);
            r.w = lrelu_add_clamp_gelu_half<SERIES>(r.w, sadd, a.slope, lo_half, hi_half);
            float *dst = ytile + ((16 * nt + col) * vol + off0);
            if (VSTORE && run >= 4) {
              store4(dst, r);
            } else {
              // Voxels past the end of a row segment continue on the next row.
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int ve = v0 + e;
                if (ve >= V) break;
                if (contig) {
                  dst[e] = r[e];
                } else {
                  const int hl = fdiv(ve, last_col ? a.divTClast : a.divTC), wl = ve - hl * cols;
                  ytile[(16 * nt + col) * vol + (h0 + hl) * a.Wo + c0 + wl] = r[e];
                }
              }
            }
          }
        }
      };

      using One = std::integral_constant<int, 1>;
      using Two = std::integral_constant<int, 2>;
      using First = std::integral_constant<bool, FAST>;
      if (MTT <= MT * WAVES) {
        // One pass per wave: the first MTT - 16 waves take two blocks, the
        // rest one (waves w, w + 4, w + 8, w + 12 share a SIMD, so each SIMD
        // gets a quarter of the blocks, rounded up).  Always the case for
        // FAST (8 rows of at most 62 voxels, plus alignment).
        const int w = __builtin_amdgcn_readfirstlane(wave), q = max(MTT - WAVES, 0);
        if (w < q) {
          pass(2 * w, First(), Two());
        } else if (q + w < MTT) {
          pass(q + w, First(), One());
        } else {
          if constexpr (FAST) fp.store(xs + ((d + KS) % SLOTS) * planestride);  // a wave with no block
        }
      } else {
        if constexpr (!FAST) {
#pragma unroll 1
          for (int mb_iv = MT * wave; mb_iv < MTT; mb_iv += MT * WAVES) pass(mb_iv, First(), Two());
        }
      }

      // Plane d + KS goes to slot (d + KS) % (KS + 1), last read by tile d - 1, which
      // every wave finished before the previous barrier.
      if constexpr (!FAST) {
        if (more) stage.store(nr, src_of(d + KS), dst_of(d + KS));
      }
      __syncthreads();  // plane d + KS visible; plane d free
    }
  }
}

template <class L, int FXC, int FTR, bool VL, bool VS, bool SER>
int launch_instance(const Conv3dArgs &a, size_t lds_bytes, const DeviceInfo &dev,
                    hipStream_t stream) {
  auto kern = conv3d_lrelu_add_clamp_gelu_kernel<L, FXC, FTR, VL, VS, SER>;
  static LaunchCache cache;
  const int per_cu = launch_setup((const void *)kern, cache, dev.device, lds_bytes, THREADS);
  if (per_cu < 0) return CCE_ERR_LAUNCH;
  int grid = dev.num_cus * per_cu;
  if (grid > a.nblocks) grid = a.nblocks;
  grid = (grid + 7) & ~7;  // the XCD remap needs a multiple of 8; surplus workgroups exit
  hipLaunchKernelGGL(kern, dim3(grid), dim3(THREADS), lds_bytes, stream, a);
  return launch_status(stream, "conv3d_lrelu_add_clamp_gelu_kernel");
}

template <class L, bool VL, bool VS, bool FIXED64>
int launch_series(const Conv3dArgs &a, size_t lds_bytes, const DeviceInfo &dev,
                  hipStream_t stream) {
  const bool series = a.lo >= -1.0f && a.hi <= 1.0f;
  // FIXED64: 64-float staged rows in 8-row tiles (W = 64, as in the page's
  // workload) get their own instance with compile-time LDS offsets.
  if constexpr (FIXED64) {
    const bool img31 = (long long)L::CI * a.D * a.H * a.W * 4 < (1LL << 31) &&
                       (long long)L::CO * a.Do * a.Ho * a.Wo * 4 < (1LL << 31);
    if (a.XC == 64 && a.TR == 8 && img31)
      return series ? launch_instance<L, 64, 8, VL, VS, true>(a, lds_bytes, dev, stream)
                    : launch_instance<L, 64, 8, VL, VS, false>(a, lds_bytes, dev, stream);
  }
  return series ? launch_instance<L, 0, 0, VL, VS, true>(a, lds_bytes, dev, stream)
                : launch_instance<L, 0, 0, VL, VS, false>(a, lds_bytes, dev, stream);
}

template <class L>
size_t ring_floats(int tr, int xc, int *planestride, int *chstride) {
  *planestride = plane_floats<L::KS>(tr, xc);
  *chstride = chan_floats<L::KS>(tr, xc);
  return (size_t)L::CI * *chstride;
}

// Tiling of one layer shape and its launch: 16-byte loads and stores where
// sizes and alignment allow, the polynomial GELU when [lo, hi] lies in
// [-1, 1].  FIXED64: also the instances with compile-time LDS offsets for
// 64-wide rows in 8-row tiles (the page's layer).  ych: output channels per
// image in y (L::CO unless the launch writes a slice of y's channels).
template <class L, bool FIXED64>
int launch_layer(const float *x, const float *w, const float *b, const float *s, float *y, int N,
                 int D, int H, int W, float slope, float lo, float hi, hipStream_t stream,
                 int ych = L::CO) {
  constexpr size_t EXTRA = L::WS_FLOATS + 2 * L::CO;  // weights, bias and s beside the ring
  DeviceInfo dev;
  if (current_device_info(&dev) != CCE_OK) return CCE_ERR_LAUNCH;
  Conv3dArgs a;
  a.x = x;
  a.w = w;
  a.b = b;
  a.s = s;
  a.y = y;
  a.ych = ych;
  a.D = D;
  a.H = H;
  a.W = W;
  a.Do = D - (L::KS - 1);
  a.Ho = H - (L::KS - 1);
  a.Wo = W - (L::KS - 1);
  a.slope = slope;
  a.lo = lo;
  a.hi = hi;
  const bool vl = (W % 4 == 0) && ((uintptr_t)x % 16 == 0);
  const size_t budget = dev.lds_per_block / sizeof(float);

  // Whole rows, 8 output rows per tile if they fit; else fewer rows; else
  // column tiles of a multiple of 4 output columns, 8 rows.
  a.TR = 0;
  a.TC = 0;
  a.XC = 0;
  size_t ring = 0;
  for (int tr = 8; tr >= 2 && a.TR == 0; tr /= 2) {
    const int xc = vl ? ((W + 3) & ~3) : W;
    ring = ring_floats<L>(tr, xc, &a.planestride, &a.chstride);
    if (EXTRA + ring <= budget) {
      a.TR = tr;
      a.TC = a.Wo;
      a.XC = xc;
    }
  }
  if (a.TR == 0) {
    a.TR = 8;
    // Staged columns: TC + KS - 1 rounded up to a multiple of 4.
    for (int tc = (a.Wo - 1) & ~3; tc >= 4; tc -= 4) {
      const int xc = (tc + L::KS - 1 + 3) & ~3;
      ring = ring_floats<L>(a.TR, xc, &a.planestride, &a.chstride);
      if (EXTRA + ring <= budget) {
        a.TC = tc;
        a.XC = xc;
        break;
      }
    }
    if (a.TC <= 0 || a.TC >= a.Wo) return CCE_ERR_UNSUPPORTED;
  }
  const size_t lds_bytes = (EXTRA + ring) * sizeof(float);
  a.rowtiles = (a.Ho + a.TR - 1) / a.TR;
  a.coltiles = (a.Wo + a.TC - 1) / a.TC;
  const long long nb = (long long)N * a.rowtiles * a.coltiles;
  if (nb >= (1LL << 31)) return CCE_ERR_TOO_LARGE;
  a.nblocks = (int)nb;
  a.divRowCol = make_fastdiv((uint32_t)(a.rowtiles * a.coltiles));
  a.divCol = make_fastdiv((uint32_t)a.coltiles);
  a.divTC = make_fastdiv((uint32_t)a.TC);
  a.divTClast = make_fastdiv((uint32_t)(a.Wo - (a.coltiles - 1) * a.TC));

  // 16-byte stores need every lane's four voxels consecutive and aligned:
  // whole-row tiles need (TR Wo) and (Ho Wo) multiples of 4; column tiles
  // need Wo % 4 == 0 (TC is a multiple of 4).
  const bool y16 = (uintptr_t)y % 16 == 0;
  const bool vs = y16 &&
                  (a.coltiles == 1 ? ((a.Ho * a.Wo) % 4 == 0 && (a.TR * a.Wo) % 4 == 0) : (a.Wo % 4 == 0));
  if (vl) return vs ? launch_series<L, true, true, FIXED64>(a, lds_bytes, dev, stream)
                    : launch_series<L, true, false, FIXED64>(a, lds_bytes, dev, stream);
  return vs ? launch_series<L, false, true, FIXED64>(a, lds_bytes, dev, stream)
            : launch_series<L, false, false, FIXED64>(a, lds_bytes, dev, stream);
}

}  // namespace

int launch_conv3d_lrelu_add_clamp_gelu(const float *x, const float *w, const float *b,
                                       const float *s, float *y, int N, int C_in, int D, int H,
                                       int W, int C_out, int k, float slope, float lo, float hi,
                                       hipStream_t stream) {
  // The page's layer, 8 -> 64 channels, 3 x 3 x 3, with every fast path.
  if (C_in == 8 && C_out == 64 && k == 3)
    return launch_layer<Layer3<8, 64, 3>, true>(x, w, b, s, y, N, D, H, W, slope, lo, hi, stream);
  // A 1 x 1 x 1 layer is a 1 x 1 Conv2d over D * H rows of W pixels: it runs
  // on the Conv2d strip kernel with this operator's epilogue.  (On this
  // kernel its two K-steps per tile left the plane staging and the per-tile
  // barrier exposed: 0.17 ms for 8 -> 64 at N = 32, 16 x 64 x 64.)
  if (k == 1)
    return launch_pointwise_lrelu_add_clamp_gelu(x, w, b, s, y, N, C_in, D * H, W, C_out, slope,
                                                 lo, hi, stream);
  // Other 3 x 3 x 3 layer shapes: C_in of 4, 8 or 16, C_out of 16, 32 or 64,
  // with the 16-byte paths and the polynomial GELU but run-time LDS offsets.
  // Measured (N = 32, 16 x 64 x 64): 4 -> 16 at 0.52 and 8 -> 32 at 0.70 of
  // peak, against 0.34 and 0.47 with scalar loads, scalar stores and erff.
#define CCE_CONV3D_LAYER(CI, CO, KS)                                                         \
  if (C_in == CI && C_out == CO && k == KS)                                                 \
    return launch_layer<Layer3<CI, CO, KS>, false>(x, w, b, s, y, N, D, H, W, slope, lo, hi, stream);
  CCE_CONV3D_LAYER(4, 16, 3) CCE_CONV3D_LAYER(4, 32, 3) CCE_CONV3D_LAYER(4, 64, 3)
  CCE_CONV3D_LAYER(8, 16, 3) CCE_CONV3D_LAYER(8, 32, 3)
  CCE_CONV3D_LAYER(16, 16, 3) CCE_CONV3D_LAYER(16, 32, 3)
#undef CCE_CONV3D_LAYER
  // 16 -> 64: its 110 KB weight leaves LDS for whole-row tiles of 4 rows
  // only up to 34-float rows; wider rows went to column tiles (8 x 12
  // voxels for W = 64, 6 of a tile's 32 block slots: 0.40 of peak at N = 32,
  // 16 x 64 x 64).  There, two launches of the 16 -> 32 kernel, each with
  // half the weight, bias and s, write output channels 0-31 and 32-63 of
  // every image from 4-row whole-row tiles (0.75 of peak; the input is read
  // twice, 16 of the 80 channels moved per output voxel).
  if (C_in == 16 && C_out == 64 && k == 3) {
    using Full = Layer3<16, 64, 3>;
    using Half = Layer3<16, 32, 3>;
    DeviceInfo dev;
    if (current_device_info(&dev) != CCE_OK) return CCE_ERR_LAUNCH;
    const bool vl = (W % 4 == 0) && ((uintptr_t)x % 16 == 0);
    int ps, cs;
    const size_t need = Full::WS_FLOATS + 2 * Full::CO + ring_floats<Full>(4, vl ? ((W + 3) & ~3) : W, &ps, &cs);
    if (need * sizeof(float) <= dev.lds_per_block)
      return launch_layer<Full, false>(x, w, b, s, y, N, D, H, W, slope, lo, hi, stream);
    const size_t vol = (size_t)(D - 2) * (H - 2) * (W - 2);
    for (int h = 0; h < 2; ++h) {
      const int st = launch_layer<Half, false>(x, w + (size_t)h * 32 * 16 * 27, b ? b + 32 * h : nullptr,
                                               s + 32 * h, y + (size_t)h * 32 * vol, N, D, H, W, slope,
                                               lo, hi, stream, 64);
      if (st != CCE_OK) return st;
    }
    return CCE_OK;
  }
  return CCE_ERR_UNSUPPORTED;
}

}  // namespace cce
