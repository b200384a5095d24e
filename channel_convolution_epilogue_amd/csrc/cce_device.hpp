// Device helpers shared by the gfx950 kernels of libcce.
//
// Matrix-core contraction: every kernel runs its convolution as an implicit
// GEMM on v_mfma_f32_16x16x4_f32 (16 pixels x 16 output channels x 4 taps per
// instruction, fp32 in and out).  Lane layout of that instruction, as used
// throughout (lane l of a 64-wide wave):
//   A operand  lane l supplies A[m = l % 16][k = l / 16]     (pixel m, tap k)
//   B operand  lane l supplies B[k = l / 16][n = l % 16]     (tap k, channel n)
//   D result   lane l holds   D[m = 4 * (l / 16) + r][n = l % 16], r = 0..3
// so each lane ends with four consecutive pixels of one output channel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cce {

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma16x16x4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f splat4(float v) { return v4f{v, v, v, v}; }

// Raw buffer accesses (MUBUF, offset addressing): a 128-bit descriptor holds
// the base address and the buffer's size in bytes, and each lane supplies a
// 32-bit byte offset.  A load whose offset lies at or past the size returns
// zeros without touching memory, so masked window loads need no branch:
// such a lane is given kBufferOOB as its offset (buffers here are smaller
// than 2^31 bytes).  Dword 3 = 0x00020000 selects 32-bit data elements.
constexpr uint32_t kBufferOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ void buffer_store1(__amdgpu_buffer_rsrc_t r, float v, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, (int)voff, 0, 0);
}

// The scalar offset of a store stays the constant 0: with an SGPR there the
// compiler inserts no wait states between a 16-byte store and a following
// VALU write of its data registers, and on gfx950 such a write was seen to
// reach memory in place of the stored data for some lanes.
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, v4f v, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, (int)voff, 0, 0);
}

// Stages a [CO][CI][TAPS] convolution weight (the torch layout) into LDS in
// MFMA B-operand order: K-step s covers input channels 4 (s / TAPS) .. + 3 at
// tap s % TAPS, and
//   ws[(s * 64 + lane) * NT + nt] = w[16 nt + lane % 16][4 (s / TAPS) + lane / 16][s % TAPS].
// The LDS bank of an element depends only on its output channel o, so
// consecutive lanes take consecutive output channels (conflict-free writes
// for C_out = 64) and walk their channel's row of CI * TAPS floats in 16-byte
// reads when w is 16-byte aligned.  Needs CI % 4 == 0, CO % 16 == 0.
//
// Two phases, so that a kernel's prologue pays one memory latency, not one
// per pass: load() issues every global read of the weight into registers
// (a compile-time number of 16-byte reads per thread), place() writes them
// to LDS.  A kernel issues its other prologue loads (bias, first input tile)
// between the two.  A weight that is not 16-byte aligned is copied float by
// float in place().
template <int CI, int CO, int TAPS, int THREADS>
struct WeightStageB {
  static constexpr int NT = CO / 16, ROW = CI * TAPS, QUADS = CO * (ROW / 4);
  static constexpr int IT = (QUADS + THREADS - 1) / THREADS;  // 16-byte reads per thread
  static_assert(CI % 4 == 0 && CO % 16 == 0, "whole K-steps and channel blocks");
  v4f v[IT];
  bool vec;

  __device__ __forceinline__ void load(const float *__restrict__ w, int tid) {
    vec = (reinterpret_cast<uintptr_t>(w) & 15) == 0;
    if (!vec) return;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int p = tid + k * THREADS;  // p = (quad j, channel o)
      if (p < QUADS) {
        const int o = p % CO, j = p / CO;
        v[k] = *reinterpret_cast<const v4f *>(w + o * ROW + 4 * j);
      }
    }
  }

  // scale: a power of two the weights are multiplied by (exactly) on the
  // way into LDS.
  __device__ __forceinline__ void place(float *ws, const float *__restrict__ w, int tid,
                                        float scale = 1.0f) const {
    auto put = [&](int o, int r, float x) {
      const int ci = r / TAPS, tap = r - ci * TAPS;
      const int s = (ci >> 2) * TAPS + tap, lane = ((ci & 3) << 4) | (o & 15);
      ws[(s * 64 + lane) * NT + (o >> 4)] = x * scale;
    };
    if (vec) {
#pragma unroll
      for (int k = 0; k < IT; ++k) {
        const int p = tid + k * THREADS;
        if (p < QUADS) {
          const int o = p % CO, j = p / CO;
          put(o, 4 * j, v[k].x);
          put(o, 4 * j + 1, v[k].y);
          put(o, 4 * j + 2, v[k].z);
          put(o, 4 * j + 3, v[k].w);
        }
      }
    } else {
      for (int p = tid; p < CO * ROW; p += THREADS) {
        const int o = p % CO, r = p / CO;
        put(o, r, w[o * ROW + r]);
      }
    }
  }
};

template <int CI, int CO, int TAPS, int THREADS>
__device__ __forceinline__ void stage_weights_b(float *ws, const float *__restrict__ w, int tid,
                                                float scale = 1.0f) {
  WeightStageB<CI, CO, TAPS, THREADS> st;
  st.load(w, tid);
  st.place(ws, w, tid, scale);
}

// A lane's MFMA B operands of one K-step for NT 16-column channel blocks,
// stored contiguously in LDS: one 16-, 8- or 4-byte LDS read.
template <int NT>
__device__ __forceinline__ void load_b(float (&bv)[NT], const float *p) {
  if constexpr (NT == 4) {
    const v4f v = *reinterpret_cast<const v4f *>(p);
    bv[0] = v.x, bv[1] = v.y, bv[2] = v.z, bv[3] = v.w;
  } else if constexpr (NT == 2) {
    const float2 v = *reinterpret_cast<const float2 *>(p);
    bv[0] = v.x, bv[1] = v.y;
  } else {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bv[nt] = p[nt];
  }
}

__device__ __forceinline__ float clampf(float v, float lo, float hi) {
  return fminf(fmaxf(v, lo), hi);
}

// GELU(t) = 0.5 t (1 + erf(t / sqrt 2)) for |t| <= 1, written as
//   GELU(t) = 0.5 t + u P(u),   u = t^2,
// with P the degree-4 polynomial that minimises max |u (P(u) - R(u))| over
// u in [0, 1], where R(u) = (GELU(t) - 0.5 t) / u = erf(t / sqrt 2) / (2 t)
// is even in t.  The coefficients are that minimax fit (a linear programme
// in double precision, channel_convolution_epilogue_amd/gelu_poly_fit.py)
// rounded to fp32; so rounded, the approximation errs by less than 2e-8 in
// GELU -- below the fp32 rounding of the evaluation itself (about 1e-7).
// Four FMAs where the Maclaurin series of erf needs seven for the same
// accuracy.
constexpr float kGeluP4 = 9.09758819e-05f, kGeluP3 = -0.00116171606f, kGeluP2 = 0.00996111613f,
                kGeluP1 = -0.0664877221f, kGeluP0 = 0.398942083f;

__device__ __forceinline__ float gelu_small(float t) {
  const float u = t * t;
  float r = kGeluP4;
  r = fmaf(r, u, kGeluP3);
  r = fmaf(r, u, kGeluP2);
  r = fmaf(r, u, kGeluP1);
  r = fmaf(r, u, kGeluP0);
  return fmaf(u, r, 0.5f * t);
}

// GELU(2 h) for |h| <= 1/2, from h itself: with u' = h^2 = u / 4 and
// Q(x) = 4 P(4 x), whose coefficients 4^(k+1) p_k are P's scaled by powers
// of two (exactly), GELU(t) = u' Q(u') + h.  Every intermediate is the one
// of gelu_small(2 h) scaled by a power of two, so the result is the same to
// the bit, and the 0.5 t product is gone.
__device__ __forceinline__ float gelu_small_half(float h) {
  const float u = h * h;
  float r = 1024.0f * kGeluP4;
  r = fmaf(r, u, 256.0f * kGeluP3);
  r = fmaf(r, u, 64.0f * kGeluP2);
  r = fmaf(r, u, 16.0f * kGeluP1);
  r = fmaf(r, u, 4.0f * kGeluP0);
  return fmaf(u, r, h);
}

// LeakyReLU -> + s -> clamp -> GELU.  SERIES: the clamp bounds lie in [-1, 1],
// so the polynomial above applies; otherwise the device library's erff.
// LeakyReLU is one median: med3(v, slope v, +inf) = max(v, slope v) when
// slope <= 1 and med3(v, slope v, -inf) = min(v, slope v) when slope > 1;
// either is v for v >= 0 and slope v for v < 0 (exactly, as |slope v| and |v|
// compare the same way after rounding).  The clamp is a median too (lo <= hi).
template <bool SERIES>
__device__ __forceinline__ float lrelu_add_clamp_gelu_value(float v, float s, float slope, float lo, float hi) {
  const float t = __builtin_amdgcn_fmed3f(v, slope * v, slope <= 1.0f ? INFINITY : -INFINITY);
  const float c = __builtin_amdgcn_fmed3f(t + s, lo, hi);
  if (SERIES) return gelu_small(c);
  return 0.5f * c * (1.0f + erff(c * 0.70710678118654752f));
}

// The same chain on halved values: h = v / 2, s_half = s / 2, lo_half and
// hi_half the halved bounds (a kernel whose weights and bias are staged at
// half scale produces h directly).  Halving commutes with every rounding in
// the chain, and GELU(c) = 0.5 c (1 + erf(c / sqrt 2)) becomes
// c' (1 + erf(c' sqrt 2)) with c' = c / 2 (fp32 sqrt 2 is exactly twice fp32
// 1 / sqrt 2), so the result equals lrelu_add_clamp_gelu_value(v, ...) bit
// for bit (unless some intermediate is subnormal, where halving can drop its
// last bit), with one multiplication fewer.
template <bool SERIES>
__device__ __forceinline__ float lrelu_add_clamp_gelu_half(float h, float s_half, float slope, float lo_half,
                                                           float hi_half) {
  const float t = __builtin_amdgcn_fmed3f(h, slope * h, slope <= 1.0f ? INFINITY : -INFINITY);
  const float c = __builtin_amdgcn_fmed3f(t + s_half, lo_half, hi_half);
  if (SERIES) return gelu_small_half(c);
  return c * (1.0f + erff(c * 1.41421356237309515f));
}

// Division of a non-negative 31-bit integer by a divisor fixed per launch,
// by multiplication (Granlund & Montgomery, "Division by invariant integers
// using multiplication", 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l for
// 0 <= n < 2^31 (the sum cannot overflow because mulhi(n, m) <= n).
struct FastDiv {
  uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, l};
}

__device__ __forceinline__ int fdiv(int n, const FastDiv &f) {
  const uint32_t t = __umulhi((uint32_t)n, f.m);
  return (int)((t + (uint32_t)n) >> f.l);
}

// 16-byte global store of four consecutive floats (address 16-byte aligned).
__device__ __forceinline__ void store4(float *p, v4f v) {
  *reinterpret_cast<v4f *>(p) = v;
}

// Stages a tile made of equal-length rows (each `len` floats, contiguous in
// global memory and in LDS) with a fixed thread -> column assignment, so that
// a whole tile's global loads can be issued into registers one tile ahead of
// use and written to LDS later.  VEC moves 16-byte quads (row lengths,
// sources and destinations four-float aligned), otherwise single floats.
// Rows beyond KPRE passes, and columns beyond one pass, fall back to
// synchronous copies in store().
template <int KPRE, bool VEC, int THREADS>
struct RowStage {
  v4f v[KPRE];
  int cw, tpr, rpp, my_row, my_col;

  __device__ __forceinline__ void init(int len, int tid) {
    cw = VEC ? (len >> 2) : len;
    tpr = cw < THREADS ? cw : THREADS;
    rpp = THREADS / tpr;
    my_row = tid / tpr;
    my_col = tid - my_row * tpr;
  }

  // src(row) -> const float* of the row's first element.
  template <class Src>
  __device__ __forceinline__ void load(int rows, Src src) {
#pragma unroll
    for (int k = 0; k < KPRE; ++k) {
      const int row = my_row + k * rpp;
      if (my_row < rpp && row < rows) {
        const float *p = src(row);
        if (VEC)
          v[k] = *reinterpret_cast<const v4f *>(p + 4 * my_col);
        else
          v[k].x = p[my_col];
      }
    }
  }

  // dst(row) -> float* of the row's first element in LDS.
  template <class Src, class Dst>
  __device__ __forceinline__ void store(int rows, Src src, Dst dst) {
#pragma unroll
    for (int k = 0; k < KPRE; ++k) {
      const int row = my_row + k * rpp;
      if (my_row < rpp && row < rows) {
        float *d = dst(row);
        if (VEC)
          *reinterpret_cast<v4f *>(d + 4 * my_col) = v[k];
        else
          d[my_col] = v[k].x;
      }
    }
    if (my_row >= rpp) return;
    for (int row = my_row, k = 0; row < rows; row += rpp, ++k) {
      const float *p = src(row);
      float *d = dst(row);
      for (int c = (k < KPRE ? my_col + tpr : my_col); c < cw; c += tpr) {
        if (VEC)
          *reinterpret_cast<v4f *>(d + 4 * c) = *reinterpret_cast<const v4f *>(p + 4 * c);
        else
          d[c] = p[c];
      }
    }
  }
};

}  // namespace cce
