/*
 * cce.h -- C ABI of the fused small-channel convolution + epilogue library
 * (libcce.so, HIP kernels for AMD MI355X / gfx950).
 *
 * Three fused operators whose kernels read the input and weights from
 * device memory and write only the final output (the convolution result
 * never reaches device memory):
 *
 *   conv2d_relu_hswish            Conv2d k x k (stride 1, padding 0) -> ReLU -> HardSwish
 *   conv3d_lrelu_add_clamp_gelu   Conv3d k^3 (stride 1, padding 0) -> LeakyReLU -> + s[c]
 *                                 -> clamp -> exact GELU
 *   convT2d_pool_htanh_mean_tanh  ConvTranspose2d -> MaxPool2d -> Hardtanh -> mean over
 *                                 (H, W) -> tanh
 *
 * and two epilogue-only operators over a convolution output computed
 * elsewhere (the unfused paths the pages fall back to):
 *
 *   pool_htanh_mean_tanh          MaxPool2d -> Hardtanh -> mean over (H, W) -> tanh
 *   lrelu_add_clamp_gelu          LeakyReLU -> + s[c] -> clamp -> exact GELU
 *
 * The operators are the three models of the POPCORNBENCH Kimi-K2.6 level-2
 * transcripts l2_p57, l2_p90 and l2_p10 (each entry point names its page).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers to contiguous fp32 data, in the
 *    layouts stated per function (NCHW / NCDHW activations).  The caller owns
 *    every buffer; the library never allocates, frees or synchronises.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously on it; the call returns before the
 *    kernel runs.
 *  - Arguments are validated on the host before any HIP call.  An invalid or
 *    unsupported call returns a negative cce_status and launches nothing.  A
 *    failed launch returns CCE_ERR_LAUNCH.  Faults inside a running kernel
 *    surface, as usual for HIP, at the caller's next synchronisation.
 *  - Calls on different streams may run concurrently, except that one
 *    convT2d workspace must not be used by two calls at the same time.
 *  - Arithmetic is fp32 (products accumulated in fp32 by the matrix cores).
 *    Results match a double-precision evaluation of the definitions within
 *    |gpu - ref| <= 1e-4 + 1e-4 * |ref| per element.
 */
#ifndef CCE_H
#define CCE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CCE_OK = 0,
  CCE_ERR_NULL = -1,        /* a required pointer is NULL */
  CCE_ERR_SHAPE = -2,       /* a size is non-positive, or the output would be empty */
  CCE_ERR_UNSUPPORTED = -3, /* valid shape outside the set the kernels are built for */
  CCE_ERR_ALIGN = -4,       /* a tensor pointer is not 4-byte aligned */
  CCE_ERR_WORKSPACE = -5,   /* workspace NULL, misaligned or smaller than required */
  CCE_ERR_LAUNCH = -6,      /* the HIP runtime rejected the launch (no device, wrong arch ...) */
  CCE_ERR_TOO_LARGE = -7,   /* an index would overflow the kernels' 32-bit arithmetic */
  CCE_ERR_SCRATCH_LIMIT = -8 /* the call needs more than the static scratch of the _noalloc entry */
} cce_status;

/* Human-readable text for a cce_status value (static storage, never NULL). */
const char *cce_status_string(int status);

/* Library ABI version: 100 * major + minor (1.1: further layer shapes for
 * Conv2d and Conv3d, any pooling window and stride for the pooled tail;
 * 1.2: further channel counts for the fused ConvTranspose2d; 1.3: 1 x 1 x 1
 * Conv3d; 1.4: convT2d_pool_htanh_mean_tanh_noalloc, and the transposed
 * conv's workspace needs no initial contents).
 *
 * Debugging: with the environment variable CCE_DEBUG set (to anything but
 * "" or "0") when the library is first used, every launch is followed by a
 * synchronisation of its stream; a kernel that faults is then reported on
 * stderr by the call that launched it, which returns CCE_ERR_LAUNCH.  Calls
 * become blocking, and must not be captured into HIP graphs, in that mode. */
int cce_version(void);

/*
 * y = HardSwish(ReLU(conv2d(x, w) + b))           -- page l2_p57
 *
 *   x  [N][C_in][H][W]                      input
 *   w  [C_out][C_in][k][k]                  conv weight (torch Conv2d layout)
 *   b  [C_out] or NULL (NULL = zero bias)   conv bias
 *   y  [N][C_out][H-k+1][W-k+1]             output
 *
 * z[n,o,h,w] = b[o] + sum_{i,kh,kw} x[n,i,h+kh,w+kw] * w[o,i,kh,kw]  (stride 1,
 * padding 0, the defaults the page's problem uses), r = max(z, 0),
 * y = r * clamp((r + 3) / 6, 0, 1).
 *
 * Supported layers: the page's C_in = 8, C_out = 64, k = 3, and C_in in
 * {4, 8, 16}, C_out in {16, 32, 64}, k in {1, 3, 5} (k = 5 only for
 * C_in <= 8); any N >= 1 and H, W >= k.  Loads are 16-byte when W % 4 == 0
 * and x is 16-byte aligned, stores when (H-k+1)*(W-k+1) % 4 == 0 and y is
 * 16-byte aligned; otherwise 4-byte (same results).  Other layers return
 * CCE_ERR_UNSUPPORTED.  One input image (C_in*H*W floats), one output image
 * and the output pixel count N*(H-k+1)*(W-k+1) must stay below 2^31, else
 * CCE_ERR_TOO_LARGE.
 */
int conv2d_relu_hswish(const float *x, const float *w, const float *b, float *y, int N, int C_in,
                       int H, int W, int C_out, int k, void *stream);

/*
 * y = GELU(clamp(LeakyReLU(conv3d(x, w) + b, slope) + s[o], lo, hi))   -- page l2_p90
 *
 *   x  [N][C_in][D][H][W]                   input
 *   w  [C_out][C_in][k][k][k]               conv weight (torch Conv3d layout)
 *   b  [C_out] or NULL (NULL = zero bias)   conv bias
 *   s  [C_out] (the [C_out,1,1,1] sum_tensor), required
 *   y  [N][C_out][D-k+1][H-k+1][W-k+1]      output
 *
 * LeakyReLU(t) = t for t >= 0, slope * t otherwise; clamp to [lo, hi];
 * GELU(t) = 0.5 t (1 + erf(t / sqrt 2)) (exact, not the tanh form).
 *
 * Supported: k = 3 or 1; C_in in {4, 8, 16}, C_out in {16, 32, 64} (the
 * page's 3 x 3 x 3, 8 -> 64 included); 16-byte loads and stores where sizes
 * and alignment allow; a fitted polynomial for GELU when [lo, hi] lies in
 * [-1, 1], erff otherwise; any N >= 1, D, H, W >= k (rows too wide for LDS are split into
 * column tiles; a 3 x 3 x 3, 16 -> 64 layer with rows wider than 34 floats runs
 * as two launches, each writing 32 of the output channels); lo <= hi and all
 * three scalars finite;
 * N*C_out*(D-k+1)*(H-k+1)*(W-k+1) < 2^31.  Anything else returns
 * CCE_ERR_UNSUPPORTED (or CCE_ERR_SHAPE / CCE_ERR_TOO_LARGE).
 */
int conv3d_lrelu_add_clamp_gelu(const float *x, const float *w, const float *b, const float *s,
                                float *y, int N, int C_in, int D, int H, int W, int C_out, int k,
                                float negative_slope, float clamp_lo, float clamp_hi, void *stream);

/*
 * y[n,o] = tanh(mean_{ph,pw} Hardtanh(MaxPool2d(convT2d(x, w) + b)))   -- page l2_p10
 *
 *   x  [N][C_in][H][W]                      input
 *   w  [C_in][C_out][k][k]                  transposed-conv weight (torch layout)
 *   b  [C_out] or NULL (NULL = zero bias)
 *   y  [N][C_out] (the [N,C_out,1,1] result)
 *
 * The transposed conv (stride s, padding p, output padding 0) has output
 * size Ho = (H-1)*s - 2p + k; at stride 1, padding 1 it equals a correlation
 * with the kernel flipped in both spatial axes and its channel axes swapped.
 * MaxPool2d(pool_k, pool_s) has output floor((Ho - pool_k) / pool_s) + 1 per
 * axis; Hardtanh clamps to [htanh_lo, htanh_hi]; the mean divides by the
 * pooled element count.
 *
 * Workspace: device memory of at least
 * convT2d_pool_htanh_mean_tanh_workspace_bytes(...) bytes, 256-byte
 * aligned, with any contents: the call first writes everything it later
 * reads there (per-image completion counters, the prepared weight, per-tile
 * partial sums), on `stream`, so one workspace may serve calls of any shapes
 * one after another.  One workspace serves one call at a time: calls that
 * overlap in time (on different streams) need one workspace each.
 *
 * Supported: k = 3, stride = 1, pad = 1, pool_k = pool_s = 2; C_in a
 * multiple of 8 in [8, 512] and C_out in {16, 32, 64} (the page's layer is
 * 64 -> 64); H, W >= 2, htanh_lo <= htanh_hi (finite), N >= 1,
 * N*C_in*H*W < 2^31.  Anything else returns CCE_ERR_UNSUPPORTED (or
 * CCE_ERR_SHAPE / CCE_ERR_TOO_LARGE).  The result is deterministic: partial
 * sums are combined in a fixed order.
 */
int convT2d_pool_htanh_mean_tanh(const float *x, const float *w, const float *b, float *y, int N,
                                 int C_in, int H, int W, int C_out, int k, int stride, int pad,
                                 int pool_k, int pool_s, float htanh_lo, float htanh_hi,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace the call above needs for these sizes (0 if the sizes
 * are invalid or unsupported). */
size_t convT2d_pool_htanh_mean_tanh_workspace_bytes(int N, int C_in, int H, int W, int C_out,
                                                    int k, int stride, int pad, int pool_k,
                                                    int pool_s);

/* Size of the static per-device scratch behind the _noalloc entry point. */
#define CCE_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * convT2d_pool_htanh_mean_tanh without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * results, bit for bit, and errors as convT2d_pool_htanh_mean_tanh, whose
 * kernels it runs.
 *
 * In place of the workspace it uses a file-scope device array of
 * CCE_NOALLOC_SCRATCH_BYTES (8 MiB) that each GPU the library runs on holds
 * from its first call until the process ends; the first call on a device
 * looks up that device's copy (hipGetSymbolAddress) and caches its address.
 * The call allocates and frees nothing and issues no memset.  A call whose
 * workspace_bytes(...) would exceed the scratch returns
 * CCE_ERR_SCRATCH_LIMIT and launches nothing (the page's layer, 64 -> 64 at
 * 256 x 256, fits up to N = 251).  All calls on one GPU share its scratch:
 * calls that overlap in time on that GPU (on different streams or threads)
 * race and give wrong results; calls on one stream, or otherwise ordered,
 * are safe.
 */
int convT2d_pool_htanh_mean_tanh_noalloc(const float *x, const float *w, const float *b, float *y,
                                         int N, int C_in, int H, int W, int C_out, int k, int stride,
                                         int pad, int pool_k, int pool_s, float htanh_lo,
                                         float htanh_hi, void *stream);

/*
 * Epilogue-only operators over a precomputed convolution output (the
 * unfused paths the pages fall back to; the fused operators above do not
 * need them).
 */

/*
 * y[n,c] = tanh(mean_{ph,pw} Hardtanh(MaxPool2d(z[n,c], pool_k, pool_s)))  -- page l2_p10's
 * fused tail over a library transposed-conv output
 *
 *   z  [N][C][H][W]   e.g. the transposed-conv output
 *   y  [N][C]         (the [N,C,1,1] result)
 *
 * Pooled size floor((H - pool_k) / pool_s) + 1 per axis (windows may overlap
 * when pool_s < pool_k, or skip elements when pool_s > pool_k); the mean
 * divides by the pooled element count.  Deterministic (fixed summation order).
 * Supported: any pool_k, pool_s >= 1 with H, W >= pool_k (else
 * CCE_ERR_SHAPE), htanh_lo <= htanh_hi (finite), N*C < 2^31 and H*W < 2^31.
 * pool_k = pool_s = 2 takes the streaming fast path.
 */
int pool_htanh_mean_tanh(const float *z, float *y, int N, int C, int H, int W, int pool_k,
                         int pool_s, float htanh_lo, float htanh_hi, void *stream);

/*
 * y = GELU(clamp(LeakyReLU(z, slope) + s[c], lo, hi)) elementwise  -- page l2_p90's
 * fallback after a library Conv3d
 *
 *   z, y  [N][C][S]   S = spatial elements per channel (e.g. D*H*W); y may equal z
 *   s     [C]         per-channel offset (the [C,1,1,1] sum_tensor)
 *
 * Supported: N, C, S >= 1, lo <= hi, all three scalars finite, N*C < 2^31.
 */
int lrelu_add_clamp_gelu(const float *z, const float *s, float *y, int N, int C, long long S,
                         float negative_slope, float clamp_lo, float clamp_hi, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CCE_H */
