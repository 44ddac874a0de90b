/*
 * swin3d_wattn.h - Swin3D shifted-window attention for AMD Instinct MI355X (gfx950).
 *
 * The operation (Flash-Aurora README, "Kernel fusion for backbone memory
 * traffic" and "CuTe DSL window attention"; the walkthrough slides,
 * "3 · Efficient inference"):
 *
 *   Q, K, V, O are grid-layout tensors [B, D, H, W, heads, head_dim],
 *   contiguous and row-major, all of one dtype. With window w = (wd, wh, ww),
 *   shift s and padded extents P_a = ceil(X_a / w_a) * w_a for X = (D, H, W):
 *     1. pad D, H, W at the high end to P (padding is never read or written);
 *     2. cyclic shift: shifted position p holds grid position (p + s) mod P;
 *     3. partition the shifted grid into windows of N = wd*wh*ww tokens
 *        (window (2, 6, 12) gives N = 144);
 *     4. per window and head: S = scale * Q K^T; add cross_region_bias to S
 *        where query and key lie in different shift regions (the Swin
 *        shifted-window mask; the pages' value is -100, added as in PyTorch's
 *        scaled_dot_product_attention); S = -inf for padding keys; row
 *        softmax in FP32; O = softmax(S) V, accumulated in FP32;
 *     5. merge the windows back, undo the shift, crop the padding.
 *   Shift regions: along an axis with s_a > 0 the shifted grid is cut into
 *   [0, P-w), [P-w, P-s), [P-s, P); a token's region is its triple of cuts.
 *   A shift is applied as given, also where an axis holds a single window.
 *
 *   The kernels do all five steps in one pass: each workgroup gathers its
 *   window straight from grid layout and scatters O back to grid layout;
 *   no windowed copy and no N x N matrix ever reaches device memory.
 *
 * Precision: bf16 I/O uses bf16 matrix-core products for Q K^T and P V with
 * FP32 accumulation and an FP32 softmax; P is rounded to bf16 (nearest-even)
 * before P V and O is rounded to bf16 (nearest-even) at the end. f32 I/O
 * computes everything in FP32 (FP32 matrix-core products, FP32 softmax);
 * f32 I/O with F32_SPLIT runs the products as three bf16 matrix-core
 * products each. The kernels load a real stand-in token for each padding
 * slot of a window (so every load is unconditional) and replace its K and V
 * rows by zeros before use, so padding adds exactly nothing: an Inf or NaN in
 * a real token affects only the outputs of its own window, as in a
 * materialised pad-shift-partition pipeline. On grids that need padding the
 * K/V-streaming kernel skips the query blocks and key chunks that hold
 * padding only (their outputs are cropped, their weights exactly zero).
 *
 * Ownership: the caller owns every device buffer. The library allocates no
 * device memory; a plan is a small immutable host object.
 *
 * Threading: swin3d_wattn_run is asynchronous on the caller's stream and
 * never synchronizes. One plan may be used from several host threads and
 * streams at once.
 *
 * Errors: every entry point returns 0 on success or a negative code below;
 * faults inside a kernel surface at the caller's next synchronization.
 */
#ifndef SWIN3D_WATTN_H
#define SWIN3D_WATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWIN3D_WATTN_OK 0
#define SWIN3D_WATTN_EINVAL (-1)      /* null pointer, a size <= 0, shift out of range,
                                         non-finite scale, misaligned or overlapping buffers */
#define SWIN3D_WATTN_EUNSUPPORTED (-2) /* valid, but no kernel for this head_dim / window / dtype */
#define SWIN3D_WATTN_ELAUNCH (-3)     /* the HIP runtime refused the launch */

typedef enum {
  SWIN3D_WATTN_F32 = 0,       /* float32 I/O, float32 arithmetic */
  SWIN3D_WATTN_BF16 = 1,      /* bfloat16 I/O, bf16 products, float32 softmax and accumulation */
  SWIN3D_WATTN_F32_SPLIT = 2  /* float32 I/O; Q K^T and P V on the matrix cores from bf16
                                 hi/lo splits of every operand (three products: hi*hi,
                                 lo*hi, hi*lo), float32 softmax and accumulation. The
                                 FP32-fidelity mode at matrix-core speed, in the role of the
                                 pages' TF32_ACC_FP32 mode (README, "Window attention
                                 kernels"); products keep ~16 significant bits */
} swin3d_wattn_dtype_t;

/* Problem description, copied into the plan by swin3d_wattn_create. */
typedef struct {
  int32_t B, D, H, W;      /* batch and grid extents of Q/K/V/O */
  int32_t heads, head_dim; /* innermost two dimensions */
  int32_t window[3];       /* (wd, wh, ww), each >= 1; (2, 6, 12) in the pages */
  int32_t shift[3];        /* 0 <= shift[a] < window[a]; (1, 3, 6) for shifted blocks */
  int32_t dtype;           /* swin3d_wattn_dtype_t */
  float scale;             /* > 0 and finite; normally 1/sqrt(head_dim) */
  float cross_region_bias; /* added to S across shift regions: -100 (pages) or -INFINITY
                              (exclusion); must be <= 0 and not NaN */
} swin3d_wattn_desc_t;

typedef struct swin3d_wattn_plan* swin3d_wattn_t;

/* Validate *desc and build a plan for the operation above: the window,
 * shift and cross-region bias fields are the parameters of the shifted-window
 * mask (Flash-Aurora README, "CuTe DSL window attention"), the dtype selects
 * a precision mode ("Window attention kernels", "Mixed-precision inference").
 * Host-only: no device is touched.
 * Supported: dtype BF16 with head_dim 32, 64 or 128, any window with
 * wd*wh*ww <= 4096 and heads < 65536 (N = 144 at head_dim 64 runs the
 * single-tile kernel, N x head_dim = 144 x 128 and 288 x 64 a whole-window
 * kernel that holds K and V of the window in LDS at two workgroups per CU;
 * every other case streams K and V through LDS in 48- or 64-key chunks, the
 * pages' multi-stage fallback); dtype F32_SPLIT with
 * head_dim 64, wd*wh*ww = 144 and heads < 65536; dtype F32 with head_dim 32
 * or 64, wd*wh*ww <= 256 and heads < 65536 (FP32 matrix cores). B*D*H*W must be < 2^31 and each
 * of D, H, W < 2^24. A launch counts the work-items of its first grid
 * dimension in 32 bits, so the windows (times the query blocks per window of
 * the streaming kernel) times threads_per_workgroup must be < 2^32; only
 * windows of a few tokens on very large grids reach that (e.g. window
 * (1, 1, 1) on 4096 x 4097 tokens), and get EUNSUPPORTED.
 * Returns 0 and stores the plan in *out, or EINVAL / EUNSUPPORTED
 * (then *out is set to NULL when out is not NULL). */
int swin3d_wattn_create(const swin3d_wattn_desc_t* desc, swin3d_wattn_t* out);

/* O = window_attention(Q, K, V) on `stream` (a hipStream_t; NULL is the
 * default stream) for the device current on the calling thread: all five
 * steps of the operation above in one pass, gathering each window straight
 * from grid layout and scattering O back (Flash-Aurora README, "Kernel fusion
 * for backbone memory traffic" and "CuTe DSL window attention").
 * q, k, v, o: device pointers to B*D*H*W*heads*head_dim elements of the
 * plan's dtype, 16-byte aligned; o must not overlap q, k or v (q, k, v may
 * alias each other). Every element of o is written exactly once.
 * Returns 0, EINVAL (null plan or pointer, misalignment, overlap) or ELAUNCH. */
int swin3d_wattn_run(swin3d_wattn_t plan, const void* q, const void* k, const void* v, void* o,
                     void* stream);

/* Token strides, in elements, of the four tensors for
 * swin3d_wattn_run_strided: element (token t, head h, dim d) of Q sits at
 * q[t * q + h * head_dim + d], and likewise for K, V and O, where token t
 * runs over B*D*H*W in row-major [B, D, H, W] order. Within a token the
 * heads * head_dim elements stay contiguous.
 *
 * This lets the path read Q, K and V straight out of a fused projection
 * output [B, D, H, W, 3, heads, head_dim] (q = base, k = base + heads*head_dim,
 * v = base + 2*heads*head_dim, all three strides 3*heads*head_dim) and write O
 * into a wider buffer, so no copy is needed on either side of the attention
 * (the layout-copy removal of the Flash-Aurora README, "Kernel fusion for
 * backbone memory traffic"). Contiguous grid-layout tensors have stride
 * heads*head_dim. */
typedef struct {
  int64_t q, k, v, o;
} swin3d_wattn_strides_t;

/* swin3d_wattn_run with explicit token strides (see swin3d_wattn_strides_t).
 * Each stride must be >= heads*head_dim, below 2^31 elements and a multiple
 * of 16 bytes, and each span (below) at most 2^46 elements; the pointers
 * 16-byte aligned. The span of a tensor is the byte range
 * [ptr, ptr + ((tokens - 1) * stride + heads*head_dim) * element size); the
 * span of O must not overlap the spans of Q, K or V, while Q, K and V may
 * overlap each other. Elements of
 * the O buffer outside the (token, head, dim) positions are never touched.
 * Returns 0, EINVAL (null plan, pointer or strides, a stride too small, too
 * large or misaligned, misalignment, overlap) or ELAUNCH. */
int swin3d_wattn_run_strided(swin3d_wattn_t plan, const void* q, const void* k, const void* v, void* o,
                             const swin3d_wattn_strides_t* strides, void* stream);

/* ---- Fused AdaLN + residual ------------------------------------------------
 * The step the pages fuse around each Swin3D attention block (Flash-Aurora
 * README, "Kernel fusion for backbone memory traffic": LayerNorm, FiLM
 * modulation and the residual add without a full-width intermediate, with
 * FP32 activations between blocks when wanted). For row t of batch element b,
 * with C channels per row, in FP32:
 *   xhat = (x - mean) / sqrt(var + eps)      mean, biased variance over C
 *   out  = res + gamma[b] * xhat + beta[b]
 */
typedef struct {
  int64_t rows;      /* rows (tokens) per batch element */
  int32_t B;         /* batch elements; gamma and beta hold one row of C per element */
  int32_t C;         /* channels per row: a multiple of 256, at most 4096 */
  int32_t x_dtype;   /* SWIN3D_WATTN_F32 or SWIN3D_WATTN_BF16 */
  int32_t res_dtype; /* likewise */
  int32_t out_dtype; /* likewise; F32 keeps the residual stream in FP32 between blocks */
  float eps;         /* > 0 and finite */
} swin3d_adaln_desc_t;

/* out = res + gamma * LayerNorm(x) + beta on `stream` (a hipStream_t).
 * x, res, out: device pointers to B*rows*C elements ([B, rows, C] row-major)
 * of their dtypes; gamma, beta: device pointers to B*C floats ([B, C]); all
 * 16-byte aligned. out may be res itself when both have the same dtype (the
 * residual stream updated in place) but must not otherwise overlap x, res,
 * gamma or beta. B*rows must be < 2^31. Asynchronous; the caller owns every
 * buffer. Returns 0, EINVAL (null, misaligned, unknown dtype, a size <= 0,
 * eps not positive and finite, overlap), EUNSUPPORTED (C not a multiple of
 * 256 or above 4096, B*rows too large) or ELAUNCH. */
int swin3d_adaln_residual(const swin3d_adaln_desc_t* desc, const void* x, const void* res,
                          const float* gamma, const float* beta, void* out, void* stream);

/* Release a plan made by swin3d_wattn_create (a host object only: the pages'
 * kernels hold no state between calls, and neither does a plan on the
 * device). NULL is a no-op. Returns 0. */
int swin3d_wattn_destroy(swin3d_wattn_t plan);

/* Static English text for a return code. */
const char* swin3d_wattn_strerror(int code);

/* Geometry of a plan, for callers that size work or report throughput. */
typedef struct {
  int32_t padded[3];        /* P = (PD, PH, PW) */
  int32_t windows_per_axis[3];
  int64_t n_windows;        /* B * prod(windows_per_axis): the folded batch of the pages */
  int64_t n_masked_windows; /* windows that hold more than one shift region or padding */
  int32_t tokens_per_window;/* N */
  int64_t tokens;           /* B*D*H*W real tokens */
  int64_t workgroups;       /* workgroups one run launches */
  int32_t threads_per_workgroup;
  int32_t kernel;           /* 1 = bf16 matrix-core kernel (N = 144, head_dim 64),
                               2 = f32 split-bf16 matrix-core kernel, 3 = bf16 matrix-core
                               kernel with K/V streamed through LDS, 4 = f32 matrix-core
                               kernel, 5 = bf16 matrix-core kernel with the whole window's
                               K/V in LDS (N x head_dim = 144 x 128 or 288 x 64) */
} swin3d_wattn_info_t;

/* Fill *info for a plan. Host-only. Returns 0 or EINVAL. */
int swin3d_wattn_get_info(swin3d_wattn_t plan, swin3d_wattn_info_t* info);

#ifdef __cplusplus
}
#endif

#endif /* SWIN3D_WATTN_H */
