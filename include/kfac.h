/*
 * kfac.h -- C ABI of the per-GPU K-FAC hot path for AMD Instinct MI355X
 * (gfx950).  One K-FAC step on one GPU is
 *
 *     kfac_factors      A and G Kronecker factors with their running average
 *     kfac_pack_sym     upper triangles of the factors <-> one fused buffer
 *     kfac_damped_inverse  (X + gamma I)^-1 of every factor, batched
 *     kfac_precondition (G + gamma I)^-1 . gradW . (A + gamma I)^-1 per layer
 *
 * and, to feed real layers, kfac_im2col / kfac_grad_rows (factor inputs from
 * a layer's input and output gradient) and kfac_grad_matrix (a layer's
 * weight and bias gradients as one matrix and back),
 * following "Accelerating Distributed K-FAC with Smart Parallelism of
 * Computing and Communication Tasks" (cited per entry point below).
 *
 * Common rules
 *   - Matrices are row-major.  "Upper" means the entries (i, j) with j >= i.
 *   - Arrays of per-layer pointers (x, m, xinv, grad, ...) and the size
 *     arrays (rows, d, ...) are HOST arrays, read during the call only.  The
 *     pointers they hold are DEVICE pointers, at least 4-byte aligned.
 *   - `workspace` is a device buffer of at least the size returned by the
 *     matching *_workspace_size() call, 256-byte aligned, owned by the
 *     caller, and must stay untouched until the enqueued work has finished.
 *     The library allocates no device memory and keeps no state between
 *     calls; calls on different streams with different workspaces may run
 *     concurrently.
 *   - Every call validates its arguments on the host first.  On an error it
 *     returns a non-zero status and enqueues nothing.  On success the work is
 *     enqueued on `stream` (0 = the null stream) and the call returns
 *     without waiting for it.
 *   - Inputs containing NaN or Inf are not screened; they propagate
 *     (the inverse reports them through `info`).
 */
#ifndef KFAC_H
#define KFAC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KFAC_OK = 0,
    KFAC_ERR_INVALID_VALUE = 1, /* bad count, size, pointer, alignment, gamma or eps */
    KFAC_ERR_WORKSPACE = 2,     /* workspace missing, misaligned or too small */
    KFAC_ERR_UNSUPPORTED = 3,   /* valid request this build cannot serve */
    KFAC_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} kfac_status_t;

typedef enum { KFAC_F32 = 0, KFAC_BF16 = 1 } kfac_dtype_t;
typedef enum { KFAC_PACK = 0, KFAC_UNPACK = 1 } kfac_pack_dir_t;

/* Largest factor dimension and largest number of layers / matrices per call. */
#define KFAC_MAX_DIM 16384
#define KFAC_MAX_COUNT 4096

/* ABI version of this header (bumped on any incompatible change). */
int kfac_abi_version(void);

/* Static, human-readable name of a status code. */
const char* kfac_status_string(kfac_status_t status);

/* ---------------------------------------------------------------- factors --
 * Kronecker factors with running average.  The page builds, per layer l, the
 * factor A from the layer's input a and the factor G from the gradient with
 * respect to the layer's output g, both symmetric (paragraph introducing the
 * Kronecker factors; the pipelining paragraph computes them in the forward
 * pre-hook and the backward hook, "Eq. (7)" and "Eq. (8)").  For each of the
 * n matrices:
 *
 *     F_i = (1 / rows_i) * X_i^T X_i
 *     M_i <- F_i                                 if first_step != 0
 *     M_i <- eps * M_i + (1 - eps) * F_i         otherwise
 *
 * x[i]   : [rows[i], d[i]] row-major, float32 (in_dtype KFAC_F32) or bfloat16
 *          (KFAC_BF16, accumulated in float32).  float32 products are formed
 *          on the bf16 matrix cores as six bf16 products of exact three-way
 *          splits of each value and carry float32 rounding.  A layer with a bias carries
 *          a trailing column of ones.
 * m[i]   : [d[i], d[i]] float32.  Only the upper triangle is read (when
 *          first_step == 0) and written; the strict lower triangle is left
 *          as it was.
 * eps    : in [0, 1].  1 <= rows[i] <= 2^31 - 1, 1 <= d[i] <= KFAC_MAX_DIM.
 * The x[i] must not overlap any m[j].  Results are deterministic: the same
 * inputs give the same bits on every run.
 */
size_t kfac_factors_workspace_size(int n, const int64_t* rows, const int64_t* d, kfac_dtype_t in_dtype);
kfac_status_t kfac_factors(int n, const void* const* x, const int64_t* rows, const int64_t* d,
                           kfac_dtype_t in_dtype, float* const* m, float eps, int first_step,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------- pack --
 * Tensor fusion of the symmetric factors: only the upper triangle including
 * the diagonal is kept, d(d+1)/2 elements per factor (tensor-fusion
 * paragraph on communicated elements; paragraph on sending only the upper
 * triangles), and consecutive factors are merged into one contiguous buffer
 * (paragraph on dynamic tensor fusion).
 *
 *     packed[off_l + i*d_l - i*(i-1)/2 + (j - i)] = M_l[i][j],  0 <= i <= j < d_l
 *     off_l = sum_{k<l} d_k (d_k + 1) / 2
 *
 * KFAC_PACK reads the upper triangles of m[l] and writes `packed`
 * (kfac_packed_size() float32 elements).  KFAC_UNPACK reads `packed` and
 * writes every element of m[l]: entry (i, j) and its mirror (j, i).  Values
 * are copied bit for bit.  The m[l] must not overlap each other or `packed`.
 * The host passes only the pointers and orders; the offsets off_l are
 * formed on the device, as a prefix sum across a wavefront.  The workspace
 * (kfac_pack_workspace_size() bytes) holds that layer table.
 */
int64_t kfac_packed_size(int n, const int64_t* d);
size_t kfac_pack_workspace_size(int n, const int64_t* d);
kfac_status_t kfac_pack_sym(int n, float* const* m, const int64_t* d, float* packed, kfac_pack_dir_t dir,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* kfac_pack_sym without a workspace, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, results and errors as kfac_pack_sym;
 * the layer table lives in a device array of the library instead (64 KiB per
 * GPU, held until the process ends).  It allocates nothing: no hipMalloc, no
 * hipFree, no allocating library call.  At most KFAC_STATIC_MAX_FACTORS
 * factors per call, else KFAC_ERR_UNSUPPORTED (nothing enqueued).  Every call
 * on one GPU shares that array, and the last call's table stays in it: calls
 * that may overlap on one GPU (different streams, or different host threads
 * without ordering) race and must not be made.
 */
#define KFAC_STATIC_MAX_FACTORS 1024
kfac_status_t kfac_pack_sym_static(int n, float* const* m, const int64_t* d, float* packed, kfac_pack_dir_t dir,
                                   hipStream_t stream);

/* Plain device-to-device copy of `bytes` bytes (16-byte loads and stores,
 * one per lane).  It computes nothing of the method: it is the measured
 * streaming rate that the HBM-bound figures of pack and unpack are set
 * against, beside the published peak.  src and dst are device pointers,
 * 16-byte aligned, not overlapping; bytes is a multiple of 16 (0 is a no-op),
 * else KFAC_ERR_INVALID_VALUE.
 */
kfac_status_t kfac_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Matrix-core rate reference.  `blocks` workgroups of four waves each run
 * `iters` rounds of four independent matrix-core products on register
 * operands, with no memory traffic besides one float per wave written to
 * `sink` (device, 4 * blocks floats, 4-byte aligned), which keeps the products
 * from being removed.  The products are v_mfma_f32_32x32x16_bf16
 * (KFAC_RATE_BF16, 32768 flops each), v_mfma_f64_16x16x4f64 (KFAC_RATE_F64,
 * 2048) or v_mfma_f32_32x32x2f32 (KFAC_RATE_F32, 4096).  It computes nothing
 * of the method: timed by the caller, it is the rate the matrix cores
 * sustain on this part under its own clock and power limits, the measured
 * reference for the matrix-core-bound stages beside the published peaks.
 * *flops (host, may be NULL) receives the flops of the call.
 * KFAC_ERR_INVALID_VALUE for an unknown kind, iters outside [1, 2^24],
 * blocks outside [1, 65536] or a null sink.
 */
typedef enum { KFAC_RATE_BF16 = 0, KFAC_RATE_F64 = 1, KFAC_RATE_F32 = 2 } kfac_rate_kind_t;
kfac_status_t kfac_matrix_rate(kfac_rate_kind_t kind, int64_t iters, int blocks, float* sink, double* flops,
                               hipStream_t stream);

/* ---------------------------------------------------------------- inverse --
 * Tikhonov-damped inverse of each factor (paragraph on damping before
 * inverting; the inverses of different layers are independent, paragraph on
 * MPD-KFAC; the inverse goes through a Cholesky decomposition, paragraph on
 * the inverse performance model).  For each of the n matrices:
 *
 *     Y_i = X_i + gamma I   (X_i read from the upper triangle of x[i])
 *     Y_i = U^T U  (Cholesky),  V = U^-1,  xinv[i] = V V^T = Y_i^-1
 *
 * The factorisation and V are computed in float64 on the GPU, where errors
 * grow with the condition number; the last product V V^T, whose error
 * relative to ||xinv||_F does not, with float32-accurate products (each
 * float32 product as six bf16 products of exact splits).  xinv[i] is written
 * as float32, both triangles, exactly symmetric.  info[i] (device int32 array of n entries) receives 0 on
 * success, or k > 0 when the leading minor of order k of Y_i is not positive
 * definite or not finite (LAPACK xPOTRF convention); xinv[i] is then
 * unspecified.  gamma must be finite and >= 0.  x[i] and xinv[j] must not
 * overlap.
 */
size_t kfac_inverse_workspace_size(int n, const int64_t* d);
kfac_status_t kfac_damped_inverse(int n, const float* const* x, const int64_t* d, float gamma,
                                  float* const* xinv, int32_t* info,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ----------------------------------------------------------- precondition --
 * Preconditioned gradient of each layer (the damped update rule that follows
 * the Kronecker inverse property (A (x) G)^-1 = A^-1 (x) G^-1):
 *
 *     out[l] = ginv[l] . grad[l] . ainv[l]
 *
 * ginv[l] : [d_g[l], d_g[l]] float32, (G + gamma I)^-1, symmetric;
 * grad[l] : [d_g[l], d_a[l]] float32 weight gradient (bias gradient in the
 *           last column for layers with a bias);
 * ainv[l] : [d_a[l], d_a[l]] float32, (A + gamma I)^-1, symmetric;
 * out[l]  : [d_g[l], d_a[l]] float32.
 * ginv and ainv must be exactly symmetric (as kfac_damped_inverse writes
 * them): the kernels read them in whichever orientation coalesces.  The two
 * products run on the bf16 matrix cores as six bf16 products of exact
 * splits per float32 product, with float32 rounding.  out[l]
 * must not overlap any input.
 */
size_t kfac_precondition_workspace_size(int n, const int64_t* d_g, const int64_t* d_a);
kfac_status_t kfac_precondition(int n, const float* const* ginv, const float* const* grad,
                                const float* const* ainv, const int64_t* d_g, const int64_t* d_a,
                                float* const* out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* ----------------------------------------------------------------- layers --
 * Factor inputs of real layers.  The page computes A_{l-1} from the layer's
 * input in the forward pre-hook and G_l from the gradient with respect to the
 * layer's output in the backward hook (pipelining paragraph; the optimizer
 * paragraph that registers both hooks on every layer).  For a convolution the
 * rows of a factor input are its patches, one row per sample and output
 * position, so that A = (1/rows) a^T a with rows = batch * H_out * W_out.
 * A fully connected layer is the 1 x 1 case: h = w = kh = kw = 1.
 */
typedef struct {
    int64_t n, c, h, w; /* input [n, c, h, w] row-major; n, c, h, w >= 1 */
    int32_t kh, kw;     /* kernel size >= 1 */
    int32_t sh, sw;     /* stride >= 1 */
    int32_t ph, pw;     /* zero padding >= 0 */
    int32_t dh, dw;     /* dilation >= 1 */
    int32_t ones;       /* 1: a trailing column of ones (the layer has a bias), else 0 */
    int32_t reserved;   /* 0 */
} kfac_conv_t;

/* Patches of each layer input as the rows of its A-factor input:
 *
 *     oh = (h + 2 ph - dh (kh - 1) - 1) / sh + 1,  ow likewise (both >= 1)
 *     a[l][(ni oh + y) ow + x][(ci kh + i) kw + j] = x[l][ni][ci][y sh - ph + i dh][x sw - pw + j dw]
 *
 * zero where the index falls outside the input, and 1 in the last column
 * when ones = 1.  a[l] is [n oh ow, c kh kw + ones] row-major, in `dtype`
 * like x[l]; values are copied bit for bit.  The column order matches a
 * weight [c_out, c, kh, kw] read as [c_out, c kh kw].  a[l] must not
 * overlap any x[j]; at most 2^31 - 1 elements per a[l] and per sample of
 * x[l] (c h w), else KFAC_ERR_INVALID_VALUE.
 */
size_t kfac_im2col_workspace_size(int n);
kfac_status_t kfac_im2col(int n, const void* const* x, const kfac_conv_t* shape, kfac_dtype_t dtype,
                          void* const* a, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Output gradients as the rows of each G-factor input:
 *
 *     g[l][b hw + p][ci] = scale * gy[l][b][ci][p]
 *
 * gy[l] : [batch[l], c[l], hw[l]] (an output gradient [b, c, H, W] with the
 *         positions flattened; a fully connected layer: hw = 1);
 * g[l]  : [batch[l] hw[l], c[l]], the product formed in float32 and stored
 *         in `dtype` like gy[l] (rounded to nearest even for bfloat16).
 * `scale` multiplies every gradient (for a loss averaged over the batch,
 * scale = batch gives per-sample gradients).  g[l] must not overlap gy[j].
 */
size_t kfac_grad_rows_workspace_size(int n);
kfac_status_t kfac_grad_rows(int n, const void* const* gy, const int64_t* batch, const int64_t* c,
                             const int64_t* hw, kfac_dtype_t dtype, float scale, void* const* g,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* A layer's weight and bias gradients as one [d_out, d_in + has_bias] matrix
 * (the gradW of kfac_precondition, bias in the last column) and back:
 *
 *     KFAC_PACK    mat[l][r][k] = wgrad[l][r][k] (k < d_in), mat[l][r][d_in] = bgrad[l][r]
 *     KFAC_UNPACK  the reverse
 *
 * wgrad[l] : [d_out, d_in] float32 (a convolution weight [c_out, c, kh, kw]
 *            with d_in = c kh kw);  bgrad[l] : [d_out] float32 or NULL (no
 *            bias, has_bias = 0).  Values are copied bit for bit; mat[l]
 *            must not overlap wgrad[j] or bgrad[j].
 */
size_t kfac_grad_matrix_workspace_size(int n);
kfac_status_t kfac_grad_matrix(int n, float* const* wgrad, float* const* bgrad, const int64_t* d_out,
                               const int64_t* d_in, float* const* mat, kfac_pack_dir_t dir,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KFAC_H */
