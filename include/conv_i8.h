/*
 * conv_i8.h — INT8 2-D convolution forward (conv_fprop) with INT32
 * accumulation and INT32 output, for AMD Instinct MI355X (gfx950).
 *
 * The operation (cuDNN docs page "Convolutions", section "Convolution Fprop",
 * and its "Python API" list: image, weight, pre_padding, post_padding, stride,
 * dilation):
 *
 *   Y[n,k,p,q] = sum_{c<C} sum_{r<R} sum_{s<S}
 *                  X[n, c, p*stride_h - pre_h + r*dil_h, q*stride_w - pre_w + s*dil_w]
 *                * W[k, c, r, s]
 *
 * where X reads as 0 outside 0 <= h < H, 0 <= w < W (zero padding).  It is a
 * cross-correlation: the filter is not flipped (the naive loop of "Building a
 * From-Scratch INT8 Strided Convolution Kernel", "Step 2", reads the input at
 * oh*stride + kh against kernel tap kh); true convolution is available
 * through conv_fprop_i8_ex_ws.  The result is exact: every product
 * of two int8 values is summed in 32-bit integers, which cannot overflow while
 * C*R*S <= 131071 (|product| <= 16384); larger reductions are refused.  The
 * plain entries never saturate and refuse an int8 output (the forum thread
 * "INT8 convolution using cuDNN Python Frontend" shows what an int8 output
 * descriptor produces there: the true sums clamped to int8 and packed into
 * the int32 buffer).  The separate requantising entries at the end of this
 * file write int8 on purpose, through an explicit epilogue.
 *
 * Output size: P = floor((H + pre_h + post_h - dil_h*(R-1) - 1) / stride_h) + 1,
 * and Q likewise; a negative numerator is an error.
 *
 * Tensors are described as in the forum thread's graph.tensor(dim, stride)
 * and the blog's "Step 1: Define the Strided Tensor Layout": four logical dims
 * plus four strides counted in ELEMENTS (not bytes).  Logical orders are
 *   image  [N, C, H, W]   int8
 *   filter [K, C, R, S]   int8
 *   output [N, K, P, Q]   int32
 * so NCHW, NHWC (channels_last), KCRS, KRSC and strided views are all just
 * stride choices.  Element (a,b,c,d) lives at ptr + a*s0 + b*s1 + c*s2 + d*s3,
 * where ptr points at element (0,0,0,0).  The stride of a dim of size 1 is
 * ignored.  Strides must be >= 0; input strides may be 0 (broadcast); the
 * output must not overlap itself.  Spatial pairs are [h, w].
 *
 * Ownership: the caller owns every buffer.  Pointers are device pointers
 * (HIP memory of the current device); the library never frees them and keeps
 * no state between calls.  All device work is enqueued on `stream` (a
 * hipStream_t; NULL means the default stream); calls return without waiting
 * for it.
 *
 * Errors: argument errors are detected on the host before any device work is
 * enqueued, and then nothing is written.  CONV_I8_ERR_HIP means a HIP call
 * failed while enqueueing; faults inside kernels surface at the caller's next
 * synchronisation of the stream.  Only the output elements the descriptor
 * addresses are written; gaps of a strided output are left untouched.
 */
#ifndef CONV_I8_H
#define CONV_I8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CONV_I8_DT_INT8 = 1,
    CONV_I8_DT_INT32 = 2
} conv_i8_dtype_t;

/* A 4-D tensor: dtype (conv_i8_dtype_t), ndim (must be 4), logical dims and
 * element strides in the logical order given above. */
typedef struct {
    int32_t dtype;
    int32_t ndim;
    int64_t dims[4];
    int64_t strides[4];
} conv_i8_desc_t;

typedef enum {
    CONV_I8_OK = 0,
    CONV_I8_ERR_NULL = 1,        /* a required pointer is NULL */
    CONV_I8_ERR_DTYPE = 2,       /* image/filter not INT8, or output not INT32 */
    CONV_I8_ERR_RANK = 3,        /* ndim != 4 */
    CONV_I8_ERR_DIMS = 4,        /* negative dim, or a filter dim R or S < 1 */
    CONV_I8_ERR_PARAM = 5,       /* stride < 1, dilation < 1 or padding < 0 */
    CONV_I8_ERR_CHANNELS = 6,    /* image C != filter C */
    CONV_I8_ERR_OUT_DIMS = 7,    /* output dims != [N, K, P, Q], or P or Q < 1 */
    CONV_I8_ERR_STRIDES = 8,     /* negative stride, or an output that overlaps itself */
    CONV_I8_ERR_RANGE = 9,       /* C*R*S > 131071: int32 sums no longer exact */
    CONV_I8_ERR_WORKSPACE = 10,  /* workspace smaller than conv_fprop_i8_workspace_size */
    CONV_I8_ERR_UNSUPPORTED = 11,/* one image or the filter spans >= 2 GiB */
    CONV_I8_ERR_HIP = 12,        /* a HIP runtime call failed */
    CONV_I8_ERR_SCRATCH = 13     /* conv_fprop_i8_noalloc: workspace needed exceeds its scratch array */
} conv_i8_status_t;

/* Largest C*R*S for which the int32 sum is exact for all int8 inputs. */
#define CONV_I8_MAX_REDUCTION 131071

/*
 * Output dims [N, K, P, Q] for an image and filter descriptor and the conv
 * parameters: the output-size formula above (cuDNN "Convolutions",
 * "Convolution Fprop", whose Python API returns the response tensor of the
 * padded, strided, dilated window; the blog's "Correctness Testing" checks a
 * 32x32 image with a 3x3 filter gives 30x30).  Validates the same fields
 * conv_fprop_i8 does except the output.  Host-only: touches no device.
 */
conv_i8_status_t conv_fprop_i8_out_dims(const conv_i8_desc_t *image,
                                        const conv_i8_desc_t *filter,
                                        const int64_t pre_padding[2],
                                        const int64_t post_padding[2],
                                        const int64_t stride[2],
                                        const int64_t dilation[2],
                                        int64_t out_dims[4]);

/*
 * The workspace query of the forum thread "INT8 convolution using cuDNN
 * Python Frontend" (question post: the graph reports its workspace size, the
 * caller allocates that many bytes and passes them to the execute call), here
 * without a graph object.
 *
 * Bytes of device workspace conv_fprop_i8_ws needs for this problem (0 when
 * both the image and the filter are already channel-innermost with C a
 * multiple of 16 and 16-byte aligned rows; otherwise room for their packed
 * N,H,W,C / K,R,S,C copies).  image_ptr and filter_ptr are only inspected for
 * their 16-byte alignment and may be NULL (then they count as aligned).
 * Host-only.
 */
conv_i8_status_t conv_fprop_i8_workspace_size(const conv_i8_desc_t *image, const void *image_ptr,
                                              const conv_i8_desc_t *filter, const void *filter_ptr,
                                              const conv_i8_desc_t *out,
                                              const int64_t pre_padding[2],
                                              const int64_t post_padding[2],
                                              const int64_t stride[2],
                                              const int64_t dilation[2],
                                              size_t *workspace_bytes);

/*
 * The execute call of the same forum question post (operands, output and the
 * caller's workspace passed together), for the operation of cuDNN
 * "Convolutions", "Convolution Fprop" (parameters of its Python API list).
 *
 * Y = conv_fprop(image, filter) into `out_ptr`, with caller-provided device
 * workspace of `workspace_bytes` bytes, 256-byte aligned (may be NULL when the
 * size needed is 0; CONV_I8_ERR_WORKSPACE if too small or misaligned).  Never
 * allocates, never synchronises: safe to record into a HIP graph.  The
 * workspace must stay untouched until the stream has run the call.
 */
conv_i8_status_t conv_fprop_i8_ws(const conv_i8_desc_t *image, const void *image_ptr,
                                  const conv_i8_desc_t *filter, const void *filter_ptr,
                                  const conv_i8_desc_t *out, void *out_ptr,
                                  const int64_t pre_padding[2],
                                  const int64_t post_padding[2],
                                  const int64_t stride[2],
                                  const int64_t dilation[2],
                                  void *workspace, size_t workspace_bytes,
                                  void *stream);

/*
 * cuDNN "Convolutions", "Convolution Fprop" as one call (the Python API's
 * parameter list: image, weight, pre_padding, post_padding, stride,
 * dilation), for callers that do not manage a workspace.
 *
 * Same as conv_fprop_i8_ws, but any workspace needed is taken with
 * hipMallocAsync on `stream` and released with hipFreeAsync after the work.
 */
conv_i8_status_t conv_fprop_i8(const conv_i8_desc_t *image, const void *image_ptr,
                               const conv_i8_desc_t *filter, const void *filter_ptr,
                               const conv_i8_desc_t *out, void *out_ptr,
                               const int64_t pre_padding[2],
                               const int64_t post_padding[2],
                               const int64_t stride[2],
                               const int64_t dilation[2],
                               void *stream);

/*
 * For callers that cannot allocate device memory: code being recorded into a
 * HIP graph, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same operation, arguments and errors as conv_fprop_i8 (no workspace
 * argument), but any workspace the problem needs (the packed channel-innermost
 * copies of an image or filter the kernels cannot read in place) comes from a
 * static device array of CONV_I8_NOALLOC_SCRATCH_BYTES bytes, one per GPU,
 * held from the first call on that GPU until the process ends.  Calls no
 * hipMalloc/hipFree and no allocating library routine.  A problem needing
 * more returns CONV_I8_ERR_SCRATCH before any device work (the
 * conv_fprop_i8_workspace_size of the same arguments tells the need).  The
 * calling thread's current device must be the device of `stream`
 * (CONV_I8_ERR_PARAM otherwise).  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race on it and must be serialised by the caller; consecutive calls
 * on one stream are fine.  The array keeps the last call's contents; nothing
 * in it needs to start at zero.
 */
#define CONV_I8_NOALLOC_SCRATCH_BYTES (16u << 20)

conv_i8_status_t conv_fprop_i8_noalloc(const conv_i8_desc_t *image, const void *image_ptr,
                                       const conv_i8_desc_t *filter, const void *filter_ptr,
                                       const conv_i8_desc_t *out, void *out_ptr,
                                       const int64_t pre_padding[2],
                                       const int64_t post_padding[2],
                                       const int64_t stride[2],
                                       const int64_t dilation[2],
                                       void *stream);

/*
 * Counterpart of the plan list of the cuDNN frontend tutorial page
 * (autotuning paragraph: plans from the heuristic modes, each one built and
 * timed): here the single plan this library picks, for inspection.
 *
 * A one-line, human-readable description of how conv_fprop_i8_ws would run
 * this problem (which operands are repacked, the tile shape, the grid).
 * Writes at most `len` bytes including the terminating NUL.  Host-only.
 */
conv_i8_status_t conv_fprop_i8_plan(const conv_i8_desc_t *image, const void *image_ptr,
                                    const conv_i8_desc_t *filter, const void *filter_ptr,
                                    const conv_i8_desc_t *out,
                                    const int64_t pre_padding[2],
                                    const int64_t post_padding[2],
                                    const int64_t stride[2],
                                    const int64_t dilation[2],
                                    char *buf, size_t len);

/*
 * The candidate plans of the cuDNN frontend tutorial page (autotuning
 * paragraph: every plan the heuristics offer is built and timed, and the
 * index of the fastest is kept): here the names of every tile shape the
 * library can run, comma-separated, in the order the planner considers
 * them.  Setting the environment variable CONV_I8_TILE to one of them makes
 * the planner use that tile wherever it applies (the plan string then names
 * it); a problem it does not fit falls back to the default tile.  Measured
 * choices for known problems are compiled into the library and take
 * precedence over its cost model.  Writes at most `len` bytes including the
 * terminating NUL (CONV_I8_ERR_PARAM if that is too short, CONV_I8_ERR_NULL
 * for a NULL buf).  Host-only.
 */
conv_i8_status_t conv_i8_tile_names(char *buf, size_t len);

/*
 * Calibration for the compute side of the roofline (the blog "Building a
 * From-Scratch INT8 Strided Convolution Kernel" measures GOPS in its
 * "Benchmarking" section and asks for hardware observability in "Extending
 * It"): the INT8 matrix-core rate this GPU reaches under load, to set beside
 * the published peak.  Launches `workgroups` workgroups of four waves on
 * `stream`; each wave issues `iters` x 8 v_mfma_i32_32x32x32_i8 back to back
 * on register operands (random bytes drawn from `seed`, or all zeros when
 * seed is 0) and every thread writes one checksum to out[] (device memory,
 * workgroups * 256 int32 elements, caller-owned).  One launch performs
 * workgroups * 4 * iters * 8 * 65536 INT8 operations; time it with events
 * on the stream.  CONV_I8_ERR_NULL for a NULL out, CONV_I8_ERR_PARAM for
 * workgroups outside [1, 2^20] or iters < 1, CONV_I8_ERR_HIP if the launch
 * fails.
 */
conv_i8_status_t conv_i8_mfma_ceiling(int workgroups, int iters, uint32_t seed, int32_t *out, void *stream);

/*
 * Requantising INT8 epilogue, fused into the convolution.
 *
 * The naive loop of "Building a From-Scratch INT8 Strided Convolution
 * Kernel" (step 2) clamps each sum to [-128, 127] and stores it as INT8, and
 * the page's roadmap ("Extending It") fuses a ReLU and a quantisation step
 * into the convolution to save the DRAM round trip of the wide sums; the
 * cuDNN frontend tutorial fuses a bias add and ReLU into a convolution and
 * scales a matmul by a host scalar alpha.  Here, for output element
 * (n, k, p, q) with exact sum acc (as in conv_fprop_i8):
 *
 *   v = fmaf((float)acc, s_k, b_k)   float conversion rounds to nearest even,
 *                                    then one fused multiply-add (one rounding)
 *   v = max(v, 0)                    only when relu != 0
 *   y = clamp(rint(v), -128, 127)    round half to even, saturate
 *
 * s_k = scale[k] when scale != NULL, else alpha; b_k = bias[k] when
 * bias != NULL, else 0.  scale and bias are device pointers to K floats,
 * 4-byte aligned, owned by the caller and read by the kernels on `stream`.
 * Non-finite factors: a value that is NaN after the multiply-add (an
 * infinite scale times a zero sum, or infinities of opposite sign) is written
 * as 0, and an infinite value saturates to -128 or 127.  With alpha = 1 and no
 * bias or relu the result is the page's saturating INT8 store.
 */
typedef struct {
    const float *scale;  /* K per-output-channel scales, or NULL: alpha for all */
    float alpha;         /* used when scale == NULL; must be finite then */
    const float *bias;   /* K per-output-channel biases, or NULL: no bias */
    int32_t relu;        /* nonzero: negative values become 0 before rounding */
} conv_i8_requant_t;

/*
 * Workspace bytes for conv_fprop_i8_requant_ws: the same rules as
 * conv_fprop_i8_workspace_size, for an INT8 output descriptor
 * (CONV_I8_ERR_DTYPE otherwise).  Host-only.
 */
conv_i8_status_t conv_fprop_i8_requant_workspace_size(const conv_i8_desc_t *image,
                                                      const void *image_ptr,
                                                      const conv_i8_desc_t *filter,
                                                      const void *filter_ptr,
                                                      const conv_i8_desc_t *out,
                                                      const int64_t pre_padding[2],
                                                      const int64_t post_padding[2],
                                                      const int64_t stride[2],
                                                      const int64_t dilation[2],
                                                      size_t *workspace_bytes);

/*
 * conv_fprop followed by the requantising epilogue above, INT8 output [N, K,
 * P, Q] with any non-overlapping strides (CONV_I8_ERR_DTYPE for any other
 * output dtype; CONV_I8_ERR_NULL for rq == NULL; CONV_I8_ERR_PARAM for a
 * misaligned scale/bias array or a non-finite alpha without a scale array).
 * Workspace, errors and stream behaviour as conv_fprop_i8_ws: never
 * allocates, never synchronises.
 */
conv_i8_status_t conv_fprop_i8_requant_ws(const conv_i8_desc_t *image, const void *image_ptr,
                                          const conv_i8_desc_t *filter, const void *filter_ptr,
                                          const conv_i8_desc_t *out, void *out_ptr,
                                          const int64_t pre_padding[2],
                                          const int64_t post_padding[2],
                                          const int64_t stride[2],
                                          const int64_t dilation[2],
                                          const conv_i8_requant_t *rq,
                                          void *workspace, size_t workspace_bytes,
                                          void *stream);

/*
 * Same as conv_fprop_i8_requant_ws, with any workspace taken and released
 * stream-ordered (hipMallocAsync / hipFreeAsync) as in conv_fprop_i8.
 */
conv_i8_status_t conv_fprop_i8_requant(const conv_i8_desc_t *image, const void *image_ptr,
                                       const conv_i8_desc_t *filter, const void *filter_ptr,
                                       const conv_i8_desc_t *out, void *out_ptr,
                                       const int64_t pre_padding[2],
                                       const int64_t post_padding[2],
                                       const int64_t stride[2],
                                       const int64_t dilation[2],
                                       const conv_i8_requant_t *rq,
                                       void *stream);

/*
 * Convolution mode.  The cuDNN "Convolutions" page lists a convolution_mode
 * parameter for "Convolution Fprop" without defining its values; read as the
 * usual pair: cross-correlation (the operation above, what every other entry
 * computes) and true convolution, which reads filter tap (R-1-r, S-1-s)
 * where cross-correlation reads (r, s):
 *
 *   Y[n,k,p,q] = sum_{c,r,s} X[n, c, p*stride_h - pre_h + r*dil_h,
 *                                q*stride_w - pre_w + s*dil_w]
 *                            * W[k, c, R-1-r, S-1-s]
 */
typedef enum {
    CONV_I8_MODE_CROSS_CORRELATION = 0,
    CONV_I8_MODE_CONVOLUTION = 1
} conv_i8_mode_t;

/*
 * Workspace bytes for conv_fprop_i8_ex_ws (the same rules as
 * conv_fprop_i8_workspace_size; the mode does not change them).  The output
 * descriptor may be INT32 or INT8.  CONV_I8_ERR_PARAM for an unknown mode.
 */
conv_i8_status_t conv_fprop_i8_ex_workspace_size(const conv_i8_desc_t *image,
                                                 const void *image_ptr,
                                                 const conv_i8_desc_t *filter,
                                                 const void *filter_ptr,
                                                 const conv_i8_desc_t *out,
                                                 const int64_t pre_padding[2],
                                                 const int64_t post_padding[2],
                                                 const int64_t stride[2],
                                                 const int64_t dilation[2],
                                                 int32_t mode,
                                                 size_t *workspace_bytes);

/*
 * The general entry: either mode (conv_i8_mode_t), and the epilogue chosen by
 * the output descriptor -- INT32 sums with rq == NULL (CONV_I8_ERR_PARAM
 * otherwise), or the requantising INT8 epilogue with rq != NULL
 * (CONV_I8_ERR_NULL otherwise); any other output dtype is
 * CONV_I8_ERR_DTYPE.  Workspace, errors and stream behaviour as
 * conv_fprop_i8_ws: never allocates, never synchronises.  With
 * CONV_I8_MODE_CROSS_CORRELATION it computes exactly what conv_fprop_i8_ws
 * or conv_fprop_i8_requant_ws compute.
 */
conv_i8_status_t conv_fprop_i8_ex_ws(const conv_i8_desc_t *image, const void *image_ptr,
                                     const conv_i8_desc_t *filter, const void *filter_ptr,
                                     const conv_i8_desc_t *out, void *out_ptr,
                                     const int64_t pre_padding[2],
                                     const int64_t post_padding[2],
                                     const int64_t stride[2],
                                     const int64_t dilation[2],
                                     int32_t mode,
                                     const conv_i8_requant_t *rq,
                                     void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * Data gradient (cuDNN "Convolutions" page, section "Convolution Dgrad": the
 * gradient with respect to the image during backpropagation, with the same
 * pre/post padding, stride, dilation and convolution mode as the forward
 * pass).  Read as the adjoint of conv_fprop: every forward term
 * X[n,c,h,w] * W[k,c,r,s] added to Y[n,k,p,q] returns dY[n,k,p,q] * W[k,c,r,s]
 * to dX[n,c,h,w]:
 *
 *   dX[n,c,h,w] = sum_{k,r,s} dY[n,k,p,q] * W[k,c,r',s']
 *       over the taps with h + pre_h - r*dil_h = p*stride_h, 0 <= p < P,
 *       and w + pre_w - s*dil_w = q*stride_w, 0 <= q < Q;
 *       (r',s') = (r,s), or (R-1-r, S-1-s) for CONV_I8_MODE_CONVOLUTION.
 *
 * loss (dY) is INT8 [N,K,P,Q], filter INT8 [K,C,R,S], dx INT32 [N,C,H,W];
 * [P, Q] must be the forward output size of [H, W] (CONV_I8_ERR_OUT_DIMS
 * otherwise; with stride > 1 several H give one P, so dx's dims decide).
 * Exact int32 sums while K*R*S <= 131071 (CONV_I8_ERR_RANGE otherwise).  Any
 * strides; dx must not overlap itself.  The work is stride_h*stride_w
 * forward convolutions, one per residue class of (h, w), each a stride-1
 * true convolution of dY with the filter transposed to [C, K, ...] and
 * subsampled to the taps that reach that class; they run one after another
 * on `stream` and share the workspace.  A filter view whose K is contiguous
 * (a KRSC filter) is read in place when K is a multiple of 64 and C of 16;
 * when every phase reads its view that way and a channel-innermost dY in
 * place, all the phases (up to four) run as one launch and no workspace is
 * needed.  Otherwise the workspace holds the packed operands of the phases;
 * with several phases, K a multiple of 16 and a channel-innermost dY, every
 * phase's packed filter view gets a region of its own, written by one repack
 * launch before the phases.  The size depends on whether the operands can be
 * read in place, so pass the pointers of the call to the size query.  Errors
 * and stream behaviour as conv_fprop_i8_ws; never allocates, never
 * synchronises.
 */
conv_i8_status_t conv_dgrad_i8_workspace_size(const conv_i8_desc_t *loss, const void *loss_ptr,
                                              const conv_i8_desc_t *filter,
                                              const void *filter_ptr,
                                              const conv_i8_desc_t *dx,
                                              const int64_t pre_padding[2],
                                              const int64_t post_padding[2],
                                              const int64_t stride[2],
                                              const int64_t dilation[2],
                                              int32_t mode,
                                              size_t *workspace_bytes);

conv_i8_status_t conv_dgrad_i8_ws(const conv_i8_desc_t *loss, const void *loss_ptr,
                                  const conv_i8_desc_t *filter, const void *filter_ptr,
                                  const conv_i8_desc_t *dx, void *dx_ptr,
                                  const int64_t pre_padding[2],
                                  const int64_t post_padding[2],
                                  const int64_t stride[2],
                                  const int64_t dilation[2],
                                  int32_t mode,
                                  void *workspace, size_t workspace_bytes,
                                  void *stream);

/* conv_dgrad_i8_ws with its workspace taken stream-ordered (hipMallocAsync). */
conv_i8_status_t conv_dgrad_i8(const conv_i8_desc_t *loss, const void *loss_ptr,
                               const conv_i8_desc_t *filter, const void *filter_ptr,
                               const conv_i8_desc_t *dx, void *dx_ptr,
                               const int64_t pre_padding[2],
                               const int64_t post_padding[2],
                               const int64_t stride[2],
                               const int64_t dilation[2],
                               int32_t mode,
                               void *stream);

/*
 * Weight gradient (cuDNN "Convolutions" page, section "Convolution Wgrad":
 * the gradient with respect to the filter from the image and the loss, with
 * the forward's padding, stride, dilation and convolution mode).  Read as
 * the adjoint of conv_fprop with respect to W:
 *
 *   dW[k,c,r',s'] = sum_{n,p,q} dY[n,k,p,q]
 *                      * X[n, c, p*stride_h - pre_h + r*dil_h, q*stride_w - pre_w + s*dil_w]
 *
 * (X is 0 outside the image), (r',s') = (r,s), or (R-1-r,S-1-s) for
 * CONV_I8_MODE_CONVOLUTION.  image INT8 [N,C,H,W], loss (dY) INT8 [N,K,P,Q]
 * with [P,Q] the forward output size, dw INT32 [K,C,R,S] (its dims give R
 * and S).  Exact int32 sums while N*P*Q <= 131071 (CONV_I8_ERR_RANGE
 * otherwise).  Any strides; dw must not overlap itself.  The work is one
 * forward convolution: the image transposed to [C, N, H, W] convolved with the
 * loss transposed to [K, N, P, Q] at stride = dilation and dilation = stride,
 * written to dW transposed to [C, K, R, S] (reversed along R and S for true
 * convolution).  Channels-last image and loss (channel stride 1, image
 * strides and the loss's pixel pitch multiples of 16 bytes, 16-byte aligned
 * pointers), C and K multiples of 16 and a dense dw of at most 128 tiles of
 * 128x128 per filter tap take one kernel instead that reads both operands in
 * place: for each tap, the product of the loss and the image pixels the tap
 * reads, over the N*P*Q output pixels.  Errors and stream behaviour as
 * conv_fprop_i8_ws; never
 * allocates, never synchronises.  The workspace holds the packed transposed
 * operands and, when the long N*P*Q reduction is split over workgroups and dw
 * is dense, one int32 partial copy of dw per split (added into dw by a
 * reduction kernel on the same stream); its contents on return are
 * unspecified.
 */
conv_i8_status_t conv_wgrad_i8_workspace_size(const conv_i8_desc_t *image, const void *image_ptr,
                                              const conv_i8_desc_t *loss, const void *loss_ptr,
                                              const conv_i8_desc_t *dw,
                                              const int64_t pre_padding[2],
                                              const int64_t post_padding[2],
                                              const int64_t stride[2],
                                              const int64_t dilation[2],
                                              int32_t mode,
                                              size_t *workspace_bytes);

conv_i8_status_t conv_wgrad_i8_ws(const conv_i8_desc_t *image, const void *image_ptr,
                                  const conv_i8_desc_t *loss, const void *loss_ptr,
                                  const conv_i8_desc_t *dw, void *dw_ptr,
                                  const int64_t pre_padding[2],
                                  const int64_t post_padding[2],
                                  const int64_t stride[2],
                                  const int64_t dilation[2],
                                  int32_t mode,
                                  void *workspace, size_t workspace_bytes,
                                  void *stream);

/* conv_wgrad_i8_ws with its workspace taken stream-ordered (hipMallocAsync). */
conv_i8_status_t conv_wgrad_i8(const conv_i8_desc_t *image, const void *image_ptr,
                               const conv_i8_desc_t *loss, const void *loss_ptr,
                               const conv_i8_desc_t *dw, void *dw_ptr,
                               const int64_t pre_padding[2],
                               const int64_t post_padding[2],
                               const int64_t stride[2],
                               const int64_t dilation[2],
                               int32_t mode,
                               void *stream);

/*
 * Counterpart of conv_fprop_i8_plan for the weight gradient (cuDNN
 * "Convolutions" page, section "Convolution Wgrad"; the plan list of the
 * cuDNN frontend tutorial page, autotuning paragraph): the description of
 * the one forward call conv_wgrad_i8_ws makes (tile, split of the N*P*Q
 * reduction, workspace), "kernel=wgrad_in_place ..." for a gradient the
 * in-place kernel serves, or "empty" for a dw with no elements.  Arguments
 * and errors as conv_wgrad_i8_workspace_size; writes at most `len` bytes
 * including the terminating NUL.  Host-only.
 */
conv_i8_status_t conv_wgrad_i8_plan(const conv_i8_desc_t *image, const void *image_ptr,
                                    const conv_i8_desc_t *loss, const void *loss_ptr,
                                    const conv_i8_desc_t *dw,
                                    const int64_t pre_padding[2],
                                    const int64_t post_padding[2],
                                    const int64_t stride[2],
                                    const int64_t dilation[2],
                                    int32_t mode,
                                    char *buf, size_t len);

/*
 * Static string naming a status code.  The forum thread's answer post traces
 * the question's wrong output to a descriptor mistake (strides that do not
 * match the NCHW layout); each refusal above is reported by name instead of
 * running on a descriptor the library cannot honour.  Unknown codes give a
 * string containing "unknown".
 */
const char *conv_i8_status_string(conv_i8_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* CONV_I8_H */
