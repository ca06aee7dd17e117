/*
 * Plain CPU oracle for INT8 convolution forward with INT32 output, and for
 * the same convolution followed by a requantising INT8 epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no source,
 * header, table or helper with the HIP library, and it is deliberately slow:
 * a direct nested loop over the definition, 64-bit accumulation, no blocking.
 *
 * What it computes (cuDNN docs page "Convolutions", section "Convolution
 * Fprop": the response is the image convolved with the filter; its Python API
 * list names pre_padding, post_padding, stride and dilation):
 *
 *   Y[n,k,p,q] = sum_{r<R} sum_{s<S} sum_{c<C}
 *                  Xpad[n, c, p*sh - ph + r*dh, q*sw - pw + s*dw] * W[k,c,r,s]
 *
 * with Xpad equal to X inside the image and 0 outside it (zero padding).
 * Readings taken where the pages leave a step open:
 *   - "convolved" is read as cross-correlation (no flip of the filter): the
 *     naive loop of "Building a From-Scratch INT8 Strided Convolution Kernel",
 *     "Step 2: Implement the Naive Strided Loop", reads input[ih+kh] against
 *     kernel[kh], and the forum page takes torch's conv2d as the truth;
 *     the cuDNN page's convolution_mode parameter (listed, never defined)
 *     is read as the usual pair: cross-correlation (mode 0, the default) or
 *     true convolution (mode 1), which reads filter tap (R-1-r, S-1-s) where
 *     cross-correlation reads (r, s) -- every entry below takes the mode;
 *   - the filter is indexed [k, c, r, s]; the same loop on that page adds the
 *     channel stride twice for the filter, which is read as a slip for the
 *     output-channel stride plus the input-channel stride;
 *   - no clamp in the plain entry: its result is INT32, not the clamped INT8
 *     of that loop (the clamp belongs to the requantising entry further down);
 *   - padding is zero; pre_padding is added before row/column 0, post_padding
 *     after the last one; spatial pairs are [h, w].
 *
 * Tensors are addressed as in "Step 1: Define the Strided Tensor Layout" of
 * the same page: logical dims plus strides counted in elements, so element
 * (a,b,c,d) of a tensor lives at ptr + a*s0 + b*s1 + c*s2 + d*s3.
 *
 * Output size per spatial dim: out = floor((in + pre + post - dil*(k-1) - 1) / stride) + 1,
 * rejected when the numerator is negative (checked before dividing).
 *
 * The loop nest follows the naive loop's order: batch, output channel, output
 * row, output column, then filter row, filter column, input channel.  OpenMP
 * splits only the (batch, output channel) pairs; each output element is
 * summed by one thread in that fixed order.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum {
    ORACLE_OK = 0,
    ORACLE_ERR_ARG = 1,      /* null pointer or negative size / parameter */
    ORACLE_ERR_SHAPE = 2,    /* channel mismatch or empty output window */
    ORACLE_ERR_OUT_DIMS = 3, /* output dims are not [N, K, P, Q] */
    ORACLE_ERR_OVERFLOW = 4  /* some sum does not fit in int32 */
};

/* Output size of one spatial dimension; -1 if the window never fits. */
static int64_t oracle_out_len(int64_t in, int64_t pre, int64_t post,
                              int64_t filt, int64_t stride, int64_t dil)
{
    int64_t span = in + pre + post - dil * (filt - 1) - 1;
    if (span < 0)
        return -1;
    return span / stride + 1;
}

int oracle_out_dims(const int64_t xdims[4], const int64_t wdims[4],
                    const int64_t pre[2], const int64_t post[2],
                    const int64_t stride[2], const int64_t dil[2],
                    int64_t ydims[4])
{
    if (!xdims || !wdims || !pre || !post || !stride || !dil || !ydims)
        return ORACLE_ERR_ARG;
    for (int i = 0; i < 4; ++i)
        if (xdims[i] < 0 || wdims[i] < 0)
            return ORACLE_ERR_ARG;
    for (int i = 0; i < 2; ++i)
        if (pre[i] < 0 || post[i] < 0 || stride[i] < 1 || dil[i] < 1)
            return ORACLE_ERR_ARG;
    if (xdims[1] != wdims[1])
        return ORACLE_ERR_SHAPE;
    int64_t p = oracle_out_len(xdims[2], pre[0], post[0], wdims[2], stride[0], dil[0]);
    int64_t q = oracle_out_len(xdims[3], pre[1], post[1], wdims[3], stride[1], dil[1]);
    if (p < 1 || q < 1)
        return ORACLE_ERR_SHAPE;
    ydims[0] = xdims[0];
    ydims[1] = wdims[0];
    ydims[2] = p;
    ydims[3] = q;
    return ORACLE_OK;
}

static int64_t oracle_elems(const int64_t d[4])
{
    return d[0] * d[1] * d[2] * d[3];
}

/* One output element, summed over the filter window in the naive loop's order. */
static int64_t oracle_point(const int8_t *x, const int64_t xd[4], const int64_t xs[4],
                            const int8_t *w, const int64_t wd[4], const int64_t ws[4],
                            int64_t n, int64_t k, int64_t p, int64_t q,
                            const int64_t pre[2], const int64_t stride[2],
                            const int64_t dil[2], int mode)
{
    const int64_t C = xd[1], H = xd[2], Wd = xd[3];
    const int64_t R = wd[2], S = wd[3];
    int64_t acc = 0;
    for (int64_t r = 0; r < R; ++r) {
        const int64_t h = p * stride[0] - pre[0] + r * dil[0];
        const int64_t fr = mode ? R - 1 - r : r;   /* filter row read at this tap */
        for (int64_t s = 0; s < S; ++s) {
            const int64_t wc = q * stride[1] - pre[1] + s * dil[1];
            const int64_t fs = mode ? S - 1 - s : s;
            if (h < 0 || h >= H || wc < 0 || wc >= Wd)
                continue; /* zero padding: the term is 0 */
            for (int64_t c = 0; c < C; ++c) {
                const int64_t xv = x[n * xs[0] + c * xs[1] + h * xs[2] + wc * xs[3]];
                const int64_t wv = w[k * ws[0] + c * ws[1] + fr * ws[2] + fs * ws[3]];
                acc += xv * wv;
            }
        }
    }
    return acc;
}

/*
 * Full convolution.  x, w, y point at element (0,0,0,0) of each tensor.
 * ydims must equal oracle_out_dims(...).  Returns ORACLE_ERR_OVERFLOW (after
 * writing the wrapped values) if any sum leaves the int32 range.
 * nthreads <= 0 uses the OpenMP default.
 */
int oracle_conv_fprop(const int8_t *x, const int64_t xdims[4], const int64_t xstr[4],
                      const int8_t *w, const int64_t wdims[4], const int64_t wstr[4],
                      int32_t *y, const int64_t ydims[4], const int64_t ystr[4],
                      const int64_t pre[2], const int64_t post[2],
                      const int64_t stride[2], const int64_t dil[2], int mode, int nthreads)
{
    int64_t want[4];
    if (!xstr || !wstr || !ystr)
        return ORACLE_ERR_ARG;
    int rc = oracle_out_dims(xdims, wdims, pre, post, stride, dil, want);
    if (rc != ORACLE_OK)
        return rc;
    /* a tensor with no elements is never read, so it may have no storage */
    if ((!x && oracle_elems(xdims) > 0) || (!w && oracle_elems(wdims) > 0) ||
        (!y && oracle_elems(ydims) > 0))
        return ORACLE_ERR_ARG;
    for (int i = 0; i < 4; ++i)
        if (ydims[i] != want[i])
            return ORACLE_ERR_OUT_DIMS;

    const int64_t N = ydims[0], K = ydims[1], P = ydims[2], Q = ydims[3];
    int overflow = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : overflow)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            for (int64_t p = 0; p < P; ++p) {
                for (int64_t q = 0; q < Q; ++q) {
                    int64_t acc = oracle_point(x, xdims, xstr, w, wdims, wstr,
                                               n, k, p, q, pre, stride, dil, mode);
                    if (acc < INT32_MIN || acc > INT32_MAX)
                        overflow = 1;
                    y[n * ystr[0] + k * ystr[1] + p * ystr[2] + q * ystr[3]] =
                        (int32_t)(uint32_t)(uint64_t)acc;
                }
            }
        }
    }
    return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;
}

/*
 * Selected output elements only: idx holds npts rows of (n, k, p, q); the
 * exact 64-bit sums go to out[i].  Used to check outputs of workloads too
 * large to recompute whole.
 */
int oracle_conv_fprop_points(const int8_t *x, const int64_t xdims[4], const int64_t xstr[4],
                             const int8_t *w, const int64_t wdims[4], const int64_t wstr[4],
                             const int64_t pre[2], const int64_t post[2],
                             const int64_t stride[2], const int64_t dil[2], int mode,
                             const int64_t *idx, int64_t npts, int64_t *out)
{
    int64_t yd[4];
    if (!xstr || !wstr || (npts > 0 && (!idx || !out)) || npts < 0)
        return ORACLE_ERR_ARG;
    int rc = oracle_out_dims(xdims, wdims, pre, post, stride, dil, yd);
    if (rc != ORACLE_OK)
        return rc;
    if ((!x && oracle_elems(xdims) > 0) || (!w && oracle_elems(wdims) > 0))
        return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t *t = idx + 4 * i;
        for (int d = 0; d < 4; ++d)
            if (t[d] < 0 || t[d] >= yd[d])
                return ORACLE_ERR_ARG;
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t *t = idx + 4 * i;
        out[i] = oracle_point(x, xdims, xstr, w, wdims, wstr, t[0], t[1], t[2], t[3],
                              pre, stride, dil, mode);
    }
    return ORACLE_OK;
}

/*
 * Requantising epilogue: INT8 output with saturation.
 *
 * "Building a From-Scratch INT8 Strided Convolution Kernel" clamps each sum
 * to [-128, 127] before storing it as INT8 (step 2, the naive loop), and its
 * roadmap ("Extending It") names fusing a ReLU and a quantisation step into
 * the convolution; the cuDNN frontend tutorial fuses a bias add and a ReLU
 * into a convolution and hangs an alpha scale off a matmul.  Where the pages
 * leave the arithmetic open, the reading taken here is, per output element
 * with exact integer sum acc and output channel k:
 *
 *   v = fmaf((float)acc, s_k, b_k)     one IEEE single rounding (fused)
 *   v = max(v, 0)                      only with relu
 *   r = nearbyintf(v)                  round half to even
 *   y = min(max(r, -128), 127)         saturate to INT8
 *
 * with s_k = scale[k] (or alpha for every k when scale is NULL) and
 * b_k = bias[k] (or 0 when bias is NULL).  (float)acc rounds to nearest
 * even; sums here stay below 2^31.  With s = 1 and no bias or relu this is
 * exactly the page's clamp.  The pages say nothing of non-finite factors;
 * the reading taken: a NaN after the multiply-add (an infinite scale times a
 * zero sum, or infinities of opposite sign) is written as 0, and an infinity
 * saturates like any large value.
 */
static int8_t oracle_requant(int64_t acc, float s, float b, int relu)
{
    float v = fmaf((float)acc, s, b);
    if (v != v)
        v = 0.0f;  /* NaN (an infinite scale or bias): written as 0 */
    if (relu && v < 0.0f)
        v = 0.0f;
    v = nearbyintf(v);
    if (v > 127.0f)
        v = 127.0f;
    if (v < -128.0f)
        v = -128.0f;
    return (int8_t)v;
}

/* The epilogue above on given sums: acc[i] of output channel ch[i]. */
int oracle_requant_values(const int64_t *acc, const int64_t *ch, int64_t n,
                          const float *scale, float alpha, const float *bias, int relu,
                          int8_t *out)
{
    if (n < 0 || (n > 0 && (!acc || !ch || !out)))
        return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) {
        const float s = scale ? scale[ch[i]] : alpha;
        const float b = bias ? bias[ch[i]] : 0.0f;
        out[i] = oracle_requant(acc[i], s, b, relu);
    }
    return ORACLE_OK;
}

/*
 * Convolution followed by the requantising epilogue, INT8 output with any
 * strides.  scale and bias hold K floats each (or are NULL).  Returns
 * ORACLE_ERR_OVERFLOW if a sum leaves the int32 range (it is still
 * requantised from the exact sum).
 */
int oracle_conv_fprop_requant(const int8_t *x, const int64_t xdims[4], const int64_t xstr[4],
                              const int8_t *w, const int64_t wdims[4], const int64_t wstr[4],
                              int8_t *y, const int64_t ydims[4], const int64_t ystr[4],
                              const int64_t pre[2], const int64_t post[2],
                              const int64_t stride[2], const int64_t dil[2],
                              const float *scale, float alpha, const float *bias, int relu,
                              int mode, int nthreads)
{
    int64_t want[4];
    if (!xstr || !wstr || !ystr)
        return ORACLE_ERR_ARG;
    int rc = oracle_out_dims(xdims, wdims, pre, post, stride, dil, want);
    if (rc != ORACLE_OK)
        return rc;
    if ((!x && oracle_elems(xdims) > 0) || (!w && oracle_elems(wdims) > 0) ||
        (!y && oracle_elems(ydims) > 0))
        return ORACLE_ERR_ARG;
    for (int i = 0; i < 4; ++i)
        if (ydims[i] != want[i])
            return ORACLE_ERR_OUT_DIMS;

    const int64_t N = ydims[0], K = ydims[1], P = ydims[2], Q = ydims[3];
    int overflow = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : overflow)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            const float s = scale ? scale[k] : alpha;
            const float b = bias ? bias[k] : 0.0f;
            for (int64_t p = 0; p < P; ++p) {
                for (int64_t q = 0; q < Q; ++q) {
                    int64_t acc = oracle_point(x, xdims, xstr, w, wdims, wstr,
                                               n, k, p, q, pre, stride, dil, mode);
                    if (acc < INT32_MIN || acc > INT32_MAX)
                        overflow = 1;
                    y[n * ystr[0] + k * ystr[1] + p * ystr[2] + q * ystr[3]] =
                        oracle_requant(acc, s, b, relu);
                }
            }
        }
    }
    return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;
}

/*
 * Data gradient (cuDNN "Convolutions" page, section "Convolution Dgrad": the
 * gradient of the loss with respect to the image, for the same padding,
 * stride, dilation and mode as the forward pass).  Read as the adjoint of
 * the forward sum above: each forward term X[n,c,h,w] * W[k,c,r,s] added to
 * Y[n,k,p,q] sends dY[n,k,p,q] * W[k,c,r,s] back to dX[n,c,h,w]:
 *
 *   dX[n,c,h,w] = sum_{k,r,s} dY[n,k,p,q] * W[k,c,r',s']
 *     over the taps with h + pre_h - r*dil_h = p*stride_h, 0 <= p < P
 *     (and likewise for w, q), (r',s') = (r,s), or (R-1-r,S-1-s) in mode 1.
 *
 * dy is [N,K,P,Q] int8, w [K,C,R,S] int8, dx [N,C,H,W] int32; P and Q must
 * be the forward output size for H and W.  One output element is summed by
 * one thread over k, then r, then s; 64-bit sums.
 */
static int64_t oracle_dgrad_point(const int8_t *dy, const int64_t dd[4], const int64_t ds[4],
                                  const int8_t *w, const int64_t wd[4], const int64_t ws[4],
                                  int64_t n, int64_t c, int64_t h, int64_t x,
                                  const int64_t pre[2], const int64_t stride[2],
                                  const int64_t dil[2], int mode)
{
    const int64_t K = wd[0], R = wd[2], S = wd[3], P = dd[2], Q = dd[3];
    int64_t acc = 0;
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t r = 0; r < R; ++r) {
            const int64_t pn = h + pre[0] - r * dil[0];     /* = p * stride_h */
            if (pn < 0 || pn % stride[0] != 0 || pn / stride[0] >= P)
                continue;
            const int64_t p = pn / stride[0];
            const int64_t fr = mode ? R - 1 - r : r;
            for (int64_t s = 0; s < S; ++s) {
                const int64_t qn = x + pre[1] - s * dil[1];
                if (qn < 0 || qn % stride[1] != 0 || qn / stride[1] >= Q)
                    continue;
                const int64_t q = qn / stride[1];
                const int64_t fs = mode ? S - 1 - s : s;
                acc += (int64_t)dy[n * ds[0] + k * ds[1] + p * ds[2] + q * ds[3]] *
                       (int64_t)w[k * ws[0] + c * ws[1] + fr * ws[2] + fs * ws[3]];
            }
        }
    }
    return acc;
}

int oracle_conv_dgrad(const int8_t *dy, const int64_t dydims[4], const int64_t dystr[4],
                      const int8_t *w, const int64_t wdims[4], const int64_t wstr[4],
                      int32_t *dx, const int64_t dxdims[4], const int64_t dxstr[4],
                      const int64_t pre[2], const int64_t post[2],
                      const int64_t stride[2], const int64_t dil[2], int mode, int nthreads)
{
    int64_t fwd[4];
    if (!dydims || !dystr || !wstr || !dxdims || !dxstr)
        return ORACLE_ERR_ARG;
    /* the forward problem dX would give: its output must be dY's shape */
    int rc = oracle_out_dims(dxdims, wdims, pre, post, stride, dil, fwd);
    if (rc != ORACLE_OK)
        return rc;
    for (int i = 0; i < 4; ++i)
        if (dydims[i] != fwd[i])
            return ORACLE_ERR_OUT_DIMS;
    if ((!dy && oracle_elems(dydims) > 0) || (!w && oracle_elems(wdims) > 0) ||
        (!dx && oracle_elems(dxdims) > 0))
        return ORACLE_ERR_ARG;

    const int64_t N = dxdims[0], C = dxdims[1], H = dxdims[2], W = dxdims[3];
    int overflow = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : overflow)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t ci = 0; ci < C; ++ci) {
            for (int64_t h = 0; h < H; ++h) {
                for (int64_t x = 0; x < W; ++x) {
                    int64_t acc = oracle_dgrad_point(dy, dydims, dystr, w, wdims, wstr,
                                                     n, ci, h, x, pre, stride, dil, mode);
                    if (acc < INT32_MIN || acc > INT32_MAX)
                        overflow = 1;
                    dx[n * dxstr[0] + ci * dxstr[1] + h * dxstr[2] + x * dxstr[3]] =
                        (int32_t)(uint32_t)(uint64_t)acc;
                }
            }
        }
    }
    return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;
}

/*
 * Weight gradient (cuDNN "Convolutions" page, section "Convolution Wgrad":
 * the gradient with respect to the filter, from the image and the loss, for
 * the forward's padding, stride, dilation and mode).  The adjoint of the
 * forward sum with respect to W: each forward term X[n,c,h,w] * W[k,c,r',s']
 * added to Y[n,k,p,q] sends X[n,c,h,w] * dY[n,k,p,q] to dW[k,c,r',s']:
 *
 *   dW[k,c,r',s'] = sum_{n,p,q} dY[n,k,p,q] * X[n,c, p*stride_h - pre_h + r*dil_h,
 *                                                     q*stride_w - pre_w + s*dil_w]
 *
 * (X is 0 outside the image), (r',s') = (r,s), or (R-1-r,S-1-s) in mode 1.
 * x is [N,C,H,W] int8, dy [N,K,P,Q] int8, dw [K,C,R,S] int32; dY's dims must
 * be the forward output dims.  Summed over n, then p, then q; 64-bit sums.
 */
int oracle_conv_wgrad(const int8_t *x, const int64_t xdims[4], const int64_t xstr[4],
                      const int8_t *dy, const int64_t dydims[4], const int64_t dystr[4],
                      int32_t *dw, const int64_t dwdims[4], const int64_t dwstr[4],
                      const int64_t pre[2], const int64_t post[2],
                      const int64_t stride[2], const int64_t dil[2], int mode, int nthreads)
{
    int64_t fwd[4];
    if (!xstr || !dydims || !dystr || !dwdims || !dwstr)
        return ORACLE_ERR_ARG;
    int rc = oracle_out_dims(xdims, dwdims, pre, post, stride, dil, fwd);
    if (rc != ORACLE_OK)
        return rc;
    for (int i = 0; i < 4; ++i)
        if (dydims[i] != fwd[i])
            return ORACLE_ERR_OUT_DIMS;
    if ((!x && oracle_elems(xdims) > 0) || (!dy && oracle_elems(dydims) > 0) ||
        (!dw && oracle_elems(dwdims) > 0))
        return ORACLE_ERR_ARG;

    const int64_t N = xdims[0], H = xdims[2], W = xdims[3];
    const int64_t K = dwdims[0], C = dwdims[1], R = dwdims[2], S = dwdims[3];
    const int64_t P = dydims[2], Q = dydims[3];
    int overflow = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : overflow)
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t ci = 0; ci < C; ++ci) {
            for (int64_t r = 0; r < R; ++r) {
                for (int64_t s = 0; s < S; ++s) {
                    int64_t acc = 0;
                    for (int64_t n = 0; n < N; ++n) {
                        for (int64_t p = 0; p < P; ++p) {
                            const int64_t h = p * stride[0] - pre[0] + r * dil[0];
                            if (h < 0 || h >= H)
                                continue;
                            for (int64_t q = 0; q < Q; ++q) {
                                const int64_t wc = q * stride[1] - pre[1] + s * dil[1];
                                if (wc < 0 || wc >= W)
                                    continue;
                                acc += (int64_t)dy[n * dystr[0] + k * dystr[1] + p * dystr[2] + q * dystr[3]] *
                                       (int64_t)x[n * xstr[0] + ci * xstr[1] + h * xstr[2] + wc * xstr[3]];
                            }
                        }
                    }
                    if (acc < INT32_MIN || acc > INT32_MAX)
                        overflow = 1;
                    const int64_t gr = mode ? R - 1 - r : r, gs = mode ? S - 1 - s : s;
                    dw[k * dwstr[0] + ci * dwstr[1] + gr * dwstr[2] + gs * dwstr[3]] =
                        (int32_t)(uint32_t)(uint64_t)acc;
                }
            }
        }
    }
    return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;
}

/* Threads an OpenMP parallel region gets by default (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
