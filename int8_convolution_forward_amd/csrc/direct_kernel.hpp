// Direct convolution for tiny problems: one thread per output element, the
// operands read in place through their element strides (any layout, any
// alignment), the sum of int8 products in int32 (cuDNN "Convolutions" page,
// "Convolution Fprop"; the naive loop of "Building a From-Scratch INT8
// Strided Convolution Kernel", step 2, with zero padding for taps outside the
// image).  A problem this small is bound by launches, not by arithmetic:
// reading the operands in place saves the repack launch the implicit-GEMM
// kernels need for layouts that are not channel-innermost.
#pragma once

#include "kernel_common.hpp"

namespace convi8 {

struct DirectArgs {
    const int8_t *x;           // image element (0,0,0,0)
    const int8_t *w;           // filter element (0,0,0,0)
    void *y;                   // output element (0,0,0,0): int32, or int8 with q8
    long long xs[4], ws[4];    // element strides [N,C,H,W], [K,C,R,S]
    long long ys[4];           // output element strides [N,K,P,Q]
    long long total;           // N*K*P*Q
    int K, C, R, S, P, Q, H, W;
    int preH, preW, strH, strW, dilH, dilW;
    int conv_mode;             // 1: tap (r, s) reads filter tap (R-1-r, S-1-s)
    int flip_out;              // 1: output (p, q) goes to (P-1-p, Q-1-q)
    const float *q_scale;      // requantisation (q8): per-channel scale or q_alpha
    const float *q_bias;
    float q_alpha;
    int q_relu;
    int q8;
};

template <int = 0>   // a template: instantiated only where it is launched
__global__ __launch_bounds__(256) void conv_direct_kernel(DirectArgs a)
{
    const long long step = (long long)gridDim.x * 256;
    for (long long o = (long long)blockIdx.x * 256 + threadIdx.x; o < a.total; o += step) {
        // o = ((n*K + k)*P + p)*Q + q
        long long r0 = o;
        const int q = (int)(r0 % a.Q);
        r0 /= a.Q;
        const int p = (int)(r0 % a.P);
        r0 /= a.P;
        const int k = (int)(r0 % a.K);
        const long long n = r0 / a.K;
        const int8_t *xn = a.x + n * a.xs[0];
        const int8_t *wk = a.w + k * a.ws[0];
        int acc = 0;
        for (int r = 0; r < a.R; ++r) {
            const int h = p * a.strH - a.preH + r * a.dilH;
            if ((unsigned)h >= (unsigned)a.H)
                continue;
            const int fr = a.conv_mode ? a.R - 1 - r : r;
            for (int s = 0; s < a.S; ++s) {
                const int wc = q * a.strW - a.preW + s * a.dilW;
                if ((unsigned)wc >= (unsigned)a.W)
                    continue;
                const int fs = a.conv_mode ? a.S - 1 - s : s;
                const int8_t *xp = xn + h * a.xs[2] + wc * a.xs[3];
                const int8_t *wp = wk + fr * a.ws[2] + fs * a.ws[3];
                for (int c = 0; c < a.C; ++c)
                    acc += (int)xp[c * a.xs[1]] * (int)wp[c * a.ws[1]];
            }
        }
        const int po = a.flip_out ? a.P - 1 - p : p;
        const int qo = a.flip_out ? a.Q - 1 - q : q;
        const long long off = n * a.ys[0] + k * a.ys[1] + po * a.ys[2] + qo * a.ys[3];
        if (a.q8) {
            const float sc = a.q_scale ? a.q_scale[k] : a.q_alpha;
            const float bi = a.q_bias ? a.q_bias[k] : 0.0f;
            ((int8_t *)a.y)[off] = (int8_t)requant_i8(acc, sc, bi, a.q_relu != 0);
        } else {
            ((int32_t *)a.y)[off] = acc;
        }
    }
}

}  // namespace convi8
