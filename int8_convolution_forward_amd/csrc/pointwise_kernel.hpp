// 1x1 INT8 convolution forward for gfx950: a streaming matrix product.
//
// With a 1x1 filter the convolution of the cuDNN "Convolutions" page
// ("Convolution Fprop") reads every input pixel once and writes every output
// pixel once: out[m, k] = sum_c x[pixel(m), c] * w[k, c].  For the few output
// channels of a pointwise (bottleneck) layer that is far below the MFMA rate
// and bound by HBM: the job is to keep enough bytes in flight.
//
// Each wave owns up to TPW 32-pixel tiles, strided by the number of waves in
// the grid (so that every CU gets work when there are fewer than 4*TPW tiles
// per CU).  It fetches the whole filter
// once into registers (the B operand of v_mfma_i32_32x32x32_i8: lane l holds
// output channel y*32 + l%32, channels ks*32 + (l/32)*16 .. +16), issues the
// 16-byte image loads of all its tiles up front (lane l: pixel l%32 of the
// tile, the same channel split), then multiplies and stores tile by tile
// (INT32 sums, or their requantised INT8 values), so the stores of the first
// tiles overlap the loads of the last.  No LDS and no barrier.  Pixels outside the image (padding, stride) and channels past C
// load out of range, i.e. zeros.
#pragma once

#include "kernel_common.hpp"

namespace convi8 {

// POL: cache policy of the output stores (kOutStoreStream when the launch's
// output has unit channel stride, else kOutStoreDefault)
template <int FN, int KS, int TPW, int POL>
__global__ __launch_bounds__(256) void conv_pointwise_kernel(IgemmArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * 4;             // tile t of this wave: wave + t*nwaves
    const int chunk = (lane >> 5) * 16;           // channel offset of this lane within a k-step

    const __amdgpu_buffer_rsrc_t flt_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.flt, (short)0, a.flt_range, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t img_brsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.img, (short)0, a.img_range, kRsrcWord3);

    // ---- filter fragments, once -------------------------------------------
    v4i bfr[KS][FN];
#pragma unroll
    for (int y = 0; y < FN; ++y) {
        const int k = y * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = ks * 32 + chunk;
            const int off = (k < a.K && c < a.C) ? k * a.fK + c : kOutOfRange;
            bfr[ks][y] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(flt_rsrc, off, 0, 0));
        }
    }

    // ---- image fragments of all this wave's tiles ---------------------------
    v4i afr[TPW][KS];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int m = (wave + t * nwaves) * 32 + (lane & 31);
        int base = kOutOfRange;
        if (m < a.M) {
            const int n = udiv(m, a.d_pq);
            const int rem = m - n * a.PQ;
            const int p = udiv(rem, a.d_q);
            const int q = rem - p * a.Q;
            const int h = p * a.strH - a.padH, w = q * a.strW - a.padW;
            if ((unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W)
                base = n * a.sN + h * a.sH + w * a.sW;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = ks * 32 + chunk;
            const int off = (base != kOutOfRange && c < a.C) ? base + c : kOutOfRange;
            afr[t][ks] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(img_brsrc, off, 0, 0));
        }
    }

    // ---- multiply and store, tile by tile ----------------------------------
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.out, (short)0, a.out_range, kRsrcWord3);
    // stores with the cache policy the launch picked for this output layout
    auto st32 = [&](int v, int off) { __builtin_amdgcn_raw_buffer_store_b32(v, out_rsrc, off, 0, POL); };
    auto st8 = [&](unsigned char v, int off) { __builtin_amdgcn_raw_buffer_store_b8(v, out_rsrc, off, 0, POL); };
    const int mrow0 = 4 * (lane >> 5);
    const bool q8 = a.q8 != 0, relu = a.q_relu != 0;
    float qs[FN], qb[FN];                         // requantising epilogue, per column block
#pragma unroll
    for (int y = 0; y < FN; ++y) {
        qs[y] = 0.0f;
        qb[y] = 0.0f;
        if (q8)
            requant_params(a, y * 32 + (lane & 31), qs[y], qb[y]);
    }
    // fully unrolled (afr[t] must stay in registers): the loop body is long
    // enough that a plain unroll hint is not always taken
#pragma clang loop unroll(full)
    for (int t = 0; t < TPW; ++t) {
        v16i acc[FN];
#pragma unroll
        for (int y = 0; y < FN; ++y)
            acc[y] = v16i{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int y = 0; y < FN; ++y)
                acc[y] = __builtin_amdgcn_mfma_i32_32x32x32_i8(afr[t][ks], bfr[ks][y], acc[y], 0, 0, 0);
        // 32x32 accumulator layout: lane l, value v -> pixel row
        // 8*(v/4) + 4*(l/32) + v%4, output channel column l%32; the output's
        // pixels are equally spaced (pix_stride elements apart)
        const int mb = (wave + t * nwaves) * 32 + mrow0;
#pragma unroll
        for (int y = 0; y < FN; ++y) {
            const int kk = y * 32 + (lane & 31);
            const bool k_ok = kk < a.K;
            if (q8 && a.q8_pack) {
                // four rows of a lane -> one dword; a quad transposes them so
                // that lane 4j+t stores channels 4j..4j+3 of row t
                const int kq = kk & ~3;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    unsigned wv = 0;
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        wv |= ((unsigned)requant_i8(acc[y][4 * i + u], qs[y], qb[y], relu) & 0xFFu) << (8 * u);
                    wv = quad_transpose_bytes(wv, lane);
                    const int m = mb + 8 * i + (lane & 3);
                    const int off = (kq < a.K && m < a.M) ? m * a.pix_stride + kq : kOutOfRange;
                    st32((int)wv, off);
                }
            } else if (q8) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = mb + 8 * (v >> 2) + (v & 3);
                    const int off = (k_ok && m < a.M) ? m * a.pix_stride + kk * a.oK : kOutOfRange;
                    st8((unsigned char)requant_i8(acc[y][v], qs[y], qb[y], relu), off);
                }
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = mb + 8 * (v >> 2) + (v & 3);
                    const int off = (k_ok && m < a.M) ? (m * a.pix_stride + kk * a.oK) * 4 : kOutOfRange;
                    st32(acc[y][v], off);
                }
            }
        }
    }
}

}  // namespace convi8
