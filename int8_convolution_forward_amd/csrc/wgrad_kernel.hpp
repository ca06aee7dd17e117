// Weight gradient read in place from channels-last operands on gfx950
// (CDNA4).
//
// dW[k, c, r, s] = sum over output pixels j = (n, p, q) of dY[j, k] *
// X[n, p*st_h - pre_h + r*dil_h, q*st_w - pre_w + s*dil_w, c] (X is 0 outside
// the image): for each filter tap a matrix product whose reduction runs over
// the pixels.  Channels-last loss and image store each pixel's channels
// contiguously, i.e. both operands come reduction-major ("k-major": a row per
// pixel, the GEMM's M or N dimension along the row).  The kernel stages 64
// pixels of both per step in LDS exactly as they lie in memory (the image row
// of pixel j is the pixel tap (r, s) of output pixel j reads, or zeros in the
// padding) and builds the MFMA fragments with transposing LDS reads
// (ds_read_b64_tr_b8), so neither operand is repacked.  For a 1x1 filter at
// stride 1 without padding (TAPS false) the image row of pixel j is pixel j
// itself and no index arithmetic is needed.
//
// Tile TM x TN of one tap of dW (TM loss channels k, TN image channels c),
// four waves 2 x 2; workgroup x = tap * tiles + tile; the pixels split over
// gridDim.y (split z runs steps [z*kchunk, (z+1)*kchunk)) and each split
// stores its partial sums into its own copy of dW, which a reduction kernel
// adds (integer adds: the sum does not depend on their order).
#pragma once

#include "kernel_common.hpp"

namespace convi8 {

struct WgradInPlaceArgs {
    const int8_t *dy;     // loss: pixel j's K channels at dy + j*dy_pitch
    const int8_t *x;      // image: pixel j's C channels at x + j*x_pitch
    int32_t *out;         // dW, or partial copy 0: (k, c) at out[k*oK + c*oC]
    int rows;             // pixels N*P*Q
    int K, C;
    int dy_pitch, x_pitch;   // bytes from one pixel to the next (multiples of 16)
    int dy_range, x_range;   // bytes the two buffer resources cover
    int oK, oC;              // element strides of dW
    int out_range;           // bytes of one copy of dW
    int tiles_n;             // tiles along C
    int nsteps;              // ceil(rows / 64)
    int kchunk;              // steps per split
    long long part_stride;   // elements from one partial copy to the next
    // taps (TAPS): pixel j = (n, p, q) of the output, tap (r, s) reads image
    // pixel (n, p*st_h + r*dil_h - pre_h, q*st_w + s*dil_w - pre_w)
    int tiles;               // tiles of one tap
    int S;                   // filter width (tap = r*S + s)
    int R;
    int PQ, Q;
    float inv_pq, inv_q;     // 1/PQ, 1/Q rounded to float (fdiv)
    int H, W;
    int sN, sH, sW;          // image strides in bytes (channel stride 1)
    int st_h, st_w, dil_h, dil_w, pre_h, pre_w;
    int oR, oS;              // element strides of dW along r and s
    int flip;                // true convolution: tap (r, s) goes to (R-1-r, S-1-s)
};

template <int TM, int TN, int NS, bool TAPS>
__global__ __launch_bounds__(256) void wgrad_inplace_kernel(WgradInPlaceArgs a)
{
    constexpr int NW = 4;                    // waves, 2 x 2
    constexpr int BK = 64;                   // pixels per step
    constexpr int GB = NW * 1024;            // bytes of one workgroup-wide load
    constexpr int AL = TM * BK / GB;         // loss loads per thread per step
    constexpr int BL = TN * BK / GB;         // image loads per thread per step
    constexpr int A_BYTES = TM * BK, B_BYTES = TN * BK;
    constexpr int SLOT = A_BYTES + B_BYTES;
    constexpr int FM = TM / 2 / 32, FN = TN / 2 / 32;
    constexpr int KS = BK / 32;              // MFMA k-steps per step
    constexpr int L = AL + BL;
    static_assert(TM == 128 && TN == 128, "rows of eight 16-byte chunks (the swizzle below)");
    static_assert(NS >= 3 && (NS - 2) * L < 64, "ring depth");

    __shared__ __attribute__((aligned(1024))) int8_t lds[NS * SLOT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = TAPS ? (int)(blockIdx.x % (unsigned)a.tiles) : (int)blockIdx.x;
    const int tap = TAPS ? (int)(blockIdx.x / (unsigned)a.tiles) : 0;
    const int m0 = (tile / a.tiles_n) * TM;
    const int n0 = (tile % a.tiles_n) * TN;
    const int tr = TAPS ? tap / a.S : 0, ts = TAPS ? tap - tr * a.S : 0;
    const int dh = tr * a.dil_h - a.pre_h, dw = ts * a.dil_w - a.pre_w;
    const int s0 = (int)blockIdx.y * a.kchunk;
    const int ns = max(min(a.kchunk, a.nsteps - s0), 0);
    const v4i dy_rsrc = make_rsrc(a.dy, a.dy_range);
    const v4i x_rsrc = make_rsrc(a.x, a.x_range);
    const unsigned lds0 = lds_address(lds);

    // Load i of this thread fills LDS row kr = (i*NW + wave)*8 + lane/8 (one
    // pixel) at 16-byte position lane%8 (a wave-wide load writes 1 KiB
    // contiguously), with the row's global chunk (lane%8) ^ (kr%8): the eight
    // rows a transposing read spans then sit at eight different positions.
    int a_off[AL], b_off[BL], a_row[AL], b_row[BL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int kr = (i * NW + wave) * 8 + (lane >> 3);
        const int col = m0 + (((lane & 7) ^ (kr & 7)) << 4);
        a_row[i] = kr;
        a_off[i] = col < a.K ? kr * a.dy_pitch + col : -1;
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        const int kr = (i * NW + wave) * 8 + (lane >> 3);
        const int col = n0 + (((lane & 7) ^ (kr & 7)) << 4);
        b_row[i] = kr;
        b_off[i] = col < a.C ? (TAPS ? col : kr * a.x_pitch + col) : -1;
    }
    // step s (local) into ring slot s % NS; pixels past the last and steps
    // past the split read zeros (out-of-range offsets)
    auto issue = [&](int s) {
        const unsigned slot = lds0 + (unsigned)((s % NS) * SLOT);
        const int j0 = (s0 + s) * BK;
        const bool live = s < ns;
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const bool ok = live && a_off[i] >= 0 && j0 + a_row[i] < a.rows;
            load16_to_lds(dy_rsrc, slot + i * GB + wave * 1024, ok ? a_off[i] + j0 * a.dy_pitch : kOutOfRange);
        }
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            const int j = j0 + b_row[i];
            bool ok = live && b_off[i] >= 0 && j < a.rows;
            int off;
            if constexpr (TAPS) {
                // the image pixel tap (r, s) of output pixel j reads
                const int n = fdiv(j, a.PQ, a.inv_pq);
                const int rem = j - n * a.PQ;
                const int p = fdiv(rem, a.Q, a.inv_q);
                const int h = p * a.st_h + dh, w = (rem - p * a.Q) * a.st_w + dw;
                ok = ok && (unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W;
                off = n * a.sN + h * a.sH + w * a.sW + b_off[i];
            } else {
                off = b_off[i] + j0 * a.x_pitch;
            }
            load16_to_lds(x_rsrc, slot + A_BYTES + i * GB + wave * 1024, ok ? off : kOutOfRange);
        }
    };

    // Fragment reads: ds_read_b64_tr_b8 hands lane i of each 16-lane group
    // byte i % 8 of the eight rows that lanes 2b + i / 8 (b = 0..7) address.
    // Lane t addresses pixel row kr + (t%16)/2 at channel col + 8 (t & 1), so
    // lane i of the group receives pixels kr .. kr+7 of channel col + i; a
    // second read 8 rows down gives pixels kr+8 .. kr+15: together the 16
    // reduction values an MFMA lane holds (channel lane % 32, pixels
    // 16 (lane / 32) .. +16 of the k-step).
    const int wm = (wave >> 1) * (TM / 2), wn = (wave & 1) * (TN / 2);
    int a_lane[FM][KS], b_lane[FN][KS];
    {
        const int j = lane & 15;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int kr = ks * 32 + (lane >> 5) * 16 + (j >> 1);
#pragma unroll
            for (int x = 0; x < FM; ++x) {
                const int col = wm + x * 32 + ((lane >> 4) & 1) * 16 + (j & 1) * 8;
                a_lane[x][ks] = kr * TM + (((col >> 4) ^ (kr & 7)) << 4) + (col & 8);
            }
#pragma unroll
            for (int y = 0; y < FN; ++y) {
                const int col = wn + y * 32 + ((lane >> 4) & 1) * 16 + (j & 1) * 8;
                b_lane[y][ks] = A_BYTES + kr * TN + (((col >> 4) ^ (kr & 7)) << 4) + (col & 8);
            }
        }
    }
    auto frag = [&](int base) {
        const int8_t *p = &lds[base];
        const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)p);
        const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(p + 8 * 128));
        return v4i{lo.x, lo.y, hi.x, hi.y};
    };

    v16i acc[FM][FN];
#pragma unroll
    for (int x = 0; x < FM; ++x)
#pragma unroll
        for (int y = 0; y < FN; ++y)
            acc[x][y] = v16i{};

#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        issue(s);
    for (int s = 0; s < ns; ++s) {
        // step s has landed (the NS-2 later ones may be in flight), and every
        // wave is done with slot (s-1) % NS, which step s+NS-1 refills
        wait_vm_lgkm0<(NS - 2) * L>();
        __builtin_amdgcn_s_barrier();
        issue(s + NS - 1);
        const int sb = (s % NS) * SLOT;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            v4i af[FM], bf[FN];
#pragma unroll
            for (int x = 0; x < FM; ++x)
                af[x] = frag(sb + a_lane[x][ks]);
#pragma unroll
            for (int y = 0; y < FN; ++y)
                bf[y] = frag(sb + b_lane[y][ks]);
#pragma unroll
            for (int x = 0; x < FM; ++x)
#pragma unroll
                for (int y = 0; y < FN; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[x], bf[y], acc[x][y], 0, 0, 0);
        }
    }
    // the trailing (out-of-range) loads land before the LDS is released
    wait_vm_lgkm0<0>();

    // 32x32 accumulator layout: lane l, value v -> row 8*(v/4) + 4*(l/32) +
    // v%4 (loss channel k), column l%32 (image channel c)
    const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.out + (long long)blockIdx.y * a.part_stride), (short)0, a.out_range, kRsrcWord3);
    const int tap_off = TAPS ? (a.flip ? a.R - 1 - tr : tr) * a.oR + (a.flip ? a.S - 1 - ts : ts) * a.oS : 0;
#pragma unroll
    for (int x = 0; x < FM; ++x)
#pragma unroll
        for (int y = 0; y < FN; ++y) {
            const int c = n0 + wn + y * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int k = m0 + wm + x * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int off = (k < a.K && c < a.C) ? (k * a.oK + c * a.oC + tap_off) * 4 : kOutOfRange;
                __builtin_amdgcn_raw_buffer_store_b32(acc[x][y][v], out_rsrc, off, 0, kOutStoreDefault);
            }
        }
}

}  // namespace convi8
