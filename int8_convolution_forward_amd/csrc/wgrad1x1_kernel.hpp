// Weight gradient of a 1x1 convolution of stride 1 without padding, read in
// place from channels-last operands on gfx950 (CDNA4).
//
// With a 1x1 filter every output pixel j = (n, p, q) reads the input pixel at
// the same place, so dW[k, c] = sum_j dY[j, k] * X[j, c]: a matrix product
// whose reduction runs over the pixels.  Channels-last loss and image store
// each pixel's channels contiguously, i.e. both operands come reduction-major
// ("k-major": a row per pixel, the GEMM's M or N dimension along the row).
// The kernel stages 64 pixels of both per step in LDS exactly as they lie in
// memory and builds the MFMA fragments with transposing LDS reads
// (ds_read_b64_tr_b8), so neither operand is repacked and each byte of the
// loss and the image is read from HBM about once per tile column or row.
//
// Tile TM x TN of dW (TM loss channels k, TN image channels c), four waves
// 2 x 2; the pixels split over gridDim.y (split z runs steps [z*kchunk,
// (z+1)*kchunk)) and each split stores its partial sums into its own copy
// of dW, which a reduction kernel adds (integer adds: the sum does not depend
// on their order).
#pragma once

#include "kernel_common.hpp"

namespace convi8 {

struct Wgrad1x1Args {
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
};

template <int TM, int TN, int NS>
__global__ __launch_bounds__(256) void wgrad1x1_kernel(Wgrad1x1Args a)
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
    const int m0 = (int)(blockIdx.x / (unsigned)a.tiles_n) * TM;
    const int n0 = (int)(blockIdx.x % (unsigned)a.tiles_n) * TN;
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
        b_off[i] = col < a.C ? kr * a.x_pitch + col : -1;
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
            const bool ok = live && b_off[i] >= 0 && j0 + b_row[i] < a.rows;
            load16_to_lds(x_rsrc, slot + A_BYTES + i * GB + wave * 1024,
                          ok ? b_off[i] + j0 * a.x_pitch : kOutOfRange);
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
#pragma unroll
    for (int x = 0; x < FM; ++x)
#pragma unroll
        for (int y = 0; y < FN; ++y) {
            const int c = n0 + wn + y * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int k = m0 + wm + x * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int off = (k < a.K && c < a.C) ? (k * a.oK + c * a.oC) * 4 : kOutOfRange;
                __builtin_amdgcn_raw_buffer_store_b32(acc[x][y][v], out_rsrc, off, 0, kOutStoreDefault);
            }
        }
}

}  // namespace convi8
