// Layout normalisation: any strided int8 [A, C, Y, X] tensor -> packed
// [A, Y, X, Cp] with the channels innermost and zero-filled up to Cp (a
// multiple of 16).  The zero channels add nothing to any sum, so the packed
// copy convolves exactly like the original.  Used for images (A=N, Y=H, X=W)
// and filters (A=K, Y=R, X=S) whose layout the implicit-GEMM kernel cannot
// read with aligned 16-byte channel vectors (NCHW, strided views, C % 16 != 0).
//
// The memory layout decides the cost here ("Building a From-Scratch INT8
// Strided Convolution Kernel", "Key Takeaways").  A workgroup moves a tile of
// 64 positions x 64 channels: 64 x-positions of one (a, y) row, or, for a
// transposed view whose first dim is the contiguous one, 64 a-values at one
// (y, x).  When one walk (along x, along c, or along a) has a small stride
// (at most 8 bytes), the tile's 64 lines along that walk are read as aligned
// 16-byte vectors into LDS (every vector holds at least one wanted byte, so
// no vector leaves the pages the tensor occupies), and the wanted bytes are
// picked out of LDS; otherwise every element is read on its own.  Each
// thread then writes one 16-byte vector of 16 consecutive channels.  One
// launch serves up to two tensors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernel_common.hpp"

namespace convi8 {

enum RepackMode : int {
    kRepackXFast = 0,   // stride along x <= 8 bytes: lines along x
    kRepackCFast = 1,   // stride along c <= 8 bytes: lines along c
    kRepackGather = 2,  // none: one load per element
    kRepackAFast = 3,   // stride along a <= 8 bytes: tiles of 64 a-values at one (y, x),
                        // lines along a (a transposed view)
};

struct RepackJob {
    const int8_t *src;               // element (0,0,0,0)
    long long s0, s1, sy, sx;        // element strides of [A, C, Y, X]
    int A, C, Y, X, Cp;
    int mode;
    int tiles_x, tiles_c;            // 64-wide tiles along x (along a for kRepackAFast) and Cp
    int pp_shift;                    // kRepackAFast: log2 of the (y, x) positions one tile
                                     // covers (Cp 16: 4 positions, Cp 32: 2; else 1)
    int tiles;                       // A*Y (or ceil(Y*X / positions)) * tiles_x * tiles_c
    Divisor d_tc, d_tx, d_o;         // tiles_c, tiles_x, and X (kRepackAFast) or Y
    int8_t *dst;                     // packed [A][Y][X][Cp]
};

constexpr int kRepackMaxJobs = 8;

// NJ job slots: 2 for a convolution's image and filter, kRepackMaxJobs for
// the filter views of a strided layer's data-gradient phases (a smaller
// argument block keeps the common launch as cheap as it can be)
template <int NJ>
struct RepackArgs {
    RepackJob job[NJ];               // tiles of job i follow those of jobs 0 .. i-1
    int njobs;
};

// LDS bytes per line for a largest line stride of STEP bytes: 63 strides,
// one byte, up to 15 bytes of alignment, rounded up to whole vectors
template <int STEP>
constexpr int repack_line()
{
    return (15 + 63 * STEP + 1 + 15) / 16 * 16;
}

template <int STEP, int NJ>
__global__ __launch_bounds__(256) void repack_to_channels_last_kernel(RepackArgs<NJ> args)
{
    constexpr int kRepackLine = repack_line<STEP>();
    __shared__ __attribute__((aligned(16))) int8_t raw[64 * kRepackLine];

    unsigned bid = blockIdx.x;               // each job has fewer than 2^31 tiles
    int ji = 0;                              // uniform: the job this workgroup serves
    while (ji + 1 < args.njobs && bid >= (unsigned)args.job[ji].tiles) {
        bid -= (unsigned)args.job[ji].tiles;
        ++ji;
    }
    const RepackJob &j = args.job[ji];

    const int tid = threadIdx.x;
    const bool af = j.mode == kRepackAFast;
    // An a-fast tile with few channels (Cp 16 or 32) covers 4 or 2
    // consecutive (y, x) positions: its 64 LDS lines are 16 or 32 channel
    // lines per position, and each output vector (16 channels) is one of a
    // position's.  Every other tile covers one outer index.
    const int pps = af ? j.pp_shift : 0;
    const int lshift = 6 - pps;              // log2 of the lines per outer index
    // tile index -> (outer, x-tile, c-tile) and outer -> (o_hi, o_lo) with
    // the host's magic-number divisors (no division chain before the loads)
    const int q1 = udiv((int)bid, j.d_tc);
    const int ct = (int)bid - q1 * j.tiles_c;
    const int outer_t = udiv(q1, j.d_tx);
    const int pt = q1 - outer_t * j.tiles_x;
    const int outer0 = outer_t << pps;       // first outer index of the tile
    const int nouter = af ? j.Y * j.X : j.A * j.Y;
    // x-tiles: outer = (a, y), the tile walks x; a-tiles: outer = (y, x), it walks a
    auto row_of = [&](int outer) {
        const int o_hi = udiv(outer, j.d_o);
        const int o_lo = outer - o_hi * (af ? j.X : j.Y);
        const int ai = af ? 0 : o_hi, yi = af ? o_hi : o_lo, xi = af ? o_lo : 0;
        return j.src + (long long)ai * j.s0 + (long long)yi * j.sy + (long long)xi * j.sx;
    };
    const int x0 = pt * 64, c0 = ct * 64;    // x0: first x (or first a) of the tile
    const int xn = min(64, (af ? j.A : j.X) - x0);  // positions in this tile
    const int cn = max(0, min(64, j.C - c0)); // real channels in this tile (the rest pad with zeros)
    const long long pstride = af ? j.s0 : j.sx;  // stride between the tile's positions

    // output vector of this thread: position x0 + xl of outer index
    // outer0 + ps, channels c0 + cg*16 .. +16
    const int xl = tid >> 2, cq = tid & 3;
    const int ps = cq >> (2 - pps), cg = cq & ((4 >> pps) - 1);
    const bool out_ok = xl < xn && outer0 + ps < nouter && c0 + cg * 16 < j.Cp;
    const int8_t *row = row_of(outer0 + (out_ok ? ps : 0));
    int v[4] = {0, 0, 0, 0};

    if (j.mode == kRepackGather) {
        if (out_ok) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int cl = cg * 16 + i;
                if (cl < cn)
                    v[i >> 2] |= (int)(uint8_t)row[(long long)(c0 + cl) * j.s1 + (long long)(x0 + xl) * pstride] << (8 * (i & 3));
            }
        }
    } else {
        // line l of the tile: channel c0+l (x-fast, a-fast) or position x0+l
        // (c-fast); it runs over the other index with stride `step`.  Four
        // threads share a line and fetch every fourth of its aligned vectors.
        // With several outer indices per tile, line l is channel line
        // l mod 2^lshift of outer index outer0 + (l >> lshift).
        const bool xf = j.mode != kRepackCFast;
        const long long lstride = xf ? j.s1 : pstride;
        const int step = (int)(xf ? pstride : j.s1);
        const int nlines = xf ? cn : xn;
        const int nalong = xf ? xn : cn;
        const long long lead_off = (long long)(xf ? x0 : c0) * step + (long long)(xf ? c0 : x0) * lstride;
        const int8_t *line0 = row + lead_off;   // line 0 of the thread's output outer index
        {
            const int l = tid >> 2, sub = tid & 3;
            const int lp = l >> lshift, ll = l & ((1 << lshift) - 1);
            if (ll < nlines && nalong > 0 && outer0 + lp < nouter) {
                const int8_t *first = (pps ? row_of(outer0 + lp) : row) + lead_off + (long long)ll * lstride;
                const uintptr_t a0 = (uintptr_t)first & ~(uintptr_t)15;
                const int nv = (int)(((((uintptr_t)first & 15) + (uintptr_t)(nalong - 1) * step) >> 4) + 1);
                for (int v16 = sub; v16 < nv; v16 += 4)
                    *(int4 *)&raw[l * kRepackLine + v16 * 16] = *(const int4 *)(a0 + (uintptr_t)v16 * 16);
            }
        }
        __syncthreads();
        if (out_ok) {
            // The offset of line l's first byte within its first aligned
            // vector (only the low four address bits matter) steps by the
            // line stride from one line to the next, and the byte of channel
            // i sits at a fixed distance from the previous one.  All sixteen
            // reads stay inside their lines (the lines past C hold whatever
            // the buffer held), so they go out unconditionally, back to back,
            // and the bytes past C are masked off afterwards.
            const unsigned b0 = (unsigned)(uintptr_t)line0, ls = (unsigned)lstride;
            if (xf) {
                // line cg*16 + i of outer index outer0 + ps, position xl
                unsigned lead = (b0 + (unsigned)(cg * 16) * ls) & 15u;
                const int8_t *p = &raw[((ps << lshift) + cg * 16) * kRepackLine + xl * step];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    v[i >> 2] |= (int)(uint8_t)p[i * kRepackLine + (int)lead] << (8 * (i & 3));
                    lead = (lead + ls) & 15u;
                }
            } else {
                // line xl, position cq*16 + i
                const unsigned lead = (b0 + (unsigned)xl * ls) & 15u;
                const int8_t *p = &raw[xl * kRepackLine + (int)lead + cq * 16 * step];
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    v[i >> 2] |= (int)(uint8_t)p[i * step] << (8 * (i & 3));
            }
            const int nvalid = min(max(cn - cg * 16, 0), 16);   // real channels of this vector
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int nb = min(max(nvalid - 4 * w, 0), 4);
                v[w] &= nb == 4 ? -1 : (int)((1u << (8 * nb)) - 1u);
            }
        }
    }
    if (out_ok) {
        // packed [A][Y][X][Cp]: outer index o is (y, x) of a-tiles, (a, y) of x-tiles
        const long long o = outer0 + ps;
        const long long pos = af ? (long long)(x0 + xl) * nouter + o : o * j.X + x0 + xl;
        int8_t *d = j.dst + pos * j.Cp + c0 + cg * 16;
        // non-temporal: the packed copy is read by the next kernel, after the
        // write-back at this kernel's end, not from this CU's caches
        typedef int i32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(i32x4{v[0], v[1], v[2], v[3]}, (i32x4 *)d);
    }
}

}  // namespace convi8
