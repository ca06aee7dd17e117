// Implicit-GEMM INT8 convolution forward for gfx950 (CDNA4).
//
// The convolution of the cuDNN "Convolutions" page ("Convolution Fprop") is
// computed as a matrix product without materialising the unrolled image:
//
//   rows    m = (n, p, q)        M = N*P*Q output pixels
//   columns k                    K output channels
//   inner   (r, s, c)            C*R*S products per output
//
// The image is read channel-innermost (N,H,W,C with C a multiple of 16 and
// every 16-channel run 16-byte aligned), the filter as K,R,S,C.  A 16-byte
// chunk of the inner dimension is then 16 consecutive channels of one pixel
// at one filter tap, which is one aligned vector load.  Where the tap falls in
// the padding (or the row is past M, the column past K, the chunk past the
// end of C*R*S) the load is given an offset beyond the buffer's range, and the
// buffer unit returns zeros: padding costs no branch and no extra traffic.
//
// Per workgroup (256 threads = 4 waves in a 2x2 grid): a TM x TN output tile.
// Each stage moves BK bytes of the inner dimension for every tile row and
// column through registers into one of two LDS buffers (double buffering, one
// barrier per stage), while the waves multiply the other buffer with
// v_mfma_i32_32x32x32_i8.  LDS rows are BK bytes with 16-byte chunks permuted
// by an XOR of the row index so that the MFMA operand reads (32 rows, one
// chunk) and the stores (consecutive chunks) are free of bank conflicts.
//
// Inner-dimension order: "blocked" when C/16 is a multiple of the chunks per
// stage: stage = (channel block, r, s) with (r, s) varying fastest, so the
// R*S stages that reuse one channel block of the same pixels run back to
// back and hit in cache.  Otherwise "flat": chunks in (r, s, c) order, a stage
// may straddle taps, and the last stage is padded with zero chunks.
//
// Epilogue: int32 results go straight from the accumulators to the output
// through its element strides.  The MFMA output column (the lane index) is
// made the output's contiguous dimension: output channels for an
// channel-innermost output, pixels for a pixel-innermost (N,K,P,Q) one, by
// swapping the MFMA operands (PIX_J).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convi8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Buffer offset that always lies outside a resource (ranges are < 2^31).
constexpr int kOutOfRange = (int)0x80000000u;
// Buffer resource word 3 for gfx9-family raw buffer access (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;

struct IgemmArgs {
    const int8_t *img;   // image, channel-innermost; (0,0,0,0) at img
    const int8_t *flt;   // filter K,R,S,C with C innermost
    int32_t *out;        // output element (0,0,0,0)
    int img_range;       // bytes addressable from img (buffer range)
    int flt_range;       // bytes addressable from flt
    int N, H, W, C;      // C: channels as stored (multiple of 16)
    int sN, sH, sW;      // image strides in bytes (channel stride is 1)
    int K, R, S;
    int fK, fR, fS;      // filter strides in bytes (channel stride is 1)
    int P, Q, PQ, M;     // M = N*P*Q
    int strH, strW, dilH, dilW, padH, padW;
    long long oN, oK, oP, oQ;  // output strides in elements
    int nstages;         // stages of BK bytes of the inner dimension
    int cc;              // C / 16
    int blocked;         // 1: stage = (channel block, r, s); 0: flat (r, s, c) order
    int tiles_n;         // column tiles
    int tiles;           // total tiles
};

__device__ __forceinline__ int swizzle_chunk(int row, int chunk, int bk)
{
    // 64-byte rows: 4 chunks; 128-byte rows: 8 chunks.  The XOR keeps any 8
    // (32 banks) or 16 (64 banks) consecutive rows' reads of one logical chunk
    // on distinct banks.
    if (bk == 64)
        return chunk ^ (((row >> 1) ^ (row >> 2)) & 3);
    return chunk ^ ((row ^ (row >> 1)) & 7);
}

// Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous
// run of tiles (column tiles of one row tile are adjacent) so that the image
// rows a run reads stay in that XCD's L2.
__device__ __forceinline__ int xcd_tile(int bid, int tiles)
{
    const int per = tiles >> 3, rem = tiles & 7;
    const int xcd = bid & 7, idx = bid >> 3;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

template <int TM, int TN, int BK, bool PIX_J>
__global__ __launch_bounds__(256) void conv_igemm_kernel(IgemmArgs a)
{
    constexpr int CPS = BK / 16;            // 16-byte chunks per row per stage
    constexpr int RPP = 256 / CPS;          // rows covered by one pass of the workgroup
    constexpr int AL = TM / RPP;            // image-row loads per thread per stage
    constexpr int BL = TN / RPP;            // filter-row loads per thread per stage
    constexpr int WM = TM / 2, WN = TN / 2; // wave tile
    constexpr int FM = WM / 32, FN = WN / 32;
    static_assert(AL >= 1 && BL >= 1 && FM >= 1 && FN >= 1, "tile too small");
    static_assert(TM % RPP == 0 && TN % RPP == 0, "tile rows must fill load passes");

    __shared__ __attribute__((aligned(16))) int8_t lds_a[2][TM * BK];
    __shared__ __attribute__((aligned(16))) int8_t lds_b[2][TN * BK];
    __shared__ long long out_row[TM];

    const int tid = threadIdx.x;
    const int tile = xcd_tile(blockIdx.x, a.tiles);
    const int m0 = (tile / a.tiles_n) * TM;
    const int n0 = (tile % a.tiles_n) * TN;

    // ---- per-row addressing, computed once ------------------------------
    const int j = tid % CPS;       // this thread's chunk within a stage
    const int rb = tid / CPS;      // this thread's first row
    int a_h0[AL], a_w0[AL], a_off[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int m = m0 + rb + i * RPP;
        if (m < a.M) {
            const int n = m / a.PQ;
            const int rem = m - n * a.PQ;
            const int p = rem / a.Q;
            const int q = rem - p * a.Q;
            a_h0[i] = p * a.strH - a.padH;
            a_w0[i] = q * a.strW - a.padW;
            a_off[i] = n * a.sN + a_h0[i] * a.sH + a_w0[i] * a.sW;
        } else {
            a_h0[i] = -0x40000000;  // never inside the image
            a_w0[i] = 0;
            a_off[i] = 0;
        }
    }
    for (int i = tid; i < TM; i += 256) {
        const int m = m0 + i;
        long long o = -1;
        if (m < a.M) {
            const int n = m / a.PQ;
            const int rem = m - n * a.PQ;
            const int p = rem / a.Q;
            const int q = rem - p * a.Q;
            o = n * a.oN + p * a.oP + q * a.oQ;
        }
        out_row[i] = o;
    }
    int b_off[BL];
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        const int k = n0 + rb + i * RPP;
        b_off[i] = k < a.K ? k * a.fK : kOutOfRange;
    }

    // ---- inner-dimension position of this thread's chunk -----------------
    int r, s, c16;
    if (a.blocked) {
        r = 0; s = 0; c16 = j;
    } else {
        const int rs = j / (a.cc > 0 ? a.cc : 1);
        c16 = j - rs * a.cc;
        r = rs / a.S;
        s = rs - r * a.S;
    }
    int rdh = r * a.dilH, sdw = s * a.dilW;

    const __amdgpu_buffer_rsrc_t img_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.img, (short)0, a.img_range, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t flt_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.flt, (short)0, a.flt_range, kRsrcWord3);

    v4i ra[AL], rbv[BL];

    auto gload = [&]() {
        const bool chunk_ok = r < a.R;
        const int itoff = rdh * a.sH + sdw * a.sW + c16 * 16;
        const int ftoff = r * a.fR + s * a.fS + c16 * 16;
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int h = a_h0[i] + rdh, w = a_w0[i] + sdw;
            const bool ok = chunk_ok && (unsigned)h < (unsigned)a.H && (unsigned)w < (unsigned)a.W;
            ra[i] = __builtin_amdgcn_raw_buffer_load_b128(img_rsrc, ok ? a_off[i] + itoff : kOutOfRange, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            const bool ok = chunk_ok && b_off[i] != kOutOfRange;
            rbv[i] = __builtin_amdgcn_raw_buffer_load_b128(flt_rsrc, ok ? b_off[i] + ftoff : kOutOfRange, 0, 0);
        }
    };
    auto step_tap = [&]() {
        ++s;
        sdw += a.dilW;
        if (s == a.S) {
            s = 0;
            sdw = 0;
            ++r;
            rdh += a.dilH;
        }
    };
    auto advance = [&]() {
        if (a.blocked) {
            step_tap();
            if (r == a.R) {
                r = 0;
                rdh = 0;
                c16 += CPS;
            }
        } else {
            c16 += CPS;
            while (c16 >= a.cc && r < a.R) {
                c16 -= a.cc;
                step_tap();
            }
        }
    };
    auto lds_store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int row = rb + i * RPP;
            *(v4i *)&lds_a[buf][row * BK + swizzle_chunk(row, j, BK) * 16] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            const int row = rb + i * RPP;
            *(v4i *)&lds_b[buf][row * BK + swizzle_chunk(row, j, BK) * 16] = rbv[i];
        }
    };

    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = (wave >> 1) * WM;
    const int wn = (wave & 1) * WN;

    v16i acc[FM][FN];
#pragma unroll
    for (int x = 0; x < FM; ++x)
#pragma unroll
        for (int y = 0; y < FN; ++y)
            acc[x][y] = v16i{};

    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const int ch = ks * 2 + (lane >> 5);
            v4i af[FM], bf[FN];
#pragma unroll
            for (int x = 0; x < FM; ++x) {
                const int row = wm + x * 32 + (lane & 31);
                af[x] = *(const v4i *)&lds_a[buf][row * BK + swizzle_chunk(row, ch, BK) * 16];
            }
#pragma unroll
            for (int y = 0; y < FN; ++y) {
                const int row = wn + y * 32 + (lane & 31);
                bf[y] = *(const v4i *)&lds_b[buf][row * BK + swizzle_chunk(row, ch, BK) * 16];
            }
#pragma unroll
            for (int x = 0; x < FM; ++x)
#pragma unroll
                for (int y = 0; y < FN; ++y)
                    acc[x][y] = PIX_J
                        ? __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[y], af[x], acc[x][y], 0, 0, 0)
                        : __builtin_amdgcn_mfma_i32_32x32x32_i8(af[x], bf[y], acc[x][y], 0, 0, 0);
        }
    };

    if (a.nstages > 0) {
        gload();
        advance();
        lds_store(0);
    }
    __syncthreads();
    for (int it = 0; it < a.nstages; ++it) {
        const int cur = it & 1;
        const bool more = it + 1 < a.nstages;
        if (more) {
            gload();
            advance();
        }
        compute(cur);
        if (more)
            lds_store(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------
    // 32x32 accumulator layout: lane l, value v -> MFMA row 8*(v/4) + 4*(l/32) + v%4,
    // MFMA column l%32.  Rows come from the first MFMA operand.
#pragma unroll
    for (int x = 0; x < FM; ++x) {
#pragma unroll
        for (int y = 0; y < FN; ++y) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int mrow = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int mcol = lane & 31;
                const int prow = wm + x * 32 + (PIX_J ? mcol : mrow);
                const int kk = n0 + wn + y * 32 + (PIX_J ? mrow : mcol);
                const long long o = out_row[prow];
                if (o >= 0 && kk < a.K)
                    a.out[o + kk * a.oK] = acc[x][y][v];
            }
        }
    }
}

}  // namespace convi8
