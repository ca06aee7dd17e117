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
// at one filter tap: one aligned vector load.  Where the tap falls in the
// padding (or the row is past M, the column past K, the chunk past the end of
// C*R*S) the load gets an offset beyond the buffer's range and the buffer
// unit returns zeros: padding costs no branch and no memory traffic.
//
// Per workgroup (256 threads = 4 waves in a 2x2 grid): a TM x TN output tile.
// Operand tiles stream from memory straight into a ring of NS LDS stages
// (buffer_load ... lds, 16 bytes per lane, no register staging), NS-1 stages
// ahead of the one being multiplied, so the load latency is covered by
// NS-1 stages of v_mfma_i32_32x32x32_i8 work.  One barrier per stage both
// publishes the stage that just landed and retires the slot the next loads
// overwrite.  LDS rows are BK bytes whose 16-byte chunks are permuted by an
// XOR of low row bits: each wave-wide direct load still fills one contiguous
// 1 KiB block (lane i -> bytes 16i..16i+15), the lane simply fetches the
// chunk that belongs there, and the MFMA operand reads (32 rows, one chunk)
// spread over all banks.
//
// Inner-dimension order: "blocked" when C/16 is a multiple of the chunks per
// stage: stage = (channel block, r, s) with (r, s) varying fastest, so the R*S
// stages that reuse one channel block of the same pixels run back to back and
// hit in cache; the stage position is then uniform across the workgroup.
// Otherwise "flat": chunks in (r, s, c) order, a stage may straddle taps, and
// each thread tracks the position of its own chunk.
//
// Epilogue: int32 results go from the accumulators to the output through its
// element strides.  The MFMA output column (the lane index) is made the
// output's contiguous dimension — output channels for a channel-innermost
// output, pixels for a pixel-innermost one — by swapping the MFMA operands.
#pragma once

#include "kernel_common.hpp"

namespace convi8 {

// KMAJ: the filter is read in place k-major (output channels contiguous, fK
// the stride of one input channel; blocked order only): a filter stage holds
// BK input-channel rows of TN output channels and its fragments are formed by
// LDS transposing reads, as in the 3x3 ring kernel.
// One workgroup's tile: workgroup bx of the launch's tiles, split by of the
// inner dimension (the kernels below run it with their block index).
template <int TM, int TN, int BK, int NS, int WGM, int WGN, bool FLAT, bool PIX_J, int EPI, bool KMAJ>
__device__ __forceinline__ void igemm_tile(const IgemmArgs &a, int bx, int by)
{
    constexpr int NW = WGM * WGN;           // waves per workgroup (WGM x WGN grid)
    constexpr int CPS = BK / 16;            // 16-byte chunks per row per stage
    constexpr int RPI = 64 / CPS;           // rows one wave-wide load fills
    constexpr int AL = TM / (NW * RPI);     // image-row loads per thread per stage
    constexpr int BL = TN / (NW * RPI);     // filter-row loads per thread per stage
    constexpr int LPS = AL + BL;            // loads per thread per stage
    constexpr int A_BYTES = TM * BK, STAGE = (TM + TN) * BK;
    constexpr int WM = TM / WGM, WN = TN / WGN; // wave tile
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int KS = BK / 32;             // MFMA k-steps per stage
    constexpr int NMF = KS * FM * FN;       // MFMAs per stage per wave
    constexpr int NRD = KS * (FM + FN);     // fragment reads per stage per wave
    static_assert(AL >= 1 && BL >= 1 && FM >= 1 && FN >= 1, "tile too small");
    static_assert(TM % (NW * RPI) == 0 && TN % (NW * RPI) == 0, "tile rows must fill wave loads");
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    static_assert(NS >= 2 && (NS - 2) * LPS < 64, "pipeline depth");
    static_assert(!KMAJ || (!FLAT && (TN == 64 || TN == 128 || TN == 256)), "k-major filter stages");
    constexpr int KRB = 1024 / TN;          // k-major: input-channel rows per 1 KB wave load

    __shared__ __attribute__((aligned(1024))) int8_t smem[NS * STAGE];
    __shared__ int out_row[PIX_J ? 1 : TM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = xcd_tile(bx, a.tiles);
    const int m0 = (tile / a.tiles_n) * TM;
    const int n0 = (tile % a.tiles_n) * TN;

    // ---- load geometry: load i of this wave fills LDS block i*NW+wave (rows
    // (i*NW+wave)*RPI ...), lane -> row + lane/CPS, physical chunk lane%CPS.
    // The logical chunk j it must fetch depends only on row bits that are
    // the same for every i, so j is one per thread.
    const int row0 = wave * RPI + lane / CPS;
    const int j = swizzle_chunk<BK>(row0, lane % CPS);

    int a_h0[AL], a_w0[AL], a_off[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int m = m0 + row0 + i * NW * RPI;
        if (m < a.M) {
            const int n = udiv(m, a.d_pq);
            const int rem = m - n * a.PQ;
            const int p = udiv(rem, a.d_q);
            const int q = rem - p * a.Q;
            a_h0[i] = p * a.strH - a.padH;
            a_w0[i] = q * a.strW - a.padW;
            a_off[i] = n * a.sN + a_h0[i] * a.sH + a_w0[i] * a.sW + (FLAT ? 0 : j * 16);
        } else {
            a_h0[i] = -0x40000000;  // never inside the image
            a_w0[i] = 0;
            a_off[i] = 0;
        }
    }
    // k-major filter rows: 16-byte chunk position q of input-channel row kr
    // holds global chunk q ^ kmaj_swz(kr), so that the eight rows of one
    // transposing read sit in eight different bank groups
    auto kmaj_swz = [](int kr) { return TN == 64 ? (kr >> 1) & 3 : kr & 7; };
    int b_off[BL];
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        if constexpr (KMAJ) {
            const int kr = (i * NW + wave) * KRB + lane / (TN / 16);
            const int col = n0 + (((lane % (TN / 16)) ^ kmaj_swz(kr)) << 4);
            b_off[i] = col < a.K ? kr * a.fK + col : kOutOfRange;
        } else {
            const int k = n0 + row0 + i * NW * RPI;
            b_off[i] = k < a.K ? k * a.fK + (FLAT ? 0 : j * 16) : kOutOfRange;
        }
    }
    if constexpr (!PIX_J) {
        if (!a.pix_linear)
            fill_out_rows<TM, 64 * NW>(a, m0, out_row);
    }

    // ---- inner-dimension position of the next stage to load ---------------
    // blocked: (r, s, cpos) uniform, cpos = channel-block byte offset, stepped
    // with selects; flat: each thread's chunk index g = stage*CPS + j is split
    // into (r, s, c16) afresh for every stage.
    // split z of the inner dimension: stages [stage0, stage_end)
    const int stage0 = by * a.kchunk;
    const int stage_end = min(a.nstages, stage0 + a.kchunk);
    int r = 0, s = 0, cpos = 0;
    int issued = stage0;
    if constexpr (!FLAT) {
        // blocked order: stage = (channel block * R + r) * S + s
        const int rs = stage0 % (a.R * a.S);
        s = rs % a.S;
        r = rs / a.S;
        cpos = stage0 / (a.R * a.S) * BK;
    }

    const unsigned smem_lds = lds_address(smem);
    const v4i img_rsrc = make_rsrc(a.img, a.img_range);
    const v4i flt_rsrc = make_rsrc(a.flt, a.flt_range);

    // per-stage load state, set by begin_stage(), used by dma_one()
    int rdh = 0, sdw = 0, itoff = 0, ftoff = 0;
    unsigned lbase = 0;

    // Loads of the next stage go to ring slot `slot`.  Past the last stage
    // (and, in flat order, for chunks past C*R*S) every load is out of range
    // and fills zeros, so each iteration keeps the same count of loads.
    auto begin_stage = [&](int slot) {
        if constexpr (FLAT) {
            const int g = issued * CPS + j;
            const int rs = fdiv(g, a.cc, a.inv_cc);
            const int c16 = g - rs * a.cc;
            r = fdiv(rs, a.S, a.inv_s);
            s = rs - r * a.S;
            cpos = c16 * 16;
        }
        const bool live = issued < stage_end && (!FLAT || r < a.R);
        rdh = live ? r * a.dilH : -0x20000000;  // dead stage: every row fails the bounds test
        sdw = s * a.dilW;
        itoff = rdh * a.sH + sdw * a.sW + cpos;
        ftoff = live ? a.flt0 + r * a.fR + s * a.fS + (KMAJ ? cpos * a.fK : cpos) : kOutOfRange;
        lbase = smem_lds + slot * STAGE + wave * 1024;
    };
    auto dma_one = [&](int i) {  // i < LPS, compile-time after unrolling
        if (i < AL) {
            const int h = a_h0[i] + rdh, w = a_w0[i] + sdw;
            const bool ok = ((unsigned)h < (unsigned)a.H) & ((unsigned)w < (unsigned)a.W);
            load16_to_lds(img_rsrc, lbase + i * NW * 1024, ok ? a_off[i] + itoff : kOutOfRange);
        } else {
            // b_off (column past K) or ftoff (dead stage) negative: out of range
            const int b = i - AL;
            load16_to_lds(flt_rsrc, lbase + A_BYTES + b * NW * 1024,
                          (b_off[b] | ftoff) < 0 ? kOutOfRange : b_off[b] + ftoff);
        }
    };
    auto end_stage = [&]() {
        ++issued;
        if constexpr (!FLAT) {
            const int s1 = s + 1;
            const bool ws = s1 == a.S;
            s = ws ? 0 : s1;
            const int r1 = r + (ws ? 1 : 0);
            const bool wr = r1 == a.R;
            r = wr ? 0 : r1;
            cpos += wr ? BK : 0;
        }
    };
    auto issue_stage = [&](int slot) {
        begin_stage(slot);
#pragma unroll
        for (int i = 0; i < LPS; ++i)
            dma_one(i);
        end_stage();
    };

    const int wm = (wave / WGN) * WM;
    const int wn = (wave % WGN) * WN;

    v16i acc[FM][FN];
#pragma unroll
    for (int x = 0; x < FM; ++x)
#pragma unroll
        for (int y = 0; y < FN; ++y)
            acc[x][y] = v16i{};

    // Operand fragments, double-buffered in registers: frag[buf][ks][0..FM)
    // from the image tile, [FM..FM+FN) from the filter tile.
    v4i frag[2][KS][FM + FN];
    auto read_one = [&](int buf, int slot, int i) {  // i < NRD
        const int ks = i / (FM + FN), f = i % (FM + FN);
        if (KMAJ && f >= FM) {
            // two transposing reads (rows kr .. kr+7, kr+8 .. kr+15): lane
            // i of each 16-lane group gets byte i % 8 of the rows lanes
            // 2b + i / 8 address, so lane j addresses row kr + j / 2 at
            // output channel col + 8 (j & 1)
            const int jj = lane & 15;
            const int col = wn + (f - FM) * 32 + ((lane >> 4) & 1) * 16 + (jj & 1) * 8;
            const int kr = ks * 32 + (lane >> 5) * 16 + (jj >> 1);
            const int8_t *p = smem + slot * STAGE + A_BYTES + kr * TN + (((col >> 4) ^ kmaj_swz(kr)) << 4) + (col & 8);
            const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)p);
            const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(p + 8 * TN));
            frag[buf][ks][f] = v4i{lo.x, lo.y, hi.x, hi.y};
            return;
        }
        const int ch = ks * 2 + (lane >> 5);
        const int row = (f < FM ? wm + f * 32 : wn + (f - FM) * 32) + (lane & 31);
        const int8_t *base = smem + slot * STAGE + (f < FM ? 0 : A_BYTES);
        frag[buf][ks][f] = *(const v4i *)&base[row * BK + swizzle_chunk<BK>(row, ch) * 16];
    };
    auto mfma_one = [&](int buf, int t) {  // t < NMF
        const int ks = t / (FM * FN), x = (t / FN) % FM, y = t % FN;
        acc[x][y] = PIX_J
            ? __builtin_amdgcn_mfma_i32_32x32x32_i8(frag[buf][ks][FM + y], frag[buf][ks][x], acc[x][y], 0, 0, 0)
            : __builtin_amdgcn_mfma_i32_32x32x32_i8(frag[buf][ks][x], frag[buf][ks][FM + y], acc[x][y], 0, 0, 0);
    };

    // One stage: the MFMAs of stage `it` (fragments in registers `buf`) are
    // interleaved with the loads of stage it+NS into the slot stage `it` has
    // just vacated and the fragment reads of stage it+1 into `buf^1`.
    // The first PRE MFMAs need only this wave's registers: they go out
    // before the wait and the barrier, so the matrix unit has work while the
    // waves line up; the loads and reads ride on the others.
    constexpr int NOTHER = LPS + NRD;
    constexpr int PRE = NMF / 4;
    int cur_slot = 0;
    auto body = [&](int buf) {
#pragma unroll
        for (int t = 0; t < PRE; ++t)
            mfma_one(buf, t);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_lgkm0<(NS - 2) * LPS>();  // own loads of stage it+1 landed; frag[buf] read
        __builtin_amdgcn_s_barrier();       // all waves: stage it+1 visible, slot it%NS free
        __builtin_amdgcn_sched_barrier(0);
        begin_stage(cur_slot);
        const int nslot = cur_slot + 1 == NS ? 0 : cur_slot + 1;
#pragma unroll
        for (int t = PRE; t < NMF; ++t) {
            mfma_one(buf, t);
#pragma unroll
            for (int o = (t - PRE) * NOTHER / (NMF - PRE); o < (t - PRE + 1) * NOTHER / (NMF - PRE); ++o) {
                if (o < LPS)
                    dma_one(o);
                else
                    read_one(buf ^ 1, nslot, o - LPS);
            }
        }
        end_stage();
        cur_slot = nslot;
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- main loop --------------------------------------------------------
    // An odd stage count runs one extra all-zero stage, so the loop body
    // (two stages, one per fragment buffer) has no branch inside it.
    const int nloop = (max(stage_end - stage0, 0) + 1) & ~1;
    if (nloop > 0) {
#pragma unroll
        for (int st = 0; st < NS; ++st)
            issue_stage(st);
        wait_vm_lgkm0<(NS - 1) * LPS>();
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int i = 0; i < NRD; ++i)
            read_one(0, 0, i);
        for (int it = 0; it < nloop; it += 2) {
            body(0);
            body(1);
        }
        // drain the trailing (out-of-range) loads before the ring is retired
        wait_vm_lgkm0<0>();
    }
    __syncthreads();

    // ---- epilogue ---------------------------------------------------------
    store_tile_any<FM, FN, PIX_J, EPI>(a, acc, m0, n0, wm, wn, lane, out_row);
}

template <int TM, int TN, int BK, int NS, int WGM, int WGN, bool FLAT, bool PIX_J, int EPI, bool KMAJ = false>
__global__ __launch_bounds__(64 * WGM * WGN) void conv_igemm_kernel(IgemmArgs a)
{
    igemm_tile<TM, TN, BK, NS, WGM, WGN, FLAT, PIX_J, EPI, KMAJ>(a, blockIdx.x, blockIdx.y);
}

// Several convolutions of one shape class in one launch (the stride phases
// of a data gradient): workgroups [first[p], first[p+1]) run phase p with its
// own arguments; every phase uses the same tile, order, layout and epilogue.
constexpr int kMaxPhases = 4;
struct IgemmPhases {
    IgemmArgs ph[kMaxPhases];
    int first[kMaxPhases + 1];
    int nph;
};
static_assert(sizeof(IgemmPhases) <= 4096, "the phases' arguments must fit one kernel argument block");

template <int TM, int TN, int BK, int NS, int WGM, int WGN, bool FLAT, bool PIX_J, int EPI, bool KMAJ>
__global__ __launch_bounds__(64 * WGM * WGN) void conv_igemm_phases_kernel(IgemmPhases m)
{
    const int b = blockIdx.x;
    int p = 0;
#pragma unroll
    for (int i = 1; i < kMaxPhases; ++i)
        p += i < m.nph && b >= m.first[i] ? 1 : 0;
    igemm_tile<TM, TN, BK, NS, WGM, WGN, FLAT, PIX_J, EPI, KMAJ>(m.ph[p], b - m.first[p], 0);
}

// Sum of the partial outputs of a split inner dimension: out[i] = the sum
// over z < nsplit of part[z*stride + i], for every i < n.  The output is
// dense, so i walks each of its elements once; int32 addition is exact and
// independent of order.  V4: n, stride and both pointers allow 16-byte
// vectors.
template <bool V4>
__global__ __launch_bounds__(256) void split_reduce_kernel(const int32_t *part, long long stride, int nsplit,
                                                           int32_t *out, long long n)
{
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const long long step = (long long)gridDim.x * 256;
    if constexpr (V4) {
        const long long n4 = n / 4, s4 = stride / 4;
        const i32x4 *p4 = (const i32x4 *)part;
        for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += step) {
            i32x4 s = p4[i];
            for (int z = 1; z < nsplit; ++z)
                s += p4[z * s4 + i];
            ((i32x4 *)out)[i] = s;
        }
    } else {
        for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += step) {
            int s = part[i];
            for (int z = 1; z < nsplit; ++z)
                s += part[z * stride + i];
            out[i] = s;
        }
    }
}

// The same sum for many copies of a small output (16-byte vectors): each
// workgroup takes 256/G vectors, its G groups of threads add copies g, g+G,
// g+2G, ... of them (four loads in flight per thread), and the G group sums
// of each vector are added through LDS.  Enough loads are then in flight for
// an output of a few thousand vectors to be summed at HBM speed.
template <int G>
__global__ __launch_bounds__(256) void split_reduce_wide_kernel(const int32_t *part, long long stride, int nsplit,
                                                                int32_t *out, long long n)
{
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    constexpr int V = 256 / G;   // vectors per workgroup
    __shared__ i32x4 red[G][V];
    const int it = threadIdx.x % V, g = threadIdx.x / V;
    const long long i = (long long)blockIdx.x * V + it;
    const long long n4 = n / 4, s4 = stride / 4;
    i32x4 s = {0, 0, 0, 0};
    if (i < n4) {
        const i32x4 *p = (const i32x4 *)part + i;
        int z = g;
        for (; z + 3 * G < nsplit; z += 4 * G) {
            const i32x4 a = p[z * s4], b = p[(z + G) * s4], c = p[(z + 2 * G) * s4], d = p[(z + 3 * G) * s4];
            s += (a + b) + (c + d);
        }
        for (; z < nsplit; z += G)
            s += p[z * s4];
    }
    red[g][it] = s;
    __syncthreads();
    if (g == 0 && i < n4) {
#pragma unroll
        for (int k = 1; k < G; ++k)
            s += red[k][it];
        ((i32x4 *)out)[i] = s;
    }
}

}  // namespace convi8
