// Footprint implicit-GEMM INT8 convolution for 3x3 filters on gfx950 (CDNA4).
//
// Same product as the im2col kernel (rows m = (n, p, q), columns k, inner
// (r, s, c)), but the image operand is not streamed once per filter tap.  For
// each block of 64 channels the kernel loads into LDS, once, every input pixel
// the tile's TM output pixels touch with any of the nine taps (the tile's
// footprint: whole padded rows, from the first pixel's top tap row to the last
// pixel's bottom tap row, zeros where the rows or columns fall in the
// padding), and builds the image operand of tap (r, s) by reading footprint
// pixel  base(m) + r*dil_h*Wf + s*dil_w  for output pixel m.  The filter still
// streams one (channel block, tap) stage at a time through an NS-slot LDS
// ring.  For a 3x3 filter this cuts the image bytes a tile moves into LDS by
// about R*S / (1 + halo overhead), which is what bounds the im2col kernel on
// large-channel layers: the per-CU load path, not the matrix cores.
//
// Everything about the schedule is fixed at compile time: the filter is 3x3,
// the main loop runs two channel blocks (18 stages) per iteration, and the
// ring depth divides 18, so ring slots, footprint buffers, tap indices and the
// number of loads in flight are constants at every stage.  The footprint of
// block c+1 goes into the other of two buffers in pieces that ride along with
// the filter loads of taps NS-1 .. 8 of block c: the first of those loads is
// issued after every wave has finished reading block c-1 (the previous user
// of that buffer), and all of them land before the first read of block c+1.
//
// LDS layout of a footprint, in 16-byte slots: pixel (row fr, column fc) at
// slot fr*Pr + fc*5 (64 channel bytes and a one-slot gap), so 16 output
// pixels along a row, read with one 16-byte chunk each, fall on 16 distinct
// bank groups (5 is odd), and the row pitch Pr is padded so that the next
// output row continues the same progression (the host picks Pr with
// stride_h*Pr = 5*stride_w*Q modulo 16 where it can).  The address of tap
// (r, s) is then a per-lane constant plus a uniform offset.  A wave-wide
// direct load fills 1 KiB = 64 consecutive slots; lanes whose slot is a gap
// (or past the footprint, or in the padding) load out of range, i.e. zeros.
#pragma once

#include <type_traits>

#include "kernel_common.hpp"

namespace convi8 {

namespace fp3x3 {

constexpr int kTaps = 9;

// f(integral_constant<int, I>) for I = B .. E-1, each a separate instantiation
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// footprint groups (workgroup-wide loads) carried by the stage at tap t
template <int NS, int NG>
constexpr int pieces_at(int t)
{
    const int first = NS - 1, n = kTaps - NS + 1;
    if (t < first)
        return 0;
    const int i = t - first;
    return (i + 1) * NG / n - i * NG / n;
}

template <int NS, int NG>
constexpr int first_piece(int t)
{
    const int first = NS - 1, n = kTaps - NS + 1;
    return t < first ? 0 : (t - first) * NG / n;
}

// loads a thread issues for a stage at tap t
template <int NS, int NG, int BL>
constexpr int loads_at(int t)
{
    return BL + pieces_at<NS, NG>(t);
}

// loads issued after those of the stage following tap t, while that stage is
// awaited: stages t+2 .. t+NS-1
template <int NS, int NG, int BL>
constexpr int outstanding_after_next(int t)
{
    int n = 0;
    for (int d = 2; d <= NS - 1; ++d)
        n += loads_at<NS, NG, BL>((t + d) % kTaps);
    return n;
}

}  // namespace fp3x3

// KSPL = 2 runs two waves per wave tile, each on one 32-channel half of
// every stage (so two waves share each SIMD with a 128x64 tile apiece); the
// halves are added through LDS at the end, each wave storing half the columns.
template <int TM, int TN, int NS, int FPIX, int WGM, int WGN, bool PIX_J, int KSPL = 1>
__global__ __launch_bounds__(64 * WGM * WGN * KSPL) void conv_footprint3x3_kernel(IgemmArgs a)
{
    using namespace fp3x3;
    constexpr int NQ = WGM * WGN;            // waves per channel half
    constexpr int NW = NQ * KSPL;
    constexpr int GB = NW * 1024;            // bytes of one workgroup-wide load
    constexpr int BK = 64;                   // channels per stage
    constexpr int PITCH = 80;                // footprint bytes per pixel (FPIX pixels fill a buffer)
    constexpr int BL = TN * BK / GB;         // filter loads per thread per stage
    constexpr int B_BYTES = TN * BK;         // one ring slot
    constexpr int NG = (FPIX * PITCH + GB - 1) / GB;
    constexpr int FBUF = NG * GB;            // one footprint buffer
    constexpr int WM = TM / WGM, WN = TN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int KS = BK / 32 / KSPL;       // MFMA k-steps per stage of one wave
    constexpr int NMF = KS * FM * FN;
    constexpr int NRD = KS * (FM + FN);
    static_assert(BL >= 1 && TN * BK % GB == 0, "filter tile must fill workgroup loads");
    static_assert((2 * kTaps) % NS == 0 && NS >= 2 && NS <= kTaps, "ring depth must divide 18");
    static_assert(FM >= 1 && FN >= 1 && NMF >= 2, "wave tile");
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    static_assert(KSPL == 1 || (KSPL == 2 && FN % 2 == 0 && NS * TN * BK >= NW * (FN / 2) * 4096),
                  "channel split: even wave-tile columns, exchange fits the ring");

    __shared__ __attribute__((aligned(1024))) int8_t ring[NS * B_BYTES];
    __shared__ __attribute__((aligned(1024))) int8_t fbuf[2 * FBUF];
    __shared__ int out_row[PIX_J ? 1 : TM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = xcd_tile(blockIdx.x, a.tiles);
    const int m0 = (tile / a.tiles_n) * TM;
    const int n0 = (tile % a.tiles_n) * TN;
    const int kg = wave / NQ;                // channel half (KSPL = 2)
    const int wq = wave % NQ;
    const int wm = (wq / WGN) * WM;
    const int wn = (wq % WGN) * WN;

    // ---- footprint geometry of this tile (uniform) ------------------------
    const int m_last = min(m0 + TM, a.M) - 1;
    const int n_a = udiv(m0, a.d_pq);
    const int p_a = udiv(m0 - n_a * a.PQ, a.d_q);
    const int hp_a = p_a * a.strH;           // first footprint row (padded coordinates of image n_a)
    const int n_b = udiv(m_last, a.d_pq);
    const int p_b = udiv(m_last - n_b * a.PQ, a.d_q);
    const int frows = (n_b - n_a) * a.Hp + p_b * a.strH + 2 * a.dilH - hp_a + 1;  // host keeps frows*Pr within the buffer

    // ---- footprint loads: group g, this thread -> 16-byte slot
    // g*GB/16 + wave*64 + lane of the buffer = footprint row slot/Pr, pixel
    // (slot%Pr)/5 of that row, chunk (slot%Pr)%5 (chunk 4 and the row's
    // tail slots are gaps)
    int foff[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int slot = g * (GB / 16) + wave * 64 + lane;
        const int fr = fdiv(slot, a.Pr, a.inv_pr);
        const int rem = slot - fr * a.Pr;
        const int fc = rem / 5;
        const int j = rem - fc * 5;
        const int hr = hp_a + fr;
        const int dn = fdiv(hr, a.Hp, a.inv_hp);
        const int h = hr - dn * a.Hp - a.padH;
        const int w = fc - a.padW;
        const bool ok = (j < 4) & (fc < a.Wf) & (fr < frows) & ((unsigned)h < (unsigned)a.H) &
                        ((unsigned)w < (unsigned)a.W);
        foff[g] = ok ? (n_a + dn) * a.sN + h * a.sH + w * a.sW + j * 16 : kOutOfRange;
    }

    // ---- filter loads: load i of this wave fills ring rows (i*NW+wave)*16 ..
    const int row0 = wave * 16 + (lane >> 2);
    const int jb = swizzle_chunk<64>(row0, lane & 3);
    int b_off[BL];
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        const int k = n0 + row0 + i * NW * 16;
        b_off[i] = k < a.K ? k * a.fK + jb * 16 : kOutOfRange;
    }
    if constexpr (!PIX_J) {
        if (!a.pix_linear)
            fill_out_rows<TM, 64 * NW>(a, m0, out_row);
    }

    // ---- operand reads: per-lane byte offsets (tap (0,0), footprint buffer 0 /
    // ring slot 0); a tap adds a uniform offset, buffers and slots a constant
    int a_lane[FM][KS];
#pragma unroll
    for (int x = 0; x < FM; ++x) {
        const int m = m0 + wm + x * 32 + (lane & 31);
        int idx = 0;
        if (m < a.M) {
            const int n = udiv(m, a.d_pq);
            const int rem = m - n * a.PQ;
            const int p = udiv(rem, a.d_q);
            const int q = rem - p * a.Q;
            idx = ((n - n_a) * a.Hp + p * a.strH - hp_a) * a.Pr + q * a.strW * 5;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            a_lane[x][ks] = (idx + (kg * KS + ks) * 2 + (lane >> 5)) * 16;
    }
    int b_lane[FN][KS];
#pragma unroll
    for (int y = 0; y < FN; ++y) {
        const int row = wn + y * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            b_lane[y][ks] = row * BK + swizzle_chunk<64>(row, (kg * KS + ks) * 2 + (lane >> 5)) * 16;
    }

    const v4i img_rsrc = make_rsrc(a.img, a.img_range);
    const v4i flt_rsrc = make_rsrc(a.flt, a.flt_range);
    const unsigned ring_lds = lds_address(ring) + wave * 1024;
    const unsigned fbuf_lds = lds_address(fbuf) + wave * 1024;
    const int nblk = a.ncblk;

    // uniform per-tap offsets: footprint bytes (read side), filter bytes (load side)
    auto tap_read = [&](int t) { return ((t / 3) * a.dilH * a.Pr + (t % 3) * a.dilW * 5) * 16; };
    auto tap_flt = [&](int t) { return a.flt0 + (t / 3) * a.fR + (t % 3) * a.fS; };

    // Loads of stage (block cb, tap t) into ring slot `slot`, plus the
    // footprint pieces of block cb+1 that ride on tap t.  Past the last block
    // every load is out of range: offsets get the resource's range added.
    auto dma_filter = [&](int slot, int cb, int t, int i) {
        const int ftoff = cb < nblk ? tap_flt(t) + cb * BK : a.flt_range;
        load16_to_lds(flt_rsrc, ring_lds + slot * B_BYTES + i * GB, b_off[i] + ftoff);
    };
    auto dma_piece = [&](int cb, int par, int g) {  // footprint group g of block cb (parity par)
        const int coff = cb < nblk ? cb * BK : a.img_range;
        load16_to_lds(img_rsrc, fbuf_lds + par * FBUF + g * GB, foff[g] + coff);
    };

    v16i acc[FM][FN];
#pragma unroll
    for (int x = 0; x < FM; ++x)
#pragma unroll
        for (int y = 0; y < FN; ++y)
            acc[x][y] = v16i{};

    v4i frag[2][KS][FM + FN];
    // fragment read i of the stage at tap t, ring slot `slot`, footprint buffer fb
    auto read_one = [&](int buf, int slot, int fb, int toff, int i) {
        const int ks = i / (FM + FN), f = i % (FM + FN);
        if (f < FM)
            frag[buf][ks][f] = *(const v4i *)&fbuf[fb * FBUF + a_lane[f][ks] + toff];
        else
            frag[buf][ks][f] = *(const v4i *)&ring[slot * B_BYTES + b_lane[f - FM][ks]];
    };
    auto mfma_one = [&](int buf, int t) {
        const int ks = t / (FM * FN), x = (t / FN) % FM, y = t % FN;
        acc[x][y] = PIX_J
            ? __builtin_amdgcn_mfma_i32_32x32x32_i8(frag[buf][ks][FM + y], frag[buf][ks][x], acc[x][y], 0, 0, 0)
            : __builtin_amdgcn_mfma_i32_32x32x32_i8(frag[buf][ks][x], frag[buf][ks][FM + y], acc[x][y], 0, 0, 0);
    };

    // ---- prologue: footprint of block 0, then stages 0 .. NS-1 -------------
#pragma unroll
    for (int g = 0; g < NG; ++g)
        dma_piece(0, 0, g);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
#pragma unroll
        for (int i = 0; i < BL; ++i)
            dma_filter(st, 0, st, i);
#pragma unroll
        for (int g = 0; g < pieces_at<NS, NG>(st); ++g)
            dma_piece(1, 1, first_piece<NS, NG>(st) + g);
    }
    {
        constexpr int ahead = [] {
            int n = 0;
            for (int st = 1; st < NS; ++st)
                n += loads_at<NS, NG, BL>(st);
            return n;
        }();
        wait_vm_lgkm0<ahead>();
    }
    __builtin_amdgcn_s_barrier();
    {
        const int t0 = tap_read(0);
#pragma unroll
        for (int i = 0; i < NRD; ++i)
            read_one(0, 0, 0, t0, i);
    }

    // ---- main loop: two channel blocks (18 stages) per iteration ----------
    // Stage u = 18*pair + v runs MFMAs on fragments read during stage u-1,
    // issues the loads of stage u+NS into the ring slot it vacated, and reads
    // the fragments of stage u+1.
    const int npairs = (nblk + 1) >> 1;
    for (int pair = 0; pair < npairs; ++pair) {
        const int cb0 = pair * 2;
        static_for<0, 2 * kTaps>([&](auto vc) {
            constexpr int v = decltype(vc)::value;
            constexpr int t = v % kTaps;
            constexpr int buf = v & 1;
            constexpr int slot = v % NS;
            // the stage being loaded: u + NS
            constexpr int lv = v + NS;
            constexpr int lt = lv % kTaps;
            const int lcb = cb0 + lv / kTaps;
            // the stage being read: u + 1
            constexpr int rv = v + 1;
            constexpr int rt = rv % kTaps;
            constexpr int rfb = (rv / kTaps) & 1;  // block parity (cb0 is even)
            constexpr int rslot = rv % NS;

            wait_vm_lgkm0<outstanding_after_next<NS, NG, BL>(t)>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            const int rtoff = tap_read(rt);
            constexpr int npc = pieces_at<NS, NG>(lt);
            constexpr int gp0 = first_piece<NS, NG>(lt);
#pragma unroll
            for (int q = 0; q < NMF; ++q) {
                mfma_one(buf, q);
                // the fragment reads of stage u+1 ride on the first half of
                // the MFMAs, so the last of them has half a stage to land
                // before the wait at the top of the next stage; the loads of
                // stage u+NS (long latency, awaited NS-1 stages later) take
                // the second half
                constexpr int H = NMF / 2, NL = BL + npc;
                if (q < H) {
#pragma unroll
                    for (int o = q * NRD / H; o < (q + 1) * NRD / H; ++o)
                        read_one(buf ^ 1, rslot, rfb, rtoff, o);
                } else {
#pragma unroll
                    for (int o = (q - H) * NL / (NMF - H); o < (q - H + 1) * NL / (NMF - H); ++o) {
                        if (o < BL)
                            dma_filter(slot, lcb, lt, o);
                        else
                            dma_piece(lcb + 1, (lv / kTaps + 1) & 1, gp0 + (o - BL));
                    }
                }
                // keep the loads and reads where they are: spread between the
                // MFMAs (left to itself the scheduler bunches the reads at the
                // end of the stage, where their latency is exposed)
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    // drain the trailing (out-of-range) loads before the LDS is released
    wait_vm_lgkm0<0>();
    __syncthreads();

    // streaming stores whatever the layout: the outputs this kernel serves
    // (forward and data gradient) have a unit-stride channel or column dim,
    // and for any other layout the policy costs speed, not correctness
    if constexpr (KSPL == 1) {
        store_tile_any<FM, FN, PIX_J>(a, acc, m0, n0, wm, wn, lane, out_row);
    } else {
        // Wave (kg, wq) keeps column half kg of its tile and hands the other
        // to wave (1-kg, wq) through the (now idle) ring, lane-major, one
        // 32-row block at a time.
        constexpr int FH = FN / 2;
        v4i *const xch = (v4i *)ring;
        auto finish = [&](auto kgc) {
            constexpr int KG = decltype(kgc)::value;
#pragma unroll
            for (int x = 0; x < FM; ++x) {
#pragma unroll
                for (int yy = 0; yy < FH; ++yy)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const v16i &c = acc[x][(1 - KG) * FH + yy];
                        xch[((wave * FH + yy) * 4 + i) * 64 + lane] =
                            v4i{c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]};
                    }
                __syncthreads();
                v16i fin[1][FH];
#pragma unroll
                for (int yy = 0; yy < FH; ++yy) {
                    fin[0][yy] = acc[x][KG * FH + yy];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const v4i p = xch[(((wave ^ NQ) * FH + yy) * 4 + i) * 64 + lane];
                        fin[0][yy][4 * i] += p.x;
                        fin[0][yy][4 * i + 1] += p.y;
                        fin[0][yy][4 * i + 2] += p.z;
                        fin[0][yy][4 * i + 3] += p.w;
                    }
                }
                __syncthreads();
                store_tile_any<1, FH, PIX_J>(a, fin, m0, n0, wm + x * 32, wn + KG * FH * 32, lane, out_row);
            }
        };
        if (kg == 0)
            finish(std::integral_constant<int, 0>{});
        else
            finish(std::integral_constant<int, 1>{});
    }
}



}  // namespace convi8
