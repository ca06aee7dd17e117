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


namespace fp9 {

// Schedule of the nine-slot variant below.  Ring slot = filter tap, so the
// load of stage (block b, tap t) for block b+1 goes into the slot it vacates.
// The footprint of block b+1 (buffer (b+1)&1, free since block b-1's last
// read) rides in kChunks pieces: the first on tap 8 of block b-1, the rest on
// taps 0 .. kChunks-2 of block b, so the last piece has 8-(kChunks-2) stages
// to land before tap 8 of block b reads block b+1.
constexpr int kChunks = 6;

// index of the footprint chunk issued at tap t (-1: none)
constexpr int chunk_at(int t)
{
    return t == 8 ? 0 : (t < kChunks - 1 ? t + 1 : -1);
}

template <int NG>
constexpr int chunk_lo(int c)
{
    return c * NG / kChunks;
}

// loads a thread issues at tap t
template <int NG, int BL>
constexpr int loads_at(int t)
{
    const int c = chunk_at(t);
    return BL + (c < 0 ? 0 : chunk_lo<NG>(c + 1) - chunk_lo<NG>(c));
}

// Loads that may still be in flight at the wait on top of the stage at tap t.
// That stage reads the fragments of the next stage: for t < 8 the filter of
// (b, t+1), issued at (b-1, t+1), so the loads of taps t+2 .. 8 of the
// previous block and 0 .. t-1 of this one may be outstanding; for t = 8 the
// filter of (b+1, 0) and the whole footprint of block b+1, whose last piece
// goes out at tap kChunks-2, so only taps kChunks-1 .. 7 may be outstanding.
template <int NG, int BL>
constexpr int allowed_at(int t)
{
    int n = 0;
    if (t < 8) {
        for (int u = t + 2; u <= 8; ++u)
            n += loads_at<NG, BL>(u);
        for (int u = 0; u < t; ++u)
            n += loads_at<NG, BL>(u);
    } else {
        for (int u = kChunks - 1; u <= 7; ++u)
            n += loads_at<NG, BL>(u);
    }
    return n;
}

// Footprint pieces a thread issues at tap t.
template <int NG>
constexpr int pieces_at(int t)
{
    const int c = chunk_at(t);
    return c < 0 ? 0 : chunk_lo<NG>(c + 1) - chunk_lo<NG>(c);
}

// Block 0.  The prologue issues the filter of (0, 0), the footprint of block
// 0, the filters of (0, 1) and (0, 2) and chunk 0 of block 1; stage (0, t)
// then issues, in this order, the filter of (0, t+3) (t <= 5), the filter of
// (1, t) and its footprint chunk.  Loads that may be outstanding at the wait
// on top of stage (0, t), which needs the filter of (0, t+1) (for t = 8: the
// filter of (1, 0) and the footprint of block 1, whose last chunk goes out at
// tap kChunks-2):
template <int NG, int BL>
constexpr int allowed_first(int t)
{
    if (t == 0)
        return BL + chunk_lo<NG>(1);
    if (t == 1)
        return chunk_lo<NG>(1) + 2 * BL + pieces_at<NG>(0);
    if (t < 8)
        return BL + pieces_at<NG>(t - 2) + (t - 1 <= 5 ? BL : 0) + BL + pieces_at<NG>(t - 1);
    int n = 0;
    for (int u = kChunks - 1; u <= 7; ++u)
        n += (u <= 5 ? BL : 0) + BL + pieces_at<NG>(u);
    return n;
}

// footprint row outside the image or past the footprint (prologue table)
constexpr int kRowOutside = -0x7fffffff - 1;

// Row blocks of the tail for a wave tile of FM 32-row fragments: two
// fragments first, then one at a time, so the last row block (whose stores
// no MFMAs hide) is a single fragment; with FM < 4 one fragment each.
constexpr int tail_blocks(int FM) { return FM >= 4 ? FM - 1 : FM; }
constexpr int tail_first(int FM, int x) { return FM >= 4 && x > 0 ? x + 1 : x; }
constexpr int tail_len(int FM, int x) { return FM >= 4 && x == 0 ? 2 : 1; }

}  // namespace fp9

// 3x3 footprint kernel with a nine-slot filter ring (one slot per tap) and a
// per-block loop.  With TAIL, the last 64-channel block runs row block by row
// block: each row block of the wave tile (64 rows when the wave has 128)
// goes through all nine taps, and its INT32 stores drain while the MFMAs of
// the next row block run (instead of the whole tile's stores after the last
// MFMA).  Four waves, 2 x 2 (WGM x WGN).
template <int TM, int TN, int FPIX, int WGM, int WGN, bool PIX_J, bool TAIL, bool KMAJ = false>
__global__ __launch_bounds__(64 * WGM * WGN) void conv_fp3x3_ring9_kernel(IgemmArgs a)
{
    CONV_I8_PHASE_DECL;   // phase stamps of instrumented builds (nothing otherwise)
    using namespace fp3x3;
    using namespace fp9;
    constexpr int NW = WGM * WGN;
    constexpr int GB = NW * 1024;            // bytes of one workgroup-wide load
    constexpr int BK = 64;                   // channels per stage
    constexpr int PITCH = 80;                // footprint bytes per pixel
    constexpr int BL = TN * BK / GB;         // filter loads per thread per stage
    constexpr int B_BYTES = TN * BK;         // one ring slot
    constexpr int NG = (FPIX * PITCH + GB - 1) / GB;
    constexpr int FBUF = NG * GB;
    constexpr int WM = TM / WGM, WN = TN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int KS = 2;                    // k-steps of 32 channels per stage
    constexpr int NMF = KS * FM * FN;
    constexpr int NRD = KS * (FM + FN);
    static_assert(BL >= 1 && TN * BK % GB == 0, "filter tile must fill workgroup loads");
    static_assert(NW == 4, "four waves");
    static_assert(FM >= 1 && FN >= 1, "wave tile");
    static_assert(!KMAJ || TN == 128, "a k-major filter slot holds 64 rows of 128 output channels");
    static_assert(allowed_at<NG, BL>(0) < 64 && allowed_at<NG, BL>(7) < 64 && allowed_first<NG, BL>(8) < 64 &&
                      2 * BL + chunk_lo<NG>(1) < 64,
                  "vmcnt range");

    __shared__ __attribute__((aligned(1024))) int8_t ring[kTaps * B_BYTES];
    __shared__ __attribute__((aligned(1024))) int8_t fbuf[2 * FBUF];
    __shared__ int out_row[PIX_J ? 1 : TM];
    __shared__ int frow_off[64 * NW];   // byte offset of each footprint row (prologue)

    // every argument the prologue needs, loaded in one round trip (left to
    // itself the compiler loads some of them only where they are first used,
    // a second round trip before the first load can be issued)
    asm volatile("" ::"s"(a.img), "s"(a.flt), "s"(a.img_range), "s"(a.flt_range), "s"(a.fK), "s"(a.flt0),
                 "s"(a.fR), "s"(a.fS), "s"(a.K), "s"(a.tiles), "s"(a.tiles_n), "s"(a.ncblk), "s"(a.sN), "s"(a.sH),
                 "s"(a.sW), "s"(a.H), "s"(a.W), "s"(a.Pr), "s"(a.Hp), "s"(a.Wf));
    asm volatile("" ::"s"(a.Q), "s"(a.PQ), "s"(a.M), "s"(a.strH), "s"(a.strW), "s"(a.dilH), "s"(a.dilW),
                 "s"(a.padH), "s"(a.padW), "s"(a.d_pq.m), "s"(a.d_pq.l), "s"(a.d_q.m), "s"(a.d_q.l),
                 "s"(a.d_tn.m), "s"(a.d_tn.l), "s"(a.inv_pr), "s"(a.inv_hp));
    CONV_I8_PHASE(ph1);   // arguments loaded
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = xcd_tile(blockIdx.x, a.tiles);
    const int tm = udiv(tile, a.d_tn);
    const int m0 = tm * TM;
    const int n0 = (tile - tm * a.tiles_n) * TN;
    const int wm = (wave / WGN) * WM;
    const int wn = (wave % WGN) * WN;

    const int row0 = wave * 16 + (lane >> 2);
    const int jb = swizzle_chunk<64>(row0, lane & 3);
    int b_off[BL];
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        if constexpr (KMAJ) {
            // k-major filter (output channels contiguous, a.fK the stride of
            // one of the block's 64 reduction rows): byte p = lane*16 of load
            // i lands at slot byte i*GB + wave*1024 + p, i.e. row kr, 16-byte
            // chunk q of 128 output channels, and holds global chunk
            // q ^ (kr & 7) of that row, so that the transposing reads of a
            // fragment (eight consecutive rows of one chunk) hit eight
            // different chunk positions
            const int kr = i * (GB / 128) + wave * 8 + (lane >> 3);
            const int col = n0 + (((lane & 7) ^ (kr & 7)) << 4);
            b_off[i] = col < a.K ? kr * a.fK + col : kOutOfRange;
        } else {
            const int k = n0 + row0 + i * NW * 16;
            b_off[i] = k < a.K ? k * a.fK + jb * 16 : kOutOfRange;
        }
    }
    int a_lane[FM][KS];
    int b_lane[FN][KS];

    const v4i img_rsrc = make_rsrc(a.img, a.img_range);
    const v4i flt_rsrc = make_rsrc(a.flt, a.flt_range);
    const unsigned ring_lds = lds_address(ring) + wave * 1024;
    const unsigned fbuf_lds = lds_address(fbuf) + wave * 1024;
    const int nblk = a.ncblk;
    const int cb_bytes = KMAJ ? BK * a.fK : BK;   // filter bytes from one channel block to the next
    const bool tail = TAIL && nblk > 0;
    const int nend = tail ? nblk - 1 : nblk;   // blocks run by the main loop

    auto tap_read = [&](int t) { return ((t / 3) * a.dilH * a.Pr + (t % 3) * a.dilW * 5) * 16; };
    auto tap_flt = [&](int t) { return a.flt0 + (t / 3) * a.fR + (t % 3) * a.fS; };
    // filter of (block cb, tap t) into ring slot t; past the last block the
    // offsets leave the range (zeros)
    auto dma_filter = [&](int cb, int t, int i) {
        const int ftoff = cb < nblk ? tap_flt(t) + cb * cb_bytes : a.flt_range;
        load16_to_lds(flt_rsrc, ring_lds + t * B_BYTES + i * GB, b_off[i] + ftoff);
    };
    int foff[NG];
    auto dma_piece = [&](int cb, int g) {  // footprint group g of block cb into buffer cb&1
        const int coff = cb < nblk ? cb * BK : a.img_range;
        load16_to_lds(img_rsrc, fbuf_lds + (cb & 1) * FBUF + g * GB, foff[g] + coff);
    };

    CONV_I8_PHASE(ph2);   // prologue loads start
    // ---- prologue: the filter of (0, 0) goes out first (its offsets are
    // ready); then the footprint of block 0, each group as soon as its
    // offsets are known, so that the address arithmetic overlaps the loads;
    // then the filters of (0, 1), (0, 2) and chunk 0 of block 1 (the other
    // taps of block 0 go out during its first stages); then the addresses
    // the LDS reads need, while the loads are in flight
#pragma unroll
    for (int i = 0; i < BL; ++i)
        dma_filter(0, 0, i);

    // footprint geometry of this tile (uniform)
    const int m_last = min(m0 + TM, a.M) - 1;
    const int n_a = udiv(m0, a.d_pq);
    const int p_a = udiv(m0 - n_a * a.PQ, a.d_q);
    const int hp_a = p_a * a.strH;
    const int n_b = udiv(m_last, a.d_pq);
    const int p_b = udiv(m_last - n_b * a.PQ, a.d_q);
    const int frows = (n_b - n_a) * a.Hp + p_b * a.strH + 2 * a.dilH - hp_a + 1;
    // Slot (16 bytes) s of the footprint is footprint row fr = s / Pr, pixel
    // column fc and 16-byte piece j of that row; footprint row fr is padded
    // row hr = hp_a + fr counted from image n_a, i.e. row h of image n_a + dn
    // with hr = dn * Hp + h + padH.  Its bytes start at
    //   (n_a + dn) sN + h sH + (fc - padW) sW + 16 j.
    // Thread t first forms the row part for footprint row t (or marks a row
    // past the footprint or outside the image) in LDS; the slots then need
    // only their column and piece, and the chains stay short: the address
    // arithmetic of all groups, and the table reads, go out before the first
    // footprint load, each group's load right after its last few operations.
    // (The slots span fewer than 64 * NW rows: Pr >= 15.)  The planner keeps
    // sW below 2^23, so fc * sW is a 24-bit multiply.
    {
        const int t = tid;
        const int hr = hp_a + t;
        const int dn = fdiv(hr, a.Hp, a.inv_hp);
        const int h = hr - dn * a.Hp - a.padH;
        frow_off[t] = (t < frows && (unsigned)h < (unsigned)a.H) ? (n_a + dn) * a.sN + h * a.sH - a.padW * a.sW
                                                                 : kRowOutside;
    }
    // the table is written (the filter loads of (0, 0) stay in flight)
    wait_vm_lgkm0<BL>();
    __builtin_amdgcn_s_barrier();
    int fcg[NG], jg[NG], rog[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int slot = g * (GB / 16) + wave * 64 + lane;
        const int fr = fdiv(slot, a.Pr, a.inv_pr);
        const int rem = slot - __mul24(fr, a.Pr);
        fcg[g] = (int)(__umul24((unsigned)rem, 52429u) >> 18);   // rem / 5 (rem < 2^16)
        jg[g] = rem - fcg[g] * 5;
        rog[g] = frow_off[min(fr, 64 * NW - 1)];
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        // slots past the footprint's rows, the fifth piece of a pixel and
        // the row padding are never read: they are skipped (or filled with
        // whatever lies there); rows and columns outside the image read
        // zeros
        const int w = fcg[g] - a.padW;
        const bool ok = (rog[g] != kRowOutside) & (jg[g] < 4) & ((unsigned)w < (unsigned)a.W);
        foff[g] = ok ? rog[g] + __mul24(fcg[g], a.sW) + jg[g] * 16 : kOutOfRange;
        dma_piece(0, g);
        __builtin_amdgcn_sched_barrier(0);
    }

    v16i acc[FM][FN];
#pragma unroll
    for (int x = 0; x < FM; ++x)
#pragma unroll
        for (int y = 0; y < FN; ++y)
            acc[x][y] = v16i{};

    // filter fragment y of k-step ks of tap t
    auto b_frag = [&](int t, int y, int ks) {
        const int8_t *p = &ring[t * B_BYTES + b_lane[y][ks]];
        if constexpr (KMAJ) {
            // two transposing reads: rows kr .. kr+7, then kr+8 .. kr+15
            const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)p);
            const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(p + 8 * TN));
            return v4i{lo.x, lo.y, hi.x, hi.y};
        } else {
            return *(const v4i *)p;
        }
    };
    v4i frag[2][KS][FM + FN];
    auto read_one = [&](int buf, int t, int fb, int i) {
        const int ks = i / (FM + FN), f = i % (FM + FN);
        if (f < FM)
            frag[buf][ks][f] = *(const v4i *)&fbuf[fb * FBUF + a_lane[f][ks] + tap_read(t)];
        else
            frag[buf][ks][f] = b_frag(t, f - FM, ks);
    };
    // MFMA q of a stage: k-step major, row blocks in order, column blocks
    // snaking (consecutive MFMAs share one operand)
    auto mfma_one = [&](int buf, int q) {
        const int ks = q / (FM * FN), x = (q / FN) % FM, yy = q % FN;
        const int y = (x & 1) ? FN - 1 - yy : yy;
        acc[x][y] = PIX_J
            ? __builtin_amdgcn_mfma_i32_32x32x32_i8(frag[buf][ks][FM + y], frag[buf][ks][x], acc[x][y], 0, 0, 0)
            : __builtin_amdgcn_mfma_i32_32x32x32_i8(frag[buf][ks][x], frag[buf][ks][FM + y], acc[x][y], 0, 0, 0);
    };

#pragma unroll
    for (int t = 1; t < 3; ++t)
#pragma unroll
        for (int i = 0; i < BL; ++i)
            dma_filter(0, t, i);
#pragma unroll
    for (int g = chunk_lo<NG>(0); g < chunk_lo<NG>(1); ++g)
        dma_piece(1, g);
    CONV_I8_PHASE(ph3);   // footprint of block 0 issued
    if constexpr (!PIX_J) {
        if (!a.pix_linear)
            fill_out_rows<TM, 64 * NW>(a, m0, out_row);
    }

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
            a_lane[x][ks] = (idx + ks * 2 + (lane >> 5)) * 16;
    }
#pragma unroll
    for (int y = 0; y < FN; ++y) {
        if constexpr (KMAJ) {
            // ds_read_b64_tr_b8 hands lane i of each 16-lane group byte i % 8
            // of the eight rows that lanes 2b + i / 8 (b = 0..7) address: lane
            // j addresses row kr + j / 2 at output channel col + 8 (j & 1),
            // so that lane i receives reduction rows kr .. kr+7 of output
            // channel col + i, the fragment an MFMA lane needs (channel
            // lane % 32, rows 16 (lane / 32) .. +16 of the k-step)
            const int j = lane & 15;
            const int col = wn + y * 32 + ((lane >> 4) & 1) * 16 + (j & 1) * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kr = ks * 32 + (lane >> 5) * 16 + (j >> 1);
                b_lane[y][ks] = kr * TN + (((col >> 4) ^ (kr & 7)) << 4) + (col & 8);
            }
        } else {
            const int row = wn + y * 32 + (lane & 31);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                b_lane[y][ks] = row * BK + swizzle_chunk<64>(row, ks * 2 + (lane >> 5)) * 16;
        }
    }

    wait_vm_lgkm0<2 * BL + chunk_lo<NG>(1)>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int i = 0; i < NRD; ++i)
        read_one(0, 0, 0, i);
    CONV_I8_PHASE(ph4);   // main loop starts

    // ---- main loop ----------------------------------------------------------
    // Stage (cb, t) runs MFMAs on fragments read during the previous stage,
    // loads the filter of (cb+1, t) into slot t plus the footprint chunk that
    // rides on tap t, and reads the fragments of the next stage.  Stage u =
    // 9 cb + t keeps its fragments in buffer u & 1; blocks go in pairs so
    // that buffer, footprint buffer and every wait count are compile-time.
    auto run_block = [&](int cb, auto parc, auto firstc) {
        constexpr int PAR = decltype(parc)::value;   // cb & 1
        constexpr bool FIRST = decltype(firstc)::value;
        static_for<0, kTaps>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            constexpr int buf = (t + PAR) & 1;
            constexpr int rt = (t + 1) % kTaps;
            constexpr int rfb = t == 8 ? PAR ^ 1 : PAR;
            constexpr int ck = chunk_at(t);
            constexpr int g0 = ck < 0 ? 0 : chunk_lo<NG>(ck);
            constexpr int g1 = ck < 0 ? 0 : chunk_lo<NG>(ck + 1);
            constexpr int XL = FIRST && t + 3 < kTaps ? BL : 0;   // block 0: the filter of (0, t+3)
            constexpr int NL = XL + BL + (g1 - g0);
            const int pcb = t == 8 ? cb + 2 : cb + 1;   // block of this tap's footprint chunk

            // The first PRE MFMAs need only this wave's registers: they go
            // out before the wait and the barrier, so the matrix unit has
            // work while the waves line up.  Then the fragment reads of the
            // next stage ride on half of the remaining MFMAs, the loads on
            // the other half.
            constexpr int PRE = NMF / 4;
            constexpr int H = PRE + (NMF - PRE) / 2;
#pragma unroll
            for (int q = 0; q < NMF; ++q) {
                if (q == PRE) {
                    wait_vm_lgkm0<FIRST ? allowed_first<NG, BL>(t) : allowed_at<NG, BL>(t)>();
                    __builtin_amdgcn_s_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                }
                mfma_one(buf, q);
                if (q < PRE) {
                } else if (q < H) {
#pragma unroll
                    for (int o = (q - PRE) * NRD / (H - PRE); o < (q - PRE + 1) * NRD / (H - PRE); ++o)
                        read_one(buf ^ 1, rt, rfb, o);
                } else {
#pragma unroll
                    for (int o = (q - H) * NL / (NMF - H); o < (q - H + 1) * NL / (NMF - H); ++o) {
                        if (o < XL)
                            dma_filter(0, t + 3, o);
                        else if (o < XL + BL)
                            dma_filter(cb + 1, t, o - XL);
                        else
                            dma_piece(pcb, g0 + (o - XL - BL));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using First = std::integral_constant<bool, true>;
    using Steady = std::integral_constant<bool, false>;
    if (nend > 0)
        run_block(0, I0{}, First{});
    int cb = 1;
    for (; cb + 1 < nend; cb += 2) {
        run_block(cb, I1{}, Steady{});
        run_block(cb + 1, I0{}, Steady{});
    }
    if (cb < nend)
        run_block(cb, I1{}, Steady{});
    CONV_I8_PHASE(ph5);   // main loop done

    if (!tail) {
        wait_vm_lgkm0<0>();
        store_tile_any<FM, FN, PIX_J>(a, acc, m0, n0, wm, wn, lane, out_row);
    } else {
        // ---- last block, row block by row block --------------------------
        // Row blocks of the wave's 32-row fragments (tail_first, tail_len):
        // with four or more fragments the first row block takes two (each
        // step then reads two image and FN filter fragments for 2 * FN
        // products, which keeps the LDS read rate under what the CU serves)
        // and the others one, so the last row block, whose stores are
        // exposed, is small.  Steps s = x * 18 + (t * 2 + ks): row block x,
        // tap t, k-step ks.  The image and filter fragments of step s+D are
        // read during step s (all nine taps of the block are in the ring).
        // The stores of row block x-1 go out spread over the steps of row
        // block x.
        const int fb = (nblk - 1) & 1;
        if (nend == 0) {
            // a single block: the main loop, which loads taps 3 .. 8 of block
            // 0, did not run
#pragma unroll
            for (int t = 3; t < kTaps; ++t)
#pragma unroll
                for (int i = 0; i < BL; ++i)
                    dma_filter(0, t, i);
        }
        wait_vm_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
        CONV_I8_PHASE(ph6);   // tail starts
        constexpr int NRB = tail_blocks(FM);
        constexpr int RBM = tail_len(FM, 0);   // fragments of the largest row block
        constexpr int NSTEP = kTaps * KS;
        constexpr int TOTAL = NRB * NSTEP;
        constexpr int D = PIX_J ? 2 : 3;   // (three would spill with the pixel-lane epilogue)
        constexpr int NR = D + 1;   // the reads D steps ahead must not land in the slot in use
        v4i ab[NR][RBM];
        v4i bb[NR][FN];
        auto read_step = [&](auto sc) {
            constexpr int s2 = decltype(sc)::value;
            constexpr int x = s2 / NSTEP, r = s2 % NSTEP;
            constexpr int t = r / KS, ks = r % KS;
#pragma unroll
            for (int i = 0; i < tail_len(FM, x); ++i)
                ab[s2 % NR][i] = *(const v4i *)&fbuf[fb * FBUF + a_lane[tail_first(FM, x) + i][ks] + tap_read(t)];
#pragma unroll
            for (int y = 0; y < FN; ++y)
                bb[s2 % NR][y] = b_frag(t, y, ks);
        };
        const __amdgpu_buffer_rsrc_t out_rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void *)a.out, (short)0, a.out_range, kRsrcWord3);
        // MODE 0: lanes walk channels, equally spaced pixels, every row of the
        // tile inside the problem: a lane base plus a uniform offset per store.
        // MODE 1: lanes walk channels, pixel offsets from the table (or rows
        // past the problem).  MODE 2: lanes walk pixels.
        const int kk0 = n0 + wn + (lane & 31);
        const int mrow0 = wm + 4 * (lane >> 5);
        // bytes per output element: INT32 sums, or INT8 through the
        // requantising epilogue (one byte store per value)
        const int es = a.q8 ? 1 : 4;
        const bool relu = a.q_relu != 0;
        // MODE 0 lane bases, computed once (the opaque asm keeps the compiler
        // from recomputing them at every store)
        int obase[FN];
#pragma unroll
        for (int y = 0; y < FN; ++y) {
            const int kk = kk0 + y * 32;
            obase[y] = kk < a.K ? ((m0 + mrow0) * a.pix_stride + kk * a.oK) * es : kOutOfRange;
            asm volatile("" : "+v"(obase[y]));
        }
        // requantisation of a lane's channel columns (lanes walk channels;
        // lanes past K read channel K-1 and store nothing)
        float qs[FN], qb[FN];
#pragma unroll
        for (int y = 0; y < FN; ++y) {
            qs[y] = 0.0f;
            qb[y] = 0.0f;
            if (!PIX_J && a.q8) {
                const int kc = min(kk0 + y * 32, a.K - 1);
                qs[y] = a.q_scale ? a.q_scale[kc] : a.q_alpha;
                qb[y] = a.q_bias ? a.q_bias[kc] : 0.0f;
            }
        }
        // MODE 2 (lanes walk pixels): each lane's pixel offset per row block,
        // or -1 past the problem
        int pixo[PIX_J ? FM : 1];
        if constexpr (PIX_J) {
#pragma unroll
            for (int x = 0; x < FM; ++x) {
                const int m = m0 + wm + x * 32 + (lane & 31);
                const int n = udiv(m, a.d_pq);
                const int rem = m - n * a.PQ;
                const int p = udiv(rem, a.d_q);
                const int q = rem - p * a.Q;
                pixo[x] = m < a.M ? n * a.oN + p * a.oP + q * a.oQ + a.out0 : -1;
                asm volatile("" : "+v"(pixo[x]));
            }
        }
        auto store_one = [&](auto modec, auto q8c, int x, int y, int v, int value) {
            constexpr int MODE = decltype(modec)::value;
            constexpr bool Q8 = decltype(q8c)::value;
            constexpr int ES = Q8 ? 1 : 4;
            const int rv = 8 * (v >> 2) + (v & 3);   // row of value v within its 32-row block
            auto put = [&](int voff, int soff, float sc, float bi) {
                if constexpr (Q8)
                    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)requant_i8(value, sc, bi, relu), out_rsrc,
                                                         voff, soff, kOutStoreStream);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(value, out_rsrc, voff, soff, kOutStoreStream);
            };
            if constexpr (MODE == 0) {
                put(obase[y], (x * 32 + rv) * a.pix_stride * ES, qs[y], qb[y]);
            } else if constexpr (MODE == 1) {
                const int kk = kk0 + y * 32;
                const int r = mrow0 + x * 32 + rv;
                int off = kOutOfRange;
                if (a.pix_linear) {
                    const int m = m0 + r;
                    off = (kk < a.K && m < a.M) ? (m * a.pix_stride + kk * a.oK) * ES : kOutOfRange;
                } else {
                    const int po = out_row[r];
                    off = (kk < a.K && po >= 0) ? (po + kk * a.oK) * ES : kOutOfRange;
                }
                put(off, 0, qs[y], qb[y]);
            } else {
                const int kk = n0 + wn + y * 32 + 4 * (lane >> 5) + rv;
                const int off = (pixo[x] >= 0 && kk < a.K) ? (pixo[x] + kk * a.oK) * ES : kOutOfRange;
                float sc = 0.0f, bi = 0.0f;
                if constexpr (Q8) {
                    // lanes walk pixels: the channel changes with the value
                    const int kc = min(kk, a.K - 1);
                    sc = a.q_scale ? a.q_scale[kc] : a.q_alpha;
                    bi = a.q_bias ? a.q_bias[kc] : 0.0f;
                }
                put(off, 0, sc, bi);
            }
        };
        // In a row block of one fragment, odd steps accumulate into a second
        // set (added in at the end of the row block): the row block has only
        // FN accumulators, and alternating two sets keeps dependent MFMAs
        // 2 * FN issues apart.
        v16i acc2[FN];
        auto run_tail = [&](auto modec, auto q8c) {
            static_for<0, D>([&](auto sc) { read_step(sc); });
            static_for<0, TOTAL>([&](auto sc) {
                constexpr int st = decltype(sc)::value;
                constexpr int x = st / NSTEP, r = st % NSTEP;
                constexpr int L = tail_len(FM, x), F = tail_first(FM, x);
                if constexpr (st + D < TOTAL)
                    read_step(std::integral_constant<int, st + D>{});
#pragma unroll
                for (int i = 0; i < L; ++i)
#pragma unroll
                    for (int y = 0; y < FN; ++y) {
                        const v4i &fa = ab[st % NR][i];
                        const v4i &fbm = bb[st % NR][y];
                        v16i &c0 = acc[F + i][y];
                        if constexpr (L > 1 || r % 2 == 0) {
                            c0 = PIX_J ? __builtin_amdgcn_mfma_i32_32x32x32_i8(fbm, fa, c0, 0, 0, 0)
                                       : __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, fbm, c0, 0, 0, 0);
                        } else {
                            const v16i c = r == 1 ? v16i{} : acc2[y];
                            acc2[y] = PIX_J ? __builtin_amdgcn_mfma_i32_32x32x32_i8(fbm, fa, c, 0, 0, 0)
                                            : __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, fbm, c, 0, 0, 0);
                        }
                    }
                if constexpr (L == 1 && r == NSTEP - 1) {
#pragma unroll
                    for (int y = 0; y < FN; ++y)
                        acc[F][y] += acc2[y];
                }
                // stores of the previous row block: 16 * FN values per
                // fragment, spread over the 18 steps
                if constexpr (x >= 1) {
                    constexpr int PF = tail_first(FM, x - 1);
                    constexpr int NV = 16 * FN * tail_len(FM, x - 1);
                    constexpr int lo = r * NV / NSTEP, hi = (r + 1) * NV / NSTEP;
#pragma unroll
                    for (int e = lo; e < hi; ++e) {
                        const int f = PF + e / (16 * FN), y = e / 16 % FN;
                        store_one(modec, q8c, f, y, e % 16, acc[f][y][e % 16]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            });
#pragma unroll
            for (int e = 0; e < 16 * FN * tail_len(FM, NRB - 1); ++e) {
                const int f = tail_first(FM, NRB - 1) + e / (16 * FN), y = e / 16 % FN;
                store_one(modec, q8c, f, y, e % 16, acc[f][y][e % 16]);
            }
        };
        auto run_mode = [&](auto q8c) {
            if (PIX_J)
                run_tail(std::integral_constant<int, 2>{}, q8c);
            else if (a.pix_linear && m0 + TM <= a.M)
                run_tail(std::integral_constant<int, 0>{}, q8c);
            else
                run_tail(std::integral_constant<int, 1>{}, q8c);
        };
        if (a.q8)
            run_mode(std::true_type{});
        else
            run_mode(std::false_type{});
    }
    CONV_I8_PHASE_FLUSH(a);
}




}  // namespace convi8
