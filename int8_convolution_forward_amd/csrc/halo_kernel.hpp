// Footprint ("halo") variant of the INT8 implicit-GEMM convolution for gfx950.
//
// For a filter with several taps, the im2col rows of neighbouring taps read
// largely the same input pixels.  This kernel loads, once per block of 64
// channels, the whole input region a tile of TM consecutive output pixels
// touches (its footprint: the padded input rows from the first pixel's top
// tap to the last pixel's bottom tap, across the full padded width, zeros for
// padding) into LDS, and builds the image operand of every tap (r, s) from it
// by reading pixel  base(m) + r*dil_h*Wf + s*dil_w  for output pixel m.  Only
// the filter still streams one (tap, channel block) stage at a time through
// the NS-slot LDS ring, as in the im2col kernel.
//
// Schedule (stage = one (channel block c, tap t) pair, C*R*S/64 stages): the
// footprint of block c+1 is loaded into the other of two footprint buffers in
// pieces, one piece riding along with the filter loads of each of the stages
// t = NS-1 ... NS-1+npieces-1 of block c.  With the ring issuing stage s while
// stage s-NS is multiplied, the first piece leaves only after every wave has
// finished reading block c-1 (which used the same buffer), and the last piece
// lands before the first fragment of block c+1 is read.  Every stage issues
// the same number of loads (stages without a piece send theirs out of range
// into a scratch block), so one compile-time s_waitcnt serves every stage.
//
// Footprint pixel fp occupies 64 bytes of LDS at fp*64, its 16-byte chunks
// permuted by bits 2..3 of fp: 16 consecutive pixels read by one LDS read
// cycle then cover all 64 banks (pixels with the same fp mod 4 get distinct
// chunk slots).
#pragma once

#include "kernel_common.hpp"

namespace convi8 {

__device__ __forceinline__ int fp_swizzle(int fp, int chunk)
{
    return chunk ^ ((fp >> 2) & 3);
}

template <int TM, int TN, int NS, int FLS, int FPIX, int WGM, int WGN, bool PIX_J>
__global__ __launch_bounds__(64 * WGM * WGN) void conv_halo_kernel(IgemmArgs a)
{
    constexpr int NW = WGM * WGN;           // waves per workgroup
    constexpr int GB = NW * 1024;           // bytes one workgroup-wide load fills
    constexpr int BK = 64;                  // channels (bytes) per stage
    constexpr int BL = TN / (NW * 16);      // filter-row loads per thread per stage
    constexpr int LPS = BL + FLS;           // loads per thread per stage
    constexpr int B_BYTES = TN * BK;        // one ring slot
    constexpr int FBUF = FPIX * 64;         // one footprint buffer
    constexpr int NG = FBUF / GB;           // load groups per footprint buffer
    constexpr int WM = TM / WGM, WN = TN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int KS = BK / 32;
    constexpr int NMF = KS * FM * FN;
    constexpr int NRD = KS * (FM + FN);
    static_assert(BL >= 1 && FM >= 1 && FN >= 1 && NG % FLS == 0 && TN % (NW * 16) == 0, "tile shape");
    static_assert(NS >= 2 && (NS - 2) * LPS + NG < 64, "pipeline depth");

    __shared__ __attribute__((aligned(1024))) int8_t ring[NS * B_BYTES];
    __shared__ __attribute__((aligned(1024))) int8_t fbuf[2 * FBUF];
    __shared__ __attribute__((aligned(1024))) int8_t scratch[GB];
    __shared__ int out_row[PIX_J ? 1 : TM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = xcd_tile(blockIdx.x, a.tiles);
    const int m0 = (tile / a.tiles_n) * TM;
    const int n0 = (tile % a.tiles_n) * TN;
    const int wm = (wave / WGN) * WM;
    const int wn = (wave % WGN) * WN;

    // ---- footprint geometry of this tile (uniform) ------------------------
    const int m_last = min(m0 + TM, a.M) - 1;
    const int n_a = udiv(m0, a.d_pq);
    const int p_a = udiv(m0 - n_a * a.PQ, a.d_q);
    const int hp_a = p_a * a.strH;          // first footprint row, padded coords of image n_a
    const int n_b = udiv(m_last, a.d_pq);
    const int p_b = udiv(m_last - n_b * a.PQ, a.d_q);
    const int frows = (n_b - n_a) * a.Hp + p_b * a.strH + (a.R - 1) * a.dilH - hp_a + 1;
    const int fpix = frows * a.Wf;          // footprint pixels (the host keeps it <= capacity)

    // ---- image operand: footprint pixel of each MFMA row at tap (0, 0) ----
    int aidx[FM];
#pragma unroll
    for (int x = 0; x < FM; ++x) {
        const int m = m0 + wm + x * 32 + (lane & 31);
        int idx = 0;
        if (m < a.M) {
            const int n = udiv(m, a.d_pq);
            const int rem = m - n * a.PQ;
            const int p = udiv(rem, a.d_q);
            const int q = rem - p * a.Q;
            idx = ((n - n_a) * a.Hp + p * a.strH - hp_a) * a.Wf + q * a.strW;
        }
        aidx[x] = idx;
    }

    // ---- footprint loads: group g of this wave fills LDS bytes
    // g*GB + wave*1024 + lane*16, i.e. pixel g*GB/64 + wave*16 + lane/4,
    // physical chunk lane%4; the logical chunk depends on pixel bits 2..3,
    // which are lane bits 4..5 for every g.
    const int jf = fp_swizzle(lane >> 2, lane & 3);
    // buffer offset of this thread's 16 bytes of group g for channel block c
    auto foot_off = [&](int c, int g) -> int {
        const int fp = g * (GB / 64) + wave * 16 + (lane >> 2);
        const int fr = fdiv(fp, a.Wf, a.inv_wf);
        const int fc = fp - fr * a.Wf;
        const int hr = hp_a + fr;
        const int dn = fdiv(hr, a.Hp, a.inv_hp);
        const int h = hr - dn * a.Hp - a.padH;
        const int w = fc - a.padW;
        const bool ok = (fp < fpix) & ((unsigned)h < (unsigned)a.H) & ((unsigned)w < (unsigned)a.W) &
                        (c * 4 + jf < a.cc);
        return ok ? (n_a + dn) * a.sN + h * a.sH + w * a.sW + (c * 4 + jf) * 16 : kOutOfRange;
    };

    // ---- filter loads (as in the im2col kernel) ---------------------------
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

    const v4i img_rsrc = make_rsrc(a.img, a.img_range);
    const v4i flt_rsrc = make_rsrc(a.flt, a.flt_range);
    const unsigned ring_lds = lds_address(ring);
    const unsigned fbuf_lds = lds_address(fbuf);
    const unsigned scratch_lds = lds_address(scratch) + wave * 1024;
    const int RS = a.R * a.S;

    // footprint load of group g for channel block c into buffer c % 2
    auto foot_one = [&](int c, int g) {
        load16_to_lds(img_rsrc, fbuf_lds + (c & 1) * FBUF + g * GB + wave * 1024, foot_off(c, g));
    };

    // issue side: stage (ic, it_) = (channel block, tap index), tap (ir, is)
    int ic = 0, itap = 0, ir = 0, is = 0, issued = 0;
    int ftoff = 0;
    unsigned lslot = 0;
    bool piece = false;
    int pg = 0;
    auto begin_stage = [&](int slot) {
        const bool live = issued < a.nstages;
        ftoff = live ? ir * a.fR + is * a.fS + ic * 64 : kOutOfRange;
        lslot = ring_lds + slot * B_BYTES + wave * 1024;
        // footprint piece of block ic+1 rides on taps NS-1 .. NS-2+npieces
        const int pc = itap - (NS - 1);
        piece = pc >= 0 && pc < a.npieces;
        pg = pc * FLS;
    };
    auto dma_one = [&](int i) {  // i < LPS
        if (i < BL) {
            load16_to_lds(flt_rsrc, lslot + i * GB,
                          (b_off[i] | ftoff) < 0 ? kOutOfRange : b_off[i] + ftoff);
        } else {
            // group pg+f of the next block's footprint, or an out-of-range
            // load into the scratch block on stages that carry no piece (and
            // past the last block, where the channel test fails)
            const int f = i - BL;
            const int g = pg + f;
            const unsigned dst = piece ? fbuf_lds + ((ic + 1) & 1) * FBUF + g * GB + wave * 1024
                                       : scratch_lds;
            load16_to_lds(img_rsrc, dst, piece ? foot_off(ic + 1, g) : kOutOfRange);
        }
    };
    auto end_stage = [&]() {
        ++issued;
        const int s1 = is + 1;
        const bool ws = s1 == a.S;
        is = ws ? 0 : s1;
        const int r1 = ir + (ws ? 1 : 0);
        const bool wr = r1 == a.R;
        ir = wr ? 0 : r1;
        const int t1 = itap + 1;
        const bool wt = t1 == RS;
        itap = wt ? 0 : t1;
        ic += wt ? 1 : 0;
    };
    auto issue_stage = [&](int slot) {
        begin_stage(slot);
#pragma unroll
        for (int i = 0; i < LPS; ++i)
            dma_one(i);
        end_stage();
    };

    // read side: the stage whose fragments are fetched next
    int rc = 0, rr = 0, rs_ = 0, rtap = 0;
    auto read_step = [&]() {
        const int s1 = rs_ + 1;
        const bool ws = s1 == a.S;
        rs_ = ws ? 0 : s1;
        const int r1 = rr + (ws ? 1 : 0);
        const bool wr = r1 == a.R;
        rr = wr ? 0 : r1;
        const int t1 = rtap + 1;
        const bool wt = t1 == RS;
        rtap = wt ? 0 : t1;
        rc += wt ? 1 : 0;
    };

    v16i acc[FM][FN];
#pragma unroll
    for (int x = 0; x < FM; ++x)
#pragma unroll
        for (int y = 0; y < FN; ++y)
            acc[x][y] = v16i{};

    v4i frag[2][KS][FM + FN];
    int tap_off = 0;
    const int8_t *fb = fbuf;
    auto read_setup = [&]() {
        tap_off = rr * a.dilH * a.Wf + rs_ * a.dilW;
        fb = fbuf + (rc & 1) * FBUF;
    };
    auto read_one = [&](int buf, int slot, int i) {  // i < NRD
        const int ks = i / (FM + FN), f = i % (FM + FN);
        const int ch = ks * 2 + (lane >> 5);
        if (f < FM) {
            const int fp = aidx[f] + tap_off;
            frag[buf][ks][f] = *(const v4i *)&fb[fp * 64 + fp_swizzle(fp, ch) * 16];
        } else {
            const int row = wn + (f - FM) * 32 + (lane & 31);
            frag[buf][ks][f] =
                *(const v4i *)&ring[slot * B_BYTES + row * 64 + swizzle_chunk<64>(row, ch) * 16];
        }
    };
    auto mfma_one = [&](int buf, int t) {  // t < NMF
        const int ks = t / (FM * FN), x = (t / FN) % FM, y = t % FN;
        acc[x][y] = PIX_J
            ? __builtin_amdgcn_mfma_i32_32x32x32_i8(frag[buf][ks][FM + y], frag[buf][ks][x], acc[x][y], 0, 0, 0)
            : __builtin_amdgcn_mfma_i32_32x32x32_i8(frag[buf][ks][x], frag[buf][ks][FM + y], acc[x][y], 0, 0, 0);
    };

    constexpr int NOTHER = LPS + NRD;
    int cur_slot = 0;
    auto body = [&](int buf) {
        wait_vm_lgkm0<(NS - 2) * LPS>();   // own loads of stage it+1 landed; frag[buf] read
        __builtin_amdgcn_s_barrier();        // all waves: stage it+1 visible, slot it%NS free
        __builtin_amdgcn_sched_barrier(0);
        begin_stage(cur_slot);
        const int nslot = cur_slot + 1 == NS ? 0 : cur_slot + 1;
        read_step();
        read_setup();
#pragma unroll
        for (int t = 0; t < NMF; ++t) {
            mfma_one(buf, t);
#pragma unroll
            for (int o = t * NOTHER / NMF; o < (t + 1) * NOTHER / NMF; ++o) {
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
    const int nloop = (a.nstages + 1) & ~1;
    if (nloop > 0) {
        // footprint of block 0, then the first NS filter stages (the last of
        // them may already carry a piece of block 1's footprint)
#pragma unroll
        for (int g = 0; g < NG; ++g)
            foot_one(0, g);
#pragma unroll
        for (int st = 0; st < NS; ++st)
            issue_stage(st);
        wait_vm_lgkm0<(NS - 1) * LPS>();
        __builtin_amdgcn_s_barrier();
        read_setup();
#pragma unroll
        for (int i = 0; i < NRD; ++i)
            read_one(0, 0, i);
        for (int it = 0; it < nloop; it += 2) {
            body(0);
            body(1);
        }
        wait_vm_lgkm0<0>();
    }
    __syncthreads();

    store_tile<FM, FN, PIX_J>(a, acc, m0, n0, wm, wn, lane, out_row);
}

}  // namespace convi8
