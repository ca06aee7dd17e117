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

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convi8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

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
    int oN, oK, oP, oQ;  // output strides in elements (one launch spans < 2^31 bytes)
    int out_range;       // bytes addressable from out
    int pix_linear;      // output pixel m = (n*P + p)*Q + q lives at m*pix_stride
    int pix_stride;
    int nstages;         // stages of BK bytes of the inner dimension
    int cc;              // C / 16
    float inv_cc, inv_s; // 1.0f / cc, 1.0f / S (flat order index split)
    int tiles_n;         // column tiles
    int tiles;           // total tiles
};

// s_waitcnt immediate (gfx9 encoding): wait until at most `vm` vector-memory
// operations are outstanding and all LDS operations are done.
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0()
{
    static_assert(VM >= 0 && VM < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (0 << 8));
}

template <int BK>
__device__ __forceinline__ int swizzle_chunk(int row, int chunk)
{
    // 64-byte rows (4 chunks) use row bits 1..3, 128-byte rows (8 chunks) row
    // bits 0..3: any 8 (32 banks) or 16 (64 banks) consecutive rows reading one
    // logical chunk land on distinct banks.
    if constexpr (BK == 64)
        return chunk ^ (((row >> 1) ^ (row >> 2)) & 3);
    else
        return chunk ^ ((row ^ (row >> 1)) & 7);
}

// Buffer resource (gfx9 layout): base address, stride 0, byte range,
// format word.  Built from kernel arguments, so it is wave-uniform.
__device__ __forceinline__ v4i make_rsrc(const void *p, int range)
{
    const unsigned long long a = (unsigned long long)p;
    v4i d;
    d.x = (int)(unsigned)a;
    d.y = (int)((a >> 32) & 0xFFFFu);
    d.z = range;
    d.w = kRsrcWord3;
    return d;
}

// 16 bytes per lane from buffer offset `voff` straight into LDS: lane i's
// bytes land at lds + 16*i (a wave fills one contiguous 1 KiB block).  An
// offset outside the range writes zeros.  Written as inline assembly so the
// compiler does not add a wait for these loads before every LDS read (it
// cannot tell which ring slot they fill); the kernel counts them itself with
// s_waitcnt vmcnt.
__device__ __forceinline__ void load16_to_lds(v4i rsrc, unsigned lds_addr, int voff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rsrc) : "memory", "m0");
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ unsigned lds_address(const void *p)
{
    return (unsigned)(unsigned long long)(lds_void *)p;
}

// floor(n / d) for 0 <= n < 2^22 and 1 <= d < 2^22, with inv = 1.0f / d
// rounded to float: the quotient of n + 1/2 stays more than 1/(2d) away
// from the next integer while the float error is below n / (d * 2^23).
__device__ __forceinline__ int fdiv(int n, int d, float inv)
{
    (void)d;
    return (int)(((float)n + 0.5f) * inv);
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

template <int TM, int TN, int BK, int NS, bool FLAT, bool PIX_J>
__global__ __launch_bounds__(256) void conv_igemm_kernel(IgemmArgs a)
{
    constexpr int CPS = BK / 16;            // 16-byte chunks per row per stage
    constexpr int RPI = 64 / CPS;           // rows one wave-wide load fills
    constexpr int AL = TM / (4 * RPI);      // image-row loads per thread per stage
    constexpr int BL = TN / (4 * RPI);      // filter-row loads per thread per stage
    constexpr int LPS = AL + BL;            // loads per thread per stage
    constexpr int A_BYTES = TM * BK, STAGE = (TM + TN) * BK;
    constexpr int WM = TM / 2, WN = TN / 2; // wave tile
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int KS = BK / 32;             // MFMA k-steps per stage
    constexpr int NMF = KS * FM * FN;       // MFMAs per stage per wave
    constexpr int NRD = KS * (FM + FN);     // fragment reads per stage per wave
    static_assert(AL >= 1 && BL >= 1 && FM >= 1 && FN >= 1, "tile too small");
    static_assert(TM % (4 * RPI) == 0 && TN % (4 * RPI) == 0, "tile rows must fill wave loads");
    static_assert(NS >= 2 && (NS - 2) * LPS < 64, "pipeline depth");

    __shared__ __attribute__((aligned(1024))) int8_t smem[NS * STAGE];
    __shared__ int out_row[PIX_J ? 1 : TM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = xcd_tile(blockIdx.x, a.tiles);
    const int m0 = (tile / a.tiles_n) * TM;
    const int n0 = (tile % a.tiles_n) * TN;

    // ---- load geometry: load i of this wave fills LDS block i*4+wave (rows
    // (i*4+wave)*RPI ...), lane -> row + lane/CPS, physical chunk lane%CPS.
    // The logical chunk j it must fetch depends only on row bits that are
    // the same for every i, so j is one per thread.
    const int row0 = wave * RPI + lane / CPS;
    const int j = swizzle_chunk<BK>(row0, lane % CPS);

    int a_h0[AL], a_w0[AL], a_off[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int m = m0 + row0 + i * 4 * RPI;
        if (m < a.M) {
            const int n = m / a.PQ;
            const int rem = m - n * a.PQ;
            const int p = rem / a.Q;
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
    int b_off[BL];
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        const int k = n0 + row0 + i * 4 * RPI;
        b_off[i] = k < a.K ? k * a.fK + (FLAT ? 0 : j * 16) : kOutOfRange;
    }
    if constexpr (!PIX_J) {
        if (!a.pix_linear) {
            for (int i = tid; i < TM; i += 256) {
                const int m = m0 + i;
                int o = -1;
                if (m < a.M) {
                    const int n = m / a.PQ;
                    const int rem = m - n * a.PQ;
                    const int p = rem / a.Q;
                    const int q = rem - p * a.Q;
                    o = n * a.oN + p * a.oP + q * a.oQ;
                }
                out_row[i] = o;
            }
        }
    }

    // ---- inner-dimension position of the next stage to load ---------------
    // blocked: (r, s, cpos) uniform, cpos = channel-block byte offset, stepped
    // with selects; flat: each thread's chunk index g = stage*CPS + j is split
    // into (r, s, c16) afresh for every stage.
    int r = 0, s = 0, cpos = 0;
    int issued = 0;

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
        const bool live = issued < a.nstages && (!FLAT || r < a.R);
        rdh = live ? r * a.dilH : -0x20000000;  // dead stage: every row fails the bounds test
        sdw = s * a.dilW;
        itoff = rdh * a.sH + sdw * a.sW + cpos;
        ftoff = live ? r * a.fR + s * a.fS + cpos : kOutOfRange;
        lbase = smem_lds + slot * STAGE + wave * 1024;
    };
    auto dma_one = [&](int i) {  // i < LPS, compile-time after unrolling
        if (i < AL) {
            const int h = a_h0[i] + rdh, w = a_w0[i] + sdw;
            const bool ok = ((unsigned)h < (unsigned)a.H) & ((unsigned)w < (unsigned)a.W);
            load16_to_lds(img_rsrc, lbase + i * 4096, ok ? a_off[i] + itoff : kOutOfRange);
        } else {
            // b_off (column past K) or ftoff (dead stage) negative: out of range
            const int b = i - AL;
            load16_to_lds(flt_rsrc, lbase + A_BYTES + b * 4096,
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

    const int wm = (wave >> 1) * WM;
    const int wn = (wave & 1) * WN;

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
    constexpr int NOTHER = LPS + NRD;
    int cur_slot = 0;
    auto body = [&](int buf) {
        wait_vm_lgkm0<(NS - 2) * LPS>();  // own loads of stage it+1 landed; frag[buf] read
        __builtin_amdgcn_s_barrier();       // all waves: stage it+1 visible, slot it%NS free
        __builtin_amdgcn_sched_barrier(0);
        begin_stage(cur_slot);
        const int nslot = cur_slot + 1 == NS ? 0 : cur_slot + 1;
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
    // An odd stage count runs one extra all-zero stage, so the loop body
    // (two stages, one per fragment buffer) has no branch inside it.
    const int nloop = (a.nstages + 1) & ~1;
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
    // 32x32 accumulator layout: lane l, value v -> MFMA row 8*(v/4) + 4*(l/32) + v%4,
    // MFMA column l%32.  Rows come from the first MFMA operand.  Elements past
    // M or K get an out-of-range offset and the buffer store drops them.
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.out, (short)0, a.out_range, kRsrcWord3);
#pragma unroll
    for (int x = 0; x < FM; ++x) {
        int pix_off_j = 0;
        bool pix_ok_j = true;
        if constexpr (PIX_J) {
            const int m = m0 + wm + x * 32 + (lane & 31);
            pix_ok_j = m < a.M;
            const int n = m / a.PQ;
            const int rem = m - n * a.PQ;
            const int p = rem / a.Q;
            const int q = rem - p * a.Q;
            pix_off_j = n * a.oN + p * a.oP + q * a.oQ;
        }
#pragma unroll
        for (int y = 0; y < FN; ++y) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int mrow = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int mcol = lane & 31;
                int off;
                if constexpr (PIX_J) {
                    const int kk = n0 + wn + y * 32 + mrow;
                    off = (pix_ok_j && kk < a.K) ? (pix_off_j + kk * a.oK) * 4 : kOutOfRange;
                } else {
                    const int prow = wm + x * 32 + mrow;
                    const int kk = n0 + wn + y * 32 + mcol;
                    int po;
                    bool ok;
                    if (a.pix_linear) {
                        ok = m0 + prow < a.M;
                        po = (m0 + prow) * a.pix_stride;
                    } else {
                        po = out_row[prow];
                        ok = po >= 0;
                    }
                    off = (ok && kk < a.K) ? (po + kk * a.oK) * 4 : kOutOfRange;
                }
                __builtin_amdgcn_raw_buffer_store_b32(acc[x][y][v], out_rsrc, off, 0, 0);
            }
        }
    }
}

}  // namespace convi8
