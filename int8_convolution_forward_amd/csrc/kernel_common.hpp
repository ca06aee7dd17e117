// Shared pieces of the INT8 conv_fprop kernels for gfx950 (CDNA4): kernel
// arguments, buffer-resource and direct-to-LDS load helpers, LDS swizzles,
// division by launch-invariant divisors, the XCD-aware tile order and the
// epilogues (INT32 sums, or requantised INT8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convi8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// Buffer offset that always lies outside a resource (ranges are < 2^31).
constexpr int kOutOfRange = (int)0x80000000u;
// Buffer resource word 3 for gfx9-family raw buffer access (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the output stores when the lanes of a store walk a
// unit-stride output dimension (IgemmArgs::out_nt): non-temporal, since the
// results are not read again by this kernel and streaming whole lines
// shortens the write-back at the end.  Stores scattered over many lines
// (e.g. a weight gradient written through a filter layout whose contiguous
// dim is the slowest part of the row index) keep the default policy, so the
// L2 merges the pieces of each line before it writes them back.
constexpr int kOutStoreStream = 2;
constexpr int kOutStoreDefault = 0;

// floor(n / d) for 0 <= n < 2^31 as (umulhi(n, m) + n) >> l, with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1 (computed on the host).
struct Divisor {
    unsigned m;
    int l;
};

__device__ __forceinline__ int udiv(int n, Divisor d)
{
    return (int)((__umulhi((unsigned)n, d.m) + (unsigned)n) >> d.l);
}

struct IgemmArgs {
    const int8_t *img;   // image, channel-innermost; (0,0,0,0) at img
    const int8_t *flt;   // filter K,R,S,C with C innermost
    int32_t *out;        // output element (0,0,0,0); int8_t when q8 is set
    int img_range;       // bytes addressable from img (buffer range)
    int flt_range;       // bytes addressable from flt
    int N, H, W, C;      // C: channels as stored (multiple of 16)
    int sN, sH, sW;      // image strides in bytes (channel stride is 1)
    int K, R, S;
    int fK, fR, fS;      // filter strides in bytes (channel stride is 1); fR, fS are
                         // negative for true convolution (taps read in reverse)
    int flt0;            // byte offset of tap (r, s) = (0, 0) as the kernels read it:
                         // 0, or (R-1)*|fR| + (S-1)*|fS| for true convolution
    int P, Q, PQ, M;     // M = N*P*Q
    int strH, strW, dilH, dilW, padH, padW;
    int oN, oK, oP, oQ;  // output strides in elements (one launch spans < 2^31 bytes);
                         // oP, oQ negative when rows and columns are written reversed
    int out0;            // element offset of output (p, q) = (0, 0) within its image:
                         // 0, or (P-1)*|oP| + (Q-1)*|oQ| for reversed rows and columns
    int out_range;       // bytes addressable from out
    int pix_linear;      // output pixel m = (n*P + p)*Q + q lives at m*pix_stride
    int pix_stride;
    int nstages;         // stages of BK bytes of the inner dimension
    int cc;              // C / 16
    float inv_cc, inv_s; // 1.0f / cc, 1.0f / S (flat order index split)
    int tiles_n;         // column tiles
    int tiles;           // total tiles
    Divisor d_pq, d_q;   // division by P*Q and by Q (pixel index -> n, p, q)
    Divisor d_tn;        // division by tiles_n (tile index -> row tile, column tile)
    // footprint kernel only
    int Hp;              // padded image height H + pre_h + post_h
    int Wf;              // footprint width (Q-1)*stride_w + (S-1)*dil_w + 1
    int Pr;              // footprint row pitch in LDS, 16-byte slots
    float inv_pr, inv_hp;
    int ncblk;           // channel blocks of 64
    int kmaj;            // 3x3 ring kernel: the filter is read k-major (output channels
                         // contiguous, fK the stride of one input channel); picks the
                         // instantiation on the host
    // requantising INT8 epilogue (q8 != 0)
    const float *q_scale; // K per-channel scales, or null: q_alpha for every channel
    const float *q_bias;  // K per-channel biases, or null: none
    float q_alpha;
    int q_relu;
    int q8;
    int q8_pack;          // channel stride 1, K, pix_stride and out 4-byte multiples:
                          // four channels of a pixel go out as one dword
    // split of the inner dimension over gridDim.y (im2col kernel): split z
    // runs stages [z*kchunk, min((z+1)*kchunk, nstages)) and adds its partial
    // sums to the (zeroed) output with int32 atomics; ksplit 1: plain stores
    int ksplit;
    int kchunk;
    int out_nt;           // lanes of a store walk a unit-stride output dim: the
                          // im2col and 1x1 kernels are launched with streaming stores
    // split with partial outputs (part != 0): split z stores plain partial
    // sums into its own copy of the output at out + z*part_stride elements
    // (a reduction kernel adds the copies); part == 0: atomics into out
    int part;
    long long part_stride;
#ifdef CONV_I8_PHASE_CLOCK
    long long *phase_clk;  // per-workgroup phase stamps (instrumented builds only)
#endif
};

// Per-workgroup phase stamps of the 3x3 ring kernel, compiled in only with
// CONV_I8_PHASE_CLOCK (int8_convolution_forward_amd/phase_clock.py builds and
// runs such a library): stamp i (shader clock, s_memtime; 0 entry, 1
// arguments loaded, 2 prologue loads start, 3 footprint of block 0 issued,
// 4 main loop starts, 5 main loop done, 6 tail starts, 11 end) goes to
// phase_clk[16 * workgroup + i], the constant 100 MHz clock at the start and
// the end to slots 14 and 15, all written by thread 0 at the end.  The
// stamps are plain locals of the kernel body (an object holding them ended
// up in scratch memory); without the macro every hook expands to nothing.
#ifdef CONV_I8_PHASE_CLOCK
#define CONV_I8_PHASE_DECL                                                                              \
    long long ph0 = __builtin_amdgcn_s_memtime(), ph_rt0 = __builtin_amdgcn_s_memrealtime(), ph1 = 0, \
              ph2 = 0, ph3 = 0, ph4 = 0, ph5 = 0, ph6 = 0
#define CONV_I8_PHASE(v) v = __builtin_amdgcn_s_memtime()
#define CONV_I8_PHASE_FLUSH(a)                                                                          \
    do {                                                                                                \
        const long long ph11 = __builtin_amdgcn_s_memtime();                                            \
        if ((a).phase_clk && threadIdx.x == 0) {                                                        \
            long long *o = (a).phase_clk + 16 * blockIdx.x;                                             \
            o[0] = ph0; o[1] = ph1; o[2] = ph2; o[3] = ph3; o[4] = ph4; o[5] = ph5; o[6] = ph6;         \
            o[11] = ph11; o[14] = ph_rt0; o[15] = __builtin_amdgcn_s_memrealtime();                     \
        }                                                                                               \
    } while (0)
#else
#define CONV_I8_PHASE_DECL
#define CONV_I8_PHASE(v)
#define CONV_I8_PHASE_FLUSH(a)
#endif

// Requantising INT8 epilogue of one exact sum: the sum as a float, one fused
// multiply-add with the channel's scale and bias, ReLU if asked, round half to
// even, saturate to [-128, 127] (a NaN becomes 0).  With scale 1 it is the
// clamped INT8 store of the naive loop in "Building a From-Scratch INT8
// Strided Convolution Kernel" (step 2); the ReLU and scale are the
// quantisation step its roadmap fuses.
__device__ __forceinline__ int requant_i8(int acc, float s, float b, bool relu)
{
    const float v = __builtin_fmaf((float)acc, s, b);
    // v_cvt_i32_f32 saturates (±inf and |v| >= 2^31 go to the int32 limits)
    // and turns a NaN (an infinite scale or bias meeting a zero or opposite
    // term) into 0, so after rounding half to even the integer median does
    // ReLU and the clamp to [-128, 127] (or [0, 127]).  Both are written as
    // instructions: C leaves a float-to-int conversion of NaN or of an
    // out-of-range value undefined.
    int r, q;
    asm("v_cvt_i32_f32 %0, %1" : "=v"(r) : "v"(__builtin_rintf(v)));
    asm("v_med3_i32 %0, %1, %2, %3" : "=v"(q) : "v"(r), "v"(relu ? 0 : -128), "v"(127));
    return q;
}

// 4x4 byte transpose within each quad of lanes: byte u of lane t's result is
// byte t of lane u's input (two DPP lane swaps, t^1 then t^2, each followed
// by a byte or half-word merge).
__device__ __forceinline__ unsigned quad_transpose_bytes(unsigned x, int lane)
{
    const unsigned p = (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
    const unsigned y = (lane & 1) ? (((p & 0xFF00FF00u) >> 8) | (x & 0xFF00FF00u))
                                  : ((x & 0x00FF00FFu) | ((p & 0x00FF00FFu) << 8));
    const unsigned q = (unsigned)__builtin_amdgcn_update_dpp(0, (int)y, 0x4E, 0xF, 0xF, false);
    return (lane & 2) ? ((q >> 16) | (y & 0xFFFF0000u)) : ((y & 0x0000FFFFu) | (q << 16));
}

// Scale and bias of output channel kk (clamped into [0, K): lanes past K
// compute a value that is never stored).
__device__ __forceinline__ void requant_params(const IgemmArgs &a, int kk, float &s, float &b)
{
    const int k = kk < a.K ? kk : a.K - 1;
    s = a.q_scale ? a.q_scale[k] : a.q_alpha;
    b = a.q_bias ? a.q_bias[k] : 0.0f;
}

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
    // XCDs below rem hold per + 1 tiles, the others per (no branch, so the
    // kernel's argument loads are not held back behind it)
    const int per = tiles >> 3, rem = tiles & 7;
    const int xcd = bid & 7, idx = bid >> 3;
    return xcd * per + min(xcd, rem) + idx;
}

// Output-row offsets (elements) of the tile's TM pixels, or -1 past M, for
// outputs whose pixels are not equally spaced.
template <int TM, int NT>
__device__ __forceinline__ void fill_out_rows(const IgemmArgs &a, int m0, int *out_row)
{
    for (int i = threadIdx.x; i < TM; i += NT) {
        const int m = m0 + i;
        int o = -1;
        if (m < a.M) {
            const int n = udiv(m, a.d_pq);
            const int rem = m - n * a.PQ;
            const int p = udiv(rem, a.d_q);
            const int q = rem - p * a.Q;
            o = n * a.oN + p * a.oP + q * a.oQ + a.out0;
        }
        out_row[i] = o;
    }
}

// Epilogue: INT32 sums, or (Q8) their requantised INT8 values.  32x32
// accumulator layout: lane l, value v -> MFMA row 8*(v/4) + 4*(l/32) + v%4,
// MFMA column l%32; rows come from the first MFMA operand.  Elements past M or
// K get an out-of-range offset and the buffer store drops them, so no branch
// guards a store.
template <int FM, int FN, bool PIX_J, bool Q8 = false, bool ATOM = false, int POL = kOutStoreStream>
__device__ __forceinline__ void store_tile(const IgemmArgs &a, v16i (&acc)[FM][FN], int m0, int n0,
                                           int wm, int wn, int lane, const int *out_row,
                                           long long zoff = 0)
{
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)(a.out + zoff), (short)0, a.out_range, kRsrcWord3);
    constexpr int ES = Q8 ? 1 : 4;           // bytes per output element
    const bool relu = a.q_relu != 0;
    auto put = [&](int v, int off, float qs, float qb) {
        if constexpr (Q8)
            __builtin_amdgcn_raw_buffer_store_b8((unsigned char)requant_i8(v, qs, qb, relu), out_rsrc,
                                                 off, 0, POL);
        else if constexpr (ATOM)
            (void)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(v, out_rsrc, off, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b32(v, out_rsrc, off, 0, POL);
    };
    const int mcol = lane & 31;
    const int mrow0 = 4 * (lane >> 5);
    if constexpr (PIX_J) {
        // lanes walk pixels: one pixel per (lane, x), channels along v
        int pix_off[FM];
        bool pix_ok[FM];
#pragma unroll
        for (int x = 0; x < FM; ++x) {
            const int m = m0 + wm + x * 32 + mcol;
            pix_ok[x] = m < a.M;
            const int n = udiv(m, a.d_pq);
            const int rem = m - n * a.PQ;
            const int p = udiv(rem, a.d_q);
            const int q = rem - p * a.Q;
            pix_off[x] = n * a.oN + p * a.oP + q * a.oQ + a.out0;
        }
#pragma unroll
        for (int y = 0; y < FN; ++y) {
            const int kb = n0 + wn + y * 32 + mrow0;
            // the 16 channels of this lane in column block y, and (Q8) their
            // scale and bias, shared by every row block x
            float qs[16], qb[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                qs[v] = 0.0f;
                qb[v] = 0.0f;
                if constexpr (Q8)
                    requant_params(a, kb + 8 * (v >> 2) + (v & 3), qs[v], qb[v]);
            }
#pragma unroll
            for (int x = 0; x < FM; ++x) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int kk = kb + 8 * (v >> 2) + (v & 3);
                    const int off = (pix_ok[x] && kk < a.K) ? (pix_off[x] + kk * a.oK) * ES : kOutOfRange;
                    put(acc[x][y][v], off, qs[v], qb[v]);
                }
            }
        }
    } else if (Q8 && a.pix_linear && a.q8_pack) {
        // lanes walk channels, pixel m at m * pix_stride, channel stride 1:
        // a lane's four consecutive rows become one dword, a quad of lanes
        // transposes them, and lane 4j+t stores channels 4j..4j+3 of row t
#pragma unroll
        for (int y = 0; y < FN; ++y) {
            const int kk = n0 + wn + y * 32 + mcol;
            const int kq = kk & ~3;
            const bool k_ok = kq < a.K;
            float qs, qb;
            requant_params(a, kk, qs, qb);
#pragma unroll
            for (int x = 0; x < FM; ++x) {
                const int mb = m0 + wm + x * 32 + mrow0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    unsigned wv = 0;
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        wv |= ((unsigned)requant_i8(acc[x][y][4 * i + u], qs, qb, relu) & 0xFFu) << (8 * u);
                    wv = quad_transpose_bytes(wv, lane);
                    const int m = mb + 8 * i + (lane & 3);
                    const int off = (k_ok && m < a.M) ? m * a.pix_stride + kq : kOutOfRange;
                    __builtin_amdgcn_raw_buffer_store_b32((int)wv, out_rsrc, off, 0, POL);
                }
            }
        }
    } else if (a.pix_linear) {
        // lanes walk channels; pixel m sits at m * pix_stride
#pragma unroll
        for (int y = 0; y < FN; ++y) {
            const int kk = n0 + wn + y * 32 + mcol;
            const bool k_ok = kk < a.K;
            const int koff = kk * a.oK;
            float qs = 0.0f, qb = 0.0f;
            if constexpr (Q8)
                requant_params(a, kk, qs, qb);
#pragma unroll
            for (int x = 0; x < FM; ++x) {
                const int mb = m0 + wm + x * 32 + mrow0;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = mb + 8 * (v >> 2) + (v & 3);
                    const int off = (k_ok && m < a.M) ? (m * a.pix_stride + koff) * ES : kOutOfRange;
                    put(acc[x][y][v], off, qs, qb);
                }
            }
        }
    } else {
        // lanes walk channels; pixel offsets from the table
#pragma unroll
        for (int y = 0; y < FN; ++y) {
            const int kk = n0 + wn + y * 32 + mcol;
            const bool k_ok = kk < a.K;
            const int koff = kk * a.oK;
            float qs = 0.0f, qb = 0.0f;
            if constexpr (Q8)
                requant_params(a, kk, qs, qb);
#pragma unroll
            for (int x = 0; x < FM; ++x) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int po = out_row[wm + x * 32 + mrow0 + 8 * (v >> 2) + (v & 3)];
                    const int off = (k_ok && po >= 0) ? (po + koff) * ES : kOutOfRange;
                    put(acc[x][y][v], off, qs, qb);
                }
            }
        }
    }
}

// Epilogue kinds a kernel is instantiated with: plain stores with the
// streaming or the default cache policy, or the stores of one split of a
// split inner dimension (partial copies, or int32 atomics into the zeroed
// output; integer adds make the result independent of their order).
constexpr int kEpiStream = 0;
constexpr int kEpiDefault = 1;
constexpr int kEpiSplit = 2;

// store_tile with the epilogue the arguments ask for
template <int FM, int FN, bool PIX_J, int EPI = kEpiStream>
__device__ __forceinline__ void store_tile_any(const IgemmArgs &a, v16i (&acc)[FM][FN], int m0, int n0,
                                               int wm, int wn, int lane, const int *out_row)
{
    constexpr int POL = EPI == kEpiStream ? kOutStoreStream : kOutStoreDefault;
    if constexpr (EPI == kEpiSplit) {
        if (a.part)
            store_tile<FM, FN, PIX_J, false, false, kOutStoreDefault>(a, acc, m0, n0, wm, wn, lane, out_row,
                                                                      (long long)blockIdx.y * a.part_stride);
        else
            store_tile<FM, FN, PIX_J, false, true>(a, acc, m0, n0, wm, wn, lane, out_row);
    } else {
        if (a.q8)
            store_tile<FM, FN, PIX_J, true, false, POL>(a, acc, m0, n0, wm, wn, lane, out_row);
        else
            store_tile<FM, FN, PIX_J, false, false, POL>(a, acc, m0, n0, wm, wn, lane, out_row);
    }
}

}  // namespace convi8
