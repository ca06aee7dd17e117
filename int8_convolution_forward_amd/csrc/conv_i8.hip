// conv_i8: host side of the INT8 conv_fprop library (gfx950).
//
// Validates the descriptors and conv parameters (all on the host, before any
// device work), decides whether the image and/or filter must first be
// repacked to a channel-innermost layout, picks a tile shape, and enqueues
// the kernels on the caller's stream.  See include/conv_i8.h for the
// contract; the operation is the one of the cuDNN "Convolutions" page,
// section "Convolution Fprop", with the parameters of its Python API list.
#include "conv_i8.h"

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <numeric>
#include <string>

#include "footprint_kernel.hpp"
#include "pointwise_kernel.hpp"
#include "igemm_kernel.hpp"
#include "repack_kernel.hpp"
#include "mfma_ceiling_kernel.hpp"
#include "direct_kernel.hpp"
#include "wgrad_kernel.hpp"

#ifdef CONV_I8_HOST_ONLY
// Host-only build of the validation and planning code (built with the host
// sanitizers on a machine without a GPU): no kernel is instantiated, so no
// device code exists, and a launch does nothing.  Never a product build.
#undef hipLaunchKernelGGL
#define hipLaunchKernelGGL(...) ((void)0)
#endif

namespace convi8 {
namespace {

constexpr int64_t kI32Max = 0x7fffffffLL;
constexpr int kCUs = 256;  // MI355X compute units (8 XCDs x 32)

struct T4 {
    int64_t d[4];
    int64_t s[4];  // element strides; 0 for dims of size <= 1
    int64_t elems() const { return d[0] * d[1] * d[2] * d[3]; }
};

bool mul_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_mul_overflow(a, b, r); }
bool add_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_add_overflow(a, b, r); }

// Largest element offset addressed by a tensor, +1 (0 if it has no elements).
bool span_of(const T4 &t, int64_t *span)
{
    for (int i = 0; i < 4; ++i)
        if (t.d[i] == 0) {
            *span = 0;
            return true;
        }
    int64_t acc = 1;
    for (int i = 0; i < 4; ++i) {
        int64_t term;
        if (!mul_ok(t.d[i] - 1, t.s[i], &term) || !add_ok(acc, term, &acc))
            return false;
    }
    *span = acc;
    return true;
}

conv_i8_status_t read_desc(const conv_i8_desc_t *desc, int32_t dtype, T4 *t)
{
    if (!desc)
        return CONV_I8_ERR_NULL;
    if (desc->ndim != 4)
        return CONV_I8_ERR_RANK;
    if (desc->dtype != dtype)
        return CONV_I8_ERR_DTYPE;
    for (int i = 0; i < 4; ++i) {
        if (desc->dims[i] < 0)
            return CONV_I8_ERR_DIMS;
        t->d[i] = desc->dims[i];
        // The stride of a dim of size 1 never multiplies a nonzero index.
        t->s[i] = desc->dims[i] > 1 ? desc->strides[i] : 0;
        if (t->s[i] < 0)
            return CONV_I8_ERR_STRIDES;
    }
    return CONV_I8_OK;
}

// True when no two logical indices of t address the same element.
bool non_overlapping(const T4 &t)
{
    for (int i = 0; i < 4; ++i)
        if (t.d[i] == 0)
            return true;  // no elements, nothing can overlap
    int idx[4] = {0, 1, 2, 3};
    std::sort(idx, idx + 4, [&](int a, int b) { return t.s[a] < t.s[b]; });
    int64_t reach = 0;  // largest offset reachable by the dims sorted so far
    for (int k = 0; k < 4; ++k) {
        const int i = idx[k];
        if (t.d[i] <= 1)
            continue;
        if (t.s[i] <= reach)
            return false;
        int64_t term;
        if (!mul_ok(t.d[i] - 1, t.s[i], &term) || !add_ok(reach, term, &reach))
            return false;
    }
    return true;
}

struct Problem {
    T4 x, w, y;
    int64_t N, C, H, W, K, R, S, P, Q;
    int64_t pre[2], post[2], str[2], dil[2];
    int64_t mode;      // CONV_I8_MODE_*: 1 reads filter tap (R-1-r, S-1-s)
    int64_t flip_out;  // 1: output (p, q) is written at (P-1-p, Q-1-q) (weight gradient
                       // of true convolution); never set by a caller's descriptor
    int64_t split_ok;  // 1: an im2col launch with few tiles and a long inner dimension may
                       // split it over gridDim.y (the output is zeroed first, partial
                       // sums added atomically); set only for the weight gradient
};

conv_i8_status_t read_params(const int64_t *pre, const int64_t *post, const int64_t *stride,
                             const int64_t *dil, Problem *pb)
{
    if (!pre || !post || !stride || !dil)
        return CONV_I8_ERR_NULL;
    for (int i = 0; i < 2; ++i) {
        if (pre[i] < 0 || post[i] < 0 || stride[i] < 1 || dil[i] < 1)
            return CONV_I8_ERR_PARAM;
        if (pre[i] > kI32Max / 4 || post[i] > kI32Max / 4 || stride[i] > kI32Max / 4 ||
            dil[i] > kI32Max / 4)
            return CONV_I8_ERR_UNSUPPORTED;
        pb->pre[i] = pre[i];
        pb->post[i] = post[i];
        pb->str[i] = stride[i];
        pb->dil[i] = dil[i];
    }
    return CONV_I8_OK;
}

// Output length of one spatial dim; -1 when the dilated window never fits.
int64_t out_len(int64_t in, int64_t pre, int64_t post, int64_t f, int64_t stride, int64_t dil)
{
    const int64_t span = in + pre + post - dil * (f - 1) - 1;
    if (span < 0)
        return -1;
    return span / stride + 1;
}

conv_i8_status_t analyze_inputs(const conv_i8_desc_t *image, const conv_i8_desc_t *filter,
                                const int64_t *pre, const int64_t *post, const int64_t *stride,
                                const int64_t *dil, Problem *pb)
{
    conv_i8_status_t st;
    if ((st = read_desc(image, CONV_I8_DT_INT8, &pb->x)) != CONV_I8_OK)
        return st;
    if ((st = read_desc(filter, CONV_I8_DT_INT8, &pb->w)) != CONV_I8_OK)
        return st;
    if ((st = read_params(pre, post, stride, dil, pb)) != CONV_I8_OK)
        return st;
    pb->N = pb->x.d[0];
    pb->C = pb->x.d[1];
    pb->H = pb->x.d[2];
    pb->W = pb->x.d[3];
    pb->K = pb->w.d[0];
    pb->R = pb->w.d[2];
    pb->S = pb->w.d[3];
    if (pb->R < 1 || pb->S < 1)
        return CONV_I8_ERR_DIMS;
    if (pb->w.d[1] != pb->C)
        return CONV_I8_ERR_CHANNELS;
    for (int i = 0; i < 4; ++i)
        if (pb->x.d[i] > kI32Max / 4 || pb->w.d[i] > kI32Max / 4)
            return CONV_I8_ERR_UNSUPPORTED;
    int64_t crs;
    if (!mul_ok(pb->C, pb->R * pb->S, &crs) || crs > CONV_I8_MAX_REDUCTION)
        return CONV_I8_ERR_RANGE;
    pb->P = out_len(pb->H, pb->pre[0], pb->post[0], pb->R, pb->str[0], pb->dil[0]);
    pb->Q = out_len(pb->W, pb->pre[1], pb->post[1], pb->S, pb->str[1], pb->dil[1]);
    if (pb->P < 1 || pb->Q < 1)
        return CONV_I8_ERR_OUT_DIMS;
    int64_t sp;
    if (!span_of(pb->x, &sp) || !span_of(pb->w, &sp))
        return CONV_I8_ERR_UNSUPPORTED;
    return CONV_I8_OK;
}

conv_i8_status_t analyze(const conv_i8_desc_t *image, const conv_i8_desc_t *filter,
                         const conv_i8_desc_t *out, const int64_t *pre, const int64_t *post,
                         const int64_t *stride, const int64_t *dil, int32_t out_dtype, int32_t mode,
                         Problem *pb)
{
    conv_i8_status_t st = analyze_inputs(image, filter, pre, post, stride, dil, pb);
    if (st != CONV_I8_OK)
        return st;
    if (mode != CONV_I8_MODE_CROSS_CORRELATION && mode != CONV_I8_MODE_CONVOLUTION)
        return CONV_I8_ERR_PARAM;
    pb->mode = mode;
    pb->flip_out = 0;
    pb->split_ok = 0;
    // The output dtype is checked like every other field: the plain entries
    // refuse an INT8 output descriptor rather than write saturated bytes into
    // it; only the requantising entries write INT8.
    if ((st = read_desc(out, out_dtype, &pb->y)) != CONV_I8_OK)
        return st;
    const int64_t want[4] = {pb->N, pb->K, pb->P, pb->Q};
    for (int i = 0; i < 4; ++i)
        if (pb->y.d[i] != want[i])
            return CONV_I8_ERR_OUT_DIMS;
    int64_t sp;
    if (!span_of(pb->y, &sp))
        return CONV_I8_ERR_UNSUPPORTED;
    if (!non_overlapping(pb->y))
        return CONV_I8_ERR_STRIDES;
    return CONV_I8_OK;
}

// ---------------------------------------------------------------------------
// Tile configurations instantiated for the implicit-GEMM kernels.
// ---------------------------------------------------------------------------
using Launcher = void (*)(bool flat, bool pix_j, dim3 grid, hipStream_t stream, const IgemmArgs &a);
// several phases of one shape class in one launch (blocked order, k-major filters)
using PhasesLauncher = void (*)(bool pix_j, dim3 grid, hipStream_t stream, const IgemmPhases &m);

// im2col tiles whose filter stages can be read k-major (blocked order only):
// 64-channel stages of 64, 128 or 256 columns
template <int TN, int BK, int EPI>
constexpr bool kmajor_tile() { return BK == 64 && (TN == 64 || TN == 128 || TN == 256); }

template <int TM, int TN, int BK, int NS, int WGM, int WGN, int EPI>
void launch_cfg_epi(bool flat, bool pix_j, dim3 grid, hipStream_t stream, const IgemmArgs &a)
{
    const dim3 block(64 * WGM * WGN);
    if constexpr (kmajor_tile<TN, BK, EPI>()) {
        // the planner asks for k-major reads only on such tiles, blocked order
        if (a.kmaj && !flat) {
            if (pix_j)
                hipLaunchKernelGGL((conv_igemm_kernel<TM, TN, BK, NS, WGM, WGN, false, true, EPI, true>), grid, block,
                                   0, stream, a);
            else
                hipLaunchKernelGGL((conv_igemm_kernel<TM, TN, BK, NS, WGM, WGN, false, false, EPI, true>), grid, block,
                                   0, stream, a);
            return;
        }
    }
    if (flat) {
        if (pix_j)
            hipLaunchKernelGGL((conv_igemm_kernel<TM, TN, BK, NS, WGM, WGN, true, true, EPI>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((conv_igemm_kernel<TM, TN, BK, NS, WGM, WGN, true, false, EPI>), grid, block, 0, stream, a);
    } else {
        if (pix_j)
            hipLaunchKernelGGL((conv_igemm_kernel<TM, TN, BK, NS, WGM, WGN, false, true, EPI>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((conv_igemm_kernel<TM, TN, BK, NS, WGM, WGN, false, false, EPI>), grid, block, 0, stream, a);
    }
}

// the epilogue a launch needs: the stores of one split of a split inner
// dimension; else streaming output stores when each store's lanes cover
// consecutive elements, the default policy (L2 merges the lines) when they
// scatter
template <int TM, int TN, int BK, int NS, int WGM = 2, int WGN = 2>
void launch_cfg(bool flat, bool pix_j, dim3 grid, hipStream_t stream, const IgemmArgs &a)
{
    if (a.ksplit > 1)
        launch_cfg_epi<TM, TN, BK, NS, WGM, WGN, kEpiSplit>(flat, pix_j, grid, stream, a);
    else if (a.out_nt)
        launch_cfg_epi<TM, TN, BK, NS, WGM, WGN, kEpiStream>(flat, pix_j, grid, stream, a);
    else
        launch_cfg_epi<TM, TN, BK, NS, WGM, WGN, kEpiDefault>(flat, pix_j, grid, stream, a);
}

// the phases of a strided data gradient in one launch: k-major filters, blocked
// order, the streaming or the default store policy (the same for every phase)
template <int TM, int TN, int BK, int NS, int WGM = 2, int WGN = 2>
void launch_phases_cfg(bool pix_j, dim3 grid, hipStream_t stream, const IgemmPhases &m)
{
    const dim3 block(64 * WGM * WGN);
    if (m.ph[0].out_nt) {
        if (pix_j)
            hipLaunchKernelGGL((conv_igemm_phases_kernel<TM, TN, BK, NS, WGM, WGN, false, true, kEpiStream, true>),
                               grid, block, 0, stream, m);
        else
            hipLaunchKernelGGL((conv_igemm_phases_kernel<TM, TN, BK, NS, WGM, WGN, false, false, kEpiStream, true>),
                               grid, block, 0, stream, m);
    } else {
        if (pix_j)
            hipLaunchKernelGGL((conv_igemm_phases_kernel<TM, TN, BK, NS, WGM, WGN, false, true, kEpiDefault, true>),
                               grid, block, 0, stream, m);
        else
            hipLaunchKernelGGL((conv_igemm_phases_kernel<TM, TN, BK, NS, WGM, WGN, false, false, kEpiDefault, true>),
                               grid, block, 0, stream, m);
    }
}

template <int TM, int TN, int NS, int FPIX, int WGM = 2, int WGN = 2, int KSPL = 1>
void launch_fp3x3(bool, bool pix_j, dim3 grid, hipStream_t stream, const IgemmArgs &a)
{
    const dim3 block(64 * WGM * WGN * KSPL);
    if (pix_j)
        hipLaunchKernelGGL((conv_footprint3x3_kernel<TM, TN, NS, FPIX, WGM, WGN, true, KSPL>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((conv_footprint3x3_kernel<TM, TN, NS, FPIX, WGM, WGN, false, KSPL>), grid, block, 0, stream, a);
}

template <int TM, int TN, int FPIX, bool TAIL>
void launch_fp9(bool, bool pix_j, dim3 grid, hipStream_t stream, const IgemmArgs &a)
{
    if constexpr (TAIL) {
        // k-major filter reads: the tail tiles only (the planner asks no other)
        if (a.kmaj) {
            if (pix_j)
                hipLaunchKernelGGL((conv_fp3x3_ring9_kernel<TM, TN, FPIX, 2, 2, true, TAIL, true>), grid, dim3(256),
                                   0, stream, a);
            else
                hipLaunchKernelGGL((conv_fp3x3_ring9_kernel<TM, TN, FPIX, 2, 2, false, TAIL, true>), grid, dim3(256),
                                   0, stream, a);
            return;
        }
    }
    if (pix_j)
        hipLaunchKernelGGL((conv_fp3x3_ring9_kernel<TM, TN, FPIX, 2, 2, true, TAIL>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((conv_fp3x3_ring9_kernel<TM, TN, FPIX, 2, 2, false, TAIL>), grid, dim3(256), 0, stream, a);
}

constexpr int kPointwiseTilesPerWave = 4;

template <int FN, int KS>
void launch_pw(bool, bool, dim3 grid, hipStream_t stream, const IgemmArgs &a)
{
    if (a.out_nt)
        hipLaunchKernelGGL((conv_pointwise_kernel<FN, KS, kPointwiseTilesPerWave, kOutStoreStream>), grid, dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((conv_pointwise_kernel<FN, KS, kPointwiseTilesPerWave, kOutStoreDefault>), grid, dim3(256), 0,
                           stream, a);
}

enum KernelKind { kIm2col = 0, kFootprint = 1, kPointwise = 2, kDirect = 3 };

struct TileCfg {
    const char *name;  // CONV_I8_TILE value that forces this shape
    int tm, tn, bk, ns;
    int waves;         // 4 (2x2 wave grid) or 8 (4x2)
    int kind;          // KernelKind: im2col, 3x3 footprint (image once per 64-channel block), 1x1
                       // streaming, direct (tiny problems, operands read in place)
    int fpix;          // footprint capacity (pixels)
    double eff;        // relative MFMA efficiency of this tile shape (cost model)
    Launcher launch;   // the kernel instantiation with exactly these parameters
    PhasesLauncher launch_phases;   // several phases in one launch, or nullptr
};

const TileCfg kTiles[] = {
    {"64x64x64", 64, 64, 64, 4, 4, kIm2col, 0, 0.40, launch_cfg<64, 64, 64, 4>, launch_phases_cfg<64, 64, 64, 4>},
    {"128x64x64", 128, 64, 64, 4, 4, kIm2col, 0, 0.48, launch_cfg<128, 64, 64, 4>,
     launch_phases_cfg<128, 64, 64, 4>},
    {"64x128x64", 64, 128, 64, 4, 4, kIm2col, 0, 0.48, launch_cfg<64, 128, 64, 4>,
     launch_phases_cfg<64, 128, 64, 4>},
    {"128x128x64", 128, 128, 64, 4, 4, kIm2col, 0, 0.59, launch_cfg<128, 128, 64, 4>,
     launch_phases_cfg<128, 128, 64, 4>},
    {"128x128x128", 128, 128, 128, 3, 4, kIm2col, 0, 0.55, launch_cfg<128, 128, 128, 3>},
    {"256x128x64", 256, 128, 64, 4, 4, kIm2col, 0, 0.52, launch_cfg<256, 128, 64, 4>},
    {"128x256x64", 128, 256, 64, 4, 4, kIm2col, 0, 0.50, launch_cfg<128, 256, 64, 4>},
    {"w256x128x64", 256, 128, 64, 4, 8, kIm2col, 0, 0.56, launch_cfg<256, 128, 64, 4, 4, 2>},
    {"w128x128x64", 128, 128, 64, 4, 8, kIm2col, 0, 0.56, launch_cfg<128, 128, 64, 4, 4, 2>},
    {"w256x128x128", 256, 128, 128, 3, 8, kIm2col, 0, 0.76, launch_cfg<256, 128, 128, 3, 4, 2>},
    // 192 output channels in one column tile (no half-empty second tile)
    {"w128x192x128", 128, 192, 128, 3, 8, kIm2col, 0, 0.62, launch_cfg<128, 192, 128, 3, 4, 2>},
    {"f256x128", 256, 128, 64, 6, 4, kFootprint, 448, 0.70, launch_fp3x3<256, 128, 6, 448>},
    {"fw256x128", 256, 128, 64, 3, 8, kFootprint, 448, 0.68, launch_fp3x3<256, 128, 3, 448, 4, 2>},
    {"f128x128", 128, 128, 64, 6, 4, kFootprint, 384, 0.62, launch_fp3x3<128, 128, 6, 384>},
    {"fk256x128", 256, 128, 64, 6, 8, kFootprint, 448, 0.60, launch_fp3x3<256, 128, 6, 448, 2, 2, 2>},
    {"fk128x128", 128, 128, 64, 6, 8, kFootprint, 384, 0.55, launch_fp3x3<128, 128, 6, 384, 2, 2, 2>},
    // nine-slot ring; "t": the last channel block row block by row block,
    // each row block stored as soon as it is done
    {"r256x128", 256, 128, 64, 9, 4, kFootprint, 448, 0.70, launch_fp9<256, 128, 448, false>},
    {"t256x128", 256, 128, 64, 9, 4, kFootprint, 448, 0.77, launch_fp9<256, 128, 448, true>},
    {"t128x128", 128, 128, 64, 9, 4, kFootprint, 384, 0.60, launch_fp9<128, 128, 384, true>},
    // 1x1 streaming kernel: tm = pixels per wave tile, tn = output channels covered,
    // bk = channels covered
    {"pw32x64", 32, 32, 64, 0, 4, kPointwise, 0, 1.0, launch_pw<1, 2>},
    {"pw32x128", 32, 32, 128, 0, 4, kPointwise, 0, 1.0, launch_pw<1, 4>},
    {"pw32x256", 32, 32, 256, 0, 4, kPointwise, 0, 1.0, launch_pw<1, 8>},
    {"pw64x64", 32, 64, 64, 0, 4, kPointwise, 0, 1.0, launch_pw<2, 2>},
    {"pw64x128", 32, 64, 128, 0, 4, kPointwise, 0, 1.0, launch_pw<2, 4>},
    {"pw64x256", 32, 64, 256, 0, 4, kPointwise, 0, 1.0, launch_pw<2, 8>},
    {"pw128x64", 32, 128, 64, 0, 4, kPointwise, 0, 1.0, launch_pw<4, 2>},
    {"pw128x128", 32, 128, 128, 0, 4, kPointwise, 0, 1.0, launch_pw<4, 4>},
    // one thread per output element, any layout read in place (no repack)
    {"direct", 1, 1, 0, 0, 4, kDirect, 0, 1.0, nullptr},
};

// The direct kernel: applicable up to kDirectMaxMacs multiply-adds (and
// kDirectMaxCRS per output element); chosen unasked up to kDirectTinyMacs
// when the implicit-GEMM path would need a repack launch first.
constexpr double kDirectMaxMacs = 268435456.0, kDirectTinyMacs = 65536.0;
constexpr int64_t kDirectMaxCRS = 4608;
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

// Measured tile choices (the autotuning step: every applicable tile timed on
// one problem, the fastest kept).  The table is written by the package's
// tune module; a forward problem that matches an entry exactly takes its tile
// ahead of the cost model (a forced CONV_I8_TILE still wins).
struct TunedTile {
    int op;            // 0: forward convolution, 1: weight gradient (its one forward call)
    int64_t N, C, H, W, K, R, S, pre_h, pre_w, post_h, post_w, str_h, str_w, dil_h, dil_w;
    int lanes;         // forward: output lanes walk channels (0) or pixels (1);
                       // weight gradient: dW channel-innermost (0) or not (1)
    const char *tile;  // nullptr ends the table
};
const TunedTile kTuned[] = {
#include "tuned_tiles.inc"
    {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, nullptr},
};

// The table's tile for a problem (its own dims, padding, stride and dilation
// as the caller gave them), or nullptr.
const char *tuned_lookup(int op, const int64_t d[7], const int64_t *pre, const int64_t *post,
                         const int64_t *str, const int64_t *dil, int lanes)
{
    for (const TunedTile *t = kTuned; t->tile; ++t)
        if (t->op == op && t->N == d[0] && t->C == d[1] && t->H == d[2] && t->W == d[3] && t->K == d[4] &&
            t->R == d[5] && t->S == d[6] && t->pre_h == pre[0] && t->pre_w == pre[1] && t->post_h == post[0] &&
            t->post_w == post[1] && t->str_h == str[0] && t->str_w == str[1] && t->dil_h == dil[0] &&
            t->dil_w == dil[1] && t->lanes == lanes)
            return t->tile;
    return nullptr;
}

const char *tuned_tile(const Problem &pb, bool pix_j)
{
    if (pb.flip_out || pb.split_ok)
        return nullptr;
    const int64_t d[7] = {pb.N, pb.C, pb.H, pb.W, pb.K, pb.R, pb.S};
    return tuned_lookup(0, d, pb.pre, pb.post, pb.str, pb.dil, pix_j ? 1 : 0);
}

// Division by a launch-invariant divisor d >= 1 for dividends below 2^31:
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1.
Divisor make_divisor(int64_t d)
{
    Divisor r{};
    int l = 0;
    while ((int64_t(1) << l) < d)
        ++l;
    r.l = l;
    r.m = (unsigned)((((unsigned __int128)1 << 32) * (((unsigned __int128)1 << l) - (unsigned __int128)d)) /
                     (unsigned __int128)d + 1);
    return r;
}

// Largest footprint (input pixels, padded rows x padded width) any tile of
// `tm` consecutive output pixels needs.  The footprint of a tile depends only
// on its start modulo P*Q (and on truncation at M), so one period of tile
// starts plus the last tile cover every case.
int64_t max_footprint(int64_t M, int64_t PQ, int64_t Q, int64_t Hp, int64_t Wf, int64_t str_h,
                      int64_t span_h, int64_t tm)
{
    auto fp_of = [&](int64_t m0) {
        const int64_t ml = std::min(m0 + tm, M) - 1;
        const int64_t na = m0 / PQ, pa = (m0 - na * PQ) / Q;
        const int64_t nb = ml / PQ, pb = (ml - nb * PQ) / Q;
        return ((nb - na) * Hp + pb * str_h + span_h - pa * str_h + 1) * Wf;
    };
    const int64_t tiles = (M + tm - 1) / tm;
    int64_t g = PQ, b = tm;
    while (b) {
        const int64_t t = g % b;
        g = b;
        b = t;
    }
    const int64_t period = PQ / g;
    int64_t best = 0;
    for (int64_t t = 0; t < std::min(tiles, period); ++t)
        best = std::max(best, fp_of(t * tm));
    if (tiles > 0)
        best = std::max(best, fp_of((tiles - 1) * tm));
    return best;
}

// Footprint row pitch in 16-byte slots: at least 5 slots per pixel, padded
// so that stride_h * Pr = 5 * stride_w * Q (mod 16) where stride_h is odd;
// then the pixels of consecutive output rows keep distinct LDS bank groups.
int64_t footprint_pitch(int64_t Wf, int64_t Q, int64_t str_h, int64_t str_w)
{
    const int64_t base = 5 * Wf;
    if (str_h % 2 == 0)
        return base;
    int64_t inv = 1;
    for (int64_t i = 1; i < 16; i += 2)
        if ((str_h * i) % 16 == 1)
            inv = i;
    const int64_t target = (5 * str_w * Q % 16) * inv % 16;
    return base + ((target - base) % 16 + 16) % 16;
}

struct Plan {
    bool repack_x = false, repack_w = false;
    int64_t Cp = 0;                    // channels as the kernel reads them
    size_t ws_x_off = 0, ws_w_off = 0, ws_bytes = 0;
    // kernel view of the image and filter (byte strides; channel stride 1)
    int64_t xsN = 0, xsH = 0, xsW = 0, x_img_span = 0;
    int64_t wsK = 0, wsR = 0, wsS = 0, w_span = 0;
    int cfg = 0;
    bool pix_j = false;
    bool blocked = true;
    int64_t nstages = 0;
    int64_t batch_chunk = 1;           // images per igemm launch
    int64_t y_img_span = 0;            // output elements one image spans
    bool pix_linear = false;           // output pixel m at m * pix_stride
    int64_t pix_stride = 0;
    int64_t Hp = 0, Wf = 0, Pr = 0;    // footprint kernel geometry
    bool kmaj = false;                 // filter read in place with its output channels
                                       // contiguous (3x3 tail tiles; wsK is then the
                                       // stride of one input channel)
    // split of a long inner dimension over gridDim.y (weight gradient)
    int64_t ksplit = 1, kchunk = 0;    // splits, stages per split
    bool part = false;                 // partial outputs in the workspace + reduction
    size_t ws_part_off = 0;
    int64_t part_span = 0;             // elements of one partial copy (one launch's output span)
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Can the kernel read this tensor directly: channels innermost, C a multiple
// of 16, and every 16-channel run 16-byte aligned?
bool direct_ok(const T4 &t, const void *ptr)
{
    const int64_t C = t.d[1];
    if (C % 16 != 0)
        return false;
    if (C > 1 && t.s[1] != 1)
        return false;
    for (int i : {0, 2, 3})
        if (t.s[i] % 16 != 0)
            return false;
    return ptr == nullptr || aligned16(ptr);
}

// Can the 3x3 tail tiles read this filter in place k-major: output channels
// contiguous (the data gradient's view [C, K, R, S] of a KRSC filter, or an
// R, S, C, K filter), K a multiple of 16, 64-channel blocks of input
// channels, and every 16-channel run 16-byte aligned?  The kernel loads rows
// of 128 output channels per input channel and transposes them in LDS.
bool kmajor_ok(const Problem &pb, const void *ptr)
{
    const T4 &t = pb.w;
    if (pb.K % 16 != 0 || pb.C % 64 != 0 || pb.C == 0 || t.s[0] != 1 || t.s[1] > kI32Max / 64)
        return false;
    for (int i : {1, 2, 3})
        if (t.s[i] % 16 != 0)
            return false;
    return ptr == nullptr || aligned16(ptr);
}

// Tiles that read a k-major filter: the 3x3 tail tiles, and im2col tiles of
// 64-channel stages over 64, 128 or 256 columns in blocked order (the
// instantiations launch_cfg_epi and launch_fp9 provide), split inner
// dimension included (the weight gradient's transposed loss).
bool tile_reads_kmajor(const TileCfg &c, const Problem &pb)
{
    if (c.kind == kFootprint)
        return c.ns == 9 && c.name[0] == 't';
    return c.kind == kIm2col && c.bk == 64 && (c.tn == 64 || c.tn == 128 || c.tn == 256) && pb.C % c.bk == 0;
}

const char *env_tile() { return getenv("CONV_I8_TILE"); }

// One repack job: [A, C, Y, X] -> [A, Y, X, Cp].  Y and X merge into one
// run of positions when their strides allow it (packed rows, or a size-1
// dim), so the lines along x are as long as possible.
RepackJob repack_job(const T4 &t, const int8_t *src, int8_t *dst, int64_t Cp, int64_t *tiles64 = nullptr)
{
    RepackJob j{};
    j.src = src;
    j.dst = dst;
    int64_t A = t.d[0], C = t.d[1], Y = t.d[2], X = t.d[3];
    int64_t s0 = t.s[0], s1 = t.s[1], sy = t.s[2], sx = t.s[3];
    if (X == 1) {
        X = Y;
        sx = sy;
        Y = 1;
        sy = 0;
    } else if (Y == 1 || sy == X * sx) {
        X = X * Y;
        Y = 1;
        sy = 0;
    }
    j.s0 = s0;
    j.s1 = s1;
    j.sy = sy;
    j.sx = sx;
    j.A = (int)A;
    j.C = (int)C;
    j.Y = (int)Y;
    j.X = (int)X;
    j.Cp = (int)Cp;
    if (X > 1 && sx <= 8 && (sx <= s1 || C == 1))
        j.mode = kRepackXFast;
    else if (C > 1 && s1 <= 8)
        j.mode = kRepackCFast;
    else if (A > 1 && s0 >= 1 && s0 <= 8)
        j.mode = kRepackAFast;  // a transposed view: tiles walk a at each (y, x)
    else
        j.mode = kRepackGather;
    const int64_t tx = ((j.mode == kRepackAFast ? A : X) + 63) / 64, tc = (Cp + 63) / 64;
    // a-fast tiles with 16 or 32 packed channels cover 4 or 2 (y, x) positions
    // (the kernel indexes the Y*X positions with 32-bit ints)
    j.pp_shift = j.mode == kRepackAFast && Cp <= 32 && Y * X <= kI32Max - 4 ? (Cp <= 16 ? 2 : 1) : 0;
    const int64_t tiles = (j.mode == kRepackAFast ? (Y * X + (1 << j.pp_shift) - 1) >> j.pp_shift : A * Y) * tx * tc;
    if (tiles64)
        *tiles64 = tiles;
    j.tiles_x = (int)tx;
    j.tiles_c = (int)tc;
    j.tiles = tiles <= kI32Max ? (int)tiles : -1;   // -1: refused at launch
    j.d_tc = make_divisor(std::max<int64_t>(tc, 1));
    j.d_tx = make_divisor(std::max<int64_t>(tx, 1));
    j.d_o = make_divisor(std::max<int64_t>(j.mode == kRepackAFast ? X : Y, 1));
    return j;
}

conv_i8_status_t make_plan(const Problem &pb, const void *x_ptr, const void *w_ptr, Plan *pl,
                           const char *tuned_override = nullptr)
{
    pl->repack_x = !direct_ok(pb.x, x_ptr);
    pl->repack_w = !direct_ok(pb.w, w_ptr);
    pl->Cp = (pb.C + 15) / 16 * 16;

    size_t off = 0;
    if (pl->repack_x) {
        int64_t b;
        if (!mul_ok(pb.N * pb.H, pb.W * pl->Cp, &b))
            return CONV_I8_ERR_UNSUPPORTED;
        pl->ws_x_off = off;
        off = align_up(off + (size_t)b, 256);
        pl->xsW = pl->Cp;
        pl->xsH = pb.W * pl->Cp;
        pl->xsN = pb.H * pb.W * pl->Cp;
        int64_t rt = 0;
        repack_job(pb.x, nullptr, nullptr, pl->Cp, &rt);
        if (rt > kI32Max || pb.H * pb.W > kI32Max || pl->Cp > kI32Max)
            return CONV_I8_ERR_UNSUPPORTED;
    } else {
        pl->xsN = pb.x.s[0];
        pl->xsH = pb.x.s[2];
        pl->xsW = pb.x.s[3];
    }
    if (pl->repack_w) {
        int64_t b;
        if (!mul_ok(pb.K * pb.R, pb.S * pl->Cp, &b))
            return CONV_I8_ERR_UNSUPPORTED;
        pl->ws_w_off = off;
        off = align_up(off + (size_t)b, 256);
        pl->wsS = pl->Cp;
        pl->wsR = pb.S * pl->Cp;
        pl->wsK = pb.R * pb.S * pl->Cp;
        int64_t rt = 0;
        repack_job(pb.w, nullptr, nullptr, pl->Cp, &rt);
        if (rt > kI32Max || pb.R * pb.S > kI32Max || pl->Cp > kI32Max)
            return CONV_I8_ERR_UNSUPPORTED;
    } else {
        pl->wsK = pb.w.s[0];
        pl->wsR = pb.w.s[2];
        pl->wsS = pb.w.s[3];
    }
    pl->ws_bytes = off;

    // Span of one image in the kernel's view, including every tap offset the
    // kernel forms (padding and dilation may reach past the image before the
    // bounds test rejects the tap): all must fit in 31 bits.
    {
        T4 v{};
        v.d[0] = 1; v.d[1] = pl->Cp; v.d[2] = pb.H; v.d[3] = pb.W;
        v.s[0] = 0; v.s[1] = 1; v.s[2] = pb.H > 1 ? pl->xsH : 0; v.s[3] = pb.W > 1 ? pl->xsW : 0;
        int64_t sp;
        if (!span_of(v, &sp) || sp > kI32Max)
            return CONV_I8_ERR_UNSUPPORTED;
        pl->x_img_span = sp;
        int64_t reach_h, reach_w;
        if (!mul_ok(pb.H + pb.pre[0] + pb.post[0] + 1, pl->xsH, &reach_h) ||
            !mul_ok(pb.W + pb.pre[1] + pb.post[1] + 1, pl->xsW, &reach_w) ||
            reach_h + reach_w + pl->Cp > kI32Max)
            return CONV_I8_ERR_UNSUPPORTED;
        T4 f{};
        f.d[0] = pb.K; f.d[1] = pl->Cp; f.d[2] = pb.R; f.d[3] = pb.S;
        f.s[0] = pb.K > 1 ? pl->wsK : 0; f.s[1] = 1;
        f.s[2] = pb.R > 1 ? pl->wsR : 0; f.s[3] = pb.S > 1 ? pl->wsS : 0;
        if (!span_of(f, &sp) || sp > kI32Max)
            return CONV_I8_ERR_UNSUPPORTED;
        pl->w_span = sp;
    }

    // Output bytes one image addresses (its N stride aside).
    {
        T4 o = pb.y;
        o.d[0] = 1;
        int64_t sp;
        if (!span_of(o, &sp) || sp > kI32Max / 4)
            return CONV_I8_ERR_UNSUPPORTED;
        pl->y_img_span = sp;
    }
    // Images per launch: the image bytes and output bytes one launch
    // addresses, and its N*P*Q rows, must stay below 2^31.
    {
        const int64_t pq = pb.P * pb.Q;
        int64_t nb = std::max<int64_t>(1, pb.N);
        if (pl->xsN > 0)
            nb = std::min<int64_t>(nb, (kI32Max - pl->x_img_span) / pl->xsN + 1);
        if (pb.y.s[0] > 0)
            nb = std::min<int64_t>(nb, (kI32Max / 4 - pl->y_img_span) / pb.y.s[0] + 1);
        nb = std::min<int64_t>(nb, kI32Max / pq);
        if (nb < 1)
            return CONV_I8_ERR_UNSUPPORTED;
        int64_t t;
        if (!mul_ok(nb, pl->xsN, &t) || nb * pq > kI32Max)
            return CONV_I8_ERR_UNSUPPORTED;
        pl->batch_chunk = nb;
    }

    // Are output pixels equally spaced in (n, p, q) order?
    {
        const int64_t N = pb.N, P = pb.P, Q = pb.Q;
        const int64_t oN = pb.y.s[0], oP = pb.y.s[2], oQ = pb.y.s[3];
        int64_t ps = Q > 1 ? oQ : P > 1 ? oP : oN;
        pl->pix_stride = ps;
        pl->pix_linear = (Q == 1 || oQ == ps) && (P == 1 || oP == Q * ps) &&
                         (N == 1 || oN == P * Q * ps) && !pb.flip_out;
    }
    // Output layout: make the MFMA column (lanes) walk the contiguous dim.
    const int64_t oK = pb.y.s[1], oQ = pb.y.s[3];
    if (oK == 1)
        pl->pix_j = false;
    else if (oQ == 1)
        pl->pix_j = true;
    else
        pl->pix_j = oQ != 0 && (oK == 0 || oQ < oK);

    // Tile choice.  Per tile, the MFMA time (tile work at one CU's share of
    // the MFMA rate, over the shape's relative efficiency) and the operand
    // load time (bytes streamed into LDS at one CU's share of the ~20 TB/s
    // L2-to-LDS rate) overlap; tiles run in rounds of 256 (one per CU).
    const int64_t cc = pl->Cp / 16;
    const int64_t M = std::min(pb.N, pl->batch_chunk) * pb.P * pb.Q;
    const int64_t RS = pb.R * pb.S;
    const int64_t Hp = pb.H + pb.pre[0] + pb.post[0];
    const int64_t Wf = (pb.Q - 1) * pb.str[1] + (pb.S - 1) * pb.dil[1] + 1;
    const double mac_per_s_cu = 4.4e15 / 2 / kCUs, bytes_per_s_cu = 20e12 / kCUs;
    int best = -1;
    double best_cost = 0;
    const char *forced = env_tile();
    const char *tuned = forced ? nullptr : tuned_override ? tuned_override : tuned_tile(pb, pl->pix_j);
    int tuned_idx = -1;
    const double macs = (double)pb.N * pb.K * pb.P * pb.Q * pb.C * pb.R * pb.S;
    const bool direct_fits = macs <= kDirectMaxMacs && pb.C * RS <= kDirectMaxCRS;
    int direct_idx = -1;
    for (int i = 0; i < kNumTiles; ++i) {
        const TileCfg &c = kTiles[i];
        if (forced && strcmp(forced, c.name) != 0)
            continue;
        if (c.kind == kDirect) {
            if (!direct_fits)
                continue;
            if (tuned && strcmp(tuned, c.name) == 0)
                tuned_idx = i;
            direct_idx = i;
            if (forced)
                best = i;
            continue;
        }
        const int cps = c.bk / 16;
        const int64_t chunks = RS * cc;
        int64_t stages = cc % cps == 0 ? RS * (cc / cps) : (chunks + cps - 1) / cps;
        double bytes;
        if (c.kind == kPointwise) {
            // 1x1 streaming kernel: the filter fits its registers, the output
            // is channel-innermost with equally spaced pixels
            if (pb.R != 1 || pb.S != 1 || pb.K > c.tn || pl->Cp > c.bk || pl->pix_j || !pl->pix_linear)
                continue;
            if (tuned && strcmp(tuned, c.name) == 0)
                tuned_idx = i;
            // HBM-bound and measured ahead of every im2col tile on 1x1 layers
            // (the tile model prices the im2col tiles' stores too low there):
            // the first one that fits is taken
            if (getenv("CONV_I8_COST"))
                fprintf(stderr, "conv_i8 cost %-14s -> preferred for 1x1\n", c.name);
            if (best < 0 || kTiles[best].kind != kPointwise) {
                best = i;
                best_cost = 0;
            }
            continue;
        }
        if (c.kind == kFootprint) {
            // footprint kernel: a 3x3 filter, 64-channel blocks, and a tile
            // footprint that fits its buffers
            if (pb.R != 3 || pb.S != 3 || cc % 4 != 0 || Hp >= (1 << 20) || Wf >= (1 << 20))
                continue;
            // the nine-slot kernel forms column offsets with a 24-bit multiply
            if (pl->xsW < 0 || pl->xsW >= (1 << 23))
                continue;
            const int64_t fmax = max_footprint(M, pb.P * pb.Q, pb.Q, Hp, Wf, pb.str[0],
                                               (pb.R - 1) * pb.dil[0], c.tm);
            const int64_t pr = footprint_pitch(Wf, pb.Q, pb.str[0], pb.str[1]);
            if ((fmax / Wf) * pr > (int64_t)c.fpix * 5)
                continue;
            bytes = (double)c.tn * stages * 64 + (double)(cc / 4) * (fmax / Wf) * pr * 16;
        } else {
            bytes = (double)(c.tm + c.tn) * stages * c.bk;
        }
        if (tuned && strcmp(tuned, c.name) == 0)
            tuned_idx = i;
        double eff = c.eff;
        if (c.kind == kIm2col && cc % cps != 0)
            eff *= chunks > 0 ? (double)chunks / (double)(stages * cps) : 1.0;
        // fitted to measured kernel times: MFMA time at the shape's efficiency
        // plus half the operand-load time (the two overlap only partly) plus
        // the tile's INT32 stores at one CU's share of ~5 TB/s
        const double t_mfma = (double)c.tm * c.tn * stages * c.bk / mac_per_s_cu / eff;
        const double t_load = bytes / bytes_per_s_cu;
        const double t_store = (double)c.tm * c.tn * 4 / (5e12 / kCUs);
        const int64_t tiles = ((M + c.tm - 1) / c.tm) * ((pb.K + c.tn - 1) / c.tn);
        const int64_t rounds = (tiles + kCUs - 1) / kCUs;
        const double cost = (double)rounds * (t_mfma + 0.5 * t_load + t_store);
        if (getenv("CONV_I8_COST"))
            fprintf(stderr, "conv_i8 cost %-14s tiles %7lld rounds %4lld mfma %.2f load %.2f store %.2f -> %.2f us\n",
                    c.name, (long long)tiles, (long long)rounds, t_mfma * 1e6, t_load * 1e6, t_store * 1e6, cost * 1e6);
        if (best < 0 || cost < best_cost * (1 - 1e-9)) {
            best = i;
            best_cost = cost;
        }
    }
    if (tuned_idx >= 0) {
        if (getenv("CONV_I8_COST"))
            fprintf(stderr, "conv_i8 cost: measured choice %s for this problem\n", kTiles[tuned_idx].name);
        best = tuned_idx;
    } else if (!forced && direct_idx >= 0 && macs <= kDirectTinyMacs && (pl->repack_x || pl->repack_w)) {
        best = direct_idx;   // one launch instead of a repack and a convolution
    }
    if (best < 0) {
        // unknown or inapplicable CONV_I8_TILE value: default shape
        best = 0;
        for (int i = 0; i < kNumTiles; ++i)
            if (strcmp(kTiles[i].name, "128x128x64") == 0)
                best = i;
    }
    pl->cfg = best;
    const TileCfg &c = kTiles[best];
    if (c.kind == kDirect) {
        // operands read in place through their strides: no repack, no
        // workspace, no batch chunks (64-bit offsets)
        pl->repack_x = pl->repack_w = false;
        pl->ws_bytes = 0;
        pl->ksplit = 1;
        pl->kchunk = 0;
        pl->part = false;
        pl->blocked = true;
        pl->nstages = 0;
        pl->batch_chunk = std::max<int64_t>(pb.N, 1);
        return CONV_I8_OK;
    }
    if (pl->repack_w && tile_reads_kmajor(c, pb) && kmajor_ok(pb, w_ptr)) {
        // the filter is read in place (no repack, its workspace region
        // dropped: it was the last one)
        int64_t sp;
        if (span_of(pb.w, &sp) && sp <= kI32Max) {
            pl->repack_w = false;
            pl->kmaj = true;
            pl->ws_bytes = pl->ws_w_off;
            pl->wsK = pb.w.s[1];
            pl->wsR = pb.w.s[2];
            pl->wsS = pb.w.s[3];
            pl->w_span = sp;
        }
    }
    const int cps = c.bk / 16;
    pl->blocked = cc % cps == 0;
    pl->nstages = pl->blocked ? RS * (cc / cps) : (RS * cc + cps - 1) / cps;
    if (c.kind == kFootprint) {
        pl->Hp = Hp;
        pl->Wf = Wf;
        pl->Pr = footprint_pitch(Wf, pb.Q, pb.str[0], pb.str[1]);
    }

    // A few tiles over a long inner dimension (the weight gradient): split it
    // over gridDim.y so that about one workgroup runs per CU, at least 16
    // stages each.  With a dense output each split writes its partial sums
    // into its own copy of the output in the workspace and a reduction kernel
    // adds the copies; otherwise the splits add into the zeroed output with
    // int32 atomics.  (Device-scope atomics are slow here: with more than half
    // of the CUs busy they cost more than the split gains, 75 -> 167 us on the
    // large-channel weight gradient's 144 tiles.)
    pl->ksplit = 1;
    pl->kchunk = 0;
    pl->part = false;
    if (pb.split_ok && c.kind == kIm2col && pb.C > 0 && pl->nstages >= 32) {
        // partial copies need one launch over a dense output: every element
        // of its span is one of its elements, written by every split
        const int64_t span = (pb.N - 1) * pb.y.s[0] + pl->y_img_span;
        const bool dense = pl->batch_chunk >= pb.N && span == pb.N * pb.K * pb.P * pb.Q;
        const int64_t tiles = ((M + c.tm - 1) / c.tm) * ((pb.K + c.tn - 1) / c.tn);
        int64_t want = tiles > 0 ? std::min<int64_t>((kCUs + tiles - 1) / tiles, pl->nstages / 16) : 1;
        if (dense && tiles > 0) {
            // With partial copies: the split count that minimises the busiest
            // CU's stages (workgroups share CUs evenly: ceil(tiles*k/CUs)
            // workgroups of ceil(stages/k) stages each) plus the reduction
            // (k copies read and the output written at ~5 TB/s, one launch).
            // A split that leaves some CUs with two workgroups and others
            // with one gains nothing over no split.
            const double t_stage = (double)c.tm * c.tn * c.bk / (4.4e15 / 2 / kCUs) / c.eff;
            double best_t = 0;
            want = 1;
            for (int64_t k = 1; k <= std::min<int64_t>(pl->nstages / 16, 32); ++k) {
                const int64_t per_cu = (tiles * k + kCUs - 1) / kCUs;
                const int64_t st = (pl->nstages + k - 1) / k;
                const double t = (double)per_cu * st * t_stage + (k > 1 ? (k + 1) * (double)span * 4 / 5e12 + 2.5e-6 : 0);
                if (k == 1 || t < best_t * (1 - 1e-9)) {
                    best_t = t;
                    want = k;
                }
            }
        }
        // with atomics a split pays only below half of the CUs busy
        if (tiles < (dense ? kCUs : kCUs / 2) && want > 1) {
            pl->kchunk = (pl->nstages + want - 1) / want;
            pl->ksplit = (pl->nstages + pl->kchunk - 1) / pl->kchunk;
            int64_t bytes;
            if (dense && mul_ok(span * 4, pl->ksplit, &bytes)) {
                pl->part = true;
                pl->part_span = span;
                pl->ws_part_off = align_up(pl->ws_bytes, 256);
                pl->ws_bytes = pl->ws_part_off + (size_t)bytes;
            }
        }
    }
    return CONV_I8_OK;
}

// Workgroups of the direct kernel: one thread per output element, at most
// four workgroups per CU (the rest is a grid-stride loop).
int64_t direct_blocks(const Problem &pb)
{
    const int64_t total = pb.N * pb.K * pb.P * pb.Q;
    return std::min<int64_t>((total + 255) / 256, 4 * kCUs);
}

conv_i8_status_t launch_direct(const Problem &pb, const void *x_ptr, const void *w_ptr, void *y_ptr,
                               hipStream_t stream, const conv_i8_requant_t *rq)
{
    const int64_t total = pb.N * pb.K * pb.P * pb.Q;
    if (total == 0)
        return CONV_I8_OK;
    DirectArgs d{};
    d.x = (const int8_t *)x_ptr;
    d.w = (const int8_t *)w_ptr;
    d.y = y_ptr;
    for (int i = 0; i < 4; ++i) {
        d.xs[i] = pb.x.s[i];
        d.ws[i] = pb.w.s[i];
        d.ys[i] = pb.y.s[i];
    }
    d.total = total;
    d.K = (int)pb.K;
    d.C = (int)pb.C;
    d.R = (int)pb.R;
    d.S = (int)pb.S;
    d.P = (int)pb.P;
    d.Q = (int)pb.Q;
    d.H = (int)pb.H;
    d.W = (int)pb.W;
    d.preH = (int)pb.pre[0];
    d.preW = (int)pb.pre[1];
    d.strH = (int)pb.str[0];
    d.strW = (int)pb.str[1];
    d.dilH = (int)pb.dil[0];
    d.dilW = (int)pb.dil[1];
    d.conv_mode = pb.mode == CONV_I8_MODE_CONVOLUTION ? 1 : 0;
    d.flip_out = pb.flip_out ? 1 : 0;
    if (rq) {
        d.q8 = 1;
        d.q_scale = rq->scale;
        d.q_bias = rq->bias;
        d.q_alpha = rq->alpha;
        d.q_relu = rq->relu ? 1 : 0;
    }
    hipLaunchKernelGGL(conv_direct_kernel<0>, dim3((unsigned)direct_blocks(pb)), dim3(256), 0, stream, d);
    return hipGetLastError() == hipSuccess ? CONV_I8_OK : CONV_I8_ERR_HIP;
}

std::string describe(const Problem &pb, const Plan &pl)
{
    const TileCfg &c = kTiles[pl.cfg];
    const int64_t M = pb.N * pb.P * pb.Q;
    const int64_t tiles = c.kind == kDirect ? direct_blocks(pb)
                                            : ((M + c.tm - 1) / c.tm) * ((pb.K + c.tn - 1) / c.tn);
    char buf[512];
    snprintf(buf, sizeof buf,
             "repack_image=%d repack_filter=%d filter_read=%s Cp=%lld tile=%s kernel=%s order=%s stages=%lld "
             "lanes=%s tiles=%lld batch_chunk=%lld workspace=%zu ksplit=%lld split_sum=%s",
             (int)pl.repack_x, (int)pl.repack_w, pl.kmaj ? "kmajor" : pl.repack_w ? "packed" : "in_place",
             (long long)pl.Cp, c.name,
             c.kind == kFootprint ? "footprint" : c.kind == kPointwise ? "pointwise" : c.kind == kDirect ? "direct" : "im2col",
             pl.blocked ? "blocked" : "flat", (long long)pl.nstages,
             pl.pix_j ? "pixels" : "channels", (long long)tiles, (long long)pl.batch_chunk,
             pl.ws_bytes, (long long)pl.ksplit, pl.ksplit < 2 ? "none" : pl.part ? "partial" : "atomic");
    return buf;
}

bool log_enabled()
{
    const char *e = getenv("CONV_I8_LOG");
    return e && *e && strcmp(e, "0") != 0;
}

template <int NJ>
conv_i8_status_t launch_repacks_n(const RepackJob *jobs, int njobs, hipStream_t stream)
{
    RepackArgs<NJ> r{};
    int64_t total = 0;
    for (int i = 0; i < njobs; ++i) {
        if (jobs[i].tiles < 0)
            return CONV_I8_ERR_UNSUPPORTED;
        if (jobs[i].tiles == 0)
            continue;
        r.job[r.njobs++] = jobs[i];
        total += jobs[i].tiles;
    }
    if (total > kI32Max)
        return CONV_I8_ERR_UNSUPPORTED;
    if (total == 0)
        return CONV_I8_OK;
    // LDS line size for the largest stride a job walks its lines with
    int64_t step = 1;
    for (int i = 0; i < r.njobs; ++i) {
        const RepackJob &j = r.job[i];
        if (j.mode != kRepackGather)
            step = std::max<int64_t>(step, j.mode == kRepackXFast ? j.sx
                                           : j.mode == kRepackAFast ? j.s0 : j.s1);
    }
    const dim3 grid((unsigned)total);
    if (step <= 2)
        hipLaunchKernelGGL((repack_to_channels_last_kernel<2, NJ>), grid, dim3(256), 0, stream, r);
    else if (step <= 4)
        hipLaunchKernelGGL((repack_to_channels_last_kernel<4, NJ>), grid, dim3(256), 0, stream, r);
    else
        hipLaunchKernelGGL((repack_to_channels_last_kernel<8, NJ>), grid, dim3(256), 0, stream, r);
    return hipGetLastError() == hipSuccess ? CONV_I8_OK : CONV_I8_ERR_HIP;
}

conv_i8_status_t launch_repacks(const RepackJob *jobs, int njobs, hipStream_t stream)
{
    if (njobs > kRepackMaxJobs)
        return CONV_I8_ERR_UNSUPPORTED;
    return njobs <= 2 ? launch_repacks_n<2>(jobs, njobs, stream)
                      : launch_repacks_n<kRepackMaxJobs>(jobs, njobs, stream);
}

#ifdef CONV_I8_PHASE_CLOCK
// Instrumented builds only: where the 3x3 ring kernel writes its
// per-workgroup phase stamps (set by conv_i8_set_phase_clock).
long long *g_phase_clk = nullptr;
#endif

// The arguments of an implicit-GEMM launch (3x3, im2col or 1x1 kernel) that
// do not depend on the batch chunk; w is the filter as the kernel reads it
// (its packed copy when the plan repacks it).
IgemmArgs make_args(const Problem &pb, const Plan &pl, const TileCfg &c, const int8_t *w, void *y_ptr,
                    const conv_i8_requant_t *rq)
{
    IgemmArgs a{};
    a.flt = w;
    a.flt_range = (int)pl.w_span;
    a.H = (int)pb.H;
    a.W = (int)pb.W;
    a.C = (int)pl.Cp;
    a.sH = (int)pl.xsH;
    a.sW = (int)pl.xsW;
    a.K = (int)pb.K;
    a.R = (int)pb.R;
    a.S = (int)pb.S;
    a.fK = (int)pl.wsK;
    a.fR = (int)pl.wsR;
    a.fS = (int)pl.wsS;
    a.kmaj = pl.kmaj ? 1 : 0;
#ifdef CONV_I8_PHASE_CLOCK
    a.phase_clk = g_phase_clk;
#endif
    if (pb.mode == CONV_I8_MODE_CONVOLUTION) {
        // true convolution: tap (r, s) reads filter tap (R-1-r, S-1-s), i.e.
        // the taps from the far corner with negated strides (the offsets stay
        // inside [0, w_span))
        a.flt0 = (int)((pb.R - 1) * pl.wsR + (pb.S - 1) * pl.wsS);
        a.fR = -a.fR;
        a.fS = -a.fS;
    }
    a.P = (int)pb.P;
    a.Q = (int)pb.Q;
    a.PQ = (int)(pb.P * pb.Q);
    a.strH = (int)pb.str[0];
    a.strW = (int)pb.str[1];
    a.dilH = (int)pb.dil[0];
    a.dilW = (int)pb.dil[1];
    a.padH = (int)pb.pre[0];
    a.padW = (int)pb.pre[1];
    a.oN = (int)pb.y.s[0];
    a.oK = (int)pb.y.s[1];
    a.oP = (int)pb.y.s[2];
    a.oQ = (int)pb.y.s[3];
    if (pb.flip_out) {
        // reversed rows and columns: offsets stay inside the image's span
        a.out0 = (int)((pb.P - 1) * pb.y.s[2] + (pb.Q - 1) * pb.y.s[3]);
        a.oP = -a.oP;
        a.oQ = -a.oQ;
    }
    a.pix_linear = pl.pix_linear ? 1 : 0;
    a.pix_stride = (int)pl.pix_stride;
    a.nstages = pb.C > 0 ? (int)pl.nstages : 0;
    a.cc = (int)(pl.Cp / 16);
    a.inv_cc = a.cc > 0 ? 1.0f / (float)a.cc : 0.0f;
    a.inv_s = 1.0f / (float)a.S;
    a.tiles_n = (int)((pb.K + c.tn - 1) / c.tn);
    a.d_tn = make_divisor(a.tiles_n > 0 ? a.tiles_n : 1);
    a.d_pq = make_divisor(pb.P * pb.Q);
    a.d_q = make_divisor(pb.Q);
    a.Hp = (int)pl.Hp;
    a.Wf = (int)pl.Wf;
    a.inv_hp = pl.Hp > 0 ? 1.0f / (float)pl.Hp : 0.0f;
    a.Pr = (int)pl.Pr;
    a.inv_pr = pl.Pr > 0 ? 1.0f / (float)pl.Pr : 0.0f;
    a.ncblk = (int)(pl.Cp / 64);
    a.ksplit = 1;
    a.kchunk = 0x7fffffff;
    // stream the output past the L2 only when each store's lanes cover
    // consecutive elements (whole lines); scattered stores are merged in L2
    a.out_nt = (pl.pix_j ? (pb.y.s[3] == 1 || pb.Q == 1) && (pb.Q > 1 || pb.y.s[2] == 1)
                         : pb.y.s[1] == 1) ? 1 : 0;
    if (rq) {
        a.q8 = 1;
        a.q_scale = rq->scale;
        a.q_bias = rq->bias;
        a.q_alpha = rq->alpha;
        a.q_relu = rq->relu ? 1 : 0;
        // dword stores of four channels: channel stride 1, equally spaced
        // pixels, and every dword 4-byte aligned and inside one pixel's K
        a.q8_pack = pl.pix_linear && !pl.pix_j && pb.y.s[1] == 1 && pl.pix_stride % 4 == 0 &&
                    pb.K % 4 == 0 && ((uintptr_t)y_ptr & 3u) == 0 ? 1 : 0;
    }
    return a;
}

// Batch chunk [n0, n0 + nb) of a launch: the image and output windows and
// the tile count (0: nothing to launch).
int64_t set_chunk(IgemmArgs &a, const Problem &pb, const Plan &pl, const TileCfg &c, const int8_t *x,
                  void *y_ptr, int64_t n0, int64_t esize)
{
    const int64_t nb = std::min(pl.batch_chunk, pb.N - n0);
    a.img = x + n0 * pl.xsN;
    a.img_range = (int)((nb - 1) * pl.xsN + pl.x_img_span);
    a.out = (int32_t *)((int8_t *)y_ptr + n0 * pb.y.s[0] * esize);
    a.out_range = (int)(((nb - 1) * pb.y.s[0] + pl.y_img_span) * esize);
    a.N = (int)nb;
    a.sN = (int)pl.xsN;
    a.M = (int)(nb * pb.P * pb.Q);
    int64_t tiles = ((a.M + c.tm - 1) / c.tm) * (int64_t)a.tiles_n;
    if (c.kind == kPointwise) {
        // workgroups of four waves, each wave up to kPointwiseTilesPerWave
        // 32-pixel tiles; at least one workgroup per CU while there is work
        const int64_t t32 = (a.M + 31) / 32;
        tiles = std::max((t32 + 4 * kPointwiseTilesPerWave - 1) / (4 * kPointwiseTilesPerWave),
                         std::min<int64_t>(kCUs, (t32 + 3) / 4));
    }
    if (tiles == 0)
        return 0;
    a.tiles = (int)tiles;
    return tiles;
}

conv_i8_status_t run(const Problem &pb, const Plan &pl, const void *x_ptr, const void *w_ptr,
                     void *y_ptr, void *ws, hipStream_t stream, const conv_i8_requant_t *rq = nullptr)
{
    if (kTiles[pl.cfg].kind == kDirect)
        return launch_direct(pb, x_ptr, w_ptr, y_ptr, stream, rq);
    const int64_t esize = rq ? 1 : 4;        // bytes per output element
    const int8_t *x = (const int8_t *)x_ptr;
    const int8_t *w = (const int8_t *)w_ptr;
    int8_t *wsb = (int8_t *)ws;
    conv_i8_status_t st;
    RepackJob jobs[2];
    int njobs = 0;
    if (pl.repack_x && pb.C > 0) {
        jobs[njobs++] = repack_job(pb.x, x, wsb + pl.ws_x_off, pl.Cp);
        x = wsb + pl.ws_x_off;
    }
    if (pl.repack_w && pb.C > 0) {
        jobs[njobs++] = repack_job(pb.w, w, wsb + pl.ws_w_off, pl.Cp);
        w = wsb + pl.ws_w_off;
    }
    if (njobs > 0 && (st = launch_repacks(jobs, njobs, stream)) != CONV_I8_OK)
        return st;
    const TileCfg &c = kTiles[pl.cfg];
    IgemmArgs a = make_args(pb, pl, c, w, y_ptr, rq);
    for (int64_t n0 = 0; n0 < pb.N; n0 += pl.batch_chunk) {
        const int64_t nb = std::min(pl.batch_chunk, pb.N - n0);
        const int64_t tiles = set_chunk(a, pb, pl, c, x, y_ptr, n0, esize);
        if (tiles == 0)
            continue;
        unsigned ksplit = 1;
        int32_t *const out_chunk = a.out;
        const int64_t chunk_span = (nb - 1) * pb.y.s[0] + pl.y_img_span;
        if (pl.ksplit > 1 && !rq && c.kind == kIm2col) {
            ksplit = (unsigned)pl.ksplit;
            a.kchunk = (int)pl.kchunk;
            a.ksplit = (int)ksplit;
            if (pl.part) {
                // partial copies in the workspace, one per split
                a.part = 1;
                a.part_stride = pl.part_span;
                a.out = (int32_t *)(wsb + pl.ws_part_off);
            } else {
                // zeros first: the same kernel with no stages stores zeros
                IgemmArgs z = a;
                z.nstages = 0;
                z.ksplit = 1;
                c.launch(!pl.blocked, pl.pix_j, dim3((unsigned)tiles), stream, z);
                if (hipGetLastError() != hipSuccess)
                    return CONV_I8_ERR_HIP;
            }
        }
        c.launch(!pl.blocked, pl.pix_j, dim3((unsigned)tiles, ksplit), stream, a);
        if (hipGetLastError() != hipSuccess)
            return CONV_I8_ERR_HIP;
        if (a.part) {
            const int32_t *part = a.out;
            const bool v4 = chunk_span % 4 == 0 && pl.part_span % 4 == 0 && ((uintptr_t)out_chunk & 15u) == 0 &&
                            ((uintptr_t)part & 15u) == 0;
            const int64_t items = v4 ? chunk_span / 4 : chunk_span;
            const dim3 grid((unsigned)std::min<int64_t>(std::max<int64_t>((items + 255) / 256, 1), 4 * kCUs));
            if (v4)
                hipLaunchKernelGGL(split_reduce_kernel<true>, grid, dim3(256), 0, stream, part,
                                   (long long)pl.part_span, (int)ksplit, out_chunk, (long long)chunk_span);
            else
                hipLaunchKernelGGL(split_reduce_kernel<false>, grid, dim3(256), 0, stream, part,
                                   (long long)pl.part_span, (int)ksplit, out_chunk, (long long)chunk_span);
            if (hipGetLastError() != hipSuccess)
                return CONV_I8_ERR_HIP;
            a.part = 0;
            a.out = out_chunk;
        }
        a.ksplit = 1;
        a.kchunk = 0x7fffffff;
    }
    return CONV_I8_OK;
}

// Plans of recent problems.  A plan depends on the problem, on whether the
// image and filter can be read in place (layout and 16-byte alignment) and on
// a forced tile; repeated calls on one shape skip the tile search.
struct PlanKey {
    Problem pb;
    int32_t x_direct, w_direct, w_kmajor;
    char tile[24];
};
constexpr int kPlanCache = 16;
std::mutex g_plan_mutex;
PlanKey g_plan_keys[kPlanCache];
Plan g_plans[kPlanCache];
int g_plan_count = 0, g_plan_next = 0;

conv_i8_status_t prepare(const conv_i8_desc_t *image, const void *image_ptr,
                         const conv_i8_desc_t *filter, const void *filter_ptr,
                         const conv_i8_desc_t *out, const int64_t *pre, const int64_t *post,
                         const int64_t *stride, const int64_t *dil, Problem *pb, Plan *pl,
                         int32_t out_dtype = CONV_I8_DT_INT32,
                         int32_t mode = CONV_I8_MODE_CROSS_CORRELATION, bool flip_out = false,
                         bool split_ok = false, const char *tuned = nullptr)
{
    // The plan does not depend on the output dtype (it works in elements) nor
    // on the mode (the kernels read the taps in either order).
    conv_i8_status_t st = analyze(image, filter, out, pre, post, stride, dil, out_dtype, mode, pb);
    if (st != CONV_I8_OK)
        return st;
    pb->flip_out = flip_out ? 1 : 0;
    pb->split_ok = split_ok ? 1 : 0;
    PlanKey key;
    memset(&key, 0, sizeof key);  // padding takes part in the comparison
    static_assert(sizeof(Problem) % 8 == 0, "Problem has no tail padding to clear");
    key.pb = *pb;
    key.x_direct = direct_ok(pb->x, image_ptr) ? 1 : 0;
    key.w_direct = direct_ok(pb->w, filter_ptr) ? 1 : 0;
    key.w_kmajor = kmajor_ok(*pb, filter_ptr) ? 1 : 0;
    const char *forced = env_tile();
    const char *name = forced ? forced : tuned;   // a tile chosen outside the planner
    if (name)
        strncpy(key.tile, name, sizeof key.tile - 1);
    const bool cache = getenv("CONV_I8_COST") == nullptr && (!name || strlen(name) < sizeof key.tile - 1);
    if (cache) {
        std::lock_guard<std::mutex> lock(g_plan_mutex);
        for (int i = 0; i < g_plan_count; ++i)
            if (memcmp(&g_plan_keys[i], &key, sizeof key) == 0) {
                *pl = g_plans[i];
                return CONV_I8_OK;
            }
    }
    st = make_plan(*pb, image_ptr, filter_ptr, pl, tuned);
    if (st == CONV_I8_OK && cache) {
        std::lock_guard<std::mutex> lock(g_plan_mutex);
        g_plan_keys[g_plan_next] = key;
        g_plans[g_plan_next] = *pl;
        g_plan_next = (g_plan_next + 1) % kPlanCache;
        g_plan_count = std::min(g_plan_count + 1, kPlanCache);
    }
    return st;
}

// Requantisation parameters: present, 4-byte aligned arrays, a finite alpha
// when there is no scale array.
conv_i8_status_t check_requant(const conv_i8_requant_t *rq)
{
    if (!rq)
        return CONV_I8_ERR_NULL;
    if (((uintptr_t)rq->scale & 3u) != 0 || ((uintptr_t)rq->bias & 3u) != 0)
        return CONV_I8_ERR_PARAM;
    if (!rq->scale && !(rq->alpha == rq->alpha && rq->alpha - rq->alpha == 0.0f))
        return CONV_I8_ERR_PARAM;
    return CONV_I8_OK;
}

conv_i8_status_t check_ptrs(const Problem &pb, const void *x, const void *w, const void *y)
{
    if (pb.y.elems() == 0)
        return CONV_I8_OK;
    if (!y)
        return CONV_I8_ERR_NULL;
    if (pb.C > 0 && ((pb.x.elems() > 0 && !x) || (pb.w.elems() > 0 && !w)))
        return CONV_I8_ERR_NULL;
    return CONV_I8_OK;
}

}  // namespace
}  // namespace convi8

using namespace convi8;

extern "C" {

conv_i8_status_t conv_fprop_i8_out_dims(const conv_i8_desc_t *image, const conv_i8_desc_t *filter,
                                        const int64_t pre_padding[2], const int64_t post_padding[2],
                                        const int64_t stride[2], const int64_t dilation[2],
                                        int64_t out_dims[4])
{
    if (!out_dims)
        return CONV_I8_ERR_NULL;
    Problem pb;
    conv_i8_status_t st = analyze_inputs(image, filter, pre_padding, post_padding, stride, dilation, &pb);
    if (st != CONV_I8_OK)
        return st;
    out_dims[0] = pb.N;
    out_dims[1] = pb.K;
    out_dims[2] = pb.P;
    out_dims[3] = pb.Q;
    return CONV_I8_OK;
}

}  // extern "C"

namespace convi8 {
namespace {

// Shared body of the workspace-size entries.
conv_i8_status_t entry_workspace_size(const conv_i8_desc_t *image, const void *image_ptr,
                                      const conv_i8_desc_t *filter, const void *filter_ptr,
                                      const conv_i8_desc_t *out, const int64_t *pre,
                                      const int64_t *post, const int64_t *stride,
                                      const int64_t *dil, int32_t out_dtype, int32_t mode,
                                      size_t *workspace_bytes, bool flip_out = false,
                                      bool split_ok = false, const char *tuned = nullptr)
{
    if (!workspace_bytes)
        return CONV_I8_ERR_NULL;
    Problem pb;
    Plan pl;
    conv_i8_status_t st = prepare(image, image_ptr, filter, filter_ptr, out, pre, post, stride,
                                  dil, &pb, &pl, out_dtype, mode, flip_out, split_ok, tuned);
    if (st != CONV_I8_OK)
        return st;
    *workspace_bytes = pb.y.elems() == 0 || pb.C == 0 ? 0 : pl.ws_bytes;
    return CONV_I8_OK;
}

// Shared body of the compute entries.  rq is set exactly when out_dtype is
// INT8.  With alloc, the workspace is taken stream-ordered here; otherwise
// the caller's is checked and used.
conv_i8_status_t entry_run(const conv_i8_desc_t *image, const void *image_ptr,
                           const conv_i8_desc_t *filter, const void *filter_ptr,
                           const conv_i8_desc_t *out, void *out_ptr, const int64_t *pre,
                           const int64_t *post, const int64_t *stride, const int64_t *dil,
                           int32_t out_dtype, int32_t mode, const conv_i8_requant_t *rq, bool alloc,
                           void *workspace, size_t workspace_bytes, void *stream,
                           bool flip_out = false, bool split_ok = false, const char *tuned = nullptr)
{
    Problem pb;
    Plan pl;
    conv_i8_status_t st = prepare(image, image_ptr, filter, filter_ptr, out, pre, post, stride,
                                  dil, &pb, &pl, out_dtype, mode, flip_out, split_ok, tuned);
    if (st != CONV_I8_OK)
        return st;
    if (out_dtype == CONV_I8_DT_INT8 && (st = check_requant(rq)) != CONV_I8_OK)
        return st;
    if ((st = check_ptrs(pb, image_ptr, filter_ptr, out_ptr)) != CONV_I8_OK)
        return st;
    if (pb.y.elems() == 0)
        return CONV_I8_OK;
    const size_t need = pb.C == 0 ? 0 : pl.ws_bytes;
    hipStream_t s = (hipStream_t)stream;
    void *ws = workspace;
    if (alloc) {
        ws = nullptr;
        if (need > 0 && hipMallocAsync(&ws, need, s) != hipSuccess)
            return CONV_I8_ERR_HIP;
    } else {
        if (workspace_bytes < need)
            return CONV_I8_ERR_WORKSPACE;
        if (need > 0 && !workspace)
            return CONV_I8_ERR_NULL;
        if (need > 0 && ((uintptr_t)workspace & 255u) != 0)
            return CONV_I8_ERR_WORKSPACE;
    }
    if (log_enabled())
        fprintf(stderr, "conv_i8%s%s: %s\n", rq ? " (requant)" : "",
                mode == CONV_I8_MODE_CONVOLUTION ? " (convolution)" : "", describe(pb, pl).c_str());
    st = run(pb, pl, image_ptr, filter_ptr, out_ptr, ws, s, out_dtype == CONV_I8_DT_INT8 ? rq : nullptr);
    if (alloc && ws && hipFreeAsync(ws, s) != hipSuccess && st == CONV_I8_OK)
        st = CONV_I8_ERR_HIP;
    return st;
}

// ---------------------------------------------------------------------------
// Allocation-free entry: the workspace is a static device array (one copy per
// GPU, alive until the process ends) instead of caller memory or
// hipMallocAsync.  Host code never passes the array's name to a kernel or a
// copy: the name is a host-side stand-in; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace
}  // namespace convi8

#ifndef CONV_I8_HOST_ONLY
static __device__ __align__(256) uint8_t scratch[CONV_I8_NOALLOC_SCRATCH_BYTES];
#endif

namespace convi8 {
namespace {

// Device address of this device's scratch array (the device current on the
// calling thread, which must be the device of the stream the call uses).
conv_i8_status_t scratch_address(void *stream, void **addr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return CONV_I8_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices)
        return CONV_I8_ERR_UNSUPPORTED;
    if (stream) {
        int sdev = -1;
        if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess)
            return CONV_I8_ERR_HIP;
        if (sdev != dev)
            return CONV_I8_ERR_PARAM;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
#ifdef CONV_I8_HOST_ONLY
        return CONV_I8_ERR_HIP;
#else
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return CONV_I8_ERR_HIP;
#endif
        g_scratch_ptr[dev] = p;
    }
    *addr = g_scratch_ptr[dev];
    return CONV_I8_OK;
}

// Output dtype and requantisation block of the extended entries: INT32
// without a block, INT8 with one.
conv_i8_status_t ex_out_dtype(const conv_i8_desc_t *out, const conv_i8_requant_t *rq, int32_t *dt)
{
    if (!out)
        return CONV_I8_ERR_NULL;
    if (out->dtype == CONV_I8_DT_INT32) {
        if (rq)
            return CONV_I8_ERR_PARAM;
        *dt = CONV_I8_DT_INT32;
        return CONV_I8_OK;
    }
    if (out->dtype == CONV_I8_DT_INT8) {
        *dt = CONV_I8_DT_INT8;
        return CONV_I8_OK;
    }
    return CONV_I8_ERR_DTYPE;
}

// ---------------------------------------------------------------------------
// Data gradient (dgrad) as forward convolutions over stride phases.
//
// dX[n,c,h,w] sums dY[n,k,p,q] * W[k,c,r,s] over the taps with
// h + pre_h - r*dil_h = p*stride_h (and likewise along w).  For the rows h of
// one residue ph = h mod stride_h, the taps that reach them are
// r = r0 + t*j (t = stride_h / g, g = gcd(dil_h, stride_h)), and row
// i = (h - ph) / stride_h reads dY row i + e - j*(dil_h / g): a stride-1
// cross-correlation of dY with the reversed sub-filter, dilation dil_h / g.
// Each (ph, pw) phase is one forward call on views: image = dY (channels K),
// filter = W transposed to [C, K, .., ..] and subsampled by t, output = the
// phase's rows and columns of dX.
// ---------------------------------------------------------------------------
struct DgradDim {
    bool zero = false;             // no tap reaches these rows: they are 0
    int64_t rows = 0;              // dX rows of the phase (Hi)
    int64_t base = 0, step = 1;    // filter taps used: base + step*j, j < taps
    int64_t taps = 0;
    int64_t dil = 1;               // dilation of the phase call
    int64_t crop = 0, used = 0;    // dY rows [crop, crop + used) are read
    int64_t pre = 0, post = 0;     // padding of the phase call
};

// One spatial dim of one phase.  flip: the dgrad is of the true-convolution
// forward (taps reversed), so the sub-filter is read forwards.
DgradDim dgrad_dim(int64_t ph, int64_t len, int64_t out_len_, int64_t pre, int64_t st, int64_t dil,
                   int64_t R, bool flip)
{
    DgradDim d;
    d.rows = ph < len ? (len - ph + st - 1) / st : 0;
    if (d.rows == 0)
        return d;
    const int64_t g = std::gcd(dil, st);
    const int64_t t = st / g;
    int64_t r0 = -1;
    for (int64_t r = 0; r < std::min(R, t); ++r)
        if ((ph + pre - r * dil) % st == 0) {
            r0 = r;
            break;
        }
    if (r0 < 0) {
        d.zero = true;
        return d;
    }
    d.taps = (R - r0 + t - 1) / t;
    d.step = t;
    d.dil = dil / g;
    // forward call read in reverse (convolution mode) for the plain dgrad;
    // with flip the reversed filter reverses back: read from the far end
    d.base = flip ? R - 1 - r0 - t * (d.taps - 1) : r0;
    const int64_t e = (ph + pre - r0 * dil) / st;       // exact
    int64_t pad = (d.taps - 1) * d.dil - e;
    int64_t used = out_len_;
    if (pad < 0) {
        d.crop = -pad;
        used -= d.crop;
        pad = 0;
    }
    if (used <= 0) {
        d.zero = true;
        return d;
    }
    int64_t post = d.rows - used - pad + d.dil * (d.taps - 1);
    if (post < 0) {
        used += post;
        post = 0;
    }
    if (used <= 0) {
        d.zero = true;
        return d;
    }
    d.used = used;
    d.pre = pad;
    d.post = post;
    return d;
}

conv_i8_desc_t make_desc(int32_t dtype, const int64_t d[4], const int64_t st[4])
{
    conv_i8_desc_t r;
    r.dtype = dtype;
    r.ndim = 4;
    for (int i = 0; i < 4; ++i) {
        r.dims[i] = d[i];
        r.strides[i] = st[i];
    }
    return r;
}

struct DgradProblem {
    T4 dy, w, dx;
    int64_t N, K, C, R, S, H, W, P, Q;
    int64_t pre[2], post[2], str[2], dil[2];
};

conv_i8_status_t dgrad_analyze(const conv_i8_desc_t *loss, const conv_i8_desc_t *filter,
                               const conv_i8_desc_t *dx, const int64_t *pre, const int64_t *post,
                               const int64_t *stride, const int64_t *dil, int32_t mode,
                               DgradProblem *dp)
{
    conv_i8_status_t st;
    if ((st = read_desc(loss, CONV_I8_DT_INT8, &dp->dy)) != CONV_I8_OK ||
        (st = read_desc(filter, CONV_I8_DT_INT8, &dp->w)) != CONV_I8_OK ||
        (st = read_desc(dx, CONV_I8_DT_INT32, &dp->dx)) != CONV_I8_OK)
        return st;
    Problem tmp;
    if ((st = read_params(pre, post, stride, dil, &tmp)) != CONV_I8_OK)
        return st;
    if (mode != CONV_I8_MODE_CROSS_CORRELATION && mode != CONV_I8_MODE_CONVOLUTION)
        return CONV_I8_ERR_PARAM;
    for (int i = 0; i < 2; ++i) {
        dp->pre[i] = tmp.pre[i];
        dp->post[i] = tmp.post[i];
        dp->str[i] = tmp.str[i];
        dp->dil[i] = tmp.dil[i];
    }
    dp->N = dp->dx.d[0];
    dp->C = dp->dx.d[1];
    dp->H = dp->dx.d[2];
    dp->W = dp->dx.d[3];
    dp->K = dp->w.d[0];
    dp->R = dp->w.d[2];
    dp->S = dp->w.d[3];
    if (dp->R < 1 || dp->S < 1)
        return CONV_I8_ERR_DIMS;
    if (dp->w.d[1] != dp->C)
        return CONV_I8_ERR_CHANNELS;
    for (int i = 0; i < 4; ++i)
        if (dp->dx.d[i] > kI32Max / 4 || dp->w.d[i] > kI32Max / 4 || dp->dy.d[i] > kI32Max / 4)
            return CONV_I8_ERR_UNSUPPORTED;
    int64_t krs;
    if (!mul_ok(dp->K, dp->R * dp->S, &krs) || krs > CONV_I8_MAX_REDUCTION)
        return CONV_I8_ERR_RANGE;
    dp->P = out_len(dp->H, dp->pre[0], dp->post[0], dp->R, dp->str[0], dp->dil[0]);
    dp->Q = out_len(dp->W, dp->pre[1], dp->post[1], dp->S, dp->str[1], dp->dil[1]);
    if (dp->P < 1 || dp->Q < 1)
        return CONV_I8_ERR_OUT_DIMS;
    const int64_t want[4] = {dp->N, dp->K, dp->P, dp->Q};
    for (int i = 0; i < 4; ++i)
        if (dp->dy.d[i] != want[i])
            return CONV_I8_ERR_OUT_DIMS;
    int64_t sp;
    if (!span_of(dp->dy, &sp) || !span_of(dp->w, &sp) || !span_of(dp->dx, &sp))
        return CONV_I8_ERR_UNSUPPORTED;
    if (!non_overlapping(dp->dx))
        return CONV_I8_ERR_STRIDES;
    return CONV_I8_OK;
}

// Visit the forward calls of a dgrad: fn(image, x_ptr, filter, w_ptr, out,
// y_ptr, pre, post, stride, dil, mode) for every phase in order.
template <class Fn>
conv_i8_status_t dgrad_phases(const DgradProblem &dp, const void *dy_ptr, const void *w_ptr,
                              void *dx_ptr, int32_t mode, Fn &&fn)
{
    const bool flip = mode == CONV_I8_MODE_CONVOLUTION;
    const int32_t sub_mode = flip ? CONV_I8_MODE_CROSS_CORRELATION : CONV_I8_MODE_CONVOLUTION;
    for (int64_t ph = 0; ph < dp.str[0]; ++ph) {
        const DgradDim a = dgrad_dim(ph, dp.H, dp.P, dp.pre[0], dp.str[0], dp.dil[0], dp.R, flip);
        if (a.rows == 0)
            continue;
        for (int64_t pw = 0; pw < dp.str[1]; ++pw) {
            const DgradDim b = dgrad_dim(pw, dp.W, dp.Q, dp.pre[1], dp.str[1], dp.dil[1], dp.S, flip);
            if (b.rows == 0)
                continue;
            const int64_t od[4] = {dp.N, dp.C, a.rows, b.rows};
            const int64_t os[4] = {dp.dx.s[0], dp.dx.s[1], dp.str[0] * dp.dx.s[2], dp.str[1] * dp.dx.s[3]};
            const conv_i8_desc_t out = make_desc(CONV_I8_DT_INT32, od, os);
            void *y = dx_ptr ? (void *)((int32_t *)dx_ptr + ph * dp.dx.s[2] + pw * dp.dx.s[3]) : nullptr;
            const int64_t one[2] = {1, 1}, zero[2] = {0, 0};
            conv_i8_status_t st;
            if (a.zero || b.zero) {
                // no tap reaches this phase: a convolution over zero channels
                // writes its zeros
                const int64_t xd[4] = {dp.N, 0, a.rows, b.rows}, xs[4] = {0, 0, 0, 0};
                const int64_t wd[4] = {dp.C, 0, 1, 1};
                const conv_i8_desc_t img = make_desc(CONV_I8_DT_INT8, xd, xs);
                const conv_i8_desc_t flt = make_desc(CONV_I8_DT_INT8, wd, xs);
                st = fn(&img, nullptr, &flt, nullptr, &out, y, zero, zero, one, one,
                        (int32_t)CONV_I8_MODE_CROSS_CORRELATION);
            } else {
                const int64_t xd[4] = {dp.N, dp.K, a.used, b.used};
                const int64_t xs[4] = {dp.dy.s[0], dp.dy.s[1], dp.dy.s[2], dp.dy.s[3]};
                const int64_t wd[4] = {dp.C, dp.K, a.taps, b.taps};
                const int64_t ws[4] = {dp.w.s[1], dp.w.s[0], a.step * dp.w.s[2], b.step * dp.w.s[3]};
                const conv_i8_desc_t img = make_desc(CONV_I8_DT_INT8, xd, xs);
                const conv_i8_desc_t flt = make_desc(CONV_I8_DT_INT8, wd, ws);
                const void *x = dy_ptr ? (const void *)((const int8_t *)dy_ptr + a.crop * dp.dy.s[2] +
                                                        b.crop * dp.dy.s[3]) : nullptr;
                const void *wp = w_ptr ? (const void *)((const int8_t *)w_ptr + a.base * dp.w.s[2] +
                                                        b.base * dp.w.s[3]) : nullptr;
                const int64_t pre2[2] = {a.pre, b.pre}, post2[2] = {a.post, b.post};
                const int64_t dil2[2] = {a.dil, b.dil};
                st = fn(&img, x, &flt, wp, &out, y, pre2, post2, one, dil2, sub_mode);
            }
            if (st != CONV_I8_OK)
                return st;
        }
    }
    return CONV_I8_OK;
}

// The filter views of a strided layer's phases, packed once for all phases.
// With several phases each phase's convolution would repack its own
// (transposed, subsampled) filter view in a launch of its own; when every
// view needs a repack (none is read k-major), the packed copies are directly
// readable (K a multiple of 16) and the phases read the loss in place (else
// each phase repacks its part of the loss, and that launch carries its filter
// too), one repack launch writes all the views into regions at the start of
// the workspace and each phase reads its region in place.
struct DgradPack {
    bool on = false;
    int n = 0;                             // phases with taps, in dgrad_phases order
    T4 view[kRepackMaxJobs];
    const void *src[kRepackMaxJobs];
    size_t off[kRepackMaxJobs];
    size_t bytes = 0;                      // all regions, 256-byte aligned
    int64_t Kp = 0;
};

conv_i8_status_t dgrad_pack_plan(const DgradProblem &dp, const void *dy_ptr, const void *w_ptr,
                                 int32_t mode, DgradPack *pk)
{
    *pk = DgradPack{};
    if (dp.str[0] * dp.str[1] < 2)
        return CONV_I8_OK;                 // one phase: nothing to share
    if (dp.K % 16 != 0 || (dp.K > 1 && dp.dy.s[1] != 1))
        return CONV_I8_OK;                 // packed views not readable in place, or the
                                           // phases repack their part of the loss anyway
    bool ok = true;
    int n = 0;
    conv_i8_status_t st = dgrad_phases(
        dp, dy_ptr, w_ptr, nullptr, mode,
        [&](const conv_i8_desc_t *img, const void *x, const conv_i8_desc_t *flt, const void *w,
            const conv_i8_desc_t *out, void *, const int64_t *pre_, const int64_t *post_,
            const int64_t *stride_, const int64_t *dil_, int32_t m) {
            if (flt->dims[1] == 0)
                return CONV_I8_OK;         // a phase no tap reaches: zero channels, no filter
            {
                // a phase whose kernel reads its filter view in place, k-major:
                // nothing to pack (the others, if any, repack their own view)
                Problem ppb;
                Plan ppl;
                if (prepare(img, x, flt, w, out, pre_, post_, stride_, dil_, &ppb, &ppl, CONV_I8_DT_INT32, m) ==
                        CONV_I8_OK &&
                    ppl.kmaj)
                    ok = false;
            }
            T4 ti;
            conv_i8_status_t s1 = read_desc(img, CONV_I8_DT_INT8, &ti);
            if (s1 != CONV_I8_OK)
                return s1;
            if (!direct_ok(ti, x))
                ok = false;                // the phase repacks its image anyway: one launch
                                           // carries both of its repacks
            if (n >= kRepackMaxJobs) {
                ok = false;
                ++n;
                return CONV_I8_OK;
            }
            T4 t;
            conv_i8_status_t s2 = read_desc(flt, CONV_I8_DT_INT8, &t);
            if (s2 != CONV_I8_OK)
                return s2;
            if (direct_ok(t, w))
                ok = false;                // already readable in place
            pk->view[n] = t;
            pk->src[n] = w;
            ++n;
            return CONV_I8_OK;
        });
    if (st != CONV_I8_OK)
        return st;
    if (!ok || n < 2 || n > kRepackMaxJobs)
        return CONV_I8_OK;
    pk->Kp = dp.K;
    size_t off = 0;
    for (int i = 0; i < n; ++i) {
        const T4 &t = pk->view[i];
        int64_t b;
        if (!mul_ok(t.d[0] * t.d[2], t.d[3] * pk->Kp, &b))
            return CONV_I8_OK;
        pk->off[i] = off;
        off = align_up(off + (size_t)b, 256);
    }
    pk->n = n;
    pk->bytes = off;
    pk->on = true;
    return CONV_I8_OK;
}

// Descriptor of phase i's packed filter: [C, K, taps_h, taps_w] with K innermost.
conv_i8_desc_t dgrad_packed_desc(const DgradPack &pk, int i)
{
    const T4 &t = pk.view[i];
    const int64_t d[4] = {t.d[0], t.d[1], t.d[2], t.d[3]};
    const int64_t st[4] = {t.d[2] * t.d[3] * pk.Kp, 1, t.d[3] * pk.Kp, pk.Kp};
    return make_desc(CONV_I8_DT_INT8, d, st);
}

// The loss of a strided layer packed once for all phases.  With several
// phases each phase reads dY in full; a dY the kernels cannot read in place
// (not channel-innermost, or misaligned) would be repacked by every phase.
// When K is a multiple of 16 it is instead packed once, channel-innermost
// ([N][P][Q][K], 256-byte aligned at the start of the workspace), and the
// phases are planned and run on that copy (so the filter pack and the
// one-launch path of a channels-last loss apply to them too).
struct DgradLossPack {
    bool on = false;
    size_t bytes = 0;                      // the region, rounded to 256 bytes
};

DgradLossPack dgrad_loss_pack(const DgradProblem &dp, const void *dy_ptr, int32_t mode, DgradProblem *dp2)
{
    DgradLossPack lp;
    *dp2 = dp;
    int64_t b;
    if (dp.str[0] * dp.str[1] < 2 || dp.K % 16 != 0 || dp.K == 0 || direct_ok(dp.dy, dy_ptr) ||
        !mul_ok(dp.N * dp.P, dp.Q * dp.K, &b) || b == 0)
        return lp;
    int64_t tiles = 0;
    repack_job(dp.dy, nullptr, nullptr, dp.K, &tiles);
    if (tiles > kI32Max || dp.P * dp.Q > kI32Max)
        return lp;
    // only when two or more phases have taps (and would each repack dY)
    int with_taps = 0;
    dgrad_phases(dp, nullptr, nullptr, nullptr, mode,
                 [&](const conv_i8_desc_t *, const void *, const conv_i8_desc_t *flt, const void *,
                     const conv_i8_desc_t *, void *, const int64_t *, const int64_t *, const int64_t *,
                     const int64_t *, int32_t) {
                     with_taps += flt->dims[1] > 0 ? 1 : 0;
                     return CONV_I8_OK;
                 });
    if (with_taps < 2)
        return lp;
    lp.on = true;
    lp.bytes = align_up((size_t)b, 256);
    const int64_t ps[4] = {dp.P * dp.Q * dp.K, 1, dp.Q * dp.K, dp.K};
    for (int i = 0; i < 4; ++i)
        dp2->dy.s[i] = ps[i];
    return lp;
}

conv_i8_status_t dgrad_workspace(const DgradProblem &dp0, const void *dy_ptr0, const void *w_ptr,
                                 int32_t mode, size_t *bytes, DgradPack *pack = nullptr,
                                 DgradLossPack *loss_pack = nullptr)
{
    DgradProblem dp;
    const DgradLossPack lp = dgrad_loss_pack(dp0, dy_ptr0, mode, &dp);
    if (loss_pack)
        *loss_pack = lp;
    // planned on the packed copy when there is one (its region is 256-byte
    // aligned: no pointer needed for the alignment checks)
    const void *dy_ptr = lp.on ? nullptr : dy_ptr0;
    DgradPack own;
    DgradPack &pk = pack ? *pack : own;
    conv_i8_status_t st = dgrad_pack_plan(dp, dy_ptr, w_ptr, mode, &pk);
    if (st != CONV_I8_OK)
        return st;
    size_t most = 0;
    int i = 0;
    st = dgrad_phases(
        dp, dy_ptr, w_ptr, nullptr, mode,
        [&](const conv_i8_desc_t *img, const void *x, const conv_i8_desc_t *flt, const void *w,
            const conv_i8_desc_t *out, void *, const int64_t *pre, const int64_t *post,
            const int64_t *stride, const int64_t *dil, int32_t m) {
            size_t n = 0;
            conv_i8_desc_t packed;
            if (pk.on && flt->dims[1] > 0) {
                packed = dgrad_packed_desc(pk, i++);
                flt = &packed;
                w = nullptr;               // the region is 256-byte aligned
            }
            conv_i8_status_t s = entry_workspace_size(img, x, flt, w, out, pre, post, stride, dil,
                                                      CONV_I8_DT_INT32, m, &n);
            most = std::max(most, n);
            return s;
        });
    *bytes = lp.bytes + pk.bytes + most;
    return st;
}

// The phases of a strided data gradient in one launch, when every phase reads
// its loss and its filter view in place (channels-last loss, k-major view)
// on one im2col tile with one store policy, in one batch chunk: workgroups
// [first[p], first[p+1]) run phase p.  The phases write disjoint elements of
// dX, so running them together gives the bytes of running them in order.
// *done is false (and nothing is launched) when the phases do not qualify.
conv_i8_status_t dgrad_one_launch(const DgradProblem &dp, const void *loss_ptr, const void *filter_ptr,
                                  void *dx_ptr, int32_t mode, hipStream_t stream, bool *done)
{
    *done = false;
    struct Phase {
        Problem pb;
        Plan pl;
        const void *x, *w;
        void *y;
    };
    Phase ph[kMaxPhases];
    int n = 0;
    bool ok = true;
    conv_i8_status_t st = dgrad_phases(
        dp, loss_ptr, filter_ptr, dx_ptr, mode,
        [&](const conv_i8_desc_t *img, const void *x, const conv_i8_desc_t *flt, const void *w,
            const conv_i8_desc_t *out, void *y, const int64_t *pre_, const int64_t *post_, const int64_t *stride_,
            const int64_t *dil_, int32_t m) {
            if (!ok)
                return CONV_I8_OK;
            if (n >= kMaxPhases || flt->dims[1] == 0) {
                ok = false;        // too many phases, or one that no tap reaches
                return CONV_I8_OK;
            }
            Phase &p = ph[n++];
            conv_i8_status_t r = prepare(img, x, flt, w, out, pre_, post_, stride_, dil_, &p.pb, &p.pl,
                                         CONV_I8_DT_INT32, m);
            if (r != CONV_I8_OK)
                return r;
            p.x = x;
            p.w = w;
            p.y = y;
            const TileCfg &c = kTiles[p.pl.cfg];
            if (!c.launch_phases || p.pl.repack_x || p.pl.repack_w || !p.pl.kmaj || !p.pl.blocked ||
                p.pl.ksplit > 1 || p.pl.batch_chunk < p.pb.N || p.pb.C == 0 || p.pb.y.elems() == 0)
                ok = false;
            if (n > 1 && (p.pl.cfg != ph[0].pl.cfg || p.pl.pix_j != ph[0].pl.pix_j))
                ok = false;
            return CONV_I8_OK;
        });
    if (st != CONV_I8_OK || !ok || n < 2)
        return st;
    const TileCfg &c = kTiles[ph[0].pl.cfg];
    IgemmPhases m{};
    int64_t total = 0;
    for (int i = 0; i < n; ++i) {
        IgemmArgs a = make_args(ph[i].pb, ph[i].pl, c, (const int8_t *)ph[i].w, ph[i].y, nullptr);
        const int64_t tiles = set_chunk(a, ph[i].pb, ph[i].pl, c, (const int8_t *)ph[i].x, ph[i].y, 0, 4);
        if (tiles == 0 || (i > 0 && a.out_nt != m.ph[0].out_nt))
            return CONV_I8_OK;   // one store policy for every phase
        m.ph[i] = a;
        m.first[i] = (int)total;
        total += tiles;
        if (total > kI32Max)
            return CONV_I8_OK;
    }
    for (int i = n; i <= kMaxPhases; ++i)
        m.first[i] = (int)total;
    m.nph = n;
    if (log_enabled()) {
        for (int i = 0; i < n; ++i)
            fprintf(stderr, "conv_i8%s: %s\n", mode == CONV_I8_MODE_CONVOLUTION ? " (convolution)" : "",
                    describe(ph[i].pb, ph[i].pl).c_str());
        fprintf(stderr, "conv_i8: %d data-gradient phases in one launch of %lld workgroups\n", n, (long long)total);
    }
    c.launch_phases(ph[0].pl.pix_j, dim3((unsigned)total), stream, m);
    if (hipGetLastError() != hipSuccess)
        return CONV_I8_ERR_HIP;
    *done = true;
    return CONV_I8_OK;
}

conv_i8_status_t dgrad_entry(const conv_i8_desc_t *loss, const void *loss_ptr,
                             const conv_i8_desc_t *filter, const void *filter_ptr,
                             const conv_i8_desc_t *dx, void *dx_ptr, const int64_t *pre,
                             const int64_t *post, const int64_t *stride, const int64_t *dil,
                             int32_t mode, bool alloc, void *workspace, size_t workspace_bytes,
                             void *stream)
{
    DgradProblem dp;
    conv_i8_status_t st = dgrad_analyze(loss, filter, dx, pre, post, stride, dil, mode, &dp);
    if (st != CONV_I8_OK)
        return st;
    if (dp.dx.elems() == 0)
        return CONV_I8_OK;
    if (!dx_ptr || (dp.K > 0 && ((dp.dy.elems() > 0 && !loss_ptr) || (dp.w.elems() > 0 && !filter_ptr))))
        return CONV_I8_ERR_NULL;
    size_t need = 0;
    DgradPack pk;
    DgradLossPack lp;
    if ((st = dgrad_workspace(dp, loss_ptr, filter_ptr, mode, &need, &pk, &lp)) != CONV_I8_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    void *ws = workspace;
    if (alloc) {
        ws = nullptr;
        if (need > 0 && hipMallocAsync(&ws, need, s) != hipSuccess)
            return CONV_I8_ERR_HIP;
    } else {
        if (workspace_bytes < need)
            return CONV_I8_ERR_WORKSPACE;
        if (need > 0 && !workspace)
            return CONV_I8_ERR_NULL;
        if (need > 0 && ((uintptr_t)workspace & 255u) != 0)
            return CONV_I8_ERR_WORKSPACE;
    }
    // workspace: [packed loss][packed filter views][the phases' own]
    int8_t *const wsb = (int8_t *)ws;
    int8_t *const ws_pk = wsb + lp.bytes;
    DgradProblem dpr = dp;                  // the problem the phases run on
    const void *dy_run = loss_ptr;
    if (lp.on) {
        dgrad_loss_pack(dp, loss_ptr, mode, &dpr);
        dy_run = wsb;
        if (log_enabled())
            fprintf(stderr, "conv_i8: data-gradient loss packed once for %lld phases\n",
                    (long long)(dp.str[0] * dp.str[1]));
    }
    {
        // the loss and every phase's filter view packed in as few launches
        // as the job slots allow
        RepackJob jobs[kRepackMaxJobs];
        int nj = 0;
        if (lp.on)
            jobs[nj++] = repack_job(dp.dy, (const int8_t *)loss_ptr, wsb, dp.K);
        for (int i = 0; pk.on && i < pk.n && st == CONV_I8_OK; ++i) {
            if (nj == kRepackMaxJobs) {
                st = launch_repacks(jobs, nj, s);
                nj = 0;
            }
            jobs[nj++] = repack_job(pk.view[i], (const int8_t *)pk.src[i], ws_pk + pk.off[i], pk.Kp);
        }
        if (nj > 0 && st == CONV_I8_OK)
            st = launch_repacks(jobs, nj, s);
    }
    if (st == CONV_I8_OK && !pk.on) {
        bool done = false;
        st = dgrad_one_launch(dpr, dy_run, filter_ptr, dx_ptr, mode, s, &done);
        if (st != CONV_I8_OK || done) {
            if (alloc && ws && hipFreeAsync(ws, s) != hipSuccess && st == CONV_I8_OK)
                st = CONV_I8_ERR_HIP;
            return st;
        }
    }
    // the phases run one after another on the stream and share the workspace
    // past the packed loss and filters
    int i = 0;
    const size_t phase_ws = need - lp.bytes - pk.bytes;
    if (st == CONV_I8_OK)
        st = dgrad_phases(dpr, dy_run, filter_ptr, dx_ptr, mode,
                          [&](const conv_i8_desc_t *img, const void *x, const conv_i8_desc_t *flt,
                              const void *w, const conv_i8_desc_t *out, void *y, const int64_t *pre_,
                              const int64_t *post_, const int64_t *stride_, const int64_t *dil_,
                              int32_t m) {
                              conv_i8_desc_t packed;
                              if (pk.on && flt->dims[1] > 0) {
                                  w = ws_pk + pk.off[i];
                                  packed = dgrad_packed_desc(pk, i++);
                                  flt = &packed;
                              }
                              return entry_run(img, x, flt, w, out, y, pre_, post_, stride_, dil_,
                                               CONV_I8_DT_INT32, m, nullptr, false,
                                               phase_ws ? ws_pk + pk.bytes : nullptr, phase_ws, stream);
                          });
    if (alloc && ws && hipFreeAsync(ws, s) != hipSuccess && st == CONV_I8_OK)
        st = CONV_I8_ERR_HIP;
    return st;
}

// ---------------------------------------------------------------------------
// Weight gradient (wgrad) as one forward convolution.
//
// dW[k,c,r,s] = sum_{n,p,q} X[n,c, p*st_h - pre_h + r*dil_h, ..] * dY[n,k,p,q]
// is a forward convolution of the image transposed to [C, N, H, W] (batch C,
// channels N) with the loss transposed to [K, N, P, Q] (a P x Q filter),
// stride dil, dilation st, the same pre-padding, written to dW transposed to
// [C, K, R, S].  Its post-padding is cut so that exactly R x S outputs come
// out (rows no output reads are cropped off the image).  The weight gradient
// of true convolution writes tap (r, s) to (R-1-r, S-1-s): the same call with
// reversed output rows and columns.
// ---------------------------------------------------------------------------
struct WgradProblem {
    T4 x, dy, dw;
    int64_t N, C, H, W, K, R, S, P, Q;
    int64_t pre[2], post[2], str[2], dil[2];
};

// The measured table's tile for a weight gradient, keyed by the gradient's
// own problem (the forward layer's dims and parameters, dW's layout).
const char *tuned_wgrad_tile(const WgradProblem &wp)
{
    const int64_t d[7] = {wp.N, wp.C, wp.H, wp.W, wp.K, wp.R, wp.S};
    return tuned_lookup(1, d, wp.pre, wp.post, wp.str, wp.dil, wp.dw.s[1] == 1 ? 0 : 1);
}

conv_i8_status_t wgrad_analyze(const conv_i8_desc_t *image, const conv_i8_desc_t *loss,
                               const conv_i8_desc_t *dw, const int64_t *pre, const int64_t *post,
                               const int64_t *stride, const int64_t *dil, int32_t mode,
                               WgradProblem *wp)
{
    conv_i8_status_t st;
    if ((st = read_desc(image, CONV_I8_DT_INT8, &wp->x)) != CONV_I8_OK ||
        (st = read_desc(loss, CONV_I8_DT_INT8, &wp->dy)) != CONV_I8_OK ||
        (st = read_desc(dw, CONV_I8_DT_INT32, &wp->dw)) != CONV_I8_OK)
        return st;
    Problem tmp;
    if ((st = read_params(pre, post, stride, dil, &tmp)) != CONV_I8_OK)
        return st;
    if (mode != CONV_I8_MODE_CROSS_CORRELATION && mode != CONV_I8_MODE_CONVOLUTION)
        return CONV_I8_ERR_PARAM;
    for (int i = 0; i < 2; ++i) {
        wp->pre[i] = tmp.pre[i];
        wp->post[i] = tmp.post[i];
        wp->str[i] = tmp.str[i];
        wp->dil[i] = tmp.dil[i];
    }
    wp->N = wp->x.d[0];
    wp->C = wp->x.d[1];
    wp->H = wp->x.d[2];
    wp->W = wp->x.d[3];
    wp->K = wp->dw.d[0];
    wp->R = wp->dw.d[2];
    wp->S = wp->dw.d[3];
    if (wp->R < 1 || wp->S < 1)
        return CONV_I8_ERR_DIMS;
    if (wp->dw.d[1] != wp->C)
        return CONV_I8_ERR_CHANNELS;
    for (int i = 0; i < 4; ++i)
        if (wp->x.d[i] > kI32Max / 4 || wp->dw.d[i] > kI32Max / 4 || wp->dy.d[i] > kI32Max / 4)
            return CONV_I8_ERR_UNSUPPORTED;
    wp->P = out_len(wp->H, wp->pre[0], wp->post[0], wp->R, wp->str[0], wp->dil[0]);
    wp->Q = out_len(wp->W, wp->pre[1], wp->post[1], wp->S, wp->str[1], wp->dil[1]);
    if (wp->P < 1 || wp->Q < 1)
        return CONV_I8_ERR_OUT_DIMS;
    const int64_t want[4] = {wp->N, wp->K, wp->P, wp->Q};
    for (int i = 0; i < 4; ++i)
        if (wp->dy.d[i] != want[i])
            return CONV_I8_ERR_OUT_DIMS;
    int64_t npq;
    if (!mul_ok(wp->N, wp->P * wp->Q, &npq) || npq > CONV_I8_MAX_REDUCTION)
        return CONV_I8_ERR_RANGE;
    int64_t sp;
    if (!span_of(wp->x, &sp) || !span_of(wp->dy, &sp) || !span_of(wp->dw, &sp))
        return CONV_I8_ERR_UNSUPPORTED;
    if (!non_overlapping(wp->dw))
        return CONV_I8_ERR_STRIDES;
    return CONV_I8_OK;
}

// The forward call of a wgrad: fn(image, x, filter, w, out, y, pre, post,
// stride, dil, flip_out).
template <class Fn>
conv_i8_status_t wgrad_call(const WgradProblem &wp, const void *x_ptr, const void *dy_ptr,
                            void *dw_ptr, int32_t mode, Fn &&fn)
{
    // image rows [0, need) are the ones the outputs read: the last output row
    // reads row (P-1)*st - pre + (R-1)*dil
    int64_t len[2], post2[2];
    bool reads = true;
    const int64_t in[2] = {wp.H, wp.W}, taps[2] = {wp.R, wp.S}, outn[2] = {wp.P, wp.Q};
    for (int i = 0; i < 2; ++i) {
        const int64_t need = (outn[i] - 1) * wp.str[i] + (taps[i] - 1) * wp.dil[i] + 1 - wp.pre[i];
        reads = reads && need > 0;
        len[i] = std::min(need, in[i]);
        post2[i] = need > in[i] ? need - in[i] : 0;
    }
    const int64_t od[4] = {wp.C, wp.K, wp.R, wp.S};
    const int64_t os[4] = {wp.dw.s[1], wp.dw.s[0], wp.dw.s[2], wp.dw.s[3]};
    const conv_i8_desc_t out = make_desc(CONV_I8_DT_INT32, od, os);
    const int64_t one[2] = {1, 1}, zero[2] = {0, 0};
    if (!reads) {
        // every tap lies in the padding: a convolution over zero channels
        // writes the zeros
        const int64_t xd[4] = {wp.C, 0, wp.R, wp.S}, z4[4] = {0, 0, 0, 0};
        const int64_t fd[4] = {wp.K, 0, 1, 1};
        const conv_i8_desc_t img = make_desc(CONV_I8_DT_INT8, xd, z4);
        const conv_i8_desc_t flt = make_desc(CONV_I8_DT_INT8, fd, z4);
        return fn(&img, nullptr, &flt, nullptr, &out, dw_ptr, zero, zero, one, one, false);
    }
    const int64_t xd[4] = {wp.C, wp.N, len[0], len[1]};
    const int64_t xs[4] = {wp.x.s[1], wp.x.s[0], wp.x.s[2], wp.x.s[3]};
    const int64_t fd[4] = {wp.K, wp.N, wp.P, wp.Q};
    const int64_t fs[4] = {wp.dy.s[1], wp.dy.s[0], wp.dy.s[2], wp.dy.s[3]};
    const conv_i8_desc_t img = make_desc(CONV_I8_DT_INT8, xd, xs);
    const conv_i8_desc_t flt = make_desc(CONV_I8_DT_INT8, fd, fs);
    const int64_t pre2[2] = {wp.pre[0], wp.pre[1]};
    const int64_t st2[2] = {wp.dil[0], wp.dil[1]}, dl2[2] = {wp.str[0], wp.str[1]};
    return fn(&img, x_ptr, &flt, dy_ptr, &out, dw_ptr, pre2, post2, st2, dl2,
              mode == CONV_I8_MODE_CONVOLUTION);
}

// A weight gradient on channels-last image and loss read in place: for each
// filter tap dW[., ., r, s] = sum over the output pixels of dY times the image
// pixel the tap reads, both operands read by wgrad_inplace_kernel as they lie
// in memory (one launch), its pixels split over workgroups whose partial
// copies of dW split_reduce_kernel adds.  The forward call of the transposed
// operands repacks both, each a full pass over HBM.  A 1x1 filter at stride 1
// without padding whose image pixels are equally spaced needs no index
// arithmetic (the image row of output pixel j is pixel j).
constexpr int kWgIpTM = 128, kWgIpTN = 128, kWgIpNS = 4;
constexpr int kWgIpTarget = kCUs, kWgIpMinSteps = 8;

struct WgradInPlacePlan {
    int64_t rows, dy_pitch, x_pitch, x_span;
    bool taps;
    int tiles, tiles_n, nsteps, ksplit, kchunk;
    size_t ws_bytes;
};

// Bytes between consecutive pixels when every pixel (n, p, q) of a
// channels-last tensor lies at (n*P*Q + p*Q + q) * pitch, or 0.
int64_t pixel_pitch(const T4 &t)
{
    if (t.s[1] != 1)
        return 0;
    const int64_t P = t.d[2], Q = t.d[3];
    const int64_t pitch = Q > 1 ? t.s[3] : P > 1 ? t.s[2] : t.d[0] > 1 ? t.s[0] : 16 * ((t.d[1] + 15) / 16);
    if (pitch <= 0 || pitch % 16 != 0)
        return 0;
    if ((P > 1 && t.s[2] != Q * pitch) || (t.d[0] > 1 && t.s[0] != P * Q * pitch))
        return 0;
    return pitch;
}

bool wgrad_inplace_plan(const WgradProblem &wp, const void *x_ptr, const void *dy_ptr, WgradInPlacePlan *q)
{
    if (env_tile())
        return false;  // a forced tile is for the forward call of the transposed operands
    if (wp.K % 16 != 0 || wp.C % 16 != 0 || ((uintptr_t)x_ptr & 15u) != 0 || ((uintptr_t)dy_ptr & 15u) != 0)
        return false;
    const int64_t rows = wp.N * wp.P * wp.Q;
    q->dy_pitch = pixel_pitch(wp.dy);
    if (rows < 1 || rows > (1 << 22) - 256 || q->dy_pitch == 0)
        return false;
    int64_t e;
    if (!mul_ok(rows - 1, q->dy_pitch, &e) || e + wp.K > kI32Max)
        return false;
    // dW dense (the partial copies and their sum walk its span)
    int64_t span;
    if (!span_of(wp.dw, &span) || span != wp.K * wp.C * wp.R * wp.S || 4 * span > kI32Max)
        return false;
    const bool unit = wp.R == 1 && wp.S == 1 && wp.str[0] == 1 && wp.str[1] == 1 && wp.pre[0] == 0 &&
                      wp.pre[1] == 0 && wp.post[0] == 0 && wp.post[1] == 0;
    q->x_pitch = unit ? pixel_pitch(wp.x) : 0;
    q->taps = q->x_pitch == 0;
    if (q->taps) {
        // image pixels through their strides: 16-byte chunks, 32-bit offsets
        if (wp.x.s[1] != 1 || wp.x.s[0] % 16 != 0 || wp.x.s[2] % 16 != 0 || wp.x.s[3] % 16 != 0)
            return false;
        if (!span_of(wp.x, &q->x_span) || q->x_span > kI32Max || wp.P * wp.Q > (1 << 22) - 256)
            return false;
    } else {
        if (!mul_ok(rows - 1, q->x_pitch, &e) || e + wp.C > kI32Max)
            return false;
        q->x_span = e + wp.C;
    }
    q->rows = rows;
    q->tiles_n = (int)((wp.C + kWgIpTN - 1) / kWgIpTN);
    q->tiles = (int)((wp.K + kWgIpTM - 1) / kWgIpTM) * q->tiles_n;
    q->nsteps = (int)((rows + 63) / 64);
    // About one workgroup per CU, each at least kWgIpMinSteps steps of 64
    // pixels; a dW of more tile-taps than half the CUs aims at two per CU (the
    // kernel's 64 KB of LDS lets two share a CU, and the second hides the
    // first's waits: the large-channel layer, 144 tile-taps, takes 53 us in
    // three splits against 98 us in one)
    const int64_t units = (int64_t)q->tiles * wp.R * wp.S;
    const int64_t target = units * 2 > kWgIpTarget ? 2 * kWgIpTarget : kWgIpTarget;
    const int want = (int)std::max<int64_t>(1, std::min<int64_t>(target / units, q->nsteps / kWgIpMinSteps));
    q->kchunk = (q->nsteps + want - 1) / want;
    q->ksplit = (q->nsteps + q->kchunk - 1) / q->kchunk;
    q->ws_bytes = q->ksplit > 1 ? (size_t)q->ksplit * (size_t)span * 4 : 0;
    return true;
}

std::string describe_wgrad_inplace(const WgradProblem &wp, const WgradInPlacePlan &q)
{
    char b[256];
    snprintf(b, sizeof b,
             "kernel=wgrad_in_place tile=%dx%d operands=in_place image_rows=%s pixels=%lld steps=%d tiles=%lld "
             "ksplit=%d split_sum=%s workspace=%zu",
             kWgIpTM, kWgIpTN, q.taps ? "per_tap" : "linear", (long long)q.rows, q.nsteps,
             (long long)q.tiles * wp.R * wp.S, q.ksplit, q.ksplit > 1 ? "partial" : "none", q.ws_bytes);
    return b;
}

conv_i8_status_t wgrad_inplace_run(const WgradProblem &wp, const WgradInPlacePlan &q, const void *x_ptr,
                                   const void *dy_ptr, void *dw_ptr, void *ws, int32_t mode, hipStream_t stream)
{
    WgradInPlaceArgs a{};
    a.dy = (const int8_t *)dy_ptr;
    a.x = (const int8_t *)x_ptr;
    a.rows = (int)q.rows;
    a.K = (int)wp.K;
    a.C = (int)wp.C;
    a.dy_pitch = (int)q.dy_pitch;
    a.x_pitch = (int)q.x_pitch;
    a.dy_range = (int)((q.rows - 1) * q.dy_pitch + wp.K);
    a.x_range = (int)q.x_span;
    a.oK = (int)wp.dw.s[0];
    a.oC = (int)wp.dw.s[1];
    const int64_t span = wp.K * wp.C * wp.R * wp.S;
    a.out_range = (int)(4 * span);
    a.tiles_n = q.tiles_n;
    a.nsteps = q.nsteps;
    a.kchunk = q.kchunk;
    a.part_stride = span;
    a.out = q.ksplit > 1 ? (int32_t *)ws : (int32_t *)dw_ptr;
    a.tiles = q.tiles;
    a.R = (int)wp.R;
    a.S = (int)wp.S;
    a.PQ = (int)(wp.P * wp.Q);
    a.Q = (int)wp.Q;
    a.inv_pq = 1.0f / (float)a.PQ;
    a.inv_q = 1.0f / (float)a.Q;
    a.H = (int)wp.H;
    a.W = (int)wp.W;
    a.sN = (int)wp.x.s[0];
    a.sH = (int)wp.x.s[2];
    a.sW = (int)wp.x.s[3];
    a.st_h = (int)wp.str[0];
    a.st_w = (int)wp.str[1];
    a.dil_h = (int)wp.dil[0];
    a.dil_w = (int)wp.dil[1];
    a.pre_h = (int)wp.pre[0];
    a.pre_w = (int)wp.pre[1];
    a.oR = (int)wp.dw.s[2];
    a.oS = (int)wp.dw.s[3];
    a.flip = mode == CONV_I8_MODE_CONVOLUTION;
    const dim3 grid((unsigned)(q.taps ? (int64_t)q.tiles * wp.R * wp.S : q.tiles), (unsigned)q.ksplit);
    if (q.taps)
        hipLaunchKernelGGL((wgrad_inplace_kernel<kWgIpTM, kWgIpTN, kWgIpNS, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((wgrad_inplace_kernel<kWgIpTM, kWgIpTN, kWgIpNS, false>), grid, dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess)
        return CONV_I8_ERR_HIP;
    if (q.ksplit > 1) {
        const int32_t *part = a.out;
        int32_t *out = (int32_t *)dw_ptr;
        const bool v4 = span % 4 == 0 && ((uintptr_t)out & 15u) == 0 && ((uintptr_t)part & 15u) == 0;
        const int64_t items = v4 ? span / 4 : span;
        const dim3 rgrid((unsigned)std::min<int64_t>(std::max<int64_t>((items + 255) / 256, 1), 4 * kCUs));
        if (v4 && q.ksplit >= 16)
            hipLaunchKernelGGL(split_reduce_wide_kernel<16>, dim3((unsigned)((items + 15) / 16)), dim3(256), 0,
                               stream, part, (long long)span, q.ksplit, out, (long long)span);
        else if (v4)
            hipLaunchKernelGGL(split_reduce_kernel<true>, rgrid, dim3(256), 0, stream, part, (long long)span,
                               q.ksplit, out, (long long)span);
        else
            hipLaunchKernelGGL(split_reduce_kernel<false>, rgrid, dim3(256), 0, stream, part, (long long)span,
                               q.ksplit, out, (long long)span);
        if (hipGetLastError() != hipSuccess)
            return CONV_I8_ERR_HIP;
    }
    return CONV_I8_OK;
}

conv_i8_status_t wgrad_entry(const conv_i8_desc_t *image, const void *image_ptr,
                             const conv_i8_desc_t *loss, const void *loss_ptr,
                             const conv_i8_desc_t *dw, void *dw_ptr, const int64_t *pre,
                             const int64_t *post, const int64_t *stride, const int64_t *dil,
                             int32_t mode, bool size_only, size_t *ws_size, bool alloc,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    WgradProblem wp;
    conv_i8_status_t st = wgrad_analyze(image, loss, dw, pre, post, stride, dil, mode, &wp);
    if (st != CONV_I8_OK)
        return st;
    if (wp.dw.elems() == 0) {
        if (ws_size)
            *ws_size = 0;
        return CONV_I8_OK;
    }
    WgradInPlacePlan q1;
    if (wgrad_inplace_plan(wp, image_ptr, loss_ptr, &q1)) {
        if (size_only) {
            *ws_size = q1.ws_bytes;
            return CONV_I8_OK;
        }
        if (!image_ptr || !loss_ptr || !dw_ptr)
            return CONV_I8_ERR_NULL;
        hipStream_t s = (hipStream_t)stream;
        void *ws = workspace;
        if (alloc) {
            ws = nullptr;
            if (q1.ws_bytes > 0 && hipMallocAsync(&ws, q1.ws_bytes, s) != hipSuccess)
                return CONV_I8_ERR_HIP;
        } else {
            if (workspace_bytes < q1.ws_bytes)
                return CONV_I8_ERR_WORKSPACE;
            if (q1.ws_bytes > 0 && !workspace)
                return CONV_I8_ERR_NULL;
            if (q1.ws_bytes > 0 && ((uintptr_t)workspace & 255u) != 0)
                return CONV_I8_ERR_WORKSPACE;
        }
        if (log_enabled())
            fprintf(stderr, "conv_i8 (weight gradient): %s\n", describe_wgrad_inplace(wp, q1).c_str());
        st = wgrad_inplace_run(wp, q1, image_ptr, loss_ptr, dw_ptr, ws, mode, s);
        if (alloc && ws && hipFreeAsync(ws, s) != hipSuccess && st == CONV_I8_OK)
            st = CONV_I8_ERR_HIP;
        return st;
    }
    const char *tuned = tuned_wgrad_tile(wp);
    if (size_only)
        return wgrad_call(wp, image_ptr, loss_ptr, nullptr, mode,
                          [&](const conv_i8_desc_t *i, const void *x, const conv_i8_desc_t *f,
                              const void *w, const conv_i8_desc_t *o, void *, const int64_t *a,
                              const int64_t *b, const int64_t *c, const int64_t *d, bool fl) {
                              // the same plan as the call below (split_ok: its
                              // partial outputs live in the workspace)
                              return entry_workspace_size(i, x, f, w, o, a, b, c, d,
                                                          CONV_I8_DT_INT32,
                                                          CONV_I8_MODE_CROSS_CORRELATION, ws_size,
                                                          fl, true, tuned);
                          });
    return wgrad_call(wp, image_ptr, loss_ptr, dw_ptr, mode,
                      [&](const conv_i8_desc_t *i, const void *x, const conv_i8_desc_t *f,
                          const void *w, const conv_i8_desc_t *o, void *y, const int64_t *a,
                          const int64_t *b, const int64_t *c, const int64_t *d, bool fl) {
                          // split_ok: the long inner dimension may be split over
                          // workgroups whose partial outputs a reduction adds (or,
                          // for an output with gaps, that add into it atomically)
                          return entry_run(i, x, f, w, o, y, a, b, c, d, CONV_I8_DT_INT32,
                                           CONV_I8_MODE_CROSS_CORRELATION, nullptr, alloc,
                                           workspace, workspace_bytes, stream, fl, true, tuned);
                      });
}

}  // namespace
}  // namespace convi8

extern "C" {

conv_i8_status_t conv_fprop_i8_workspace_size(const conv_i8_desc_t *image, const void *image_ptr,
                                              const conv_i8_desc_t *filter, const void *filter_ptr,
                                              const conv_i8_desc_t *out,
                                              const int64_t pre_padding[2],
                                              const int64_t post_padding[2],
                                              const int64_t stride[2], const int64_t dilation[2],
                                              size_t *workspace_bytes)
{
    return entry_workspace_size(image, image_ptr, filter, filter_ptr, out, pre_padding, post_padding,
                                stride, dilation, CONV_I8_DT_INT32, CONV_I8_MODE_CROSS_CORRELATION,
                                workspace_bytes);
}

conv_i8_status_t conv_fprop_i8_plan(const conv_i8_desc_t *image, const void *image_ptr,
                                    const conv_i8_desc_t *filter, const void *filter_ptr,
                                    const conv_i8_desc_t *out, const int64_t pre_padding[2],
                                    const int64_t post_padding[2], const int64_t stride[2],
                                    const int64_t dilation[2], char *buf, size_t len)
{
    if (!buf || len == 0)
        return CONV_I8_ERR_NULL;
    Problem pb;
    Plan pl;
    conv_i8_status_t st = prepare(image, image_ptr, filter, filter_ptr, out, pre_padding,
                                  post_padding, stride, dilation, &pb, &pl);
    if (st != CONV_I8_OK)
        return st;
    snprintf(buf, len, "%s", describe(pb, pl).c_str());
    return CONV_I8_OK;
}

conv_i8_status_t conv_fprop_i8_ws(const conv_i8_desc_t *image, const void *image_ptr,
                                  const conv_i8_desc_t *filter, const void *filter_ptr,
                                  const conv_i8_desc_t *out, void *out_ptr,
                                  const int64_t pre_padding[2], const int64_t post_padding[2],
                                  const int64_t stride[2], const int64_t dilation[2],
                                  void *workspace, size_t workspace_bytes, void *stream)
{
    return entry_run(image, image_ptr, filter, filter_ptr, out, out_ptr, pre_padding, post_padding,
                     stride, dilation, CONV_I8_DT_INT32, CONV_I8_MODE_CROSS_CORRELATION, nullptr,
                     false, workspace, workspace_bytes, stream);
}

conv_i8_status_t conv_fprop_i8(const conv_i8_desc_t *image, const void *image_ptr,
                               const conv_i8_desc_t *filter, const void *filter_ptr,
                               const conv_i8_desc_t *out, void *out_ptr,
                               const int64_t pre_padding[2], const int64_t post_padding[2],
                               const int64_t stride[2], const int64_t dilation[2], void *stream)
{
    return entry_run(image, image_ptr, filter, filter_ptr, out, out_ptr, pre_padding, post_padding,
                     stride, dilation, CONV_I8_DT_INT32, CONV_I8_MODE_CROSS_CORRELATION, nullptr,
                     true, nullptr, 0, stream);
}

conv_i8_status_t conv_fprop_i8_noalloc(const conv_i8_desc_t *image, const void *image_ptr,
                                       const conv_i8_desc_t *filter, const void *filter_ptr,
                                       const conv_i8_desc_t *out, void *out_ptr,
                                       const int64_t pre_padding[2], const int64_t post_padding[2],
                                       const int64_t stride[2], const int64_t dilation[2],
                                       void *stream)
{
    using namespace convi8;
    size_t need = 0;
    conv_i8_status_t st = entry_workspace_size(image, image_ptr, filter, filter_ptr, out, pre_padding,
                                               post_padding, stride, dilation, CONV_I8_DT_INT32,
                                               CONV_I8_MODE_CROSS_CORRELATION, &need);
    if (st != CONV_I8_OK)
        return st;
    if (need > (size_t)CONV_I8_NOALLOC_SCRATCH_BYTES)
        return CONV_I8_ERR_SCRATCH;
    void *ws = nullptr;
    if ((st = scratch_address(stream, &ws)) != CONV_I8_OK)
        return st;
    return entry_run(image, image_ptr, filter, filter_ptr, out, out_ptr, pre_padding, post_padding,
                     stride, dilation, CONV_I8_DT_INT32, CONV_I8_MODE_CROSS_CORRELATION, nullptr,
                     false, ws, (size_t)CONV_I8_NOALLOC_SCRATCH_BYTES, stream);
}

conv_i8_status_t conv_fprop_i8_requant_workspace_size(
    const conv_i8_desc_t *image, const void *image_ptr, const conv_i8_desc_t *filter,
    const void *filter_ptr, const conv_i8_desc_t *out, const int64_t pre_padding[2],
    const int64_t post_padding[2], const int64_t stride[2], const int64_t dilation[2],
    size_t *workspace_bytes)
{
    return entry_workspace_size(image, image_ptr, filter, filter_ptr, out, pre_padding, post_padding,
                                stride, dilation, CONV_I8_DT_INT8, CONV_I8_MODE_CROSS_CORRELATION,
                                workspace_bytes);
}

conv_i8_status_t conv_fprop_i8_requant_ws(const conv_i8_desc_t *image, const void *image_ptr,
                                          const conv_i8_desc_t *filter, const void *filter_ptr,
                                          const conv_i8_desc_t *out, void *out_ptr,
                                          const int64_t pre_padding[2],
                                          const int64_t post_padding[2], const int64_t stride[2],
                                          const int64_t dilation[2], const conv_i8_requant_t *rq,
                                          void *workspace, size_t workspace_bytes, void *stream)
{
    return entry_run(image, image_ptr, filter, filter_ptr, out, out_ptr, pre_padding, post_padding,
                     stride, dilation, CONV_I8_DT_INT8, CONV_I8_MODE_CROSS_CORRELATION, rq, false,
                     workspace, workspace_bytes, stream);
}

conv_i8_status_t conv_fprop_i8_requant(const conv_i8_desc_t *image, const void *image_ptr,
                                       const conv_i8_desc_t *filter, const void *filter_ptr,
                                       const conv_i8_desc_t *out, void *out_ptr,
                                       const int64_t pre_padding[2], const int64_t post_padding[2],
                                       const int64_t stride[2], const int64_t dilation[2],
                                       const conv_i8_requant_t *rq, void *stream)
{
    return entry_run(image, image_ptr, filter, filter_ptr, out, out_ptr, pre_padding, post_padding,
                     stride, dilation, CONV_I8_DT_INT8, CONV_I8_MODE_CROSS_CORRELATION, rq, true,
                     nullptr, 0, stream);
}

conv_i8_status_t conv_fprop_i8_ex_workspace_size(const conv_i8_desc_t *image, const void *image_ptr,
                                                 const conv_i8_desc_t *filter,
                                                 const void *filter_ptr, const conv_i8_desc_t *out,
                                                 const int64_t pre_padding[2],
                                                 const int64_t post_padding[2],
                                                 const int64_t stride[2],
                                                 const int64_t dilation[2], int32_t mode,
                                                 size_t *workspace_bytes)
{
    int32_t dt = 0;
    // the output dtype decides the epilogue; either is fine for the size
    if (!out)
        return CONV_I8_ERR_NULL;
    dt = out->dtype == CONV_I8_DT_INT8 ? CONV_I8_DT_INT8 : CONV_I8_DT_INT32;
    return entry_workspace_size(image, image_ptr, filter, filter_ptr, out, pre_padding, post_padding,
                                stride, dilation, dt, mode, workspace_bytes);
}

conv_i8_status_t conv_fprop_i8_ex_ws(const conv_i8_desc_t *image, const void *image_ptr,
                                     const conv_i8_desc_t *filter, const void *filter_ptr,
                                     const conv_i8_desc_t *out, void *out_ptr,
                                     const int64_t pre_padding[2], const int64_t post_padding[2],
                                     const int64_t stride[2], const int64_t dilation[2],
                                     int32_t mode, const conv_i8_requant_t *rq, void *workspace,
                                     size_t workspace_bytes, void *stream)
{
    int32_t dt = 0;
    conv_i8_status_t st = ex_out_dtype(out, rq, &dt);
    if (st != CONV_I8_OK)
        return st;
    return entry_run(image, image_ptr, filter, filter_ptr, out, out_ptr, pre_padding, post_padding,
                     stride, dilation, dt, mode, rq, false, workspace, workspace_bytes, stream);
}

conv_i8_status_t conv_dgrad_i8_workspace_size(const conv_i8_desc_t *loss, const void *loss_ptr,
                                              const conv_i8_desc_t *filter, const void *filter_ptr,
                                              const conv_i8_desc_t *dx,
                                              const int64_t pre_padding[2],
                                              const int64_t post_padding[2],
                                              const int64_t stride[2], const int64_t dilation[2],
                                              int32_t mode, size_t *workspace_bytes)
{
    if (!workspace_bytes)
        return CONV_I8_ERR_NULL;
    DgradProblem dp;
    conv_i8_status_t st = dgrad_analyze(loss, filter, dx, pre_padding, post_padding, stride, dilation,
                                        mode, &dp);
    if (st != CONV_I8_OK)
        return st;
    if (dp.dx.elems() == 0) {
        *workspace_bytes = 0;
        return CONV_I8_OK;
    }
    return dgrad_workspace(dp, loss_ptr, filter_ptr, mode, workspace_bytes);
}

conv_i8_status_t conv_dgrad_i8_ws(const conv_i8_desc_t *loss, const void *loss_ptr,
                                  const conv_i8_desc_t *filter, const void *filter_ptr,
                                  const conv_i8_desc_t *dx, void *dx_ptr,
                                  const int64_t pre_padding[2], const int64_t post_padding[2],
                                  const int64_t stride[2], const int64_t dilation[2], int32_t mode,
                                  void *workspace, size_t workspace_bytes, void *stream)
{
    return dgrad_entry(loss, loss_ptr, filter, filter_ptr, dx, dx_ptr, pre_padding, post_padding,
                       stride, dilation, mode, false, workspace, workspace_bytes, stream);
}

conv_i8_status_t conv_dgrad_i8(const conv_i8_desc_t *loss, const void *loss_ptr,
                               const conv_i8_desc_t *filter, const void *filter_ptr,
                               const conv_i8_desc_t *dx, void *dx_ptr,
                               const int64_t pre_padding[2], const int64_t post_padding[2],
                               const int64_t stride[2], const int64_t dilation[2], int32_t mode,
                               void *stream)
{
    return dgrad_entry(loss, loss_ptr, filter, filter_ptr, dx, dx_ptr, pre_padding, post_padding,
                       stride, dilation, mode, true, nullptr, 0, stream);
}

conv_i8_status_t conv_wgrad_i8_plan(const conv_i8_desc_t *image, const void *image_ptr,
                                    const conv_i8_desc_t *loss, const void *loss_ptr,
                                    const conv_i8_desc_t *dw, const int64_t pre_padding[2],
                                    const int64_t post_padding[2], const int64_t stride[2],
                                    const int64_t dilation[2], int32_t mode, char *buf, size_t len)
{
    if (!buf || len == 0)
        return CONV_I8_ERR_NULL;
    WgradProblem wp;
    conv_i8_status_t st = wgrad_analyze(image, loss, dw, pre_padding, post_padding, stride, dilation,
                                        mode, &wp);
    if (st != CONV_I8_OK)
        return st;
    if (wp.dw.elems() == 0) {
        snprintf(buf, len, "empty");
        return CONV_I8_OK;
    }
    WgradInPlacePlan q1;
    if (wgrad_inplace_plan(wp, image_ptr, loss_ptr, &q1)) {
        snprintf(buf, len, "%s", describe_wgrad_inplace(wp, q1).c_str());
        return CONV_I8_OK;
    }
    const char *tuned = tuned_wgrad_tile(wp);
    return wgrad_call(wp, image_ptr, loss_ptr, nullptr, mode,
                      [&](const conv_i8_desc_t *i, const void *x, const conv_i8_desc_t *f,
                          const void *w, const conv_i8_desc_t *o, void *, const int64_t *a,
                          const int64_t *b, const int64_t *c, const int64_t *d, bool fl) {
                          Problem pb;
                          Plan pl;
                          conv_i8_status_t r = prepare(i, x, f, w, o, a, b, c, d, &pb, &pl,
                                                       CONV_I8_DT_INT32,
                                                       CONV_I8_MODE_CROSS_CORRELATION, fl, true,
                                                       tuned);
                          if (r == CONV_I8_OK)
                              snprintf(buf, len, "%s", describe(pb, pl).c_str());
                          return r;
                      });
}

conv_i8_status_t conv_wgrad_i8_workspace_size(const conv_i8_desc_t *image, const void *image_ptr,
                                              const conv_i8_desc_t *loss, const void *loss_ptr,
                                              const conv_i8_desc_t *dw,
                                              const int64_t pre_padding[2],
                                              const int64_t post_padding[2],
                                              const int64_t stride[2], const int64_t dilation[2],
                                              int32_t mode, size_t *workspace_bytes)
{
    if (!workspace_bytes)
        return CONV_I8_ERR_NULL;
    return wgrad_entry(image, image_ptr, loss, loss_ptr, dw, nullptr, pre_padding, post_padding,
                       stride, dilation, mode, true, workspace_bytes, false, nullptr, 0, nullptr);
}

conv_i8_status_t conv_wgrad_i8_ws(const conv_i8_desc_t *image, const void *image_ptr,
                                  const conv_i8_desc_t *loss, const void *loss_ptr,
                                  const conv_i8_desc_t *dw, void *dw_ptr,
                                  const int64_t pre_padding[2], const int64_t post_padding[2],
                                  const int64_t stride[2], const int64_t dilation[2], int32_t mode,
                                  void *workspace, size_t workspace_bytes, void *stream)
{
    return wgrad_entry(image, image_ptr, loss, loss_ptr, dw, dw_ptr, pre_padding, post_padding,
                       stride, dilation, mode, false, nullptr, false, workspace, workspace_bytes,
                       stream);
}

conv_i8_status_t conv_wgrad_i8(const conv_i8_desc_t *image, const void *image_ptr,
                               const conv_i8_desc_t *loss, const void *loss_ptr,
                               const conv_i8_desc_t *dw, void *dw_ptr,
                               const int64_t pre_padding[2], const int64_t post_padding[2],
                               const int64_t stride[2], const int64_t dilation[2], int32_t mode,
                               void *stream)
{
    return wgrad_entry(image, image_ptr, loss, loss_ptr, dw, dw_ptr, pre_padding, post_padding,
                       stride, dilation, mode, false, nullptr, true, nullptr, 0, stream);
}

conv_i8_status_t conv_i8_mfma_ceiling(int workgroups, int iters, uint32_t seed, int32_t *out, void *stream)
{
    if (!out)
        return CONV_I8_ERR_NULL;
    if (workgroups < 1 || workgroups > (1 << 20) || iters < 1)
        return CONV_I8_ERR_PARAM;
    hipLaunchKernelGGL(convi8::mfma_ceiling_kernel<0>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, iters,
                       (unsigned)seed, (int *)out);
    return hipGetLastError() == hipSuccess ? CONV_I8_OK : CONV_I8_ERR_HIP;
}

#ifdef CONV_I8_PHASE_CLOCK
// Instrumented builds only (CONV_I8_PHASE_CLOCK; not part of the product
// library or its header): a device buffer of 16 int64 per workgroup that
// every later 3x3 ring kernel launch fills with its phase stamps, or null.
conv_i8_status_t conv_i8_set_phase_clock(void *buf)
{
    g_phase_clk = (long long *)buf;
    return CONV_I8_OK;
}
#endif

conv_i8_status_t conv_i8_tile_names(char *buf, size_t len)
{
    if (!buf)
        return CONV_I8_ERR_NULL;
    size_t used = 0;
    for (int i = 0; i < kNumTiles; ++i) {
        const size_t n = strlen(kTiles[i].name) + (i ? 1 : 0);
        if (used + n + 1 > len)
            return CONV_I8_ERR_PARAM;
        if (i)
            buf[used++] = ',';
        memcpy(buf + used, kTiles[i].name, n - (i ? 1 : 0));
        used += n - (i ? 1 : 0);
    }
    if (used + 1 > len)
        return CONV_I8_ERR_PARAM;
    buf[used] = 0;
    return CONV_I8_OK;
}

const char *conv_i8_status_string(conv_i8_status_t status)
{
    // a caller may pass any int: read its bits, never the enum value (a value
    // outside the enumerators' range is undefined behaviour in C++)
    static_assert(sizeof(conv_i8_status_t) == sizeof(int), "the status enum is int-sized");
    int code;
    memcpy(&code, &status, sizeof code);
    switch (code) {
    case CONV_I8_OK: return "CONV_I8_OK";
    case CONV_I8_ERR_NULL: return "CONV_I8_ERR_NULL: a required pointer is NULL";
    case CONV_I8_ERR_DTYPE: return "CONV_I8_ERR_DTYPE: image/filter must be INT8 and the output INT32 (INT8 for the requantising entries)";
    case CONV_I8_ERR_RANK: return "CONV_I8_ERR_RANK: descriptors must have ndim == 4";
    case CONV_I8_ERR_DIMS: return "CONV_I8_ERR_DIMS: negative dim, or filter R or S < 1";
    case CONV_I8_ERR_PARAM: return "CONV_I8_ERR_PARAM: stride and dilation must be >= 1, padding >= 0; requantisation arrays 4-byte aligned, alpha finite";
    case CONV_I8_ERR_CHANNELS: return "CONV_I8_ERR_CHANNELS: image C != filter C";
    case CONV_I8_ERR_OUT_DIMS: return "CONV_I8_ERR_OUT_DIMS: output dims must be [N, K, P, Q] with P, Q >= 1";
    case CONV_I8_ERR_STRIDES: return "CONV_I8_ERR_STRIDES: negative stride or self-overlapping output";
    case CONV_I8_ERR_RANGE: return "CONV_I8_ERR_RANGE: C*R*S > 131071, int32 sums would not be exact";
    case CONV_I8_ERR_WORKSPACE: return "CONV_I8_ERR_WORKSPACE: workspace too small or not 256-byte aligned";
    case CONV_I8_ERR_UNSUPPORTED: return "CONV_I8_ERR_UNSUPPORTED: a single image or the filter spans >= 2 GiB";
    case CONV_I8_ERR_HIP: return "CONV_I8_ERR_HIP: a HIP runtime call failed";
    case CONV_I8_ERR_SCRATCH: return "CONV_I8_ERR_SCRATCH: the problem needs more workspace than conv_fprop_i8_noalloc's static scratch array holds (CONV_I8_NOALLOC_SCRATCH_BYTES); call conv_fprop_i8_ws with a caller workspace instead";
    }
    return "unknown conv_i8 status";
}

}  // extern "C"
