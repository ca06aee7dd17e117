// INT8 matrix-core rate under load, for the compute side of the roofline.
//
// Every wave issues v_mfma_i32_32x32x32_i8 back to back on register operands
// (eight independent accumulators, four operand pairs in rotation so that the
// multiplier inputs change from one instruction to the next as they do when
// fragments stream from LDS), with random bytes or zeros as operands.  On a
// given number of workgroups, one per CU, the rate this reaches is what an
// MFMA-bound kernel on that many CUs can reach at best: the clock falls under
// the power limit as the matrix units toggle more bits, so random operands
// run slower than zeros, and more busy CUs run each one slower.
#pragma once

#include "kernel_common.hpp"

namespace convi8 {

__device__ __forceinline__ unsigned ceiling_mix(unsigned x)
{
    // integer hash (xorshift-multiply rounds) for the operand bytes
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

template <int = 0>   // a template: instantiated only where it is launched
__global__ __launch_bounds__(256) void mfma_ceiling_kernel(int iters, unsigned seed, int *out)
{
    constexpr int NACC = 8, NOP = 4;
    const unsigned gid = blockIdx.x * 256u + threadIdx.x;
    v4i a[NOP], b[NOP];
#pragma unroll
    for (int o = 0; o < NOP; ++o)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[o][i] = seed ? (int)ceiling_mix(seed + gid * 32u + o * 8u + i) : 0;
            b[o][i] = seed ? (int)ceiling_mix(seed + gid * 32u + o * 8u + 4u + i) : 0;
        }
    v16i acc[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j)
        acc[j] = v16i{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < NACC; ++j)
            acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j % NOP], b[(j + j / NOP) % NOP], acc[j], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            s += acc[j][e];
    out[gid] = s;
}

}  // namespace convi8
