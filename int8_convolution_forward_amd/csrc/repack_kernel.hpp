// Layout normalisation: any strided int8 [A, C, Y, X] tensor -> packed
// [A, Y, X, Cp] with the channels innermost and zero-filled up to Cp (a
// multiple of 16).  The zero channels add nothing to any sum, so the packed
// copy convolves exactly like the original.  Used for images (A=N, Y=H, X=W)
// and filters (A=K, Y=R, X=S) whose layout the implicit-GEMM kernel cannot
// read with aligned 16-byte channel vectors (NCHW, strided views, C % 16 != 0).
//
// The memory layout decides the cost here ("Building a From-Scratch INT8
// Strided Convolution Kernel", "Key Takeaways"): a 64(x) x 64(c) tile is read
// with consecutive lanes walking whichever of x or c has the smaller stride,
// transposed through LDS, and written as 16-byte channel vectors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convi8 {

struct RepackArgs {
    const int8_t *src;               // element (0,0,0,0)
    long long s0, s1, s2, s3;        // element strides of [A, C, Y, X]
    int A, C, Y, X, Cp;
    int x_fast;                      // 1: lanes walk x when reading, else c
    int8_t *dst;                     // packed [A][Y][X][Cp]
};

__global__ __launch_bounds__(256) void repack_to_channels_last_kernel(RepackArgs a)
{
    constexpr int T = 64;
    constexpr int LD = T + 4;  // row pitch in bytes (4-byte multiple, staggers banks)
    __shared__ __attribute__((aligned(16))) int8_t tile[T * LD];  // [x][c]

    const int tid = threadIdx.x;
    const int ay = blockIdx.x;       // grid: (A*Y, ceil(X/64), ceil(Cp/64))
    const int x0 = blockIdx.y * T;
    const int c0 = blockIdx.z * T;
    const int ai = ay / a.Y;
    const int yi = ay - ai * a.Y;
    const int8_t *base = a.src + ai * a.s0 + yi * a.s2;

#pragma unroll 4
    for (int i = 0; i < (T * T) / 256; ++i) {
        const int idx = i * 256 + tid;
        int xl, cl;
        if (a.x_fast) {
            xl = idx & (T - 1);
            cl = idx >> 6;
        } else {
            cl = idx & (T - 1);
            xl = idx >> 6;
        }
        const int c = c0 + cl, x = x0 + xl;
        int8_t v = 0;
        if (c < a.C && x < a.X)
            v = base[c * a.s1 + x * a.s3];
        tile[xl * LD + cl] = v;
    }
    __syncthreads();

    const int xl = tid >> 2;
    const int cl = (tid & 3) * 16;
    const int x = x0 + xl, c = c0 + cl;
    if (x < a.X && c < a.Cp) {
        const int *srow = (const int *)&tile[xl * LD + cl];
        int4 v;
        v.x = srow[0];
        v.y = srow[1];
        v.z = srow[2];
        v.w = srow[3];
        int8_t *d = a.dst + (((long long)ai * a.Y + yi) * a.X + x) * a.Cp + c;
        *(int4 *)d = v;
    }
}

}  // namespace convi8
