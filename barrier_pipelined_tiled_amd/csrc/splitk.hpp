// splitk.hpp -- the second step of split-K for the pipelined kernels.
//
// A call whose output has too few tiles to give every CU a workgroup runs
// the pipelined kernel once over S K-ranges at a time, each range as one
// entry of the kernel's batch, writing an fp32 partial product per range
// into the call's workspace ([split][M][N], rows of N).  This kernel then
// adds the S partials of every output in split order (so the result does
// not depend on timing) and stores C, converted with round-to-nearest-even.
// (Split-K itself is not on the pages: their GEMM fills the GPU with output
// tiles alone; the GEMM page's tile-walk section counts workgroups against
// the GPU's cores the same way.)
#pragma once

#include "device_common.hpp"
#include "gemm_skinny.hpp"     // store8

namespace bpt {

struct SplitSumArgs {
    const float* partial;   // [split][M][N] fp32; N % 8 == 0
    void* C;
    long long M, N, ldc;
    int splits;
    int c_vec;              // C's base and rows allow 16-byte stores
};

// one thread per 8 consecutive outputs of a row
template <typename OutT>
__global__ __launch_bounds__(256) void splitk_sum_kernel(SplitSumArgs a) {
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long per_row = a.N / 8;
    if (gid >= a.M * per_row) return;
    const long long row = gid / per_row;
    const long long col = (gid - row * per_row) * 8;
    const long long plane = a.M * a.N;
    const float* p = a.partial + row * a.N + col;
    float4_t lo = *(const float4_t*)p, hi = *(const float4_t*)(p + 4);
    for (int s = 1; s < a.splits; ++s) {
        lo += *(const float4_t*)(p + s * plane);
        hi += *(const float4_t*)(p + s * plane + 4);
    }
    OutT* dst = static_cast<OutT*>(a.C) + row * a.ldc + col;
    if (a.c_vec) {
        store8<OutT>(dst, lo, hi);
        return;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        dst[q] = cvt_out<OutT>(lo[q]);
        dst[4 + q] = cvt_out<OutT>(hi[q]);
    }
}

}  // namespace bpt
