// repack.hpp -- zero-padded, aligned copies of A and B for shapes the
// pipelined kernels cannot read in place.
//
// The pipelined kernels copy 16-byte chunks of 8 elements global -> LDS, so
// they need 16-byte aligned rows (base and leading dimension multiples of 8
// elements) and K, N that do not cut a chunk (K % 8 == 0, N % 8 == 0).  A
// call outside that -- an odd N or K, a leading dimension that is not a
// multiple of 8, an unaligned base -- is first copied into a workspace as
// A' (M x K', K' = K rounded up to 8) and B' (K' x N', N' = N rounded up to
// 8), zeros in the padding, then multiplied by the pipelined kernel, which
// stores C at its true N.  The zeros add nothing to any sum: A'B' restricted
// to the first N columns is AB.  This copy is memory-bound and reads each
// operand once.
#pragma once
#include "device_common.hpp"

namespace bpt {

struct RepackArgs {
    const void* src;
    void* dst;
    long long ld, stride;      // source leading dimension and batch stride (elements)
    long long ldd, strided;    // destination leading dimension (multiple of 8) and stride
    int rows, cols;            // source extent
    int rows_p, cols_p;        // destination extent (cols_p % 8 == 0)
    long long total8;          // batch * rows_p * cols_p / 8
};

// Thread g writes destination elements 8g .. 8g+7 of the padded matrices
// (batch-major, then row-major) with one 16-byte store; each element is the
// source element at the same (batch, row, column), or zero past the source.
// Elements are moved as 16-bit patterns, whatever their type.
__global__ __launch_bounds__(256) void repack_pad_kernel(RepackArgs a) {
    typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
    const unsigned short* src = static_cast<const unsigned short*>(a.src);
    unsigned short* dst = static_cast<unsigned short*>(a.dst);
    const long long per_row = a.cols_p / 8;
    const long long per_mat = (long long)a.rows_p * per_row;
    for (long long g = (long long)blockIdx.x * 256 + threadIdx.x; g < a.total8; g += (long long)gridDim.x * 256) {
        const long long b = g / per_mat;
        const long long rem = g - b * per_mat;
        const int r = (int)(rem / per_row);
        const int c0 = (int)(rem - (long long)r * per_row) * 8;
        u16x8_t v;
        const unsigned short* s = src + b * a.stride + (long long)r * a.ld;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (r < a.rows && c0 + e < a.cols) ? s[c0 + e] : (unsigned short)0;
        *(u16x8_t*)(dst + b * a.strided + (long long)r * a.ldd + c0) = v;
    }
}

}  // namespace bpt
