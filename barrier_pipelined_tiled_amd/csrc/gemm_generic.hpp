// gemm_generic.hpp -- guarded GEMM for any shape, leading dimension and
// alignment.  It serves the calls the pipelined kernels decline: a K that is
// not a multiple of the K-tile, unaligned bases, odd leading dimensions, or
// operands too large for 32-bit buffer offsets.  Element loads with bounds
// checks, one LDS stage, one MFMA 32x32x16 block per wave.
#pragma once
#include "device_common.hpp"

namespace bpt {

struct GenericArgs {
    const void* A;
    const void* B;
    void* C;
    long long M, N, K;
    long long lda, ldb, ldc;
    long long strideA, strideB, strideC;
    int tiles_n;
};

// 64x64 output tile, 4 waves in 2x2, K-step 16.  LDS holds A as [m][k] and B
// transposed as [n][k] so that each lane's 8 k-values are contiguous.  BT:
// B is given transposed (N x K row-major, ldb >= K), C = A * B^T.
template <typename T, typename OutT, bool BT = false>
__global__ __launch_bounds__(256) void gemm_generic_kernel(GenericArgs args) {
    typedef typename Mfma<T>::frag_t frag_t;
    constexpr int BMg = 64, BNg = 64, BKg = 16, PAD = 8;
    __shared__ __attribute__((aligned(16))) T As[BMg][BKg + PAD];
    __shared__ __attribute__((aligned(16))) T Bs[BNg][BKg + PAD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const long long tm = blockIdx.x / args.tiles_n, tn = blockIdx.x % args.tiles_n;
    const long long m0 = tm * BMg, n0 = tn * BNg;
    const long long batch = blockIdx.y;
    const T* Ab = static_cast<const T*>(args.A) + batch * args.strideA;
    const T* Bb = static_cast<const T*>(args.B) + batch * args.strideB;
    const T zero = (T)0.0f;

    float16_t acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (long long k0 = 0; k0 < args.K; k0 += BKg) {
        // 1024 elements of A and 1024 of B per step, 4 of each per thread
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int e = tid + q * 256;
            int r = e / BKg, c = e % BKg;                  // A: row r, k c
            long long gm = m0 + r, gk = k0 + c;
            As[r][c] = (gm < args.M && gk < args.K) ? Ab[gm * args.lda + gk] : zero;
            if constexpr (BT) {
                int nb = e / BKg, kb = e % BKg;            // Bt: row (col of C) nb, k kb
                long long bk = k0 + kb, bn = n0 + nb;
                Bs[nb][kb] = (bk < args.K && bn < args.N) ? Bb[bn * args.ldb + bk] : zero;
            } else {
                int kb = e / BNg, nb = e % BNg;            // B: k kb, col nb
                long long bk = k0 + kb, bn = n0 + nb;
                Bs[nb][kb] = (bk < args.K && bn < args.N) ? Bb[bk * args.ldb + bn] : zero;
            }
        }
        __syncthreads();
        frag_t a = *(const frag_t*)&As[wm * 32 + (lane % 32)][8 * (lane / 32)];
        frag_t b = *(const frag_t*)&Bs[wn * 32 + (lane % 32)][8 * (lane / 32)];
        acc = Mfma<T>::mma32(a, b, acc);
        __syncthreads();
    }
    OutT* Cb = static_cast<OutT*>(args.C) + batch * args.strideC;
    const long long col = n0 + wn * 32 + (lane % 32);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        long long row = m0 + wm * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
        if (row < args.M && col < args.N) Cb[row * args.ldc + col] = cvt_out<OutT>(acc[r]);
    }
}

// C = 0 over an M x N window with leading dimension ldc (the empty sum, K = 0).
template <typename OutT>
__global__ void fill_zero_kernel(OutT* C, long long M, long long N, long long ldc, long long strideC) {
    long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    long long total = M * N;
    OutT* Cb = C + (long long)blockIdx.y * strideC;
    for (; idx < total; idx += (long long)gridDim.x * blockDim.x) {
        long long r = idx / N, c = idx % N;
        Cb[r * ldc + c] = (OutT)0.0f;
    }
}

}  // namespace bpt
