// gemm_apair.hpp -- the 256 x 256 pipelined GEMM with A staged a K-tile pair
// at a time (C = A * B, B row-major K x N).
//
// The 32-wide K-tile of the 4-stage kernel copies A as 64-byte pieces of its
// rows, half a 128-byte line each.  Here A is copied two K-tiles at a time:
// one copy moves 8 rows x 128 bytes, whole lines, into a "pair" stage of
// 256 rows x 64 k, which K-tiles 2p and 2p+1 both read.  B keeps its ring of
// four 32-wide stages (its rows are 512 bytes already).  Measured in a
// development copy, whole-line A copies alone took 4096^3 from 1155 to 1181
// TFLOP/s and the 4096 x 4096 x 16384 shape from 1240 to 1275.
//
// Ring and schedule (otherwise as gemm_pipelined_kernel, whose comments
// describe the publish points, the window and the copy slices):
// * Tile j reads B stage j % 4 and A pair stage (j/2) % 3.  The copy group
//   of tile g (g = j + 4, started in tile j's window) holds B(g) and, when g
//   is even, the A pair g/2: 12 copies per wave for an even group, 4 for an
//   odd one.  Three pair stages are needed: while an odd tile j is consumed,
//   pairs (j-1)/2, (j+1)/2 and (j+3)/2 are all live.  96 KiB of A and 64 KiB
//   of B fill the 160 KiB of LDS, so this variant takes no K tail (host:
//   K % 64 == 0, K >= 192).
// * publish(j+1) lets the groups of tiles j+2 and j+3 stay in flight: one
//   even and one odd group whatever j is, so the wait count is constant.
//   Only the split of a group's copies over the two k-steps depends on its
//   parity, so the loop runs two tiles per iteration.
// * BT: B given transposed (N x K row-major).  Its 32-wide K-tiles are then
//   K-contiguous rows like A's: copied with A's 32-wide swizzle into the
//   same 16 KiB B stages and read with one ds_read_b128 per fragment, as in
//   the pipelined kernel's BT form.  Only A gets whole-line pairs (B pairs
//   would need another 96 KiB).
#pragma once
#include <utility>

#include "device_common.hpp"
#include "gemm_pipelined.hpp"

namespace bpt {

template <typename T, typename OutT, bool BT = false>
struct ApairGemm {
    typedef PipelinedGemm<T, 256, 256, 32, 4, 2, 2, OutT, BT> P;      // wave tiles, B layout, epilogue
    static constexpr int BM = 256, BN = 256, BK = 32, STAGES = 4, KS = 2;
    static constexpr int MB = P::MB, NB = P::NB, TM = P::TM, TN = P::TN;
    static constexpr int AP_BYTES = BM * 2 * BK * 2;       // one pair stage: 256 rows x 128 bytes
    static constexpr int AP_STAGES = 3;
    static constexpr int B_BYTES = BK * BN * 2;            // one B stage
    static constexpr int B_BASE = AP_STAGES * AP_BYTES;
    static constexpr int RING_BYTES = B_BASE + STAGES * B_BYTES;
    static constexpr int LDS_BYTES = RING_BYTES > P::EPI_BYTES ? RING_BYTES : P::EPI_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static constexpr int A_INST = AP_BYTES / 1024 / 4;     // pair copies per wave (8)
    static constexpr int B_INST = B_BYTES / 1024 / 4;      // B copies per wave (4)
    static constexpr int LE = A_INST + B_INST;             // copies of an even group
    static constexpr int LO = B_INST;                      // copies of an odd group
    static constexpr int VMS = LE + LO;                    // publish(j+1): groups j+2, j+3 in flight
    static_assert(LE % KS == 0 && LO % KS == 0, "groups split evenly over the k-steps");
    static_assert((2 * LE + 2 * LO) < 64, "vmcnt is 6 bits");
    static constexpr int NMMA = MB * NB;
    static constexpr int NREAD = MB + (BT ? 1 : 2) * NB;
    static constexpr int RPM = (NREAD + (NMMA / 2) - 1) / (NMMA / 2);
    typedef typename Mfma<T>::frag_t frag_t;
};

template <typename T, typename OutT, bool BT = false>
__global__ __launch_bounds__(256, 1) void gemm_apair_kernel(GemmArgs args) {
    typedef ApairGemm<T, OutT, BT> G;
    typedef typename G::frag_t frag_t;
    constexpr int MB = G::MB, NB = G::NB, BK = G::BK, BN = G::BN, KS = G::KS;
    __shared__ __attribute__((aligned(1024))) char lds_raw[G::LDS_BYTES];
    BPT_LDS char* lds = (BPT_LDS char*)lds_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / 2;
    const int wn = wave % 2;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
    const int m0 = tm * G::BM;
    const int n0 = tn * BN;
    const int batch = blockIdx.y;

    const T* Ab = static_cast<const T*>(args.A) + batch * args.strideA;
    const T* Bb = static_cast<const T*>(args.B) + batch * args.strideB;
    const int M = args.M, N = args.N, K = args.K;
    const int lda = args.lda, ldb = args.ldb;
    const int4_t rsA = make_rsrc(Ab, (uint32_t)(((M - 1) * (long long)lda + K) * 2));
    const int NB_ = args.nb;
    // BT: B's resource starts at row n0 of B^T, so rows past N read as zero
    const int4_t rsB = BT ? make_rsrc(Bb + (long long)n0 * ldb, (uint32_t)(((N - n0 - 1) * (long long)ldb + K) * 2))
                          : make_rsrc(Bb, (uint32_t)(((K - 1) * (long long)ldb + NB_) * 2));

    // pair copies: 8 rows of 8 chunks (128 bytes) per instruction, chunk
    // swizzled as the 64-wide K-tile variant's A (rows past M read zero)
    uint32_t voffA[G::A_INST];
#pragma unroll
    for (int i = 0; i < G::A_INST; ++i) {
        const int row = (wave * G::A_INST + i) * 8 + lane / 8;
        const int chunk = (lane % 8) ^ swz_a<64>(row);
        voffA[i] = (uint32_t)(((m0 + row) * lda + chunk * 8) * 2);
    }
    // B copies as in the 32-wide pipelined kernel (columns past the width
    // fetch the last in-bounds piece; never stored).  BT: rows of B^T (the
    // columns of C) in 64-byte pieces, swizzled as A's 32-wide K-tiles.
    uint32_t voffB[G::B_INST];
#pragma unroll
    for (int i = 0; i < G::B_INST; ++i) {
        if constexpr (BT) {
            const int row = (wave * G::B_INST + i) * G::P::B_ROWS_PER_INST + lane / G::P::B_CHUNKS;
            const int chunk = (lane % G::P::B_CHUNKS) ^ swz_a<BK>(row);
            voffB[i] = (uint32_t)((row * ldb + chunk * 8) * 2);
        } else {
            const int row = (wave * G::B_INST + i) * 2 + lane / 32;
            const int chunk = (lane % 32) ^ swz_b(row);
            int col = n0 + chunk * 8;
            if (col >= NB_) col = NB_ - 8;
            voffB[i] = (uint32_t)((row * ldb + col) * 2);
        }
    }
    const uint32_t pair_step = 2 * BK * 2;                 // bytes of A per pair
    const uint32_t b_step = BT ? (uint32_t)BK * 2 : (uint32_t)BK * ldb * 2;   // bytes of B per K-tile

    // A block mb of K-tile parity t, k-step ks: row wm*TM + mb*32 + l%32,
    // logical chunk 4t + 2ks + l/32 of the 128-byte row, swizzled
    uint32_t rdA[2][KS];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int row = wm * G::TM + (lane % 32);
            const int chunk = (4 * t + 2 * ks + lane / 32) ^ swz_a<64>(row);
            rdA[t][ks] = (uint32_t)(row * 128 + chunk * 16);
        }
    // B block nb: transposing half-reads, as in the pipelined kernel
    uint32_t rdB[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int g = lane / 16, j = lane % 16;
        const int krow = 8 * (g / 2) + j / 4;
        const int col = wn * G::TN + nb * 32 + 16 * (g % 2) + 4 * (j % 4);
        const int chunk = (col / 8) ^ swz_b(krow);
        rdB[nb] = (uint32_t)(G::B_BASE + krow * BN * 2 + chunk * 16 + (col % 8) * 2);
    }
    // BT: B block nb, k-step ks is read like A: row (column of C) wn*TN +
    // nb*32 + lane%32 of the [BN][BK] stage, k ks*16 + 8*(lane/32)
    uint32_t rdBt[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int row = wn * G::TN + (lane % 32);
        const int chunk = (ks * 2 + lane / 32) ^ swz_a<BK>(row);
        rdBt[ks] = (uint32_t)(G::B_BASE + (row * BK + chunk * 8) * 2);
    }

    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));

    // copy i of a group: pair copies first (even groups), then B
    auto dma_one = [&]<bool EVEN>(int i, int bst, int ast, uint32_t kA, uint32_t kB) __attribute__((always_inline)) {
        if (EVEN && i < G::A_INST)
            dma16(rsA, lds0 + ast * G::AP_BYTES + (wave * G::A_INST + i) * 1024, voffA[i], kA);
        else {
            const int b = EVEN ? i - G::A_INST : i;
            dma16(rsB, lds0 + G::B_BASE + bst * G::B_BYTES + (wave * G::B_INST + b) * 1024, voffB[b], kB);
        }
    };

    float16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[i][j] = float16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    frag_t fa[2][MB];
    short4_t fbl[2][NB], fbh[2][NB];
    frag_t fbt[2][NB];                     // BT: B in one read

    // LDS read p of k-step ks of a tile (A pair stage ast, parity t; B stage bst) into set s
    auto read_piece = [&](int ast, int t, int bst, int ks, int p, int s) __attribute__((always_inline)) {
        if (p < MB) {
            fa[s][p] = *(BPT_LDS frag_t*)(lds + ast * G::AP_BYTES + rdA[t][ks] + p * 32 * 128);
        } else if constexpr (BT) {
            fbt[s][p - MB] = *(BPT_LDS frag_t*)(lds + bst * G::B_BYTES + rdBt[ks] + (p - MB) * 32 * BK * 2);
        } else {
            const int nb = (p - MB) / 2, h = (p - MB) % 2;
            BPT_LDS short4_t* q = (BPT_LDS short4_t*)(lds + bst * G::B_BYTES + rdB[nb] + ks * 16 * BN * 2 + h * 4 * BN * 2);
            if (h == 0) fbl[s][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
            else fbh[s][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
        }
    };

    // one k-step on fragment set s: MFMAs interleaved with the reads of the
    // next k-step (into set s^1) and with copies [d0, d0 + SLICE) of a group
    auto kstep = [&]<int SLICE, bool EVEN>(int s, bool reads, int rast, int rt, int rbst, int rks, int d0, int bst,
                                            int ast, uint32_t kA, uint32_t kB) __attribute__((always_inline)) {
        constexpr int DEVERY = SLICE > 0 ? G::NMMA / SLICE : 1;
        constexpr int DOFF = DEVERY / 2;
#pragma unroll
        for (int q = 0; q < G::NMMA; ++q) {
            if (reads) {
#pragma unroll
                for (int r = 0; r < G::RPM; ++r)
                    if (q * G::RPM + r < G::NREAD) read_piece(rast, rt, rbst, rks, q * G::RPM + r, s ^ 1);
            }
            const int mb = q / NB, nb = q % NB;
            frag_t b;
            if constexpr (BT)
                b = fbt[s][nb];
            else
                b = __builtin_bit_cast(frag_t, __builtin_shufflevector(fbl[s][nb], fbh[s][nb], 0, 1, 2, 3, 4, 5, 6, 7));
            acc[mb][nb] = Mfma<T>::mma32(b, fa[s][mb], acc[mb][nb]);
            if constexpr (SLICE > 0) {
                const int slot = q - DOFF;
                if (slot >= 0 && slot % DEVERY == 0 && slot / DEVERY < SLICE)
                    dma_one.template operator()<EVEN>(d0 + slot / DEVERY, bst, ast, kA, kB);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int nk = K / BK;                 // host: K % 64 == 0, nk >= 6

    // prologue: groups of tiles 0 .. 3 (pairs 0 and 1 with groups 0 and 2)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const uint32_t kB = g * b_step, kA = (g / 2) * pair_step;
        if (g % 2 == 0) {
#pragma unroll
            for (int i = 0; i < G::LE; ++i) dma_one.template operator()<true>(i, g, g / 2, kA, kB);
        } else {
#pragma unroll
            for (int i = 0; i < G::LO; ++i) dma_one.template operator()<false>(i, g, 0, kA, kB);
        }
    }
    publish<G::LO + G::LE + G::LO>();      // group 0 (tile 0) landed for every wave
#pragma unroll
    for (int p = 0; p < G::NREAD; ++p) read_piece(0, 0, 0, 0, p, 0);

    int bs = 0;                            // B stage of the tile being consumed
    int as = 0;                            // its A pair stage
    uint32_t kBn = 4 * b_step, kAn = 2 * pair_step;   // next group's offsets (group 4, pair 2)
    int bsp = 0, asp = 0;                  // pending group: stages and offsets
    uint32_t kBp = 0, kAp = 0;

    // tile j of parity P.  WIN: start group j+4 (parity P) in the window;
    // PEND: finish group j+3 (parity 1-P) in k-step 0; VM: publish(j+1)
    // wait; LAST: no publish, no next reads.
    auto tile = [&]<int P, bool WIN, bool PEND, int VM, bool LAST>() __attribute__((always_inline)) {
        constexpr int LPEND = P == 1 ? G::LE : G::LO;       // size of group j+3
        constexpr int LWIN = P == 0 ? G::LE : G::LO;        // size of group j+4
        kstep.template operator()<PEND ? LPEND / 2 : 0, P == 1>(0, true, as, P, bs, 1, LPEND / 2, bsp, asp, kAp, kBp);
        if constexpr (!LAST) {
            publish<VM>();
            const int bn = (bs + 1) & 3;
            const int an = P == 1 ? (as == 2 ? 0 : as + 1) : as;
            const int aw = as == 0 ? 2 : as - 1;           // pair stage of group j+4: (as + 2) % 3
            kstep.template operator()<WIN ? LWIN / 2 : 0, P == 0>(1, true, an, 1 - P, bn, 0, 0, bs, aw, kAn, kBn);
            if constexpr (WIN) {
                bsp = bs;
                asp = aw;
                kBp = kBn;
                kAp = kAn;
                kBn += b_step;
                if constexpr (P == 0) kAn += pair_step;
            }
            bs = bn;
            as = an;
        } else {
            kstep.template operator()<0, false>(1, false, 0, 0, 0, 0, 0, 0, 0, 0, 0);
        }
    };

    tile.template operator()<0, true, false, G::VMS, false>();              // j = 0
    int j = 1;
    for (; j < nk - 5; j += 2) {
        tile.template operator()<1, true, true, G::VMS, false>();
        tile.template operator()<0, true, true, G::VMS, false>();
    }
    tile.template operator()<1, true, true, G::VMS, false>();               // j = nk-5
    tile.template operator()<0, false, true, G::VMS, false>();              // j = nk-4: last group finishes
    tile.template operator()<1, false, false, G::LO, false>();              // j = nk-3: group nk-1 in flight
    tile.template operator()<0, false, false, 0, false>();                  // j = nk-2
    tile.template operator()<1, false, false, 0, true>();                   // j = nk-1

    pipelined_epilogue<typename G::P, OutT>(args, acc, lds, lane, wave, wm, wn, m0, n0, batch);
}

}  // namespace bpt
