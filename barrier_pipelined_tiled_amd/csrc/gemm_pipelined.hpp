// gemm_pipelined.hpp -- the software-pipelined tiled GEMM for gfx950.
//
// C = A * B, A row-major M x K (lda), B row-major K x N (ldb), C row-major
// M x N (ldc); fp16 or bf16 inputs, fp32 accumulation on the matrix cores.
//
// What the pages describe and how it is rebuilt here:
//
// * "Xe2 Nbarrier Pipelining", section "Core Concept: Split Barrier": a
//   barrier is split into a non-blocking arrive after the shared-memory
//   writes and a blocking wait before the reads, with independent loads and
//   ALU work placed in between.  The NVIDIA mbarrier page ("Phase Completion
//   Condition") makes the same idea precise: a stage is ready when every
//   expected arrival has happened AND every asynchronous transfer byte has
//   landed.  gfx950 has neither a split barrier nor a transaction counter,
//   only s_barrier and the per-wave vmcnt.  So each K-tile's LDS stage is
//   published by two steps: (1) the wave waits until its own LDS-DMA copies
//   for that stage have landed (s_waitcnt vmcnt(n), the tx-count half), then
//   (2) one s_barrier (the arrival half).  The "window" between publish and
//   consume holds the issue of the next stage's global->LDS copies, which
//   then fly during the whole MFMA phase of the current stage.
// * The same page, "What Doesn't Work: Double-Arrive Deadlock", and the
//   GEMM page's "Hardware limits": every wave executes exactly the same
//   sequence of barriers -- the loop below has no wave-dependent branch.
// * "Xe2 ESIMD GEMM", "Inner-loop rules": no conditionals in the K-loop
//   (the drain iterations are peeled into their own phase with static wait
//   counts) and incremented offsets (the buffer descriptors are built once
//   and only the scalar k offset advances, cf. "Payload CSE").
// * "Xe2 ESIMD GEMM", "DPAS / VNNI": the pages pack B for the matrix engine.
//   Here B stays row-major [k][n] in LDS and ds_read_b64_tr_b16 delivers it
//   transposed into the MFMA B-operand layout.
//
// Tiling: BM x BN workgroup tile, 4 waves in a WM x WN grid, each wave owns
// (BM/WM) x (BN/WN) built from 32x32 MFMA blocks (v_mfma_f32_32x32x16).
// STAGES LDS buffers of (BM + BN) * BK halves each form the staging ring.
#pragma once
#include <utility>

#include "device_common.hpp"

namespace bpt {

struct GemmArgs {
    const void* A;
    const void* B;
    void* C;
    int M, N, K;
    int lda, ldb, ldc;
    long long strideA, strideB, strideC;   // elements between batch entries
    int tiles_m, tiles_n;
    int group_m;                           // tile rows per group in the walk order
};

// ---------------------------------------------------------------------------
// Tile walk (which output tile a workgroup computes).
//
// Workgroups are handed to the 8 XCDs round-robin (id % 8), and each XCD has
// its own L2.  The id is first permuted so that XCD x receives a contiguous
// run of logical ids, then logical ids walk the tile grid in groups of
// group_m tile-rows, column by column inside a group, so the tiles one XCD
// holds at a time share few A row-panels and B column-panels.
// ---------------------------------------------------------------------------
__device__ inline void tile_of(int pid, int num, int tiles_m, int tiles_n, int group_m,
                               int& tm, int& tn) {
    if ((num & 7) == 0) {
        int per_xcd = num >> 3;
        pid = (pid & 7) * per_xcd + (pid >> 3);
    }
    int per_group = group_m * tiles_n;
    int group = pid / per_group;
    int first_m = group * group_m;
    int rows_here = min(tiles_m - first_m, group_m);
    int in_group = pid - group * per_group;
    tm = first_m + in_group % rows_here;
    tn = in_group / rows_here;
}

// XOR swizzles of 16-byte chunks inside an LDS tile row.  The LDS-DMA copy
// fixes where a lane's 16 bytes land (base + 16*lane), so the swizzle is
// applied by choosing which global chunk each lane fetches.
//
// A tile rows are BK=64 halves (8 chunks).  ds_read_b128 of 32 consecutive
// rows at one k-chunk must spread over the banks: chunk ^ f(row) with
// f(row) = (row & 7) ^ ((row >> 3) & 1) gives distinct banks for any 8
// consecutive rows (32-bank view) and any 16 consecutive rows (64-bank view).
__device__ inline int swz_a64(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// B tile rows are BN halves (>= 16 chunks).  ds_read_b64_tr_b16 makes each
// 16-lane group read 4 consecutive k rows x 32 bytes; f(k & 3) from
// {0, 6, 10, 12} puts those 4 rows on disjoint banks in both views, and the
// two 16-lane groups of a half-wave (next 16 columns) as well.
__device__ inline int swz_b(int k) {
    return ((k & 1) ? 6 : 0) ^ ((k & 2) ? 10 : 0);
}

template <typename T, int BM, int BN, int BK, int STAGES, int WM, int WN, typename OutT>
struct PipelinedGemm {
    static_assert(WM * WN == 4, "four waves per workgroup");
    static_assert(BK == 64, "A swizzle is written for 64-wide K tiles");
    static constexpr int kThreads = 256;
    static constexpr int TM = BM / WM;          // wave tile rows
    static constexpr int TN = BN / WN;          // wave tile cols
    static constexpr int MB = TM / 32;          // 32x32 blocks per wave (m)
    static constexpr int NB = TN / 32;          // 32x32 blocks per wave (n)
    static constexpr int KS = BK / 16;          // MFMA k-steps per tile
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(BN >= 128, "B swizzle needs >= 16 chunks per row");

    static constexpr int A_STAGE = BM * BK;     // halves
    static constexpr int B_STAGE = BK * BN;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int LDS_HALVES = STAGES * STAGE;

    // LDS-DMA bookkeeping: one wave instruction moves 1 KiB = 512 halves.
    static constexpr int A_INST = A_STAGE / 512;           // per workgroup
    static constexpr int B_INST = B_STAGE / 512;
    static constexpr int A_INST_W = A_INST / 4;            // per wave
    static constexpr int B_INST_W = B_INST / 4;
    static constexpr int LOADS_PER_STAGE = A_INST_W + B_INST_W;  // vmcnt units per stage
    static constexpr int A_ROWS_PER_INST = 512 / BK;       // 8
    static constexpr int B_ROWS_PER_INST = 512 / BN;       // 2 for BN=256
    static constexpr int B_CHUNKS = BN / 8;
    static_assert(A_INST % 4 == 0 && B_INST % 4 == 0, "stage must split evenly over 4 waves");
    static_assert(LOADS_PER_STAGE * (STAGES - 1) < 64, "vmcnt is 6 bits");
    static_assert(KS % 2 == 0, "fragment double-buffering alternates sets per k-step");

    typedef typename Mfma<T>::frag_t frag_t;
};

template <typename T, int BM, int BN, int BK, int STAGES, int WM, int WN, typename OutT>
__global__ __launch_bounds__(256, 1) void gemm_pipelined_kernel(GemmArgs args) {
    typedef PipelinedGemm<T, BM, BN, BK, STAGES, WM, WN, OutT> G;
    typedef typename G::frag_t frag_t;
    __shared__ __attribute__((aligned(1024))) T lds[G::LDS_HALVES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int wm = wave / WN;
    const int wn = wave % WN;

    // ---- a2: tile mapping --------------------------------------------------
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int batch = blockIdx.y;

    const T* Ab = static_cast<const T*>(args.A) + batch * args.strideA;
    const T* Bb = static_cast<const T*>(args.B) + batch * args.strideB;
    const int M = args.M, N = args.N, K = args.K;
    const int lda = args.lda, ldb = args.ldb;

    // ---- a3: descriptors once, per-lane offsets once -------------------------
    // Extent of each operand in bytes: anything at or beyond reads as zero.
    const int4_t rsA = make_rsrc(Ab, (uint32_t)(((M - 1) * (long long)lda + K) * 2));
    const int4_t rsB = make_rsrc(Bb, (uint32_t)(((K - 1) * (long long)ldb + N) * 2));

    uint32_t voffA[G::A_INST_W];
#pragma unroll
    for (int i = 0; i < G::A_INST_W; ++i) {
        int row = (wave * G::A_INST_W + i) * G::A_ROWS_PER_INST + lane / 8;
        int chunk = (lane % 8) ^ swz_a64(row);
        voffA[i] = (uint32_t)(((m0 + row) * lda + chunk * 8) * 2);
    }
    uint32_t voffB[G::B_INST_W];
#pragma unroll
    for (int i = 0; i < G::B_INST_W; ++i) {
        int row = (wave * G::B_INST_W + i) * G::B_ROWS_PER_INST + lane / G::B_CHUNKS;
        int chunk = (lane % G::B_CHUNKS) ^ swz_b(row);
        voffB[i] = (uint32_t)((row * ldb + n0 + chunk * 8) * 2);
    }
    const uint32_t a_step = BK * 2;                        // bytes per K-tile
    const uint32_t b_step = (uint32_t)BK * ldb * 2;

    // LDS read offsets (bytes, within a stage) for the MFMA operands.
    // A block mb, k-step ks: row = wm*TM + mb*32 + lane%32, k = ks*16 + 8*(lane/32).
    uint32_t rdA[G::KS];
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
        int row = wm * G::TM + (lane % 32);
        int chunk = (ks * 2 + lane / 32) ^ swz_a64(row);
        rdA[ks] = (uint32_t)((row * BK + chunk * 8) * 2);
    }
    // B block nb: a 16-lane group g reads rows k = ks*16 + 8*(g/2) + 4*h + j/4
    // and columns n = nb*32 + 16*(g%2) + 4*(j%4) (j = lane % 16); the
    // transpose read hands lane j the 4 k-values of column nb*32+16*(g%2)+j.
    uint32_t rdB[G::NB];
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) {
        int g = lane / 16, j = lane % 16;
        int krow = 8 * (g / 2) + j / 4;
        int col = wn * G::TN + nb * 32 + 16 * (g % 2) + 4 * (j % 4);
        int chunk = (col / 8) ^ swz_b(krow);
        rdB[nb] = (uint32_t)(G::A_STAGE * 2 + krow * BN * 2 + chunk * 16 + (col % 8) * 2);
    }

    BPT_LDS char* lds_bytes = (BPT_LDS char*)lds;

    // LDS byte address of the ring (uniform)
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_bytes));
    constexpr int STAGE_BYTES = G::STAGE * 2;
    constexpr int LPS = G::LOADS_PER_STAGE;

    // copy number i (0 .. LPS-1) of this wave for the tile at k offsets
    // (kA, kB) into ring stage `stage`: A instructions first, then B
    auto dma_one = [&](int stage, int i, uint32_t kA, uint32_t kB) {
        const uint32_t sbase = lds0 + stage * STAGE_BYTES;
        if (i < G::A_INST_W)
            dma16(rsA, sbase + (wave * G::A_INST_W + i) * 1024, voffA[i], kA);
        else
            dma16(rsB, sbase + G::A_STAGE * 2 + (wave * G::B_INST_W + (i - G::A_INST_W)) * 1024,
                  voffB[i - G::A_INST_W], kB);
    };

    float16_t acc[G::MB][G::NB];
#pragma unroll
    for (int i = 0; i < G::MB; ++i)
#pragma unroll
        for (int j = 0; j < G::NB; ++j)
            acc[i][j] = float16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                                  0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    // Operand fragments of one MFMA k-step, double-buffered in registers.
    frag_t fa0[G::MB], fb0[G::NB], fa1[G::MB], fb1[G::NB];

    auto load_frags = [&](int stage, int ks, frag_t (&a)[G::MB], frag_t (&b)[G::NB]) {
        BPT_LDS char* sbase = lds_bytes + stage * STAGE_BYTES;
#pragma unroll
        for (int mb = 0; mb < G::MB; ++mb)
            a[mb] = *(BPT_LDS frag_t*)(sbase + rdA[ks] + mb * 32 * BK * 2);
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
            BPT_LDS char* p = sbase + rdB[nb] + ks * 16 * BN * 2;
            short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BPT_LDS short4_t*)p);
            short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BPT_LDS short4_t*)(p + 4 * BN * 2));
            b[nb] = __builtin_bit_cast(frag_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };

    // All MFMAs of one k-step; when `with_dma`, the next-next tile's copies
    // are issued between them (ceil(LPS / MFMAs) per MFMA).
    constexpr int NMMA = G::MB * G::NB;
    constexpr int DMA_PER_MMA = (LPS + NMMA - 1) / NMMA;
    auto mma_step = [&](frag_t (&a)[G::MB], frag_t (&b)[G::NB], bool with_dma, int stage,
                        uint32_t kA, uint32_t kB) {
#pragma unroll
        for (int q = 0; q < NMMA; ++q) {
            const int mb = q / G::NB, nb = q % G::NB;
            acc[mb][nb] = Mfma<T>::mma32(a[mb], b[nb], acc[mb][nb]);
            if (with_dma) {
#pragma unroll
                for (int r = 0; r < DMA_PER_MMA; ++r)
                    if (q * DMA_PER_MMA + r < LPS) dma_one(stage, q * DMA_PER_MMA + r, kA, kB);
                __builtin_amdgcn_sched_barrier(0);     // keep copies spread between MFMAs
            }
        }
    };

    // ---- a4/a5: prologue, steady state, drain --------------------------------
    //
    // Tile j lives in ring stage j % STAGES.  Per tile, k-steps 0 .. KS-2 read
    // the next k-step's fragments while the MFMAs of the current one run.
    // Then comes the publish point of tile j+1 and its window:
    //   publish(j+1): own copies of tile j+1 landed + s_barrier.  Every wave
    //                 has also finished its reads of tile j's stage.
    //   window:       read tile j+1's first fragments, then run tile j's last
    //                 k-step from registers while issuing the copies of tile
    //                 j+STAGES into the stage tile j just vacated.
    // The copies of a tile are in flight for STAGES-1 full tiles of MFMA work.
    const int nk = K / BK;                 // host guarantees K % BK == 0 and nk >= STAGES
    uint32_t kA = 0, kB = 0;               // byte offsets of the next tile to copy
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
#pragma unroll
        for (int i = 0; i < LPS; ++i) dma_one(s, i, kA, kB);
        kA += a_step;
        kB += b_step;
    }
    publish<LPS * (STAGES - 1)>();         // tile 0 is in LDS for every wave
    load_frags(0, 0, fa0, fb0);
    int sc = 0;                            // stage of the tile being consumed

    // one tile; DMA: issue tile j+STAGES in the window; VM: vmcnt for
    // publish(j+1); LAST: final tile (no publish, no next reads)
    auto tile = [&]<bool DMA, int VM, bool LAST>() {
#pragma unroll
        for (int ks = 0; ks < G::KS - 1; ++ks) {
            // the next k-step's reads are issued before this k-step's MFMAs
            // (the fence stops the scheduler from sinking them to their use)
            if (ks % 2 == 0) {
                load_frags(sc, ks + 1, fa1, fb1);
                __builtin_amdgcn_sched_barrier(0);
                mma_step(fa0, fb0, false, 0, 0, 0);
            } else {
                load_frags(sc, ks + 1, fa0, fb0);
                __builtin_amdgcn_sched_barrier(0);
                mma_step(fa1, fb1, false, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (!LAST) {
            publish<VM>();
            const int sn = (sc + 1 == STAGES) ? 0 : sc + 1;
            load_frags(sn, 0, fa0, fb0);
            __builtin_amdgcn_sched_barrier(0);
            mma_step(fa1, fb1, DMA, sc, kA, kB);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (DMA) {
                kA += a_step;
                kB += b_step;
            }
            sc = sn;
        } else {
            mma_step(fa1, fb1, false, 0, 0, 0);
        }
    };

    for (int j = 0; j < nk - STAGES; ++j) tile.template operator()<true, LPS * (STAGES - 2), false>();
    // drain: the last STAGES tiles issue no copies; the wait counts fall to 0
    [&]<int... D>(std::integer_sequence<int, D...>) {
        ((D < STAGES - 1 ? tile.template operator()<false, LPS * (STAGES - 2 - (D < STAGES - 1 ? D : 0)), false>()
                         : tile.template operator()<false, 0, true>()),
         ...);
    }(std::make_integer_sequence<int, STAGES>{});

    // ---- a8: epilogue ---------------------------------------------------------
    // 32x32 block result layout: lane l, register r holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
    OutT* Cb = static_cast<OutT*>(args.C) + batch * args.strideC;
    const int ldc = args.ldc;
    const bool full = (m0 + BM <= M) && (n0 + BN <= N);
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) {
            int col = n0 + wn * G::TN + nb * 32 + (lane % 32);
            int rbase = m0 + wm * G::TM + mb * 32 + 4 * (lane / 32);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int row = rbase + 8 * (r / 4) + (r % 4);
                if (full || (row < M && col < N))
                    Cb[(long long)row * ldc + col] = cvt_out<OutT>(acc[mb][nb][r]);
            }
        }
}

}  // namespace bpt
