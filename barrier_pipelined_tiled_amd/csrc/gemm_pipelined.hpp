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
//   (2) one s_barrier (the arrival half).
// * The window between publish and consume ("What goes between arrive and
//   wait"): right after the publish of tile j+1 each wave starts reading
//   tile j+1's first operand fragments, runs the last k-step of tile j from
//   registers (it touches no LDS), and in between issues the copies of tile
//   j+STAGES into the stage tile j has just vacated.  Nothing in the window
//   reads LDS another wave is writing or writes LDS another wave reads.
// * "What Doesn't Work: Double-Arrive Deadlock" and the GEMM page's
//   "Hardware limits": every wave executes exactly the same sequence of
//   barriers -- the loop has no wave-dependent branch.
// * "Xe2 ESIMD GEMM", "Inner-loop rules": no conditionals in the K-loop (the
//   drain tiles are peeled into their own phase with static wait counts) and
//   incremented offsets (buffer descriptors are built once and only the
//   scalar k offset advances, cf. "Payload CSE").
// * "Xe2 ESIMD GEMM", "DPAS / VNNI": the pages pack B for the matrix engine.
//   Here B stays row-major [k][n] in LDS and ds_read_b64_tr_b16 delivers it
//   transposed into the MFMA operand layout.
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
    int c_vec;                             // C rows 16-byte aligned: vector stores allowed
    int nb;                                // columns of B (N, or N rounded up to 8 when B
                                           // is a zero-padded copy); N bounds the C stores
};

// ---------------------------------------------------------------------------
// Tile walk (which output tile a workgroup computes).
//
// Workgroups are handed to the 8 XCDs round-robin (id % 8), and each XCD has
// its own L2.  The id is first permuted so that XCD x receives a contiguous
// run of logical ids (tile_of), then logical ids walk the tile grid in groups
// of group_m tile-rows, column by column inside a group (group_walk), so the
// tiles one XCD holds at a time share few A row-panels and B column-panels.
// ---------------------------------------------------------------------------
__device__ inline void group_walk(int pid, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
    int per_group = group_m * tiles_n;
    int group = pid / per_group;
    int first_m = group * group_m;
    int rows_here = min(tiles_m - first_m, group_m);
    int in_group = pid - group * per_group;
    tm = first_m + in_group % rows_here;
    tn = in_group / rows_here;
}

__device__ inline void tile_of(int pid, int num, int tiles_m, int tiles_n, int group_m,
                               int& tm, int& tn) {
    if ((num & 7) == 0) {
        int per_xcd = num >> 3;
        pid = (pid & 7) * per_xcd + (pid >> 3);
    }
    group_walk(pid, tiles_m, tiles_n, group_m, tm, tn);
}

// XOR swizzles of 16-byte chunks inside an LDS tile row.  The LDS-DMA copy
// fixes where a lane's 16 bytes land (base + 16*lane), so the swizzle is
// applied by choosing which global chunk each lane fetches.
//
// A rows are BK halves, read by ds_read_b128 as 32 consecutive rows at one
// k-chunk (lanes 0-31) and the next chunk of the same rows (lanes 32-63):
//   BK = 64 (8 chunks, 128 B rows): chunk ^ ((row & 7) ^ ((row >> 3) & 1))
//   BK = 32 (4 chunks,  64 B rows): chunk ^ ((row >> 2) & 3)
// Both were measured conflict-free (SQ_LDS_BANK_CONFLICT 0, 4 LDS cycles
// per instruction) by a probe running the read pattern alone.  For 64-byte
// rows, chunk ^ (((row >> 1) ^ (row >> 3)) & 3), which a 64-bank model calls
// conflict-free, measured 2-way (8 cycles), and no swizzle 4-way.
template <int BK>
__device__ inline int swz_a(int row);
template <>
__device__ inline int swz_a<64>(int row) { return (row & 7) ^ ((row >> 3) & 1); }
template <>
__device__ inline int swz_a<32>(int row) { return (row >> 2) & 3; }

// B rows are BN halves (>= 16 chunks).  ds_read_b64_tr_b16 makes each
// 16-lane group read 4 consecutive k rows x 32 bytes; f(k & 3) from
// {0, 6, 10, 12} puts those 4 rows on disjoint banks in both views, and the
// two 16-lane groups of a half-wave (next 16 columns) as well.
__device__ inline int swz_b(int k) {
    return ((k & 1) ? 6 : 0) ^ ((k & 2) ? 10 : 0);
}

// BT: B is given transposed, N x K row-major (C = A * B^T).  Its tiles are
// then K-contiguous like A's: copied and swizzled as A, read with
// ds_read_b128 straight into the MFMA operand, no transposing read.
template <typename T, int BM, int BN, int BK, int STAGES, int WM, int WN, typename OutT, bool BT = false>
struct PipelinedGemm {
    static_assert(WM * WN == 4, "four waves per workgroup");
    static_assert(BK == 64 || BK == 32, "A swizzles exist for 32- and 64-wide K tiles");
    static_assert(STAGES >= 2, "the window needs at least two stages");
    static constexpr int TM = BM / WM;          // wave tile rows
    static constexpr int TN = BN / WN;          // wave tile cols
    static constexpr int MB = TM / 32;          // 32x32 blocks per wave (m)
    static constexpr int NB = TN / 32;          // 32x32 blocks per wave (n)
    static constexpr int KS = BK / 16;          // MFMA k-steps per tile
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(BT || BN >= 128, "B swizzle needs >= 16 chunks per row");
    static_assert(KS % 2 == 0, "fragment double-buffering alternates sets per k-step");

    static constexpr int A_STAGE = BM * BK;     // halves
    static constexpr int B_STAGE = BK * BN;
    static constexpr int STAGE_BYTES = (A_STAGE + B_STAGE) * 2;
    static constexpr int RING_BYTES = STAGES * STAGE_BYTES;

    // LDS-DMA bookkeeping: one wave instruction moves 1 KiB = 512 halves.
    static constexpr int A_INST_W = A_STAGE / 512 / 4;     // per wave
    static constexpr int B_INST_W = B_STAGE / 512 / 4;
    static constexpr int LPS = A_INST_W + B_INST_W;         // vmcnt units per stage per wave
    static constexpr int A_CHUNKS = BK / 8;                 // 16-byte chunks per A row
    static constexpr int A_ROWS_PER_INST = 64 / A_CHUNKS;
    static constexpr int B_CHUNKS = BT ? BK / 8 : BN / 8;   // 16-byte chunks per B tile row
    static constexpr int B_ROWS_PER_INST = 64 / B_CHUNKS;
    static_assert(A_STAGE % 2048 == 0 && B_STAGE % 2048 == 0, "stage must split evenly over 4 waves");
    static_assert(LPS * STAGES < 64, "vmcnt is 6 bits");

    // per k-step: MFMAs, LDS reads (A fragments + B fragments: two transposing
    // half-reads each, or one read when B is given transposed)
    static constexpr int NMMA = MB * NB;
    static constexpr int NREAD = MB + (BT ? 1 : 2) * NB;
    static constexpr int RPM = (NREAD + (NMMA / 2) - 1) / (NMMA / 2);   // reads per MFMA
    // copies of one group are spread over the KS k-steps of a tile: DSLICE per
    // k-step, one every DEVERY MFMA slots, starting DOFF slots in
    static constexpr int DSLICE = LPS / KS;
    static constexpr int DPQ = (DSLICE + NMMA - 1) / NMMA;              // copies per MFMA slot
    static constexpr int DEVERY = (NMMA * DPQ) / DSLICE;
    static constexpr int DOFF = DEVERY / 2;
    static_assert(LPS % KS == 0, "copies split evenly over the k-steps");

    // epilogue staging: each wave writes its tile to LDS, then stores rows
    // with 16-byte accesses; 4-byte outputs go in two passes.
    static constexpr int EPI_PASSES = sizeof(OutT) == 4 ? 2 : 1;
    static constexpr int EPI_ROWS = TM / EPI_PASSES;
    static constexpr int EPI_PITCH = TN * (int)sizeof(OutT) + 16;   // bytes, padded
    static constexpr int EPI_BYTES = 4 * EPI_ROWS * EPI_PITCH;
    // K % BK != 0: the partial last K-tile gets a stage of its own behind the
    // ring, when that fits
    static constexpr bool TAIL = RING_BYTES + STAGE_BYTES <= 160 * 1024;
    static constexpr int MAIN_BYTES = RING_BYTES + (TAIL ? STAGE_BYTES : 0);
    static constexpr int LDS_BYTES = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");

    typedef typename Mfma<T>::frag_t frag_t;
};

// ---- a8: epilogue ------------------------------------------------------------
// (shared by the pipelined kernels; G supplies the wave tile and staging
// geometry)
template <typename G, typename OutT>
__device__ inline void pipelined_epilogue(const GemmArgs& args, const float16_t (&acc)[G::MB][G::NB],
                                          BPT_LDS char* lds, int lane, int wave, int wm, int wn, int m0,
                                          int n0, int batch) {
    constexpr int MB = G::MB, NB = G::NB;
    const int M = args.M, N = args.N;
    // Result layout (B fragment as first MFMA operand): lane l, register r of
    // block (mb, nb) holds row mb*32 + l%32, column nb*32 + 8*(r/4) +
    // 4*(l/32) + r%4 of the wave tile.  Each wave stages its tile in LDS
    // (row-major, padded rows) and then writes whole rows, 16 bytes a lane.
    publish<0>();                          // every wave is done with the ring
    OutT* Cb = static_cast<OutT*>(args.C) + batch * args.strideC;
    const int ldc = args.ldc;
    const int row0 = m0 + wm * G::TM;      // first C row / column of this wave
    const int col0 = n0 + wn * G::TN;
    const bool vec = args.c_vec && (row0 + G::TM <= M) && (col0 + G::TN <= N);
    BPT_LDS char* stage_w = lds + wave * (G::EPI_ROWS * G::EPI_PITCH);
    constexpr int OB = (int)sizeof(OutT);
    constexpr int CH_PER_ROW = G::TN * OB / 16;            // 16-byte chunks per wave-tile row
    constexpr int ROWS_PER_IT = 64 / CH_PER_ROW;
    typedef OutT out4_t __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int pass = 0; pass < G::EPI_PASSES; ++pass) {
        constexpr int MBP = MB / G::EPI_PASSES;
#pragma unroll
        for (int mbp = 0; mbp < MBP; ++mbp) {
            const int mb = pass * MBP + mbp;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    out4_t v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = cvt_out<OutT>(acc[mb][nb][4 * g + e]);
                    const int r = mbp * 32 + (lane % 32);
                    const int c = nb * 32 + 8 * g + 4 * (lane / 32);
                    *(BPT_LDS out4_t*)(stage_w + r * G::EPI_PITCH + c * OB) = v;
                }
        }
        wave_lds_handoff();                        // rows written by other lanes are read below
#pragma unroll
        for (int it = 0; it < G::EPI_ROWS / ROWS_PER_IT; ++it) {
            const int r = it * ROWS_PER_IT + lane / CH_PER_ROW;
            const int ch = lane % CH_PER_ROW;
            int4_t v = *(BPT_LDS int4_t*)(stage_w + r * G::EPI_PITCH + ch * 16);
            const int grow = row0 + pass * G::EPI_ROWS + r;
            const int gcol = col0 + ch * (16 / OB);
            OutT* dst = Cb + (long long)grow * ldc + gcol;
            // a 16-byte chunk is wholly inside C or outside when N % 8 == 0;
            // only repacked calls (N % 8 != 0) have chunks that straddle N
            if (vec || (grow < M && gcol < N)) {
                if (args.c_vec && gcol + 16 / OB <= N) {
                    // non-temporal: C is written once and never read back
                    // here; stores that do not allocate in the L2 measured
                    // 8% faster on the batched shape (2 GiB of C per call),
                    // 1.5-2% on 4096^3 and the long-K shape
                    __builtin_nontemporal_store(v, (int4_t*)dst);
                } else {
                    OutT vals[16 / OB];
                    __builtin_memcpy(vals, &v, 16);
#pragma unroll 1
                    for (int e = 0; e < 16 / OB; ++e)
                        if (gcol + e < N) dst[e] = vals[e];
                }
            }
        }
        wave_lds_handoff();                        // the next pass overwrites what was just read
    }
}

template <typename T, int BM, int BN, int BK, int STAGES, int WM, int WN, typename OutT, bool BT = false>
__global__ __launch_bounds__(256, 1) void gemm_pipelined_kernel(GemmArgs args) {
    typedef PipelinedGemm<T, BM, BN, BK, STAGES, WM, WN, OutT, BT> G;
    typedef typename G::frag_t frag_t;
    constexpr int MB = G::MB, NB = G::NB, LPS = G::LPS;
    __shared__ __attribute__((aligned(1024))) char lds_raw[G::LDS_BYTES];
    BPT_LDS char* lds = (BPT_LDS char*)lds_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int wm = wave / WN;
    const int wn = wave % WN;

    // ---- a2: tile mapping ----------------------------------------------------
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
    const int NB_ = args.nb;               // host: NB_ % 8 == 0, N <= NB_ <= ldb (not BT)
    // BT: B's resource starts at row n0 of B^T, so rows past N read as zero
    const int4_t rsB = BT ? make_rsrc(Bb + (long long)n0 * ldb, (uint32_t)(((N - n0 - 1) * (long long)ldb + K) * 2))
                          : make_rsrc(Bb, (uint32_t)(((K - 1) * (long long)ldb + NB_) * 2));

    uint32_t voffA[G::A_INST_W];
#pragma unroll
    for (int i = 0; i < G::A_INST_W; ++i) {
        int row = (wave * G::A_INST_W + i) * G::A_ROWS_PER_INST + lane / G::A_CHUNKS;
        int chunk = (lane % G::A_CHUNKS) ^ swz_a<BK>(row);
        voffA[i] = (uint32_t)(((m0 + row) * lda + chunk * 8) * 2);
    }
    // A lane whose 8 columns of B start at or past B's width fetches the last
    // in-bounds chunk instead (host: the width is a multiple of 8), so no copy
    // ever reads past the end of B; those columns of C are never stored.
    uint32_t voffB[G::B_INST_W];
#pragma unroll
    for (int i = 0; i < G::B_INST_W; ++i) {
        int row = (wave * G::B_INST_W + i) * G::B_ROWS_PER_INST + lane / G::B_CHUNKS;
        if constexpr (BT) {                // row = column of C, chunks along k
            int chunk = (lane % G::B_CHUNKS) ^ swz_a<BK>(row);
            voffB[i] = (uint32_t)((row * ldb + chunk * 8) * 2);
        } else {
            int chunk = (lane % G::B_CHUNKS) ^ swz_b(row);
            int col = n0 + chunk * 8;
            if (col >= NB_) col = NB_ - 8;
            voffB[i] = (uint32_t)((row * ldb + col) * 2);
        }
    }
    const uint32_t a_step = BK * 2;                        // bytes per K-tile
    const uint32_t b_step = BT ? (uint32_t)BK * 2 : (uint32_t)BK * ldb * 2;

    // LDS read offsets (bytes, within a stage) for the MFMA operands.
    // A block mb, k-step ks: row wm*TM + mb*32 + lane%32, k ks*16 + 8*(lane/32).
    uint32_t rdA[G::KS];
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
        int row = wm * G::TM + (lane % 32);
        int chunk = (ks * 2 + lane / 32) ^ swz_a<BK>(row);
        rdA[ks] = (uint32_t)((row * BK + chunk * 8) * 2);
    }
    // B block nb: a 16-lane group g reads rows k = ks*16 + 8*(g/2) + 4*h + j/4
    // and columns n = nb*32 + 16*(g%2) + 4*(j%4) (j = lane % 16); the
    // transpose read hands lane j the 4 k-values of column nb*32+16*(g%2)+j.
    uint32_t rdB[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        int g = lane / 16, j = lane % 16;
        int krow = 8 * (g / 2) + j / 4;
        int col = wn * G::TN + nb * 32 + 16 * (g % 2) + 4 * (j % 4);
        int chunk = (col / 8) ^ swz_b(krow);
        rdB[nb] = (uint32_t)(G::A_STAGE * 2 + krow * BN * 2 + chunk * 16 + (col % 8) * 2);
    }
    // BT: B block nb, k-step ks is read like A: row (column of C) wn*TN +
    // nb*32 + lane%32 of the [BN][BK] tile, k ks*16 + 8*(lane/32)
    uint32_t rdBt[G::KS];
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
        int row = wn * G::TN + (lane % 32);
        int chunk = (ks * 2 + lane / 32) ^ swz_a<BK>(row);
        rdBt[ks] = (uint32_t)(G::A_STAGE * 2 + (row * BK + chunk * 8) * 2);
    }

    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));

    // copy number i (0 .. LPS-1) of this wave for the tile at k offsets
    // (kA, kB) into ring stage `stage`: A instructions first, then B
    auto dma_one = [&](int stage, int i, uint32_t kA, uint32_t kB) __attribute__((always_inline)) {
        const uint32_t sbase = lds0 + stage * G::STAGE_BYTES;
        if (i < G::A_INST_W)
            dma16(rsA, sbase + (wave * G::A_INST_W + i) * 1024, voffA[i], kA);
        else
            dma16(rsB, sbase + G::A_STAGE * 2 + (wave * G::B_INST_W + (i - G::A_INST_W)) * 1024,
                  voffB[i - G::A_INST_W], kB);
    };

    float16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[i][j] = float16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                                  0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    // Operand fragments of one k-step, double-buffered: set 0 and set 1.
    frag_t fa[2][MB];
    short4_t fbl[2][NB], fbh[2][NB];       // B as two transposing half-reads
    frag_t fbt[2][NB];                     // BT: B in one read

    // LDS read number p (0 .. NREAD-1) of k-step ks of ring stage st into set s
    auto read_piece = [&](int st, int ks, int p, int s) __attribute__((always_inline)) {
        BPT_LDS char* sbase = lds + st * G::STAGE_BYTES;
        if (p < MB) {
            fa[s][p] = *(BPT_LDS frag_t*)(sbase + rdA[ks] + p * 32 * BK * 2);
        } else if constexpr (BT) {
            fbt[s][p - MB] = *(BPT_LDS frag_t*)(sbase + rdBt[ks] + (p - MB) * 32 * BK * 2);
        } else {
            const int nb = (p - MB) / 2, h = (p - MB) % 2;
            BPT_LDS short4_t* q = (BPT_LDS short4_t*)(sbase + rdB[nb] + ks * 16 * BN * 2 + h * 4 * BN * 2);
            if (h == 0) fbl[s][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
            else fbh[s][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
        }
    };

    // One k-step: the MFMAs on fragment set s, interleaved with RPM LDS reads
    // per MFMA for (rst, rks) into the other set (when `reads`) and with
    // copies number [d0, d0 + DSLICE) of the group for stage dst (when
    // `dma`), one every NMMA/DSLICE MFMAs.  The MFMA takes the B fragment as
    // its first operand, so that each lane's result holds four consecutive
    // columns of one row of C.
    auto kstep = [&](int s, bool reads, int rst, int rks, bool dma, int dst, int d0, uint32_t kA,
                     uint32_t kB) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < G::NMMA; ++q) {
            if (reads) {
#pragma unroll
                for (int r = 0; r < G::RPM; ++r)
                    if (q * G::RPM + r < G::NREAD) read_piece(rst, rks, q * G::RPM + r, s ^ 1);
            }
            const int mb = q / NB, nb = q % NB;
            frag_t b;
            if constexpr (BT)
                b = fbt[s][nb];
            else
                b = __builtin_bit_cast(frag_t, __builtin_shufflevector(fbl[s][nb], fbh[s][nb],
                                                                       0, 1, 2, 3, 4, 5, 6, 7));
            acc[mb][nb] = Mfma<T>::mma32(b, fa[s][mb], acc[mb][nb]);
            if (dma) {
#pragma unroll
                for (int r = 0; r < G::DPQ; ++r) {
                    const int slot = q * G::DPQ + r - G::DOFF;   // copy slot within the slice
                    if (slot >= 0 && slot % G::DEVERY == 0 && slot / G::DEVERY < G::DSLICE)
                        dma_one(dst, d0 + slot / G::DEVERY, kA, kB);
                }
            }
            __builtin_amdgcn_sched_barrier(0);   // keep this interleave as written
        }
    };

    // ---- a4/a5: prologue, steady state, drain --------------------------------
    //
    // Tile j lives in ring stage j % STAGES.  Per tile, k-steps 0 .. KS-2 read
    // the next k-step's fragments while the MFMAs of the current one run.
    // Then comes the publish point of tile j+1 and its window:
    //   publish(j+1): own copies of tile j+1 landed + s_barrier.  Every wave
    //                 has also finished its reads of tile j's stage.
    //   window:       read tile j+1's first fragments, run tile j's last
    //                 k-step from registers, and start the copies of tile
    //                 j+STAGES into the stage tile j just vacated.
    // The copies of tile j+STAGES are spread in KS slices: slice 0 in the
    // window, slices 1 .. KS-1 in k-steps 0 .. KS-2 of tile j+1, so the load
    // path never sees a burst.  All of them are issued before publish(j+2),
    // which therefore still waits for exactly STAGES-2 younger groups.
    const int nk = K / BK;                 // full K-tiles; host guarantees nk >= STAGES

    // ---- K tail: K = nk*BK + ktail, 0 < ktail < BK, ktail % 8 == 0 (host) -----
    // The partial K-tile is copied first, into stage STAGES, with every copy
    // of k >= K pointed past num_records so it reads zeros (A chunks of 8 k
    // values and B rows are wholly valid or wholly not).  Being the oldest
    // copies in flight, they have landed once the first publish below has
    // waited for tile 0, and its barrier shows them to every wave.  The tail
    // K-tile is consumed after the last full one.
    const int ktail = K - nk * BK;
    if constexpr (G::TAIL) {
        if (ktail != 0) {
            const uint32_t tbase = lds0 + STAGES * G::STAGE_BYTES;
            const uint32_t tkA = (uint32_t)(nk * BK * 2);
            const uint32_t tkB = BT ? tkA : (uint32_t)nk * BK * ldb * 2;
            constexpr uint32_t kPast = 0x80000000u;        // beyond any extent the host allows
#pragma unroll
            for (int i = 0; i < G::A_INST_W; ++i) {
                int row = (wave * G::A_INST_W + i) * G::A_ROWS_PER_INST + lane / G::A_CHUNKS;
                int chunk = (lane % G::A_CHUNKS) ^ swz_a<BK>(row);
                dma16(rsA, tbase + (wave * G::A_INST_W + i) * 1024, chunk * 8 < ktail ? voffA[i] : kPast, tkA);
            }
#pragma unroll
            for (int i = 0; i < G::B_INST_W; ++i) {
                int row = (wave * G::B_INST_W + i) * G::B_ROWS_PER_INST + lane / G::B_CHUNKS;
                bool valid;
                if constexpr (BT)                          // chunks of 8 k values, as for A
                    valid = ((lane % G::B_CHUNKS) ^ swz_a<BK>(row)) * 8 < ktail;
                else                                       // rows of k
                    valid = row < ktail;
                dma16(rsB, tbase + G::A_STAGE * 2 + (wave * G::B_INST_W + i) * 1024, valid ? voffB[i] : kPast, tkB);
            }
        }
    }
    uint32_t kA = 0, kB = 0;               // byte offsets of the next tile to copy
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
#pragma unroll
        for (int i = 0; i < LPS; ++i) dma_one(s, i, kA, kB);
        kA += a_step;
        kB += b_step;
    }
    publish<LPS * (STAGES - 1)>();         // tile 0 is in LDS for every wave
#pragma unroll
    for (int p = 0; p < G::NREAD; ++p) read_piece(0, 0, p, 0);
    int sc = 0;                            // stage of the tile being consumed
    int sp = 0;                            // stage of the group still being copied
    uint32_t kAp = 0, kBp = 0;             // and its k offsets

    // one tile.  WIN: start a new group (tile j+STAGES) in the window; PEND:
    // finish the group started in the previous window during k-steps
    // 0 .. KS-2; VM: vmcnt for publish(j+1); LAST: final tile (no publish, no
    // next reads).
    auto tile = [&]<bool WIN, bool PEND, int VM, bool LAST>() __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < G::KS - 1; ++ks)
            kstep(ks & 1, true, sc, ks + 1, PEND, sp, (ks + 1) * G::DSLICE, kAp, kBp);
        if constexpr (!LAST) {
            publish<VM>();
            const int sn = (sc + 1 == STAGES) ? 0 : sc + 1;
            kstep(1, true, sn, 0, WIN, sc, 0, kA, kB);
            if constexpr (WIN) {
                sp = sc;
                kAp = kA;
                kBp = kB;
                kA += a_step;
                kB += b_step;
            }
            sc = sn;
        } else {
            kstep(1, false, 0, 0, false, 0, 0, 0, 0);
        }
    };

    constexpr int VMS = LPS * (STAGES - 2);
    if (nk > STAGES) {
        tile.template operator()<true, false, VMS, false>();
        for (int j = 1; j < nk - STAGES; ++j) tile.template operator()<true, true, VMS, false>();
        tile.template operator()<false, true, VMS, false>();      // drain tile 0 finishes the last group
    } else {
        tile.template operator()<false, false, VMS, false>();
    }
    // the rest of the drain, tiles d = 1 .. STAGES-1 of it: no copies; the
    // wait count of publish falls by one group per tile, and the last tile
    // publishes nothing
    constexpr auto drain_vm = [](int d) constexpr { return d < STAGES - 1 ? LPS * (STAGES - 2 - d) : 0; };
    [&]<int... D>(std::integer_sequence<int, D...>) {
        ((D + 1 < STAGES - 1 ? tile.template operator()<false, false, drain_vm(D + 1), false>()
                             : tile.template operator()<false, false, 0, true>()),
         ...);
    }(std::make_integer_sequence<int, STAGES - 1>{});

    // the tail K-tile, from its own stage (landed and published long ago)
    if constexpr (G::TAIL) {
        if (ktail != 0) {
#pragma unroll
            for (int p = 0; p < G::NREAD; ++p) read_piece(STAGES, 0, p, 0);
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks) kstep(ks & 1, ks + 1 < G::KS, STAGES, ks + 1, false, 0, 0, 0, 0);
        }
    }

    // ---- a8: epilogue ---------------------------------------------------------
    pipelined_epilogue<G, OutT>(args, acc, lds, lane, wave, wm, wn, m0, n0, batch);
}

}  // namespace bpt
