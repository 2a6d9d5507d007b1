// gemm_persist.hpp -- persistent GEMM for short K (C = A * B, B row-major
// K x N), 16-bit C: one workgroup per CU walks many 256 x 128 output tiles,
// and the C tile of one output tile is stored while the next one computes.
//
// With K = 256 (the batched attention-score shape) a tile is 8 K-tiles of
// 32, and storing its C takes about as long as computing it (K = 128: 4).  A workgroup
// per tile pays prologue, K-loop and C stores one after the other, and its
// CU cannot start the next tile before the stores are acknowledged.  Here
// the K-tile ring runs on across tile boundaries -- the copies of the next
// tile start four K-tiles before the current one ends, through that tile's
// own buffer descriptors -- and the finished accumulators are packed to 16
// bits into a staging area of LDS beside the ring when the next tile's first
// products overwrite them.  Each wave then stores its part of the tile in
// 16-byte row pieces (8 whole 128-byte lines per instruction), spread over
// the next tile's first 8 K-tiles (all of them when K = 128), right after a
// publish.  (Stores straight from registers write 8 bytes of 32 different
// rows per instruction; they measured three times slower than the stores
// they were meant to hide.)  The last tile takes the usual epilogue.
//
// The tile is 256 x 128 (4 waves of 128 x 64) rather than 256 x 256: the
// ring of 4 stages (96 KiB) and the staged tile (64 KiB) then fill the LDS
// exactly.  The ring is the pipelined kernel's: 4 stages of one A and one B
// K-tile, group j+4 copied into the stage tile j leaves, slice 0 in tile j's
// window and the rest in tile j+1's first k-step; publish(j+1) lets groups
// j+2 and j+3 stay in flight.
//
// Stores share the vmcnt counter with the copies, and only loads are known
// to complete in issue order among themselves.  Every publish still waits
// for exactly "all but the younger copies", which is right whatever the
// stores do: a younger copy completes only after every older one, and the
// count also covers any store still in flight.  Copies for tiles past the
// last one go through a descriptor with no records (zeros, no memory
// traffic), so the loop has one form and every wait count stays constant.
//
// Walk: the workgroups of one XCD take turns along one contiguous eighth of
// the tiles (persist_logical), so with a batch that is a multiple of 8 each
// XCD owns whole batch entries and its L2 fetches their A and B once.
//
// Host: M % 256 == 0, N % 128 == 0, K == 32 * NK, 16-byte aligned rows,
// gridDim.x <= total tiles.
#pragma once
#include <utility>

#include "device_common.hpp"
#include "gemm_pipelined.hpp"

namespace bpt {

// The logical tile (batch entry major, then the grouped walk inside it) that
// workgroup wg of `grid` computes on its it-th turn, or -1 when it has none.
// Workgroups go to the XCDs round-robin (wg % 8).  When grid is a multiple
// of 8, XCD x owns logical tiles [x*E, (x+1)*E) with E = ceil(total / 8),
// taken by its grid/8 workgroups in turn, so the tiles it holds at any time
// are consecutive in the walk and, with 8 | batch, all of its tiles belong
// to batch entries no other XCD reads.  Otherwise: tile wg + it*grid.
__device__ inline int persist_logical(int wg, int grid, int it, int total) {
    if ((grid & 7) == 0) {
        const int per_xcd = (total + 7) >> 3;
        const int hi = min(total, ((wg & 7) + 1) * per_xcd);
        const int L = (wg & 7) * per_xcd + (wg >> 3) + it * (grid >> 3);
        return L < hi ? L : -1;
    }
    const int L = wg + it * grid;
    return L < total ? L : -1;
}

// How many turns workgroup wg has: the its with persist_logical >= 0.
__device__ inline int persist_turns(int wg, int grid, int total) {
    int first, end, step;
    if ((grid & 7) == 0) {
        const int per_xcd = (total + 7) >> 3;
        first = (wg & 7) * per_xcd + (wg >> 3);
        end = min(total, ((wg & 7) + 1) * per_xcd);
        step = grid >> 3;
    } else {
        first = wg;
        end = total;
        step = grid;
    }
    return first < end ? (end - first + step - 1) / step : 0;
}

template <typename T, typename OutT, int NK>
__global__ __launch_bounds__(256, 1) void gemm_persist_kernel(GemmArgs args, int total) {
    constexpr int BM = 256, BN = 128, BK = 32, STAGES = 4;
    typedef PipelinedGemm<T, BM, BN, BK, STAGES, 2, 2, OutT, false> G;
    typedef typename G::frag_t frag_t;
    static_assert(sizeof(OutT) == 2, "16-bit C: ring and staged tile fill the LDS");
    static_assert(NK % STAGES == 0, "whole rings per tile");
    static_assert(G::KS == 2, "one pending slice per group");
    constexpr int MB = G::MB, NB = G::NB, LPS = G::LPS, DS = G::DSLICE;
    // staging: each wave's 128 x 64 tile as 128 rows of 128 bytes; 16-byte
    // chunk q of row r sits at chunk q ^ ((r >> 1) & 7), and rows with bit
    // 4 set swap the two 8-byte halves of each chunk.  Then the 32 lanes of
    // an 8-byte write (32 rows, one half chunk) and the 16 lanes of a
    // 16-byte read (two whole rows) each cover the 64 banks once.
    constexpr int STG_WAVE = G::TM * G::TN * 2;
    constexpr int STG_BASE = STAGES * G::STAGE_BYTES;
    constexpr int LDS_BYTES = STG_BASE + 4 * STG_WAVE;
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
    static_assert(G::TN * 2 == 128, "staging rows of 8 chunks");
    __shared__ __attribute__((aligned(1024))) char lds_raw[LDS_BYTES];
    BPT_LDS char* lds = (BPT_LDS char*)lds_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / 2;
    const int wn = wave % 2;
    const int lda = args.lda, ldb = args.ldb, ldc = args.ldc, K = args.K;
    const int per = args.tiles_m * args.tiles_n;
    const int wg = blockIdx.x, grid = gridDim.x;
    const int turns = persist_turns(wg, grid, total);
    if (turns == 0) return;                // host: grid <= total; uniform

    // copy offsets relative to the tile's corner (the descriptors start there)
    uint32_t voffA[G::A_INST_W];
#pragma unroll
    for (int i = 0; i < G::A_INST_W; ++i) {
        const int row = (wave * G::A_INST_W + i) * G::A_ROWS_PER_INST + lane / G::A_CHUNKS;
        const int chunk = (lane % G::A_CHUNKS) ^ swz_a<BK>(row);
        voffA[i] = (uint32_t)((row * lda + chunk * 8) * 2);
    }
    uint32_t voffB[G::B_INST_W];
#pragma unroll
    for (int i = 0; i < G::B_INST_W; ++i) {
        const int row = (wave * G::B_INST_W + i) * G::B_ROWS_PER_INST + lane / G::B_CHUNKS;
        const int chunk = (lane % G::B_CHUNKS) ^ swz_b(row);
        voffB[i] = (uint32_t)((row * ldb + chunk * 8) * 2);
    }
    const uint32_t a_step = BK * 2;
    const uint32_t b_step = (uint32_t)BK * ldb * 2;
    uint32_t rdA[G::KS];
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
        const int row = wm * G::TM + (lane % 32);
        const int chunk = (ks * 2 + lane / 32) ^ swz_a<BK>(row);
        rdA[ks] = (uint32_t)((row * BK + chunk * 8) * 2);
    }
    uint32_t rdB[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int g = lane / 16, j = lane % 16;
        const int krow = 8 * (g / 2) + j / 4;
        const int col = wn * G::TN + nb * 32 + 16 * (g % 2) + 4 * (j % 4);
        const int chunk = (col / 8) ^ swz_b(krow);
        rdB[nb] = (uint32_t)(G::A_STAGE * 2 + krow * BN * 2 + chunk * 16 + (col % 8) * 2);
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));

    // the batch entry and corner of logical tile L.  The divisions run on a
    // VGPR copy of L (every lane the same) and only the results come back
    // to SGPRs: their temporaries would otherwise take the SGPRs that hold
    // the two tiles' descriptors across the loop, and spill.
    auto corner = [&](int L, int& batch, int& m0, int& n0) __attribute__((always_inline)) {
        int Lv;
        asm volatile("v_mov_b32 %0, %1" : "=v"(Lv) : "s"(L));
        const int bv = Lv / per;
        int tm, tn;
        group_walk(Lv - bv * per, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
        batch = __builtin_amdgcn_readfirstlane(bv);
        m0 = __builtin_amdgcn_readfirstlane(tm) * BM;
        n0 = __builtin_amdgcn_readfirstlane(tn) * BN;
    };
    // tile number `it` of this workgroup: descriptors starting at its corner
    // (no records past the last tile) and this wave's corner of its C
    struct Tile {
        int4_t ra, rb;
        OutT* c;
    };
    auto tile_at = [&](int it) __attribute__((always_inline)) {
        Tile t;
        const int L = persist_logical(wg, grid, it, total);
        if (L >= 0) {
            int batch, m0, n0;
            corner(L, batch, m0, n0);
            const T* a0 = static_cast<const T*>(args.A) + batch * args.strideA + (long long)m0 * lda;
            const T* b0 = static_cast<const T*>(args.B) + batch * args.strideB + n0;
            t.ra = make_rsrc(a0, (uint32_t)(((BM - 1) * (long long)lda + K) * 2));
            t.rb = make_rsrc(b0, (uint32_t)(((K - 1) * (long long)ldb + BN) * 2));
            t.c = static_cast<OutT*>(args.C) + batch * args.strideC + (long long)(m0 + wm * G::TM) * ldc + n0 +
                  wn * G::TN;
        } else {
            t.ra = t.rb = make_rsrc(args.A, 0u);
            t.c = nullptr;
        }
        return t;
    };

    // copy i (A copies first) of the group of K-tile kt of tile t, into
    // stage kt % STAGES
    // (the LDS base and the B row step pass through an empty asm so that the
    // compiler recomputes each copy's destination and k offset with one
    // scalar op instead of holding all 4 stages x 6 copies x 8 K-tiles of
    // them in SGPRs across the tile loop, which spilled)
    auto dma_one = [&](const Tile& t, int i, int kt) __attribute__((always_inline)) {
        uint32_t l0 = lds0, bstep = b_step;
        asm volatile("" : "+s"(l0), "+s"(bstep));
        const uint32_t sbase = l0 + (kt % STAGES) * G::STAGE_BYTES;
        if (i < G::A_INST_W)
            dma16(t.ra, sbase + (wave * G::A_INST_W + i) * 1024, voffA[i], kt * a_step);
        else
            dma16(t.rb, sbase + G::A_STAGE * 2 + (wave * G::B_INST_W + (i - G::A_INST_W)) * 1024,
                  voffB[i - G::A_INST_W], kt * bstep);
    };

    float16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[i][j] = float16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    typedef OutT out4_t __attribute__((ext_vector_type(4)));
    BPT_LDS char* stg = lds + STG_BASE + wave * STG_WAVE;
    auto stg_chunk = [](int r, int q) __attribute__((always_inline)) { return r * 128 + ((q ^ ((r >> 1) & 7)) * 16); };

    frag_t fa[2][MB];
    short4_t fbl[2][NB], fbh[2][NB];
    auto read_piece = [&](int st, int ks, int p, int s) __attribute__((always_inline)) {
        BPT_LDS char* sbase = lds + st * G::STAGE_BYTES;
        if (p < MB) {
            fa[s][p] = *(BPT_LDS frag_t*)(sbase + rdA[ks] + p * 32 * BK * 2);
        } else {
            const int nb = (p - MB) / 2, h = (p - MB) % 2;
            BPT_LDS short4_t* q = (BPT_LDS short4_t*)(sbase + rdB[nb] + ks * 16 * BN * 2 + h * 4 * BN * 2);
            if (h == 0) fbl[s][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
            else fbh[s][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
        }
    };

    // One k-step on fragment set s, with the reads of k-step rks of stage
    // rst into set s^1 and copies [d0, d0 + DS) of the group of K-tile dkt of
    // tile dt.  FIRST: the tile's first k-step -- each accumulator block is
    // converted into the staging area just before its first product, which
    // starts from zero.
    auto kstep = [&]<bool FIRST>(int s, int rst, int rks, const Tile& dt, int d0, int dkt) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < G::NMMA; ++q) {
#pragma unroll
            for (int r = 0; r < G::RPM; ++r)
                if (q * G::RPM + r < G::NREAD) read_piece(rst, rks, q * G::RPM + r, s ^ 1);
            const int mb = q / NB, nb = q % NB;
            const frag_t b =
                __builtin_bit_cast(frag_t, __builtin_shufflevector(fbl[s][nb], fbh[s][nb], 0, 1, 2, 3, 4, 5, 6, 7));
            if constexpr (FIRST) {
                // lane l: row mb*32 + l%32, columns nb*32 + 8g + 4(l/32) .. +3
                const int r = mb * 32 + (lane % 32);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    out4_t v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = cvt_out<OutT>(acc[mb][nb][4 * g + e]);
                    *(BPT_LDS out4_t*)(stg + stg_chunk(r, nb * 4 + g) + ((lane / 32) ^ ((r >> 4) & 1)) * 8) = v;
                }
                acc[mb][nb] = Mfma<T>::mma32(b, fa[s][mb], float16_t{});
            } else {
                acc[mb][nb] = Mfma<T>::mma32(b, fa[s][mb], acc[mb][nb]);
            }
#pragma unroll
            for (int r = 0; r < G::DPQ; ++r) {
                const int slot = q * G::DPQ + r - G::DOFF;
                if (slot >= 0 && slot % G::DEVERY == 0 && slot / G::DEVERY < DS)
                    dma_one(dt, d0 + slot / G::DEVERY, dkt);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // The staged previous tile goes out in SLICES slices, one in each of the
    // next tile's first SLICES K-tiles: slice sl is rows 8 SPS sl .. +8 SPS-1
    // of the wave tile, 8 rows of 8 chunks per instruction.
    constexpr int SLICES = NK < 8 ? NK : 8;
    constexpr int SPS = G::TM / 8 / SLICES;            // store instructions per slice
    int4_t sv[SPS];
    auto load_slice = [&](int sl) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < SPS; ++h) {
            const int r = (sl * SPS + h) * 8 + lane / 8;
            int4_t v = *(BPT_LDS int4_t*)(stg + stg_chunk(r, lane % 8));
            sv[h] = (r & 16) ? int4_t{v[2], v[3], v[0], v[1]} : v;     // undo the half swap
        }
    };
    auto store_slice = [&](int sl, OutT* pc) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < SPS; ++h) {
            const int r = (sl * SPS + h) * 8 + lane / 8;
            OutT* dst = pc + (long long)r * ldc + (lane % 8) * 8;
            __builtin_nontemporal_store(sv[h], (int4_t*)dst);
        }
    };

    // ---- prologue: groups of K-tiles 0 .. 2 and slice 0 of group 3 ----------
    // (every K-tile's first k-step issues the other slice of group kt+3)
    Tile cur = tile_at(0);
    Tile nxt = tile_at(1);
    OutT* prv = cur.c;                     // this wave's C of the tile in the staging area
#pragma unroll
    for (int g = 0; g < STAGES - 1; ++g)
#pragma unroll
        for (int i = 0; i < LPS; ++i) dma_one(cur, i, g);
#pragma unroll
    for (int i = 0; i < DS; ++i) dma_one(cur, i, STAGES - 1);
    publish<LPS * (STAGES - 2) + DS>();    // group 0 landed for every wave
#pragma unroll
    for (int p = 0; p < G::NREAD; ++p) read_piece(0, 0, p, 0);

    // K-tile KT of the current tile: k-step 0 finishes the group of K-tile
    // KT+3, publish(KT+1), k-step 1 starts the group of K-tile KT+4 (both
    // possibly of the next tile) in the stage KT just left
    auto ktile = [&]<int KT>(int it) __attribute__((always_inline)) {
        constexpr int PK = KT + STAGES - 1, WK = KT + STAGES;
        const Tile& pt = PK < NK ? cur : nxt;
        const Tile& wt = WK < NK ? cur : nxt;
        kstep.template operator()<KT == 0>(0, KT % STAGES, 1, pt, DS, PK % NK);
        if constexpr (KT == 0) wave_lds_handoff();             // rows staged by other lanes are read below
        if constexpr (KT < SLICES) load_slice(KT);             // waited for by the publish
        publish<LPS * (STAGES - 2)>();
        if constexpr (KT < SLICES) {
            if (it > 0) store_slice(KT, prv);
        }
        kstep.template operator()<false>(1, (KT + 1) % STAGES, 0, wt, 0, WK % NK);
    };

    for (int it = 0; it < turns; ++it) {
        [&]<int... KT>(std::integer_sequence<int, KT...>) {
            (ktile.template operator()<KT>(it), ...);
        }(std::make_integer_sequence<int, NK>{});
        prv = cur.c;
        cur = nxt;
        nxt = tile_at(it + 2);
    }
    // the copies past the last tile read zeros; the epilogue's publish<0>
    // lets them land before it reuses LDS, then stores the last tile
    int lb, lm0, ln0;
    corner(persist_logical(wg, grid, turns - 1, total), lb, lm0, ln0);
    pipelined_epilogue<G, OutT>(args, acc, lds, lane, wave, wm, wn, lm0, ln0, lb);
}

// ---- the same kernel with A staged in K-tile pairs ---------------------------
//
// A 32-wide K-tile of A is a 64-byte piece of each of 256 rows, half a
// 128-byte line, and a copy instruction touches 16 such half lines.  Each
// instruction's cost goes with the lines it touches (a probe writing 2 GiB
// measured 5.6 TB/s with whole lines per instruction and 1.2 TB/s with
// 32-byte pieces of 32 rows), and the copies of this kernel's K-tiles plus
// its C stores keep the CU's vector memory path busy.  Here A is copied two
// K-tiles at a time, 8 rows x 128 bytes per instruction, as in the A-pair
// pipelined kernel.
//
// LDS: two A pair stages (256 rows x 64 k, 32 KiB each), four B stages
// (32 x 128, 8 KiB each) and the 64 KiB staging area: 160 KiB.  Global
// K-tile j reads B stage j % 4 and A pair stage (j / 2) % 2.  Copies go out
// in windows: the window of K-tile i holds B(i+4) and, for odd i, A pair
// (i+3)/2 (two copies, or ten), half of it issued in k-step 1 of K-tile i
// (right after publish(i+1)) and half in k-step 0 of K-tile i+1.  A pair
// (i+3)/2 refills the stage of pair (i-1)/2 = K-tiles i-1 and i, whose
// reads all retired before publish(i+1); B(i+4) refills K-tile i's B
// stage.  publish(j+1) needs B(j+1) (window j-3) and, for even j+1, A pair
// (j+1)/2 (window j-2); only window j-1 is younger for odd j (2 copies), and
// windows j-2 and j-1 (2 + 10) for even j.  NK is even, so the parity of j
// is that of the K-tile inside the tile and the waits are compile-time.
template <typename T, typename OutT, int NK>
__global__ __launch_bounds__(256, 1) void gemm_persist_apair_kernel(GemmArgs args, int total) {
    constexpr int BM = 256, BN = 128, BK = 32, BSTAGES = 4;
    typedef PipelinedGemm<T, BM, BN, BK, BSTAGES, 2, 2, OutT, false> G;
    typedef typename G::frag_t frag_t;
    static_assert(sizeof(OutT) == 2, "16-bit C: ring and staged tile fill the LDS");
    static_assert(NK % 4 == 0, "whole B rings and A pairs per tile");
    static_assert(G::KS == 2, "two k-steps per K-tile");
    constexpr int MB = G::MB, NB = G::NB;
    constexpr int AP_BYTES = BM * 2 * BK * 2;            // one A pair stage
    constexpr int B_BYTES = BK * BN * 2;                 // one B stage
    constexpr int B_BASE = 2 * AP_BYTES;
    constexpr int A_INST = AP_BYTES / 1024 / 4;          // pair copies per wave (8)
    constexpr int B_INST = B_BYTES / 1024 / 4;           // B copies per wave (2)
    constexpr int STG_WAVE = G::TM * G::TN * 2;
    constexpr int STG_BASE = B_BASE + BSTAGES * B_BYTES;
    constexpr int LDS_BYTES = STG_BASE + 4 * STG_WAVE;
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
    static_assert(G::TN * 2 == 128, "staging rows of 8 chunks");
    // window sizes and the wait counts derived above
    constexpr auto wsize = [](int i) constexpr { return (i & 1) ? B_INST + A_INST : B_INST; };
    constexpr int VM_EVEN = wsize(0) + wsize(1);         // publish(j+1), j even
    constexpr int VM_ODD = wsize(0);                     // publish(j+1), j odd
    static_assert(VM_EVEN + wsize(1) < 64, "vmcnt is 6 bits");
    __shared__ __attribute__((aligned(1024))) char lds_raw[LDS_BYTES];
    BPT_LDS char* lds = (BPT_LDS char*)lds_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / 2;
    const int wn = wave % 2;
    const int lda = args.lda, ldb = args.ldb, ldc = args.ldc, K = args.K;
    const int per = args.tiles_m * args.tiles_n;
    const int wg = blockIdx.x, grid = gridDim.x;
    const int turns = persist_turns(wg, grid, total);
    if (turns == 0) return;                // host: grid <= total; uniform

    // pair copies: 8 rows of 8 chunks (whole 128-byte lines) per instruction
    uint32_t voffA[A_INST];
#pragma unroll
    for (int i = 0; i < A_INST; ++i) {
        const int row = (wave * A_INST + i) * 8 + lane / 8;
        const int chunk = (lane % 8) ^ swz_a<64>(row);
        voffA[i] = (uint32_t)((row * lda + chunk * 8) * 2);
    }
    uint32_t voffB[B_INST];
#pragma unroll
    for (int i = 0; i < B_INST; ++i) {
        const int row = (wave * B_INST + i) * G::B_ROWS_PER_INST + lane / G::B_CHUNKS;
        const int chunk = (lane % G::B_CHUNKS) ^ swz_b(row);
        voffB[i] = (uint32_t)((row * ldb + chunk * 8) * 2);
    }
    const uint32_t pair_step = 2 * BK * 2;
    const uint32_t b_step = (uint32_t)BK * ldb * 2;
    // A block mb of K-tile parity t, k-step ks: row wm*TM + mb*32 + l%32,
    // logical chunk 4t + 2ks + l/32 of the 128-byte row, swizzled
    uint32_t rdA[2][G::KS];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            const int row = wm * G::TM + (lane % 32);
            const int chunk = (4 * t + 2 * ks + lane / 32) ^ swz_a<64>(row);
            rdA[t][ks] = (uint32_t)(row * 128 + chunk * 16);
        }
    uint32_t rdB[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int g = lane / 16, j = lane % 16;
        const int krow = 8 * (g / 2) + j / 4;
        const int col = wn * G::TN + nb * 32 + 16 * (g % 2) + 4 * (j % 4);
        const int chunk = (col / 8) ^ swz_b(krow);
        rdB[nb] = (uint32_t)(B_BASE + krow * BN * 2 + chunk * 16 + (col % 8) * 2);
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));

    // the batch entry and corner of logical tile L (divisions on a VGPR copy
    // of L, as in gemm_persist_kernel)
    auto corner = [&](int L, int& batch, int& m0, int& n0) __attribute__((always_inline)) {
        int Lv;
        asm volatile("v_mov_b32 %0, %1" : "=v"(Lv) : "s"(L));
        const int bv = Lv / per;
        int tm, tn;
        group_walk(Lv - bv * per, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
        batch = __builtin_amdgcn_readfirstlane(bv);
        m0 = __builtin_amdgcn_readfirstlane(tm) * BM;
        n0 = __builtin_amdgcn_readfirstlane(tn) * BN;
    };
    struct Tile {
        int4_t ra, rb;
        OutT* c;
    };
    auto tile_at = [&](int it) __attribute__((always_inline)) {
        Tile t;
        const int L = persist_logical(wg, grid, it, total);
        if (L >= 0) {
            int batch, m0, n0;
            corner(L, batch, m0, n0);
            const T* a0 = static_cast<const T*>(args.A) + batch * args.strideA + (long long)m0 * lda;
            const T* b0 = static_cast<const T*>(args.B) + batch * args.strideB + n0;
            t.ra = make_rsrc(a0, (uint32_t)(((BM - 1) * (long long)lda + K) * 2));
            t.rb = make_rsrc(b0, (uint32_t)(((K - 1) * (long long)ldb + BN) * 2));
            t.c = static_cast<OutT*>(args.C) + batch * args.strideC + (long long)(m0 + wm * G::TM) * ldc + n0 +
                  wn * G::TN;
        } else {
            t.ra = t.rb = make_rsrc(args.A, 0u);
            t.c = nullptr;
        }
        return t;
    };

    // copy c of the window of tile-local K-tile i (i = -1 .. NK-1): B copies
    // first, then the A pair copies (odd i).  Its B is K-tile i+4 and its A
    // pair (i+3)/2, both counted from the current tile's start, so those
    // past the tile belong to the next one.
    auto dma_win = [&]<int I>(int c, const Tile& cur, const Tile& nxt) __attribute__((always_inline)) {
        uint32_t l0 = lds0, bstep = b_step;
        asm volatile("" : "+s"(l0), "+s"(bstep));
        if (c < B_INST) {
            constexpr int KB = I + 4;
            const Tile& t = KB < NK ? cur : nxt;
            constexpr int kb = KB % NK;
            dma16(t.rb, l0 + B_BASE + (KB % BSTAGES) * B_BYTES + (wave * B_INST + c) * 1024, voffB[c],
                  kb * bstep);
        } else {
            constexpr int PQ = (I + 3) / 2;
            const Tile& t = 2 * PQ < NK ? cur : nxt;
            constexpr int pq = PQ % (NK / 2);
            const int a = c - B_INST;
            dma16(t.ra, l0 + (PQ % 2) * AP_BYTES + (wave * A_INST + a) * 1024, voffA[a], pq * pair_step);
        }
    };

    float16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[i][j] = float16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    typedef OutT out4_t __attribute__((ext_vector_type(4)));
    BPT_LDS char* stg = lds + STG_BASE + wave * STG_WAVE;
    auto stg_chunk = [](int r, int q) __attribute__((always_inline)) { return r * 128 + ((q ^ ((r >> 1) & 7)) * 16); };

    frag_t fa[2][MB];
    short4_t fbl[2][NB], fbh[2][NB];
    // read p of k-step ks of K-tile KTR (tile-local) into set s
    auto read_piece = [&]<int KTR>(int ks, int p, int s) __attribute__((always_inline)) {
        if (p < MB) {
            fa[s][p] = *(BPT_LDS frag_t*)(lds + ((KTR / 2) % 2) * AP_BYTES + rdA[KTR % 2][ks] + p * 32 * 128);
        } else {
            const int nb = (p - MB) / 2, h = (p - MB) % 2;
            BPT_LDS short4_t* q =
                (BPT_LDS short4_t*)(lds + (KTR % BSTAGES) * B_BYTES + rdB[nb] + ks * 16 * BN * 2 + h * 4 * BN * 2);
            if (h == 0) fbl[s][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
            else fbh[s][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
        }
    };

    // One k-step on fragment set s, with the reads of k-step rks of K-tile
    // KTR into set s^1 and copies [C0, C1) of window WI spread over its
    // MFMAs.  FIRST: the tile's first k-step (C staging, as in
    // gemm_persist_kernel).
    auto kstep = [&]<bool FIRST, int KTR, int WI, int C0, int C1>(int s, int rks, const Tile& cur, const Tile& nxt)
        __attribute__((always_inline)) {
        constexpr int NC = C1 - C0;
#pragma unroll
        for (int q = 0; q < G::NMMA; ++q) {
#pragma unroll
            for (int r = 0; r < G::RPM; ++r)
                if (q * G::RPM + r < G::NREAD) read_piece.template operator()<KTR>(rks, q * G::RPM + r, s ^ 1);
            const int mb = q / NB, nb = q % NB;
            const frag_t b =
                __builtin_bit_cast(frag_t, __builtin_shufflevector(fbl[s][nb], fbh[s][nb], 0, 1, 2, 3, 4, 5, 6, 7));
            if constexpr (FIRST) {
                const int r = mb * 32 + (lane % 32);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    out4_t v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = cvt_out<OutT>(acc[mb][nb][4 * g + e]);
                    *(BPT_LDS out4_t*)(stg + stg_chunk(r, nb * 4 + g) + ((lane / 32) ^ ((r >> 4) & 1)) * 8) = v;
                }
                acc[mb][nb] = Mfma<T>::mma32(b, fa[s][mb], float16_t{});
            } else {
                acc[mb][nb] = Mfma<T>::mma32(b, fa[s][mb], acc[mb][nb]);
            }
            // copies: copy number x of NC right after MFMA (x * NMMA) / NC
            if constexpr (NC > 0) {
#pragma unroll
                for (int x = 0; x < NC; ++x)
                    if ((x * G::NMMA) / NC == q) dma_win.template operator()<WI>(C0 + x, cur, nxt);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    constexpr int SLICES = NK < 8 ? NK : 8;
    constexpr int SPS = G::TM / 8 / SLICES;
    int4_t sv[SPS];
    auto load_slice = [&](int sl) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < SPS; ++h) {
            const int r = (sl * SPS + h) * 8 + lane / 8;
            int4_t v = *(BPT_LDS int4_t*)(stg + stg_chunk(r, lane % 8));
            sv[h] = (r & 16) ? int4_t{v[2], v[3], v[0], v[1]} : v;
        }
    };
    auto store_slice = [&](int sl, OutT* pc) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < SPS; ++h) {
            const int r = (sl * SPS + h) * 8 + lane / 8;
            OutT* dst = pc + (long long)r * ldc + (lane % 8) * 8;
            __builtin_nontemporal_store(sv[h], (int4_t*)dst);
        }
    };

    // ---- prologue: windows -4 .. -2 whole and the first half of window -1
    // (the current tile's B(0 .. 3) and A pairs 0 and 1); k-step 0 of K-tile
    // 0 issues the rest.  Then group 0 (B(0), A pair 0) has landed once the
    // younger copies number at most wsize(-2) + wsize(-1)/2.
    Tile cur = tile_at(0);
    Tile nxt = tile_at(1);
    OutT* prv = cur.c;
    [&]<int... I>(std::integer_sequence<int, I...>) {
        ((
             [&] {
                 constexpr int W = I - 4;
#pragma unroll
                 for (int c = 0; c < (W == -1 ? wsize(W) / 2 : wsize(W)); ++c)
                     dma_win.template operator()<W>(c, cur, nxt);
             }()),
         ...);
    }(std::make_integer_sequence<int, 4>{});
    publish<wsize(-2) + wsize(-1) / 2>();
#pragma unroll
    for (int p = 0; p < G::NREAD; ++p) read_piece.template operator()<0>(0, p, 0);

    // tile-local K-tile KT: k-step 0 (reads of its k-step 1, second half of
    // window KT-1), publish(KT+1), k-step 1 (reads of K-tile KT+1's k-step
    // 0 -- the next tile's first when KT = NK-1 -- first half of window KT)
    auto ktile = [&]<int KT>(int it) __attribute__((always_inline)) {
        constexpr int WP = KT - 1;
        kstep.template operator()<KT == 0, KT, WP, wsize(WP) / 2, wsize(WP)>(0, 1, cur, nxt);
        if constexpr (KT == 0) wave_lds_handoff();
        if constexpr (KT < SLICES) load_slice(KT);
        publish<(KT % 2 == 0) ? VM_EVEN : VM_ODD>();
        if constexpr (KT < SLICES) {
            if (it > 0) store_slice(KT, prv);
        }
        kstep.template operator()<false, (KT + 1) % NK, KT, 0, wsize(KT) / 2>(1, 0, cur, nxt);
    };

    for (int it = 0; it < turns; ++it) {
        [&]<int... KT>(std::integer_sequence<int, KT...>) {
            (ktile.template operator()<KT>(it), ...);
        }(std::make_integer_sequence<int, NK>{});
        prv = cur.c;
        cur = nxt;
        nxt = tile_at(it + 2);
    }
    int lb, lm0, ln0;
    corner(persist_logical(wg, grid, turns - 1, total), lb, lm0, ln0);
    pipelined_epilogue<G, OutT>(args, acc, lds, lane, wave, wm, wn, lm0, ln0, lb);
}

}  // namespace bpt
