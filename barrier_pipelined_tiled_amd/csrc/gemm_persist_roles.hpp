// gemm_persist_roles.hpp -- the persistent short-K kernel with wave roles
// (C = A * B, B row-major K x N, 16-bit C, K = 128 or 256).
//
// The other persistent kernels have every wave copy, multiply and store.
// Copies and stores then share each wave's vmcnt counter, and a publish,
// which must know that this wave's copies of a stage have landed, may leave
// in flight only as many operations as there are younger copies: every C
// store still unacknowledged takes one of those places ("Xe2 Nbarrier
// Pipelining", Producer-Consumer Pattern: give the loads to waves of their
// own).  Here a workgroup has 8 waves, two per SIMD:
//
// * waves 0-3 multiply.  The tile is 128 x 256; wave w owns its columns
//   64w .. 64w+63 over all 128 rows (4 x 2 blocks of 32 x 32, 128 fp32
//   accumulators).  They issue no global memory operation at all, so they
//   never wait on vmcnt: they read the A panel and the B stages from LDS and
//   hand the previous tile's C to the store waves through LDS.
// * waves 4-5 copy: each row block's A panel (128 x K, kept in LDS while
//   the workgroup walks that row's column tiles) and the B K-tiles (32 x 256,
//   16 KiB) through a 4-stage ring.  Their vmcnt counts copies only, so a
//   publish waits for exactly the stage it needs.
// * waves 6-7 store.  Their vmcnt counts stores only, and they never wait
//   on it: C leaves at the rate the memory system takes it.
//
// Step g (K-tile g of the workgroup's walk) starts with publish(g): the
// copy waves wait until K-tile g's copies have landed (vmcnt), the other
// waves until their LDS reads and writes are done (lgkmcnt), then one
// s_barrier.  After it the copy waves issue K-tile g+3 into the stage
// K-tile g-1 left; the compute waves run k-step 1 of K-tile g-1 (reading
// K-tile g's first fragments) and k-step 0 of K-tile g (reading its
// second), and write RPK = 128/NK rows of the previous tile's C (packed to
// 16 bits when this tile's first products overwrite the accumulators) into
// C slot g % 2; the store waves read slot (g-1) % 2, written during step
// g-1, and store its rows as whole 128-byte lines.  A slot is rewritten two
// steps after it was filled, after the store waves' reads of it retired.
//
// A new row block: its A panel replaces the old one a pair stage (64 k) at
// a time while the old row block's last tile runs, each pair as soon as that
// tile has read it for the last time; the ordinary publish waits cover the
// new pairs (see the copy loop), so no wave waits for a whole panel.
//
// The last tile's C goes out in NK more steps without products, and one
// more step stores the last slot, so every wave executes the same
// (turns + 1) * NK + 1 publishes.
//
// LDS (K = 256): panel 64 KiB (4 pair stages of 128 rows x 64 k, as the
// A-pair kernel lays them out), B ring 64 KiB, two C slots of 8 KiB; 144 KiB.
// K = 128: 32 + 64 + 32 KiB.
//
// Walk: groups of one row block and all its column tiles; group r of
// workgroup wg is persist_logical(wg, grid, r, ngroups), so at any time the
// 32 workgroups of an XCD hold 32 consecutive row blocks (one batch entry
// of 4096 rows), whose B the XCD's L2 then holds once.  Each workgroup walks
// the column tiles starting at its slot in the XCD (wg >> 3): walked in the
// same order, all 32 first touched each new B column tile together and
// waited out its HBM latency one tile after another (0.98 against 0.68 ms
// on 64 x 4096^2 x 256 with B not in the caches).
//
// Host: M % 128 == 0, N % 256 == 0, K == 32 * NK, 16-byte aligned rows and
// bases, gridDim.x % 8 == 0 and <= ngroups, gn == N / 256.
#pragma once
#include <utility>

#include "device_common.hpp"
#include "gemm_persist.hpp"

namespace bpt {

template <typename T, typename OutT, int NK>
__global__ __launch_bounds__(512, 1) void gemm_persist_roles_kernel(GemmArgs args, int ngroups, int gn) {
    constexpr int BM = 128, BN = 256, BK = 32, BSTAGES = 4;
    constexpr int TN = 64, MB = BM / 32, NB = TN / 32;   // compute wave: 128 x 64, 4 x 2 blocks
    constexpr int NMMA = MB * NB;                        // MFMAs per k-step
    constexpr int AP_BYTES = BM * 2 * BK * 2;            // a pair stage: 128 rows x 64 k
    constexpr int PANEL = (NK / 2) * AP_BYTES;
    constexpr int B_BYTES = BK * BN * 2;                 // a B K-tile: 32 x 256
    constexpr int B_BASE = PANEL;
    constexpr int RPK = BM / NK;                         // rows of C each compute wave sends per step
    constexpr int WSLOT = RPK * TN * 2;                  // its part of a slot
    constexpr int SLOT = 4 * WSLOT;
    constexpr int STG_BASE = B_BASE + BSTAGES * B_BYTES;
    constexpr int LDS_BYTES = STG_BASE + 2 * SLOT;
    constexpr int WIN = B_BYTES / 1024 / 2;              // copies per copy wave per K-tile
    constexpr int PAIR_INST = AP_BYTES / 1024;           // copies per pair stage
    constexpr int VM = (BSTAGES - 2) * WIN;              // younger copies at a publish
    constexpr int RD = WSLOT / 1024;                     // 1 KiB reads per wave part of a slot
    static_assert(NK == 4 || NK == 8, "K = 128 or 256");
    static_assert(sizeof(OutT) == 2, "16-bit C: slots of 128-byte rows");
    static_assert(RPK == 16 || RPK == 32, "half or whole 32-row blocks per step");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
    static_assert(VM + WIN < 64 && 2 * PAIR_INST + 3 * WIN < 64, "vmcnt");
    typedef typename Mfma<T>::frag_t frag_t;
    __shared__ __attribute__((aligned(1024))) char lds_raw[LDS_BYTES];
    BPT_LDS char* lds = (BPT_LDS char*)lds_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wg = blockIdx.x, grid = gridDim.x;
    const int turns = persist_turns(wg, grid, ngroups) * gn;     // tiles of this workgroup
    if (turns == 0) return;                // host: grid <= ngroups; uniform
    const int t_mma = turns * NK;          // steps with products
    const int ksteps_total = t_mma + NK;   // + the steps that send the last tile
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));

    auto publish_lgkm = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // batch entry and corner of tile number `it` of this workgroup (the
    // divisions run on VGPR copies, as in the other persistent kernels)
    auto corner = [&](int it, int& batch, int& m0, int& n0) __attribute__((always_inline)) {
        int itv;
        asm volatile("v_mov_b32 %0, %1" : "=v"(itv) : "s"(it));
        const int rv = itv / gn;
        const int r = __builtin_amdgcn_readfirstlane(rv);
        // column tiles in a rotated order, starting at the workgroup's slot
        // in its XCD: the XCD's workgroups then first touch different B
        // column tiles at the same time instead of each new one together
        int ctv;
        asm volatile("v_mov_b32 %0, %1" : "=v"(ctv) : "s"(it - r * gn + (wg >> 3)));
        const int ct = __builtin_amdgcn_readfirstlane(ctv % gn);
        const int gi = persist_logical(wg, grid, r, ngroups);
        int gv;
        asm volatile("v_mov_b32 %0, %1" : "=v"(gv) : "s"(gi));
        const int bv = gv / args.tiles_m;
        batch = __builtin_amdgcn_readfirstlane(bv);
        m0 = (gi - batch * args.tiles_m) * BM;
        n0 = ct * BN;
    };

    if (wave >= 4 && wave < 6) {
        // ---- copy waves ---------------------------------------------------
        const int cw = wave - 4;
        const int ldb = args.ldb, lda = args.lda, K = args.K;
        // B: copy c = cw * WIN + i of a K-tile holds its rows 2c, 2c+1; lane p
        // lands in 16-byte slot p%32 of row 2c + p/32 and brings the logical
        // chunk swizzled there (the pipelined kernel's swz_b)
        uint32_t voffB[WIN];
#pragma unroll
        for (int i = 0; i < WIN; ++i) {
            const int row = 2 * (cw * WIN + i) + lane / 32;
            const int chunk = (lane % 32) ^ swz_b(row);
            voffB[i] = (uint32_t)((row * ldb + chunk * 8) * 2);
        }
        const uint32_t b_step = (uint32_t)BK * ldb * 2;
        // K-tile g into stage g % 4; past the last tile through a descriptor
        // with no records (lands zeros, no traffic), so every publish waits
        // with the same count.  The descriptor is built once per tile (the
        // corner's divisions cost a few hundred cycles).
        int w_it = -1;
        int4_t rs = make_rsrc(args.B, 0u);
        auto window = [&](int g) __attribute__((always_inline)) {
            const int it = g / NK, k = g - it * NK;
            if (it != w_it) {
                w_it = it;
                if (it < turns) {
                    int batch, m0, n0;
                    corner(it, batch, m0, n0);
                    const T* b0 = static_cast<const T*>(args.B) + batch * args.strideB + n0;
                    rs = make_rsrc(b0, (uint32_t)(((K - 1) * (long long)ldb + BN) * 2));
                } else {
                    rs = make_rsrc(args.B, 0u);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) rs[q] = __builtin_amdgcn_readfirstlane(rs[q]);
            }
            const uint32_t st = lds0 + B_BASE + (g & (BSTAGES - 1)) * B_BYTES + cw * WIN * 1024;
#pragma unroll
            for (int i = 0; i < WIN; ++i) dma16(rs, st + i * 1024, voffB[i], (uint32_t)k * b_step);
        };
        // pair stage p of tile it's A panel: k 64p .. 64p+63 of the row
        // block's 128 rows, 8 rows of 128 bytes per copy, this wave's half
        auto pair = [&](int it, int p) __attribute__((always_inline)) {
            int batch, m0, n0;
            corner(it, batch, m0, n0);
            const T* a0 = static_cast<const T*>(args.A) + batch * args.strideA + (long long)m0 * lda;
            int4_t ra = make_rsrc(a0, (uint32_t)(((BM - 1) * (long long)lda + K) * 2));
#pragma unroll
            for (int q = 0; q < 4; ++q) ra[q] = __builtin_amdgcn_readfirstlane(ra[q]);
#pragma unroll
            for (int i = 0; i < PAIR_INST / 2; ++i) {
                const int ii = cw * (PAIR_INST / 2) + i;
                const int row = ii * 8 + lane / 8;
                const int chunk = (lane % 8) ^ swz_a<64>(row);
                dma16(ra, lds0 + p * AP_BYTES + ii * 1024, (uint32_t)((row * lda + chunk * 8) * 2),
                      (uint32_t)(p * 2 * BK * 2));
            }
        };
#pragma unroll
        for (int p = 0; p < NK / 2; ++p) pair(0, p);
#pragma unroll
        for (int g = 0; g < BSTAGES - 1; ++g) window(g);
        for (int g = 0; g <= ksteps_total; ++g) {
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
            // The next row block's panel, one pair stage at a time as the old
            // one's free up: pair p is last read in K-tiles 2p, 2p+1 of a
            // row block's last tile, so after publish(2p+2) it is free (p <
            // NK/2-1 in that tile, the last pair after publish(0) of the next
            // tile).  It is first read after publish(2p) of the next tile,
            // which waits until at most two windows of copies are in flight;
            // at least two were issued after the pair, and copies land in
            // order, so the pair has landed by then: no wait of its own.
            const int it = g / NK, kt = g - it * NK;
            if (it + 1 < turns && (it + 1) % gn == 0 && kt >= 2 && kt % 2 == 0) pair(it + 1, kt / 2 - 1);
            if (it < turns && it > 0 && it % gn == 0 && kt == 0) pair(it, NK / 2 - 1);
            window(g + BSTAGES - 1);
        }
        wait_vm<0>();                      // no copy writes LDS after the workgroup ends
        return;
    }

    if (wave >= 6) {
        // ---- store waves --------------------------------------------------
        const int sw = wave - 6;
        const int ldc = args.ldc;
        auto stg_chunk = [](int r, int q) __attribute__((always_inline)) {
            return r * 128 + ((q ^ ((r >> 1) & 7)) * 16);
        };
        // the tile whose rows are being stored, its C corner found once
        int c_it = -1;
        OutT* ctile = nullptr;
        for (int g = 0; g <= ksteps_total; ++g) {
            publish_lgkm();
            // slot (g-1) % 2 holds rows ((g-1) % NK) * RPK .. of tile (g-1)/NK - 1
            if (g >= NK + 1) {
                const int src = g - 1;
                const int it = src / NK - 1, k = src - (src / NK) * NK;
                const BPT_LDS char* s = lds + STG_BASE + (src & 1) * SLOT;
                int4_t v[2 * RD];
#pragma unroll
                for (int x = 0; x < 2 * RD; ++x) {
                    const int part = 2 * sw + x / RD, h = x % RD;
                    const int r2 = h * 8 + lane / 8;
                    const int4_t u = *(const BPT_LDS int4_t*)(s + part * WSLOT + stg_chunk(r2, lane % 8));
                    const bool swapped = (((RPK == 32 ? r2 >> 4 : lane % 8) ^ r2) & 1) != 0;
                    v[x] = swapped ? int4_t{u[2], u[3], u[0], u[1]} : u;
                }
                if (it != c_it) {
                    c_it = it;
                    int batch, m0, n0;
                    corner(it, batch, m0, n0);
                    ctile = static_cast<OutT*>(args.C) + batch * args.strideC + (long long)m0 * ldc + n0;
                }
                OutT* c0 = ctile + (long long)(k * RPK) * ldc;
#pragma unroll
                for (int x = 0; x < 2 * RD; ++x) {
                    const int part = 2 * sw + x / RD, h = x % RD;
                    const int r2 = h * 8 + lane / 8;
                    __builtin_nontemporal_store(v[x], (int4_t*)(c0 + (long long)r2 * ldc + part * TN + (lane % 8) * 8));
                }
            }
        }
        return;
    }

    // ---- compute waves --------------------------------------------------------
    const int wn = wave;                   // columns 64 wn .. 64 wn + 63
    // A block mb of K-tile parity t, k-step ks: row mb*32 + l%32, logical
    // chunk 4t + 2ks + l/32 of the 128-byte pair row, swizzled as copied
    uint32_t rdA[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int row = lane % 32;
            const int chunk = (4 * t + 2 * ks + lane / 32) ^ swz_a<64>(row);
            rdA[t][ks] = (uint32_t)(row * 128 + chunk * 16);
        }
    // B block nb, transposing reads: 16-lane group g, lane j reads k row
    // 8(g/2) + j/4 (+4 for the upper half, +16 per k-step) at column
    // 64 wn + 32 nb + 16(g%2) + 4(j%4)
    uint32_t rdB[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int g = lane / 16, j = lane % 16;
        const int krow = 8 * (g / 2) + j / 4;
        const int col = wn * TN + nb * 32 + 16 * (g % 2) + 4 * (j % 4);
        const int chunk = (col / 8) ^ swz_b(krow);
        rdB[nb] = (uint32_t)(B_BASE + krow * BN * 2 + chunk * 16 + (col % 8) * 2);
    }

    float16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
            acc[i][j] = float16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    typedef OutT out4_t __attribute__((ext_vector_type(4)));
    out4_t held[MB][NB][4];                              // the previous tile's C, 16-bit
    frag_t fa[2][MB];
    short4_t fbl[2][NB], fbh[2][NB];

    // read p of k-step ks of K-tile g (tile-local index KT) into set s
    auto read_piece = [&]<int KT>(int g, int ks, int p, int s) __attribute__((always_inline)) {
        if (p < MB) {
            fa[s][p] = *(BPT_LDS frag_t*)(lds + (KT / 2) * AP_BYTES + rdA[KT % 2][ks] + p * 32 * 128);
        } else {
            const int nb = (p - MB) / 2, h = (p - MB) % 2;
            BPT_LDS short4_t* q = (BPT_LDS short4_t*)(lds + (g & (BSTAGES - 1)) * B_BYTES + rdB[nb] +
                                                      ks * 16 * BN * 2 + h * 4 * BN * 2);
            if (h == 0) fbl[s][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
            else fbh[s][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
        }
    };
    static_assert(MB + 2 * NB == NMMA, "one fragment read per MFMA");

    // The held rows of step KS (RPK rows from KS*RPK on) into this wave's
    // part of slot `sb`; the order of writes is the A-resident kernel's
    // (gemm_persist_ares.hpp): lane l holds row PM*32 + l%32, 16-byte chunk
    // nb*4 + g of the 128-byte row, 8-byte half l/32; slot row r goes to
    // chunk q ^ ((r >> 1) & 7), and with RPK = 16 a v_permlane16_swap of
    // chunks 2p and 2p+1 first puts the step's 16 rows into one register of
    // all 64 lanes.  The two 8-byte halves of a chunk trade places on odd
    // rows: an 8-byte LDS write serves 16 lanes per cycle over 128 bytes of
    // banks, so the 16 rows of one write must land on 16 distinct 8-byte
    // positions modulo 128 bytes (the chunk swizzle alone gives 8, and a
    // write took twice its cycles under SQ_LDS_BANK_CONFLICT).
    auto stg_chunk = [](int r, int q) __attribute__((always_inline)) { return r * 128 + ((q ^ ((r >> 1) & 7)) * 16); };
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    auto stage_write = [&]<int KS>(BPT_LDS char* slot, int x) __attribute__((always_inline)) {
        constexpr int PM = KS * RPK / 32, H = (KS * RPK % 32) / 16;
        if constexpr (RPK == 32) {
            const int nb = x / 4, g = x % 4, r = lane % 32;
            *(BPT_LDS out4_t*)(slot + stg_chunk(r, nb * 4 + g) + ((lane / 32) ^ ((r >> 4) & 1) ^ (r & 1)) * 8) =
                held[PM][nb][g];
        } else {
            if (H == 0 && x < NB) {
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    u32x2_t a = __builtin_bit_cast(u32x2_t, held[PM][x][2 * p]);
                    u32x2_t b = __builtin_bit_cast(u32x2_t, held[PM][x][2 * p + 1]);
#pragma unroll
                    for (int d = 0; d < 2; ++d) {
                        const auto sw = __builtin_amdgcn_permlane16_swap(a[d], b[d], false, false);
                        a[d] = sw[0];
                        b[d] = sw[1];
                    }
                    held[PM][x][2 * p] = __builtin_bit_cast(out4_t, a);
                    held[PM][x][2 * p + 1] = __builtin_bit_cast(out4_t, b);
                }
            }
            if (x >= 2 && x < 2 + 2 * NB) {
                const int nb = (x - 2) / 2, p = (x - 2) % 2;
                const int r = lane % 16, q = nb * 4 + 2 * p + (lane / 16) % 2;
                *(BPT_LDS out4_t*)(slot + stg_chunk(r, q) + ((lane / 32) ^ (q & 1) ^ (r & 1)) * 8) = held[PM][nb][2 * p + H];
            }
        }
    };
    static_assert(NMMA >= 2 + 2 * NB && NMMA >= NB * 4 / (RPK == 32 ? 1 : 2), "staging writes ride on the MFMAs");

    // One k-step on fragment set s: MFMA q with read q of k-step rks of
    // K-tile rg (tile-local RKT) into set s^1 when READ, the accumulators
    // packed into `held` just before the tile's first products when FIRST,
    // and staging write q of step SKT when STG.
    auto kstep = [&]<bool FIRST, int RKT, int SKT>(int s, bool read, int rg, int rks, bool stg, BPT_LDS char* slot)
        __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < NMMA; ++q) {
            // the B pieces first: the next k-step's first two MFMAs need
            // both B blocks and A block 0, later ones one more A block each
            if (read) read_piece.template operator()<RKT>(rg, rks, q < 2 * NB ? MB + q : q - 2 * NB, s ^ 1);
            const int mb = q / NB, nb = q % NB;
            const frag_t b =
                __builtin_bit_cast(frag_t, __builtin_shufflevector(fbl[s][nb], fbh[s][nb], 0, 1, 2, 3, 4, 5, 6, 7));
            if constexpr (FIRST) {
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int e = 0; e < 4; ++e) held[mb][nb][g][e] = cvt_out<OutT>(acc[mb][nb][4 * g + e]);
                acc[mb][nb] = Mfma<T>::mma32(b, fa[s][mb], float16_t{});
            } else {
                acc[mb][nb] = Mfma<T>::mma32(b, fa[s][mb], acc[mb][nb]);
            }
            if (stg) stage_write.template operator()<SKT>(slot, q);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // step g = it * NK + KT.  MODE 0: the first tile (no previous C, no
    // k-step before its first); 1: a later tile; 2: the NK steps after the
    // last tile, which send its C without products.  Peeled at compile time:
    // with run-time conditions around the k-steps the compiler kept merged
    // copies of the accumulators and fragments and spilled.
    auto step = [&]<int KT, int MODE>(int it) __attribute__((always_inline)) {
        const int g = it * NK + KT;
        publish_lgkm();
        BPT_LDS char* slot = lds + STG_BASE + (g & 1) * SLOT + wave * WSLOT;
        if constexpr (MODE == 0 && KT == 0) {
#pragma unroll
            for (int p = 0; p < NMMA; ++p) read_piece.template operator()<0>(0, 0, p, 0);
        }
        // k-step 1 of K-tile g-1, reading K-tile g's first fragments
        if constexpr ((MODE == 0 && KT > 0) || MODE == 1)
            kstep.template operator()<false, KT, KT>(1, true, g, 0, false, slot);
        if constexpr (MODE == 2 && KT == 0) kstep.template operator()<false, KT, KT>(1, false, g, 0, false, slot);
        if constexpr (MODE < 2) {
            // k-step 0 of K-tile g, reading its second fragments, and the
            // previous tile's rows KT*RPK .. into the slot
            kstep.template operator()<MODE == 1 && KT == 0, KT, KT>(0, true, g, 1, MODE == 1, slot);
        } else {
            // the last tile's rows, without products
            if constexpr (KT == 0) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
                            for (int e = 0; e < 4; ++e) held[mb][nb][g4][e] = cvt_out<OutT>(acc[mb][nb][4 * g4 + e]);
            }
#pragma unroll
            for (int x = 0; x < NMMA; ++x) stage_write.template operator()<KT>(slot, x);
        }
    };
    auto tile = [&]<int MODE>(int it) __attribute__((always_inline)) {
        [&]<int... KT>(std::integer_sequence<int, KT...>) {
            (step.template operator()<KT, MODE>(it), ...);
        }(std::make_integer_sequence<int, NK>{});
    };
    tile.template operator()<0>(0);
    for (int it = 1; it < turns; ++it) tile.template operator()<1>(it);
    tile.template operator()<2>(turns);
    publish_lgkm();                        // step (turns + 1) * NK: the store waves store the last slot
}

}  // namespace bpt
