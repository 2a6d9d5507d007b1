// gemm_persist_ares.hpp -- the persistent short-K kernel with the A panel
// resident in LDS (C = A * B, B row-major K x N, 16-bit C, K = 128 or 256).
//
// In the persistent kernels of gemm_persist.hpp every 256 x 128 tile copies
// its A block (256 x K) and B block (K x 128) from L2 into LDS and writes its
// C block: with K = 256 that is 128 + 64 KiB in and 64 KiB out per tile, and
// measured without the A copies the same kernel ran 0.51 ms instead of 0.81
// on 64 x 4096^2 x 256 -- the stream of copies, not the products, sets the
// pace.  Here a workgroup walks the column tiles of one row block in a row
// (a "group"), keeps that block's A panel in LDS for the whole group and
// streams only B: A is copied once per group instead of once per tile.
//
// LDS (K = 256): the A panel as 4 pair stages of 256 rows x 64 k (128 KiB,
// laid out as the A-pair kernel's stages), a 3-stage B ring (24 KiB) and a
// 2 KiB C staging slot per wave.  With K = 128: a 64 KiB panel, 4 B stages
// and 4 KiB slots.  There is no room to stage a whole C tile, so the
// finished accumulators are packed to 16 bits into registers when the next
// tile's first products overwrite them, and each wave sends out RPK =
// 128/NK of its 128 rows in every K-tile of the next tile: its 8 writes of
// them into its slot ride between the first k-step's MFMAs, the read back
// as whole 128-byte row pieces comes before the publish and the stores (8
// whole lines per instruction, as before) after it.  Every wave does the
// same in every K-tile, and no slot is shared.  With RPK = 16 a K-tile takes
// half of a 32-row block, whose rows sit in half of each 32-lane group: a
// v_permlane16_swap of the pieces of chunks 2p and 2p+1 puts rows 0..15 of
// both chunks into one register of all 64 lanes and rows 16..31 into the
// other, so the writes need no lane mask (no exec writes in the loop).
//
// B stages: tile-local K-tile k of the tile with base b uses stage
// (b + k) % BSTAGES, b advancing by NK per tile; with NK = 8 and 3 stages
// the base rotates, and it is a scalar of the loop.  The window of K-tile i
// refills K-tile i's stage with B(i + BSTAGES) (of the next tile when past
// NK), half after publish(i+1) and half in the first k-step of K-tile i+1,
// so publish(j+1) lets 2 (BSTAGES - 2) younger copies fly.
//
// Stores share the vmcnt counter with the copies and may complete out of
// order with respect to them, so a publish can let only as many operations
// fly as there are copies younger than the ones it needs; a store still in
// flight takes one of those places, and with 3 stages there are 2.  At
// K = 256 that costs more than the A copies save: on 64 x 4096^2 x 256 the
// kernel ran 0.45 ms without its stores and 0.90 ms with them, against
// 0.82 ms for the A-pair kernel (whose windows of 10 A copies leave room
// for the stores every other K-tile); issuing each whole window before the
// stores made it 1.11 ms.  With K = 128 (4 stages) it is the faster one,
// 0.466 against 0.493 ms on 64 x 4096^2 x 128.
//
// A new group: after its tile's last products a full publish (every copy,
// store and LDS read of every wave retired, then a barrier) frees the old
// panel; the panel copies go out and a second full publish makes them
// visible.  The A fragments read ahead for the new tile from the old panel
// are read again.  Waiting for everything leaves the later wait counts
// right: they only ever allow fewer copies in flight than there are.
//
// Walk: group g = (batch entry, row block, column range of gn tiles); the
// groups go to XCDs and workgroups as tiles do in the other persistent
// kernels (persist_logical over groups), so at any time one XCD's 32
// workgroups hold consecutive groups -- with 16 row blocks split in two
// column ranges, the 32 groups of one batch entry, whose B the XCD's L2
// then holds once.
//
// Host: M % 256 == 0, N % 128 == 0, K == 32 * NK, tiles_n == nsplit * gn,
// 16-byte aligned rows, gridDim.x <= ngroups.
#pragma once
#include <utility>

#include "device_common.hpp"
#include "gemm_persist.hpp"

namespace bpt {

template <typename T, typename OutT, int NK>
__global__ __launch_bounds__(256, 1) void gemm_persist_ares_kernel(GemmArgs args, int ngroups, int gn, int nsplit) {
    constexpr int BM = 256, BN = 128, BK = 32;
    constexpr int BSTAGES = NK == 8 ? 3 : 4;
    typedef PipelinedGemm<T, BM, BN, BK, BSTAGES, 2, 2, OutT, false> G;
    typedef typename G::frag_t frag_t;
    static_assert(sizeof(OutT) == 2, "16-bit C: staged in 128-byte rows of 64 values");
    static_assert(NK == 4 || NK == 8, "K = 128 or 256");
    static_assert(G::KS == 2, "two k-steps per K-tile");
    static_assert(G::TN * 2 == 128, "staging rows of 8 chunks");
    constexpr int MB = G::MB, NB = G::NB;
    constexpr int AP_BYTES = BM * 2 * BK * 2;            // one A pair stage (256 rows x 64 k)
    constexpr int B_BYTES = BK * BN * 2;                 // one B stage
    constexpr int B_BASE = (NK / 2) * AP_BYTES;
    constexpr int A_INST = AP_BYTES / 1024 / 4;          // pair copies per wave (8)
    constexpr int B_INST = B_BYTES / 1024 / 4;           // B copies per wave per K-tile (2)
    constexpr int RPK = G::TM / NK;                      // held rows each wave sends out per K-tile
    constexpr int SLOT = RPK * 128;                      // RPK rows x 64 values
    constexpr int RD = SLOT / 1024;                      // read-backs (and stores) per lane per K-tile
    constexpr int STG_BASE = B_BASE + BSTAGES * B_BYTES;
    constexpr int LDS_BYTES = STG_BASE + 4 * SLOT;
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
    static_assert(RPK == 16 || RPK == 32, "half or whole 32-row blocks per K-tile");
    static_assert(G::NMMA == NB * 4, "one staging write per MFMA of a k-step");
    constexpr int VM = (BSTAGES - 2) * B_INST;           // younger copies at publish(j+1)
    constexpr int VM_PRO = VM + B_INST / 2;              // ... at the prologue's publish(0)
    static_assert(B_INST == 2, "windows of one copy per half");
    __shared__ __attribute__((aligned(1024))) char lds_raw[LDS_BYTES];
    BPT_LDS char* lds = (BPT_LDS char*)lds_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / 2;
    const int wn = wave % 2;
    const int lda = args.lda, ldb = args.ldb, ldc = args.ldc, K = args.K;
    const int per_g = args.tiles_m * nsplit;             // groups per batch entry
    const int wg = blockIdx.x, grid = gridDim.x;
    const int turns = persist_turns(wg, grid, ngroups) * gn;
    if (turns == 0) return;                // host: grid <= ngroups; uniform

    uint32_t voffB[B_INST];
#pragma unroll
    for (int i = 0; i < B_INST; ++i) {
        const int row = (wave * B_INST + i) * G::B_ROWS_PER_INST + lane / G::B_CHUNKS;
        const int chunk = (lane % G::B_CHUNKS) ^ swz_b(row);
        voffB[i] = (uint32_t)((row * ldb + chunk * 8) * 2);
    }
    const uint32_t b_step = (uint32_t)BK * ldb * 2;
    // A block mb of K-tile parity t, k-step ks: row wm*TM + mb*32 + l%32,
    // logical chunk 4t + 2ks + l/32 of the 128-byte pair row, swizzled
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

    // batch entry and corner of this workgroup's tile number `it` (the
    // divisions run on VGPR copies, as in the other persistent kernels)
    auto corner = [&](int it, int& batch, int& m0, int& n0) __attribute__((always_inline)) {
        int itv;
        asm volatile("v_mov_b32 %0, %1" : "=v"(itv) : "s"(it));
        const int rv = itv / gn;
        const int r = __builtin_amdgcn_readfirstlane(rv);
        const int tt = it - r * gn;
        const int gi = persist_logical(wg, grid, r, ngroups);
        int gv;
        asm volatile("v_mov_b32 %0, %1" : "=v"(gv) : "s"(gi));
        const int bv = gv / per_g;
        const int rem = gv - bv * per_g;
        const int tmv = rem / nsplit;
        const int nsv = rem - tmv * nsplit;
        batch = __builtin_amdgcn_readfirstlane(bv);
        m0 = __builtin_amdgcn_readfirstlane(tmv) * BM;
        n0 = (__builtin_amdgcn_readfirstlane(nsv) * gn + tt) * BN;
    };
    struct Tile {
        int4_t rb;
        OutT* c;
    };
    auto tile_at = [&](int it) __attribute__((always_inline)) {
        Tile t;
        if (it < turns) {
            int batch, m0, n0;
            corner(it, batch, m0, n0);
            const T* b0 = static_cast<const T*>(args.B) + batch * args.strideB + n0;
            t.rb = make_rsrc(b0, (uint32_t)(((K - 1) * (long long)ldb + BN) * 2));
            t.c = static_cast<OutT*>(args.C) + batch * args.strideC + (long long)(m0 + wm * G::TM) * ldc + n0 +
                  wn * G::TN;
        } else {
            t.rb = make_rsrc(args.B, 0u);   // no records: copies land zeros, no traffic
            t.c = nullptr;
        }
        return t;
    };
    // the A panel of tile `it`'s group: NK/2 pair stages, 8 rows x 128 bytes
    // (whole lines) per copy.  The per-lane offsets come from a lane number
    // read afresh, so they hold no registers between groups.
    auto load_panel = [&](int it) __attribute__((always_inline)) {
        int batch, m0, n0;
        corner(it, batch, m0, n0);
        const T* a0 = static_cast<const T*>(args.A) + batch * args.strideA + (long long)m0 * lda;
        const int4_t ra = make_rsrc(a0, (uint32_t)(((BM - 1) * (long long)lda + K) * 2));
        int ln;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
#pragma unroll
        for (int i = 0; i < A_INST; ++i) {
            const int row = (wave * A_INST + i) * 8 + ln / 8;
            const int chunk = (ln % 8) ^ swz_a<64>(row);
            const uint32_t voff = (uint32_t)((row * lda + chunk * 8) * 2);
#pragma unroll
            for (int p = 0; p < NK / 2; ++p)
                dma16(ra, lds0 + p * AP_BYTES + (wave * A_INST + i) * 1024, voff, (uint32_t)(p * 2 * BK * 2));
        }
    };

    // B stage of tile-local K-tile KB (>= NK: the next tile's), for the
    // current tile's stage base
    int bst = 0;
    auto bstage = [&]<int KB>() __attribute__((always_inline)) -> int {
        if constexpr (NK % BSTAGES == 0) {
            return KB % BSTAGES;
        } else {
            const int s = bst + KB % BSTAGES;
            return s >= BSTAGES ? s - BSTAGES : s;
        }
    };
    // copy c of the window of tile-local K-tile I (I = -BSTAGES .. NK-1):
    // B(I + BSTAGES) into the stage K-tile I leaves
    auto dma_win = [&]<int I>(int c, const Tile& cur, const Tile& nxt) __attribute__((always_inline)) {
        constexpr int KB = I + BSTAGES;
        const Tile& t = KB < NK ? cur : nxt;
        uint32_t l0 = lds0 + B_BASE + bstage.template operator()<KB>() * B_BYTES, bstep = b_step;
        asm volatile("" : "+s"(l0), "+s"(bstep));
        // the descriptor is uniform, but carried through the tile loop the
        // compiler may hold it in vector registers; the copy needs scalars
        int4_t rs = t.rb;
#pragma unroll
        for (int k = 0; k < 4; ++k) rs[k] = __builtin_amdgcn_readfirstlane(rs[k]);
        dma16(rs, l0 + (wave * B_INST + c) * 1024, voffB[c], (KB % NK) * bstep);
    };

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
    // read p of k-step ks of tile-local K-tile KTR (NK: the next tile's
    // first) into set s
    auto read_piece = [&]<int KTR>(int ks, int p, int s) __attribute__((always_inline)) {
        if (p < MB) {
            constexpr int KA = KTR % NK;
            fa[s][p] = *(BPT_LDS frag_t*)(lds + (KA / 2) * AP_BYTES + rdA[KA % 2][ks] + p * 32 * 128);
        } else {
            const int nb = (p - MB) / 2, h = (p - MB) % 2;
            BPT_LDS short4_t* q = (BPT_LDS short4_t*)(lds + bstage.template operator()<KTR>() * B_BYTES + rdB[nb] +
                                                      ks * 16 * BN * 2 + h * 4 * BN * 2);
            if (h == 0) fbl[s][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
            else fbh[s][nb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
        }
    };

    // The held rows of K-tile KS (RPK rows from KS*RPK on), in 32-row block
    // PM of the wave tile.  Lane l holds row PM*32 + l%32, 16-byte chunk q =
    // nb*4 + g of the 128-byte row, 8-byte half l/32 (held[PM][nb][g]).  Slot
    // row r goes to chunk q ^ ((r >> 1) & 7).  RPK = 32: r = l%32, halves
    // swapped for r >= 16; the write after MFMA x of the first k-step is
    // piece x = nb*4 + g.  RPK = 16: after MFMA nb of the block's first
    // K-tile the pieces g = 2p, 2p+1 swap their odd and even 16-lane rows;
    // then piece 2p + H holds, in lane l, slot row l%16 (block row 16H +
    // l%16) of chunk nb*4 + 2p + (l/16)%2, half l/32, and is written after
    // MFMA 2 + 2nb + p, halves swapped in odd chunks.  Either way the 32
    // lanes of a write half cover the 64 banks once.
    BPT_LDS char* const slot = lds + STG_BASE + wave * SLOT;
    auto stg_chunk = [](int r, int q) __attribute__((always_inline)) { return r * 128 + ((q ^ ((r >> 1) & 7)) * 16); };
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    auto stage_write = [&]<int KS>(int x) __attribute__((always_inline)) {
        constexpr int PM = KS * RPK / 32, H = (KS * RPK % 32) / 16;
        if constexpr (RPK == 32) {
            const int nb = x / 4, g = x % 4, r = lane % 32;
            *(BPT_LDS out4_t*)(slot + stg_chunk(r, nb * 4 + g) + ((lane / 32) ^ ((r >> 4) & 1)) * 8) = held[PM][nb][g];
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
                *(BPT_LDS out4_t*)(slot + stg_chunk(r, q) + ((lane / 32) ^ (q & 1)) * 8) = held[PM][nb][2 * p + H];
            }
        }
    };

    // One k-step on fragment set s, with the reads of k-step rks of K-tile
    // KTR into set s^1 and copies [C0, C1) of window WI spread over its
    // MFMAs.  FIRST: the tile's first k-step, which packs the finished
    // accumulators into `held` just before its products overwrite them.
    // STG: the K-tile's staging writes ride after the MFMAs (when stg).
    auto kstep = [&]<bool FIRST, bool STG, int KTR, int WI, int C0, int C1>(int s, int rks, const Tile& cur,
                                                                              const Tile& nxt, bool stg)
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
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int e = 0; e < 4; ++e) held[mb][nb][g][e] = cvt_out<OutT>(acc[mb][nb][4 * g + e]);
                acc[mb][nb] = Mfma<T>::mma32(b, fa[s][mb], float16_t{});
            } else {
                acc[mb][nb] = Mfma<T>::mma32(b, fa[s][mb], acc[mb][nb]);
            }
            if constexpr (NC > 0) {
#pragma unroll
                for (int x = 0; x < NC; ++x)
                    if ((x * G::NMMA) / NC == q) dma_win.template operator()<WI>(C0 + x, cur, nxt);
            }
            if constexpr (STG) {
                if (stg) stage_write.template operator()<KTR>(q);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // read the slot back as RD x 8 rows of 8 16-byte chunks (halves swapped
    // back where they were written swapped) and, after the publish,
    // store them: rows KS*RPK .. of the previous tile's wave tile
    int4_t sv[RD];
    auto stage_read = [&]() __attribute__((always_inline)) {
        wave_lds_handoff();                              // rows written by other lanes are read below
#pragma unroll
        for (int h = 0; h < RD; ++h) {
            const int r2 = h * 8 + lane / 8;
            int4_t v = *(BPT_LDS int4_t*)(slot + stg_chunk(r2, lane % 8));
            const bool swapped = RPK == 32 ? (r2 & 16) != 0 : (lane % 8) % 2 != 0;
            sv[h] = swapped ? int4_t{v[2], v[3], v[0], v[1]} : v;
        }
    };
    auto stage_store = [&]<int KS>(OutT* pc) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < RD; ++h) {
            const int r2 = h * 8 + lane / 8;
            OutT* dst = pc + (long long)(KS * RPK + r2) * ldc + (lane % 8) * 8;
            __builtin_nontemporal_store(sv[h], (int4_t*)dst);
        }
    };

    // ---- prologue: the first group's panel, windows -BSTAGES .. -2 whole
    // and the first half of window -1; then B(0) and the panel have landed
    // once VM_PRO younger copies remain.
    Tile cur = tile_at(0);
    Tile nxt = tile_at(1);
    OutT* prv = cur.c;
    load_panel(0);
    [&]<int... I>(std::integer_sequence<int, I...>) {
        ((
             [&] {
                 constexpr int W = I - BSTAGES;
#pragma unroll
                 for (int c = 0; c < (W == -1 ? B_INST / 2 : B_INST); ++c) dma_win.template operator()<W>(c, cur, nxt);
             }()),
         ...);
    }(std::make_integer_sequence<int, BSTAGES>{});
    publish<VM_PRO>();
#pragma unroll
    for (int p = 0; p < G::NREAD; ++p) read_piece.template operator()<0>(0, p, 0);

    // tile-local K-tile KT: k-step 0 (reads of its k-step 1, second half of
    // window KT-1, the staging writes of rows KT*RPK ..), their read back,
    // publish(KT+1), the stores, k-step 1 (reads of K-tile KT+1's k-step 0 --
    // the next tile's first when KT = NK-1 -- first half of window KT)
    auto ktile = [&]<int KT>(int it) __attribute__((always_inline)) {
        const bool stg = it > 0;                         // uniform: a previous tile exists
        kstep.template operator()<KT == 0, true, KT, KT - 1, B_INST / 2, B_INST>(0, 1, cur, nxt, stg);
        if (stg) stage_read();
        publish<VM>();
        if (stg) stage_store.template operator()<KT>(prv);
        kstep.template operator()<false, false, KT + 1, KT, 0, B_INST / 2>(1, 0, cur, nxt, false);
    };

    for (int it = 0; it < turns; ++it) {
        [&]<int... KT>(std::integer_sequence<int, KT...>) {
            (ktile.template operator()<KT>(it), ...);
        }(std::make_integer_sequence<int, NK>{});
        prv = cur.c;
        cur = nxt;
        nxt = tile_at(it + 2);
        if constexpr (NK % BSTAGES != 0) {
            bst += NK % BSTAGES;
            if (bst >= BSTAGES) bst -= BSTAGES;
        }
        if (it + 1 < turns && (it + 1) % gn == 0) {
            // a new group: every wave is done with the old panel (and every
            // copy and store has landed), copy the new one, wait for it, and
            // read the new tile's first A fragments again
            publish<0>();
            load_panel(it + 1);
            publish<0>();
#pragma unroll
            for (int p = 0; p < MB; ++p) read_piece.template operator()<0>(0, p, 0);
        }
    }
    int lb, lm0, ln0;
    corner(turns - 1, lb, lm0, ln0);
    pipelined_epilogue<G, OutT>(args, acc, lds, lane, wave, wm, wn, lm0, ln0, lb);
}

}  // namespace bpt
