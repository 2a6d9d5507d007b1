// attention.hpp -- fused scaled dot-product attention, forward:
//     O = softmax(scale * Q K^T) V
// for BH independent (batch x head) problems of Sq query rows, Skv keys and
// head dimension D (128 or 256), fp16 or bf16 in, fp32 accumulation.
//
// This is the second workload of the pages: the "Xe2 Nbarrier Pipelining" page
// (section "Proven Pattern: SDP Kernel Split Barrier B") describes an
// HD = 256 flash-attention kernel whose loop runs QK products, the softmax,
// a trip of S through shared memory, then the PV products, with the loads of
// V and the prefetch of the next K placed between the barrier's arrive and
// its wait.  On gfx950 the same schedule is rebuilt as follows.
//
// * Workgroup: WAVES waves of 32 query rows; wave w owns rows 32w .. 32w+31
//   and keeps its Q fragments in registers for the whole key loop.  Every
//   softmax statistic of a row lives in that row's two lanes (l and l+32),
//   so no reduction crosses waves -- the pages' barrier for the shared
//   softmax maximum has nothing to do here.  Two waves share each SIMD
//   (waves w and w + WAVES/2), which needs a wave to fit in 256 registers;
//   at head dimension 256 that holds for 32-key blocks.
// * K and V blocks of BN keys are staged global->LDS by LDS-DMA in a ring of
//   STAGES stages.  Block j is published by a vmcnt wait plus one s_barrier;
//   the copies of block j+STAGES-1 into the stage block j-1 left (the
//   window) go out between block j's first products, and the rest of its
//   math follows.
// * The K and V fragments for the matrix products are read from LDS two
//   MFMAs ahead of their use.  With both fragment reads and the O and Q
//   registers a wave holds, the compiler otherwise kept one fragment in
//   flight and waited for each read right before its MFMA.
// * S never goes through LDS.  S^T = K Q^T is formed with K as the MFMA's
//   row operand, so lane l holds query row l%32 and 16 keys of each 32 keys
//   of a block.  Those are exactly the keys its half of the wave must supply
//   to the PV product if the key order inside each 16-key step is permuted
//   (keys 4h..4h+3 and 8+4h..8+4h+3 for half h), and V is read from LDS with
//   the same permutation (transposing reads of rows 4h.. and 8+4h..).  So P
//   goes from the S accumulators to the PV operand in registers.
// * Online softmax in base 2 with a lazy rescale: a row's running maximum m
//   is raised (and its O and sum scaled by 2^(m_old - m_new)) only when some
//   row of the wave sees a logit more than 2^8 above its m; otherwise the
//   block's weights are taken against the stale m (each at most 2^8).  O / l
//   is the same either way.  Every operand of the loop (O, S, Q, the
//   fragments and the row state) fits in a wave's 256 ordinary registers,
//   where the MFMAs accumulate; nothing moves between register files.
// * Wave priority (s_setprio) favours matrix products.  After each block's
//   barrier the two waves of a SIMD start in step; raising the priority of
//   the wave issuing MFMAs keeps the matrix core fed while the other runs
//   its softmax.  At D = 128 each wave raises it for its two product phases;
//   at D = 256 one wave of each pair (w < WAVES/2) keeps the higher priority
//   throughout, which measured better there.
// * The last key block, when Skv is not a multiple of BN, is peeled from the
//   loop and masks keys >= Skv to -inf; K and V rows past Skv read as zero
//   (the buffer range check).
#pragma once
#include "device_common.hpp"
#include "gemm_pipelined.hpp"   // swz_b

namespace bpt {

struct AttnArgs {
    const void* Q;
    const void* K;
    const void* V;
    void* O;
    int Sq, Skv;
    int ldq, ldk, ldv, ldo;                 // row strides (elements)
    long long sQ, sK, sV, sO;               // per (batch x head) strides (elements)
    float c2;                               // scale * log2(e)
    int q_tiles;                            // ceil(Sq / BM)
};

// WAVES_ waves of 32 query rows each, key blocks of BN_ keys, a ring of
// STAGES_ K+V stages
template <typename T, int D, int WAVES_, int BN_, int STAGES_>
struct AttnFwd {
    static_assert(D == 128 || D == 256, "head dimensions 128 and 256");
    static_assert(BN_ == 32 || BN_ == 64, "key blocks of 32 or 64");
    static_assert(STAGES_ == 2 || STAGES_ == 4, "power-of-two rings");
    static constexpr int WAVES = WAVES_, BM = 32 * WAVES_, BN = BN_, STAGES = STAGES_;
    static constexpr int KB = BN / 32;                  // 32-key halves of a block
    static constexpr int PVS = BN / 16;                 // 16-key steps of the PV product
    static constexpr int DC = D / 8;                    // 16-byte chunks per row
    static constexpr int ROWS_PER_KIB = 1024 / (D * 2); // rows one wave-wide copy covers
    static constexpr int TILE = BN * D * 2;             // one K or V block in LDS
    static constexpr int STAGE = 2 * TILE;
    static constexpr int LDS_BYTES = STAGES * STAGE;
    static constexpr int COPIES = TILE / 1024 / WAVES;  // per wave per tile
    static constexpr int TS = D / 16;                   // k-steps of Q K^T
    static constexpr int DB = D / 32;                   // 32-wide d blocks of O
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(COPIES >= 1, "every wave copies");
    static constexpr int VM_AHEAD = (STAGES - 2) * 2 * COPIES;   // younger copies a publish lets fly
    static_assert(VM_AHEAD + 2 * COPIES < 64, "vmcnt");
};

// K rows are read 32 at a time at one 16-byte chunk (ds_read_b128 into the
// MFMA row operand): chunk ^ (row & 15) spreads 16 consecutive rows over
// all 64 banks.  V rows are read by 4-row transposing reads, for which the
// GEMM's B swizzle (swz_b) already spreads the rows.
__device__ inline int attn_swz_k(int row) { return row & 15; }

// POS: scale >= 0 (the row maximum of the logits is the maximum of the raw
// products; for a negative scale it is the minimum).  RAGGED: Skv is not a
// multiple of BN, and the last block runs as a masked copy of the block code
// after the loop.  The host picks the instance, so the loop has no
// condition on it ("Xe2 ESIMD GEMM", Inner-loop rules): at D = 256 the
// masked copy makes the compiler spill O registers around the loop exit,
// and only the RAGGED instance pays for that.
template <typename T, int D, typename OutT, bool POS, int WAVES, int BN_, int STAGES, bool RAGGED>
__global__ __launch_bounds__(WAVES * 64, 1) void attention_fwd_kernel(AttnArgs a) {
    typedef AttnFwd<T, D, WAVES, BN_, STAGES> G;
    typedef typename Mfma<T>::frag_t frag_t;
    constexpr int BN = G::BN, TS = G::TS, DB = G::DB;
    __shared__ __attribute__((aligned(1024))) char lds_raw[G::LDS_BYTES];
    BPT_LDS char* lds = (BPT_LDS char*)lds_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;                             // half of the wave
    constexpr bool kPhasePrio = D == 128;                // else priority by wave pair
    if (!kPhasePrio && wave < WAVES / 2) __builtin_amdgcn_s_setprio(1);
    const float kNegInf = -__builtin_inff();
    const float kFar = POS ? kNegInf : __builtin_inff(); // a raw product no row max can pick

    // XCD-aware order: a run of consecutive (head, query tile) pairs -- the
    // tiles of one head, sharing its K and V -- stays on one XCD's L2
    int pid = blockIdx.x;
    const int num = gridDim.x;
    if ((num & 7) == 0) pid = (pid & 7) * (num >> 3) + (pid >> 3);
    const int bh = pid / a.q_tiles;
    const int q0 = (pid - bh * a.q_tiles) * G::BM;
    const int Sq = a.Sq, Skv = a.Skv;

    const T* Qb = static_cast<const T*>(a.Q) + bh * a.sQ + (long long)q0 * a.ldq;
    const T* Kb = static_cast<const T*>(a.K) + bh * a.sK;
    const T* Vb = static_cast<const T*>(a.V) + bh * a.sV;

    // ---- Q fragments: row 32w + l%32, d = 16t + 8h .. +7 (zero past Sq) ----
    frag_t qf[TS];
    {
        const int rows = Sq - q0;                        // >= 1
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T*>(Qb), 0, (int)(((long long)(rows - 1) * a.ldq + D) * 2), kBufferWord3);
        const uint32_t vq = (uint32_t)(((wave * 32 + (lane & 31)) * a.ldq + 8 * h) * 2);
#pragma unroll
        for (int t = 0; t < TS; ++t)
            qf[t] = __builtin_bit_cast(frag_t, __builtin_amdgcn_raw_buffer_load_b128(rq, vq + t * 32, 0, 0));        // Let Q land here, with a wait the compiler sees: otherwise its wait
        // counting carries the Q loads into the key loop as pending and puts
        // vmcnt waits before their first uses there, which at run time also
        // wait for the K/V copies just issued (LDS-DMA copies count in vmcnt
        // but are invisible to the compiler).
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }

    float16_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        oacc[db] = float16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf;                               // running max of the row (base 2)
    float l_half = 0.f;                                  // this half's share of the row sum

    const int nblk = (Skv + BN - 1) / BN;
    if (nblk > 0) {
        const int4_t rsK = make_rsrc(Kb, (uint32_t)(((long long)(Skv - 1) * a.ldk + D) * 2));
        const int4_t rsV = make_rsrc(Vb, (uint32_t)(((long long)(Skv - 1) * a.ldv + D) * 2));
        // copies: wave w brings KiB w*COPIES + i of each tile; lane p lands at
        // 16-byte slot p of it = row i*ROWS_PER_KIB + p/DC (of the wave's
        // rows), physical chunk p%DC, holding logical chunk (p%DC) ^ swz(row)
        uint32_t voffK[G::COPIES], voffV[G::COPIES];
#pragma unroll
        for (int i = 0; i < G::COPIES; ++i) {
            const int row = (wave * G::COPIES + i) * G::ROWS_PER_KIB + lane / G::DC;
            const int pc = lane % G::DC;
            voffK[i] = (uint32_t)((row * a.ldk + 8 * (pc ^ attn_swz_k(row))) * 2);
            voffV[i] = (uint32_t)((row * a.ldv + 8 * (pc ^ swz_b(row))) * 2);
        }
        const uint32_t ldsb = __builtin_amdgcn_readfirstlane(lds_addr(lds));
        const uint32_t kstepK = (uint32_t)(BN * a.ldk * 2), kstepV = (uint32_t)(BN * a.ldv * 2);
        // block j into stage j % STAGES (blocks past the last read zeros):
        // copy c < COPIES is a KiB of K, the others of V
        auto copy = [&](int j, int c) __attribute__((always_inline)) {
            const uint32_t st = ldsb + (j & (STAGES - 1)) * G::STAGE + wave * G::COPIES * 1024;
            if (c < G::COPIES)
                dma16(rsK, st + c * 1024, voffK[c] + j * kstepK, 0);
            else
                dma16(rsV, st + G::TILE + (c - G::COPIES) * 1024, voffV[c - G::COPIES] + j * kstepV, 0);
        };
        auto issue = [&](int j) __attribute__((always_inline)) {
#pragma unroll
            for (int c = 0; c < 2 * G::COPIES; ++c) copy(j, c);
        };

        // fragment reads.  K (row operand of S^T = K Q^T): key 32kb + l%32,
        // logical chunk 2t + h, physical (2t + h) ^ (l & 15).  2t and h are
        // disjoint bits, so the physical chunk is 2t ^ y with y = h ^ (l & 15),
        // and the byte address row + 16 (2t ^ y) = (row + 16 y) ^ 32t: one
        // base register and one XOR per read (stage and kb offsets lie above
        // the XOR's bits).
        const uint32_t kbase = (uint32_t)((lane & 31) * D * 2 + 16 * (h ^ attn_swz_k(lane)));
        // V (row operand of O^T = V^T P^T), transposing 4-row reads: 16-lane
        // group g, lane j reads row 4(g/2) + j/4 (+8 for the upper four keys,
        // +16ks) at columns 32db + 16(g%2) + 4(j%4); chunk 4db + x with
        // x = 2(g%2) + (j%4)/2, swizzled by s = swz_b(j/4):
        // (4db + x) ^ s = 4(db ^ (s>>2)) + (x ^ (s&3)).  The byte address is
        // vbase ^ 64(db & 3), plus 256 for db >= 4.
        const int g = lane >> 4, jj = lane & 15;
        const int sv = swz_b(jj >> 2);
        const int xv = 2 * (g & 1) + ((jj & 3) >> 1);
        const uint32_t vbase = (uint32_t)((4 * (g >> 1) + (jj >> 2)) * D * 2 + 64 * (sv >> 2) +
                                          16 * (xv ^ (sv & 3)) + 8 * (jj & 1));

        // S^T for keys BN j .. BN j + BN-1 (KB 32-key halves)
        // Each fragment read goes out PD MFMAs ahead of its use, so its
        // latency runs under earlier MFMAs instead of stalling the wave.  The
        // scheduling fences keep that order (without the one before the
        // MFMA, the compiler moved the read below it).
        constexpr int PD = 2;
        // With COPY, the copies of block cj go out between the products, one
        // after every SPREAD-th MFMA: issued together after the barrier, the
        // eight waves' copies queued behind each other for the address unit
        // and held each wave 150-350 cycles before its first product.
        auto qk = [&]<bool COPY>(int j, int cj, float16_t (&s)[G::KB]) __attribute__((always_inline)) {
            const uint32_t kj = kbase + (uint32_t)((j & (STAGES - 1)) * G::STAGE);
            constexpr int N = TS * G::KB;
            auto kread = [&](int i) __attribute__((always_inline)) {
                const int t = i / G::KB, kb = i % G::KB;
                return *(BPT_LDS frag_t*)(lds + (kj ^ (32u * t)) + kb * 32 * D * 2);
            };
#pragma unroll
            for (int kb = 0; kb < G::KB; ++kb)
                s[kb] = float16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            frag_t kf[PD + 1];
#pragma unroll
            for (int i = 0; i < PD; ++i) kf[i] = kread(i);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                if (i + PD < N) kf[(i + PD) % (PD + 1)] = kread(i + PD);
                __builtin_amdgcn_sched_barrier(0);
                const int t = i / G::KB, kb = i % G::KB;
                s[kb] = Mfma<T>::mma32(kf[i % (PD + 1)], qf[t], s[kb]);
                __builtin_amdgcn_sched_barrier(0);
                constexpr int SPREAD = N / (2 * G::COPIES);
                static_assert(SPREAD >= 1 && N % (2 * G::COPIES) == 0, "copies spread evenly over the products");
                if constexpr (COPY)
                    if (i % SPREAD == 1 % SPREAD) copy(cj, i / SPREAD);
            }
        };
        // the online softmax of block j: running max, rescale of O and the
        // row sum, and the weights P as PV operands
        auto softmax = [&]<bool MASK>(int j, const float16_t (&s)[G::KB], frag_t (&pf)[G::PVS])
            __attribute__((always_inline)) {
            // the row maximum of the logits in base 2, from the raw products
            // (the scale is monotone; keys >= Skv excluded when MASK); register
            // r of half kb holds key BN j + 32kb + 8(r/4) + 4h + r%4
            auto masked = [&](int kb, int r) __attribute__((always_inline)) {
                return MASK && j * BN + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3) >= Skv;
            };
            float mraw = kFar;
#pragma unroll
            for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x = masked(kb, r) ? kFar : s[kb][r];
                    mraw = POS ? __builtin_fmaxf(mraw, x) : __builtin_fminf(mraw, x);
                }
            // join the row's two lanes (l and l+32): v_permlane32_swap of the
            // value with itself leaves the lower half's values in one result
            // and the upper half's in the other, in every lane, and max/min
            // of the two is the row's in both halves -- no LDS round trip
            // (a shuffle through ds_bpermute sat on the softmax's critical
            // path)
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, mraw),
                                                                 __builtin_bit_cast(unsigned, mraw), false, false);
                const float lo = __builtin_bit_cast(float, (unsigned)sw[0]);
                const float hi = __builtin_bit_cast(float, (unsigned)sw[1]);
                mraw = POS ? __builtin_fmaxf(lo, hi) : __builtin_fminf(lo, hi);
            }
            const float mloc = mraw * a.c2;
            // raise the running max only when some row would otherwise see a
            // weight above 2^8
            if (__builtin_amdgcn_ballot_w64(mloc > m_run + 8.0f) != 0) {
                const float m_new = __builtin_fmaxf(m_run, mloc);
                // a row with no key yet (max still -inf) has nothing to scale
                const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                l_half *= alpha;
                // a plain multiply: every operand of the loop fits in the
                // 256 ordinary registers, so the products accumulate there
                // and nothing moves between register files
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            }
            // weights p = 2^(s c2 - m) (one FMA into the exponent), rounded to
            // the input type for the PV operands (keys 16ks .. 16ks+15 of the
            // block are registers 8(ks&1) .. +7 of half ks>>1); the row sum
            // adds the rounded weights, the values the PV product uses
            const float nmref = m_run == kNegInf ? 0.f : -m_run;
#pragma unroll
            for (int ks = 0; ks < G::PVS; ++ks)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int kb = ks >> 1, r = 8 * (ks & 1) + i;
                    const float e2 = masked(kb, r) ? kNegInf : __builtin_fmaf(s[kb][r], a.c2, nmref);
                    pf[ks][i] = (typename Mfma<T>::elem_t)__builtin_amdgcn_exp2f(e2);
                }
            float psum = l_half;
#pragma unroll
            for (int ks = 0; ks < G::PVS; ++ks)
#pragma unroll
                for (int i = 0; i < 4; ++i) psum = Mfma<T>::dot2(pf[ks][2 * i], pf[ks][2 * i + 1], psum);
            l_half = psum;
        };
        // O^T += V^T P^T for block j
        auto pv = [&](int j, const frag_t (&pf)[G::PVS]) __attribute__((always_inline)) {
            const uint32_t vj = vbase + (uint32_t)((j & (STAGES - 1)) * G::STAGE + G::TILE);
            constexpr int N = G::PVS * DB;
            auto vread = [&](int i) __attribute__((always_inline)) {
                const int ks = i / DB, db = i % DB;
                BPT_LDS char* p = lds + (vj ^ (64u * (db & 3))) + (db >> 2) * 256 + ks * 16 * D * 2;
                short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BPT_LDS short4_t*)p);
                short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BPT_LDS short4_t*)(p + 8 * D * 2));
                return __builtin_bit_cast(frag_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            };
            frag_t vf[PD + 1];
#pragma unroll
            for (int i = 0; i < PD; ++i) vf[i] = vread(i);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                if (i + PD < N) vf[(i + PD) % (PD + 1)] = vread(i + PD);
                __builtin_amdgcn_sched_barrier(0);
                const int ks = i / DB, db = i % DB;
                oacc[db] = Mfma<T>::mma32(vf[i % (PD + 1)], pf[ks], oacc[db]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // Ring of STAGES: blocks 0 .. STAGES-2 are copied ahead; step j
        // publishes block j, then, during its S products, copies block
        // j+STAGES-1 into the stage block j-1 left.  Copies are issued past
        // the last block too (they
        // read zeros), so every publish lets the same STAGES-2 younger
        // blocks stay in flight.
        // publish block j: this wave's copies of it landed (vmcnt), every
        // wave's copies landed and every wave is done with block j-1
        // (s_barrier)
        auto publish = [&]() __attribute__((always_inline)) {
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(G::VM_AHEAD) : "memory");
        };
#pragma unroll
        for (int b = 0; b < STAGES - 1; ++b) issue(b);
        // host: RAGGED == (Skv % BN != 0)
        const int nfull = RAGGED ? nblk - 1 : nblk;
        float16_t s[G::KB];
        frag_t pf[G::PVS];
        int j = 0;
        for (; j < nfull; ++j) {
            publish();
            if constexpr (kPhasePrio) __builtin_amdgcn_s_setprio(1);
            qk.template operator()<true>(j, j + STAGES - 1, s);
            if constexpr (kPhasePrio) __builtin_amdgcn_s_setprio(0);
            softmax.template operator()<false>(j, s, pf);
            if constexpr (kPhasePrio) __builtin_amdgcn_s_setprio(1);
            pv(j, pf);
            if constexpr (kPhasePrio) __builtin_amdgcn_s_setprio(0);
        }
        if constexpr (RAGGED) {
            publish();
            qk.template operator()<false>(j, 0, s);
            softmax.template operator()<true>(j, s, pf);
            pv(j, pf);
        }
        // no copy may still be writing LDS when the workgroup ends
        wait_vm<0>();
    }

    // ---- O = O / l, rows < Sq ------------------------------------------------
    // the lane number read afresh: kept from the start, it and its half
    // would hold two registers through the key loop, which at D = 256 has
    // none to spare (the compiler spilled them)
    int lane_e;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
    const int he = lane_e >> 5;
    const float l_row = l_half + __shfl_xor(l_half, 32);
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    const int qrow = q0 + wave * 32 + (lane_e & 31);
    if (qrow < Sq) {
        OutT* orow = static_cast<OutT*>(a.O) + bh * a.sO + (long long)qrow * a.ldo;
        typedef OutT out4_t __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                out4_t v;
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = cvt_out<OutT>(oacc[db][4 * r4 + q] * inv);
                // plain stores: each lane writes 8-byte pieces of its row, which
                // the L2 merges (non-temporal stores measured 2% slower here)
                *(out4_t*)(orow + 32 * db + 8 * r4 + 4 * he) = v;
            }
    }
}

}  // namespace bpt
