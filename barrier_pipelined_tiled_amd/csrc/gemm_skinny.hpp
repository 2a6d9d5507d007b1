// gemm_skinny.hpp -- the memory-bound GEMM for few rows of A (decode-like
// shapes, e.g. 64 x 8192 x 8192): C (M x N) = A (M x K) * B (K x N).
//
// Such a product is bound by streaming B (K x N) from HBM once; A is small and
// stays in L2.  Two workgroup layouts are here.  In gemm_skinny_kernel a
// workgroup owns a 64 x BN output block (BN = 32 NB columns) over a range of
// K, and its waves split that range once more ("split-K inside the
// workgroup").  (gemm_skinny_ring_kernel, further down and the faster of the
// two, splits the columns over the waves instead and shares one ring; it is
// described there.)  Each wave streams its share through private LDS
// rings -- SB stages for B chunks and SA slots for A chunks -- filled by
// LDS-DMA, so the loop needs no workgroup barrier: a stage is published to the
// only wave that reads it by that wave's own vmcnt wait (the "bytes pending"
// half of the mbarrier page's completion rule; nobody else has to arrive).
// Everything asynchronous lands in LDS, never in registers, so no copy of an
// in-flight register can be made.  The wave partials are summed through LDS
// in a fixed wave order.
//
// HBM streams best when each workgroup reads wide pieces of a B row (a
// 256-byte piece reads at about 1.4x the rate of a 64-byte one), but a 128-
// column block leaves too few workgroups to occupy every CU on most shapes.
// So K may also be split across `splits` workgroups per block: each writes
// its fp32 partial block to a workspace, and a second, small kernel adds the
// `splits` partials of every block in split order (deterministic), converts
// and stores C.  The kernel boundary orders the two; a release/acquire pair
// inside one kernel would cost an L2 write-back per workgroup, several times
// the cost of the extra launch.
#pragma once
#include <utility>

#include "device_common.hpp"
#include "gemm_pipelined.hpp"   // swz_a

namespace bpt {

struct SkinnyArgs {
    const void* A;
    const void* B;
    void* C;
    int M, N, K;
    int lda, ldb, ldc;
    long long strideA, strideB, strideC;
    int tiles_n;            // column blocks of BN
    int splits;             // workgroups per block along K (1: no workspace)
    float* partial;         // splits > 1: [block][split][64][BN] fp32
};

template <typename T, int WAVES, int KC, int SB, int SA, int NB, typename OutT>
struct SkinnyGemm {
    static_assert(KC == 32 || KC == 64, "A swizzles exist for 64- and 128-byte rows");
    static_assert(SA >= 2 && SA - 1 <= SB - 2, "A runs PA = SA-1 chunks ahead, B at least one further");
    static_assert(NB == 1 || NB == 4, "B layouts exist for 64- and 256-byte rows");
    static constexpr int BM = 64, BN = 32 * NB;     // 2 x NB blocks of 32x32
    static constexpr int PA = SA - 1;               // A prefetch distance (chunks)
    static constexpr int KSTEPS = KC / 16;          // MFMA k-steps per chunk
    static constexpr int A_BYTES = BM * KC * 2;     // one A chunk
    static constexpr int B_BYTES = KC * BN * 2;     // one B chunk
    static constexpr int LA = A_BYTES / 1024;       // copies per A chunk
    static constexpr int LB = B_BYTES / 1024;       // copies per B chunk
    static constexpr int A_CHUNKS = KC / 8;         // 16-byte pieces per A row
    static constexpr int A_ROWS_PER_INST = 64 / A_CHUNKS;
    static constexpr int B_PIECES = BN / 8;         // 16-byte pieces per B row
    static constexpr int B_ROWS_PER_INST = 64 / B_PIECES;
    static constexpr int WAVE_LDS = SA * A_BYTES + SB * B_BYTES;
    static constexpr int RING_BYTES = WAVES * WAVE_LDS;
    // wave partials in LDS, rows padded by 16 bytes: the 32 rows one store
    // instruction writes then fall on different banks
    static constexpr int RED_PITCH = BN * 4 + 16;
    static constexpr int RED_WAVE = BM * RED_PITCH;
    static constexpr int RED_BYTES = WAVES * RED_WAVE;
    static constexpr int LDS_BYTES = RING_BYTES > RED_BYTES ? RING_BYTES : RED_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    // Issue order per chunk x is A(x+PA) (if it exists) then B(x+SB-1) (if it
    // exists).  Chunk c needs A(c) and the older B(c); A(c) came from chunk
    // c-PA.  vmcnt allowed at the top of chunk c = the copies issued after
    // A(c).  Steady state: B of chunk c-PA plus PA-1 full chunks.
    static constexpr int VM_STEADY = LB + (PA - 1) * (LA + LB);
    static_assert(VM_STEADY < 64, "vmcnt is 6 bits");
    // drain chunk d (0 .. SB-2), d counted from the first chunk with no B to
    // issue; x are chunk positions relative to it (negative = steady)
    static constexpr int vm_drain(int d) {
        int n = (d - PA < 0) ? LB : 0;              // the rest of chunk d-PA
        for (int x = d - PA + 1; x <= d - 1; ++x) n += ((x + PA < SB - 1) ? LA : 0) + ((x < 0) ? LB : 0);
        return n;
    }
    typedef typename Mfma<T>::frag_t frag_t;
};

// Compile-time check of the wait counts above: replay the issue order of a
// wave with nch chunks copy by copy and find, for every chunk, how many
// copies were issued after the last copy that chunk needs.
template <int SB, int PA, int LA, int LB, int VM_STEADY, int (*VM_DRAIN)(int)>
constexpr bool skinny_waits_match(int nch) {
    int kind[4096] = {}, chunk[4096] = {}, n = 0;        // issue log (kind 0 = A, 1 = B)
    auto push = [&](int k, int c, int cnt) {
        for (int i = 0; i < cnt; ++i) { kind[n] = k; chunk[n] = c; ++n; }
    };
    auto allowed = [&](int c) {                           // copies after the last one chunk c needs
        int last = -1;
        for (int i = 0; i < n; ++i)
            if (chunk[i] == c) last = i;
        return n - 1 - last;
    };
    for (int x = -(SB - 1); x < 0; ++x) {
        if (x + PA >= 0) push(0, x + PA, LA);
        push(1, x + SB - 1, LB);
    }
    int c = 0;
    for (; c + SB - 1 < nch; ++c) {
        if (allowed(c) != VM_STEADY) return false;
        push(0, c + PA, LA);
        push(1, c + SB - 1, LB);
    }
    for (int d = 0; d < SB - 1; ++d) {
        if (allowed(c + d) != VM_DRAIN(d)) return false;
        if (c + d + PA < nch) push(0, c + d + PA, LA);
    }
    return true;
}

// B rows of a 128-column block (16 pieces of 16 bytes): piece p of k row k
// sits at p ^ swz_b(k), the layout of the pipelined kernel's B tiles, which
// keeps both the copies and the transposed fragment reads conflict-free.
// 32-column rows (4 pieces) need none: 4 rows fill the 64 banks.
template <int NB>
__device__ inline int skinny_swz_b(int k) {
    if constexpr (NB == 4) return swz_b(k);
    return 0;
}

template <typename T, int WAVES, int KC, int SB, int SA, int NB, typename OutT>
__global__ __launch_bounds__(WAVES * 64, 1) void gemm_skinny_kernel(SkinnyArgs args) {
    typedef SkinnyGemm<T, WAVES, KC, SB, SA, NB, OutT> G;
    constexpr int PA = G::PA;
    static_assert(skinny_waits_match<SB, PA, G::LA, G::LB, G::VM_STEADY, &G::vm_drain>(SB) &&
                      skinny_waits_match<SB, PA, G::LA, G::LB, G::VM_STEADY, &G::vm_drain>(SB + 1) &&
                      skinny_waits_match<SB, PA, G::LA, G::LB, G::VM_STEADY, &G::vm_drain>(SB + 5),
                  "vmcnt counts disagree with the replayed issue order");
    typedef typename G::frag_t frag_t;
    constexpr int BN = G::BN;
    constexpr int BLOCK = G::BM * BN;               // outputs per block
    __shared__ __attribute__((aligned(1024))) char lds_raw[G::LDS_BYTES];
    BPT_LDS char* lds = (BPT_LDS char*)lds_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int splits = args.splits;

    // XCD-aware order: a run of consecutive workgroups -- neighbouring column
    // blocks with all their splits -- stays on one XCD, so neighbouring B
    // pieces share one L2.
    int pid = blockIdx.x;
    const int num = gridDim.x;
    if ((num & 7) == 0) pid = (pid & 7) * (num >> 3) + (pid >> 3);
    const int tile = pid / splits, split = pid - tile * splits;
    const int n0 = tile * BN;
    const int m0 = blockIdx.y * G::BM;
    const int batch = blockIdx.z;

    const T* Ab = static_cast<const T*>(args.A) + batch * args.strideA;
    const T* Bb = static_cast<const T*>(args.B) + batch * args.strideB;
    const int M = args.M, N = args.N, K = args.K, lda = args.lda, ldb = args.ldb;
    const int4_t rsA = make_rsrc(Ab, (uint32_t)(((M - 1) * (long long)lda + K) * 2));
    const int4_t rsB = make_rsrc(Bb, (uint32_t)(((K - 1) * (long long)ldb + N) * 2));

    // this workgroup's K range, and this wave's chunks in it, interleaved:
    // chunk c of wave w is chunk c*WAVES + w of the range, so the waves of a
    // workgroup read neighbouring rows of B at about the same time
    const int kwg = K / splits;                     // host: kwg % (WAVES*KC) == 0
    const int nchunks = kwg / (WAVES * KC);         // host: nchunks >= SB
    const int kbase = split * kwg + wave * KC;

    // A copies: chunk rows m (KC halves each); lane p of copy i brings row
    // i*A_ROWS_PER_INST + p/A_CHUNKS and lands at 16-byte slot p%A_CHUNKS of
    // it; the global piece it fetches is swizzled.  Rows >= M start past
    // num_records and read zeros.
    uint32_t voffA[G::LA];
#pragma unroll
    for (int i = 0; i < G::LA; ++i) {
        const int row = G::A_ROWS_PER_INST * i + lane / G::A_CHUNKS;
        const int chunk = (lane % G::A_CHUNKS) ^ swz_a<KC>(row);
        voffA[i] = (uint32_t)(((m0 + row) * lda + kbase + chunk * 8) * 2);
    }
    // B copies: chunk rows k of BN columns; lane p of copy i brings row
    // i*B_ROWS_PER_INST + p/B_PIECES into LDS piece p%B_PIECES of it, which
    // holds global piece (p%B_PIECES) ^ swz(k).  A lane whose 8 columns start
    // at or past N fetches the last in-bounds piece instead (host: N % 8 ==
    // 0); those columns are never stored.
    uint32_t voffB[G::LB];
#pragma unroll
    for (int i = 0; i < G::LB; ++i) {
        const int row = G::B_ROWS_PER_INST * i + lane / G::B_PIECES;
        int col = n0 + 8 * ((lane % G::B_PIECES) ^ skinny_swz_b<NB>(row));
        if (col >= N) col = N - 8;
        voffB[i] = (uint32_t)(((kbase + row) * ldb + col) * 2);
    }
    const uint32_t astep = WAVES * KC * 2;          // bytes per chunk along K
    const uint32_t bstep = (uint32_t)WAVES * KC * ldb * 2;

    // this wave's LDS: A slots [0, SA*A_BYTES), then B stages
    const uint32_t wlds = __builtin_amdgcn_readfirstlane(lds_addr(lds)) + wave * G::WAVE_LDS;
    BPT_LDS char* wlds_p = lds + wave * G::WAVE_LDS;

    auto issue_a = [&](int c) __attribute__((always_inline)) {
        const uint32_t dst = wlds + (c % SA) * G::A_BYTES;
#pragma unroll
        for (int i = 0; i < G::LA; ++i) dma16(rsA, dst + i * 1024, voffA[i], c * astep);
    };
    auto issue_b = [&](int c) __attribute__((always_inline)) {
        const uint32_t dst = wlds + SA * G::A_BYTES + (c % SB) * G::B_BYTES;
#pragma unroll
        for (int i = 0; i < G::LB; ++i) dma16(rsB, dst + i * 1024, voffB[i], c * bstep);
    };

    // fragment reads.  A (row block mb, k-step kk): row mb*32 + l%32, chunk
    // kk*2 + l/32, swizzled.  B block nb: a 16-lane group g reads rows kk*16 +
    // 8*(g/2) + 4h + j/4 and columns nb*32 + 16*(g%2) + 4*(j%4) (j = l%16),
    // transposed, i.e. logical piece 4nb + 2(g%2) + (j%4)/2, half (j%2); the
    // row's low two bits are j/4 for every kk and h, so is its swizzle.
    uint32_t rdA[G::KSTEPS];
#pragma unroll
    for (int kk = 0; kk < G::KSTEPS; ++kk) {
        const int row = lane % 32;                  // + mb*32 keeps the swizzle
        rdA[kk] = (uint32_t)(row * KC * 2 + (((kk * 2 + lane / 32) ^ swz_a<KC>(row)) * 16));
    }
    const int g = lane / 16, j = lane % 16;
    uint32_t rdB[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int piece = (4 * nb + 2 * (g % 2) + (j % 4) / 2) ^ skinny_swz_b<NB>(j / 4);
        rdB[nb] = (uint32_t)((8 * (g / 2) + j / 4) * BN * 2 + piece * 16 + (j % 2) * 8);
    }

    float16_t acc[2][NB];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = float16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int c) __attribute__((always_inline)) {
        BPT_LDS char* ap = wlds_p + (c % SA) * G::A_BYTES;
        BPT_LDS char* bp = wlds_p + SA * G::A_BYTES + (c % SB) * G::B_BYTES;
#pragma unroll
        for (int kk = 0; kk < G::KSTEPS; ++kk) {
            frag_t a[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) a[mb] = *(BPT_LDS frag_t*)(ap + rdA[kk] + mb * 32 * KC * 2);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                BPT_LDS char* p = bp + rdB[nb] + kk * 16 * BN * 2;
                short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BPT_LDS short4_t*)p);
                short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BPT_LDS short4_t*)(p + 4 * BN * 2));
                frag_t b = __builtin_bit_cast(frag_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) acc[mb][nb] = Mfma<T>::mma32(b, a[mb], acc[mb][nb]);
            }
        }
    };

    // Chunk c: B in stage c % SB, A in slot c % SA.  Chunk c waits for its
    // copies (vmcnt counts, see SkinnyGemm), retires its own reads of chunk
    // c-1 (lgkmcnt(0)) -- whose slot and stage are refilled next -- issues
    // A(c+PA) and B(c+SB-1), then computes.
    //
    // prologue = the pattern of chunks -(SB-1) .. -1
#pragma unroll
    for (int x = -(SB - 1); x < 0; ++x) {
        if (x + PA >= 0) issue_a(x + PA);
        issue_b(x + SB - 1);
    }

    int c = 0;
    for (; c + SB - 1 < nchunks; ++c) {             // steady: both copies exist
        wait_vm<G::VM_STEADY>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue_a(c + PA);
        issue_b(c + SB - 1);
        compute(c);
    }
    // drain, the last SB-1 chunks: no B left to issue, A while it exists
    auto drain_step = [&]<int D>() __attribute__((always_inline)) {
        wait_vm<G::vm_drain(D)>();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if constexpr (D + PA < SB - 1) issue_a(c + D + PA);
        compute(c + D);
    };
    [&]<int... D>(std::integer_sequence<int, D...>) {
        (drain_step.template operator()<D>(), ...);
    }(std::make_integer_sequence<int, SB - 1>{});

    // ---- the WAVES partial blocks, summed in fixed order --------------------
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // partial of this wave, row-major [64][BN] fp32 with RED_PITCH-byte rows
    // (lane's 4 consecutive columns per register group: the B-first MFMA
    // layout)
    BPT_LDS char* red = lds + wave * G::RED_WAVE;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                float4_t v = {acc[mb][nb][4 * gq], acc[mb][nb][4 * gq + 1], acc[mb][nb][4 * gq + 2],
                              acc[mb][nb][4 * gq + 3]};
                const int r = mb * 32 + lane % 32, col = nb * 32 + 8 * gq + 4 * (lane / 32);
                *(BPT_LDS float4_t*)(red + r * G::RED_PITCH + col * 4) = v;
            }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    OutT* Cb = static_cast<OutT*>(args.C) + batch * args.strideC;
    auto store_c = [&](int e, float4_t s) __attribute__((always_inline)) {
        const int r = e / BN, col = e % BN;
        const int grow = m0 + r, gcol = n0 + col;
        if (grow < M) {
            OutT* dst = Cb + (long long)grow * args.ldc + gcol;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (gcol + q < N) dst[q] = cvt_out<OutT>(s[q]);
        }
    };
    constexpr int STEP = WAVES * 64 * 4;            // 4 outputs per thread per pass
    auto wave_sum = [&](int e) __attribute__((always_inline)) {
        BPT_LDS char* q = lds + (e / BN) * G::RED_PITCH + (e % BN) * 4;
        float4_t s = *(BPT_LDS float4_t*)q;
#pragma unroll
        for (int w = 1; w < WAVES; ++w) s += *(BPT_LDS float4_t*)(q + w * G::RED_WAVE);
        return s;
    };
    if (splits == 1) {
        for (int e = tid * 4; e < BLOCK; e += STEP) store_c(e, wave_sum(e));
        return;
    }

    // ---- K split across workgroups: the partial goes to the workspace -------
    const long long blk = ((long long)batch * gridDim.y + blockIdx.y) * args.tiles_n + tile;
    float* part = args.partial + (blk * splits + split) * BLOCK;
    // plain stores: the sum kernel reads these right back (non-temporal
    // stores measured 1% slower per call here)
    for (int e = tid * 4; e < BLOCK; e += STEP) *(float4_t*)(part + e) = wave_sum(e);
}

// ---- the shared-ring skinny kernel -------------------------------------------
//
// Same block (64 x 128 outputs over a K range, K split over workgroups) and
// the same workspace and sum kernel as the wide kernel above, but the waves
// split the 128 columns instead of K: wave w owns columns 32w .. 32w+31 and
// every wave reads the same A chunk.  One ring of STAGES stages then serves
// the whole workgroup (A chunk + B chunk per stage), and the wave partials
// need no sum.  (Deeper rings, which this layout has room for, measured
// slower on 64 x 8192 x 8192 than 4 stages of 32-deep chunks.)  A stage
// is published like the pipelined kernel's: each wave's own copies landed
// (vmcnt) and its reads of the previous stage retired (lgkmcnt), then one
// s_barrier.  Copies issued for chunks past the workgroup's range go through
// a descriptor with no records: they land zeros, touch no memory and keep
// every wait count the same, so the loop has one form from first to last.
template <typename T, int KC, int STAGES, typename OutT>
struct SkinnyRing {
    static_assert(KC == 32 || KC == 64, "A swizzles exist for 64- and 128-byte rows");
    static constexpr int WAVES = 4, BM = 64, BN = 128;
    static constexpr int KSTEPS = KC / 16;
    static constexpr int A_BYTES = BM * KC * 2;
    static constexpr int B_BYTES = KC * BN * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LA = A_BYTES / 1024 / WAVES;   // copies per wave per stage
    static constexpr int LB = B_BYTES / 1024 / WAVES;
    static constexpr int LPS = LA + LB;
    static constexpr int A_CHUNKS = KC / 8;             // 16-byte pieces per A row
    static constexpr int A_ROWS_PER_INST = 64 / A_CHUNKS;
    static constexpr int B_ROWS_PER_INST = 4;           // 256-byte B rows
    static constexpr int LDS_BYTES = STAGES * STAGE;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    // at the top of chunk c the copies of chunks c+1 .. c+STAGES-2 may still
    // be in flight
    static constexpr int VM = (STAGES - 2) * LPS;
    static_assert(STAGES >= 2 && (STAGES - 1) * LPS < 64, "vmcnt is 6 bits");
    typedef typename Mfma<T>::frag_t frag_t;
};

template <typename T, int KC, int STAGES, typename OutT>
__global__ __launch_bounds__(256, 1) void gemm_skinny_ring_kernel(SkinnyArgs args) {
    typedef SkinnyRing<T, KC, STAGES, OutT> G;
    typedef typename G::frag_t frag_t;
    constexpr int BN = G::BN;
    constexpr int BLOCK = G::BM * BN;
    __shared__ __attribute__((aligned(1024))) char lds_raw[G::LDS_BYTES];
    BPT_LDS char* lds = (BPT_LDS char*)lds_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int splits = args.splits;

    // XCD-aware order, as in the wide kernel
    int pid = blockIdx.x;
    const int num = gridDim.x;
    if ((num & 7) == 0) pid = (pid & 7) * (num >> 3) + (pid >> 3);
    const int tile = pid / splits, split = pid - tile * splits;
    const int n0 = tile * BN;
    const int m0 = blockIdx.y * G::BM;
    const int batch = blockIdx.z;

    const T* Ab = static_cast<const T*>(args.A) + batch * args.strideA;
    const T* Bb = static_cast<const T*>(args.B) + batch * args.strideB;
    const int M = args.M, N = args.N, K = args.K, lda = args.lda, ldb = args.ldb;
    const int4_t rsA = make_rsrc(Ab, (uint32_t)(((M - 1) * (long long)lda + K) * 2));
    const int4_t rsB = make_rsrc(Bb, (uint32_t)(((K - 1) * (long long)ldb + N) * 2));
    const int4_t rsZ = make_rsrc(Bb, 0u);           // every access out of range: zeros

    const int kwg = K / splits;                     // host: kwg % KC == 0
    const int nchunks = kwg / KC;
    const int kbase = split * kwg;

    // copy i of wave w moves KiB number w*LA + i of the stage's A chunk, or
    // w*LB + i of its B chunk; pieces are swizzled as in the wide kernel
    uint32_t voffA[G::LA];
#pragma unroll
    for (int i = 0; i < G::LA; ++i) {
        const int row = (wave * G::LA + i) * G::A_ROWS_PER_INST + lane / G::A_CHUNKS;
        const int chunk = (lane % G::A_CHUNKS) ^ swz_a<KC>(row);
        voffA[i] = (uint32_t)(((m0 + row) * lda + kbase + chunk * 8) * 2);
    }
    uint32_t voffB[G::LB];
#pragma unroll
    for (int i = 0; i < G::LB; ++i) {
        const int row = (wave * G::LB + i) * G::B_ROWS_PER_INST + lane / 16;
        int col = n0 + 8 * ((lane % 16) ^ swz_b(row));
        if (col >= N) col = N - 8;
        voffB[i] = (uint32_t)(((kbase + row) * ldb + col) * 2);
    }
    const uint32_t astep = KC * 2;
    const uint32_t bstep = (uint32_t)KC * ldb * 2;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));

    auto issue = [&](int c) __attribute__((always_inline)) {
        const uint32_t dst = lds0 + (c % STAGES) * G::STAGE;
        if (c < nchunks) {                          // uniform
#pragma unroll
            for (int i = 0; i < G::LA; ++i) dma16(rsA, dst + (wave * G::LA + i) * 1024, voffA[i], c * astep);
#pragma unroll
            for (int i = 0; i < G::LB; ++i)
                dma16(rsB, dst + G::A_BYTES + (wave * G::LB + i) * 1024, voffB[i], c * bstep);
        } else {
#pragma unroll
            for (int i = 0; i < G::LPS; ++i) dma16(rsZ, dst + (wave * G::LPS + i) * 1024 % G::STAGE, 0u, 0u);
        }
    };

    // fragment reads: A as in the wide kernel; B block nb = wave
    uint32_t rdA[G::KSTEPS];
#pragma unroll
    for (int kk = 0; kk < G::KSTEPS; ++kk) {
        const int row = lane % 32;
        rdA[kk] = (uint32_t)(row * KC * 2 + (((kk * 2 + lane / 32) ^ swz_a<KC>(row)) * 16));
    }
    const int g = lane / 16, j = lane % 16;
    const int piece = (4 * wave + 2 * (g % 2) + (j % 4) / 2) ^ swz_b(j / 4);
    const uint32_t rdB = (uint32_t)(G::A_BYTES + (8 * (g / 2) + j / 4) * BN * 2 + piece * 16 + (j % 2) * 8);

    float16_t acc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
        acc[mb] = float16_t{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int c) __attribute__((always_inline)) {
        BPT_LDS char* sp = lds + (c % STAGES) * G::STAGE;
#pragma unroll
        for (int kk = 0; kk < G::KSTEPS; ++kk) {
            frag_t a[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) a[mb] = *(BPT_LDS frag_t*)(sp + rdA[kk] + mb * 32 * KC * 2);
            BPT_LDS char* p = sp + rdB + kk * 16 * BN * 2;
            short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BPT_LDS short4_t*)p);
            short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BPT_LDS short4_t*)(p + 4 * BN * 2));
            frag_t b = __builtin_bit_cast(frag_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) acc[mb] = Mfma<T>::mma32(b, a[mb], acc[mb]);
        }
    };

    // chunk c lives in stage c % STAGES; the copies of chunk c + STAGES - 1
    // refill the stage of chunk c - 1, which every wave has left by the
    // time the barrier of chunk c passes
#pragma unroll
    for (int x = 0; x < STAGES - 1; ++x) issue(x);
    for (int c = 0; c < nchunks; ++c) {
        publish<G::VM>();
        issue(c + STAGES - 1);
        compute(c);
    }
    wait_vm<0>();                                   // the trailing zero copies

    // lane l, register 4q+e of block mb: row mb*32 + l%32, column 32*wave +
    // 8q + 4(l/32) + e of the block (the B-first MFMA layout)
    OutT* Cb = static_cast<OutT*>(args.C) + batch * args.strideC;
    if (splits == 1) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int grow = m0 + mb * 32 + lane % 32;
                const int gcol = n0 + 32 * wave + 8 * q + 4 * (lane / 32);
                if (grow < M) {
                    OutT* dst = Cb + (long long)grow * args.ldc + gcol;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (gcol + e < N) dst[e] = cvt_out<OutT>(acc[mb][4 * q + e]);
                }
            }
        return;
    }
    const long long blk = ((long long)batch * gridDim.y + blockIdx.y) * args.tiles_n + tile;
    float* part = args.partial + (blk * splits + split) * BLOCK;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = mb * 32 + lane % 32, col = 32 * wave + 8 * q + 4 * (lane / 32);
            float4_t v = {acc[mb][4 * q], acc[mb][4 * q + 1], acc[mb][4 * q + 2], acc[mb][4 * q + 3]};
            *(float4_t*)(part + r * BN + col) = v;
        }
}

struct SkinnySumArgs {
    const float* partial;   // [block][split][64][BN] fp32, blocks ordered (batch, row block, column block)
    void* C;
    int M, N, ldc;
    long long strideC;
    int tiles_n, tiles_m;
    long long blocks;       // blocks of this launch
    int c_vec;              // C rows and batch entries start 16-byte aligned
};

// Eight outputs of C, one or two 16-byte non-temporal stores: C is written
// once and not read back here, and streaming stores that do not allocate in
// the L2 measured faster for every GEMM output tried.
template <typename OutT>
__device__ inline void store8(OutT* dst, float4_t lo, float4_t hi) {
    if constexpr (sizeof(OutT) == 4) {
        __builtin_nontemporal_store(lo, (float4_t*)dst);
        __builtin_nontemporal_store(hi, (float4_t*)(dst + 4));
    } else {
        typedef OutT out8_t __attribute__((ext_vector_type(8)));
        out8_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[q] = cvt_out<OutT>(lo[q]);
            v[q + 4] = cvt_out<OutT>(hi[q]);
        }
        __builtin_nontemporal_store(v, (out8_t*)dst);
    }
}

// C block = sum over splits of the partial blocks, in split order.  One
// thread per 8 consecutive outputs of a block row: 2S 16-byte loads issued
// together, one 16-byte (or two) store when C's rows allow it.
template <int BN, int S, typename OutT>
__global__ __launch_bounds__(256) void skinny_sum_kernel(SkinnySumArgs args) {
    constexpr int BLOCK = 64 * BN;
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long blk = gid / (BLOCK / 8);
    if (blk >= args.blocks) return;
    const int e = (int)(gid - blk * (BLOCK / 8)) * 8;
    const float* p = args.partial + blk * S * BLOCK + e;
    float4_t lo, hi;
    if constexpr (S <= 8) {
        float4_t v[S][2];
#pragma unroll
        for (int q = 0; q < S; ++q) {
            v[q][0] = *(const float4_t*)(p + q * BLOCK);
            v[q][1] = *(const float4_t*)(p + q * BLOCK + 4);
        }
        lo = v[0][0];
        hi = v[0][1];
#pragma unroll
        for (int q = 1; q < S; ++q) {
            lo += v[q][0];
            hi += v[q][1];
        }
    } else {
        // more splits than registers for all of them: groups of 8 loads,
        // still added in split order
#pragma unroll
        for (int g = 0; g < S; g += 8) {
            float4_t v[8][2];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                v[q][0] = *(const float4_t*)(p + (g + q) * BLOCK);
                v[q][1] = *(const float4_t*)(p + (g + q) * BLOCK + 4);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (g + q == 0) {
                    lo = v[q][0];
                    hi = v[q][1];
                } else {
                    lo += v[q][0];
                    hi += v[q][1];
                }
            }
        }
    }
    const int tn = (int)(blk % args.tiles_n);
    const long long rest = blk / args.tiles_n;
    const int tm = (int)(rest % args.tiles_m);
    const long long batch = rest / args.tiles_m;
    const int row = tm * 64 + e / BN, col = tn * BN + e % BN;
    if (row >= args.M) return;
    OutT* dst = static_cast<OutT*>(args.C) + batch * args.strideC + (long long)row * args.ldc + col;
    if (args.c_vec && col + 8 <= args.N) {
        store8<OutT>(dst, lo, hi);
        return;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (col + q < args.N) dst[q] = cvt_out<OutT>(lo[q]);
        if (col + 4 + q < args.N) dst[4 + q] = cvt_out<OutT>(hi[q]);
    }
}

}  // namespace bpt
