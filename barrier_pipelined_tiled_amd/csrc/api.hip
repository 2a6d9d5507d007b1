// api.hip -- host side of the C ABI: argument validation, variant choice on
// the host (the "Xe2 ESIMD GEMM" page, "Inner-loop rules" and "SPIR-V linker
// errors": runtime conditionals belong on the host, kernels are compile-time
// variants) and the asynchronous launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/bpt_gemm.h"
#include "attention.hpp"
#include "gemm_apair.hpp"
#include "gemm_persist.hpp"
#include "gemm_persist_ares.hpp"
#include "gemm_persist_roles.hpp"
#include "gemm_generic.hpp"
#include "gemm_pipelined.hpp"
#include "gemm_skinny.hpp"
#include "repack.hpp"
#include "splitk.hpp"

namespace {

thread_local std::string g_last_error;

bpt_status fail(bpt_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bpt_status fail(bpt_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

enum Variant {
    V_AUTO = 0,
    V_GENERIC = 1,          // guarded 64x64, any shape / alignment
    V_PIPE_256_K64_S2 = 2,  // 256x256 tile, BK 64, 2 stages
    V_PIPE_128_K64_S2 = 3,  // 128x128 tile, BK 64, 2 stages
    V_PIPE_256_K32_S4 = 4,  // 256x256 tile, BK 32, 4 stages
    V_PIPE_256_K32_S5 = 5,  // 256x256 tile, BK 32, 5 stages
    V_PIPE_128_K32_S4 = 6,  // 128x128 tile, BK 32, 4 stages
    V_SKINNY = 7,           // 64x32 block over all of K, 4 waves split K, per-wave LDS rings
    V_SKINNY_WIDE = 8,      // 64x128 block, K also split over workgroups, + split-sum kernel
    V_REPACK = 9,           // zero-padded aligned copies of A and B, then a pipelined kernel
    // B given transposed (N x K): C = A * B^T
    V_BT_256_K32_S4 = 10,   // 256x256 tile, BK 32, 4 stages
    V_BT_128_K32_S4 = 11,   // 128x128 tile, BK 32, 4 stages
    V_BT_GENERIC = 12,      // guarded 64x64, any shape / alignment
    V_BT_256_K64_S2 = 13,   // 256x256 tile, BK 64 (128-byte rows of A and Bt), 2 stages
    V_PIPE_256_K32_S4_AP = 14,  // 256x256 tile, BK 32, 4 B stages, A copied in K-tile pairs (whole lines)
    V_SKINNY_RING = 15,     // 64x128 block, waves split the columns, one shared 4-stage ring, + split-sum kernel
    V_PERSIST = 16,         // persistent 256x128 kernel for K = 128/256, 16-bit C stored during the next tile
    V_BT_256_K32_S4_AP = 17,  // B transposed: 256x256 tile, A in K-tile pairs, B^T in 4 32-wide stages
    V_SPLITK = 18,          // few output tiles: K split over the pipelined kernel's batch, + split-sum kernel
    V_PERSIST_AP = 19,      // the persistent short-K kernel with A copied in K-tile pairs (whole lines)
    V_PERSIST_AR = 20,      // the persistent short-K kernel walking row blocks with their A panel kept in LDS
    V_PERSIST_RL = 21,      // the A-resident short-K kernel with wave roles: compute, copy and store waves
    V_COUNT = 21
};

bool is_bt_variant(int v) { return (v >= V_BT_256_K32_S4 && v <= V_BT_256_K64_S2) || v == V_BT_256_K32_S4_AP; }

const char* const kVariantNames[] = {
    "auto",
    "generic_64x64x16",
    "pipelined_256x256x64_s2",
    "pipelined_128x128x64_s2",
    "pipelined_256x256x32_s4",
    "pipelined_256x256x32_s5",
    "pipelined_128x128x32_s4",
    "skinny_64x32_w4_k64_s4",
    "skinny_64x128_w4_k32_s4_splitk",
    "repack_pipelined",
    "pipelined_bt_256x256x32_s4",
    "pipelined_bt_128x128x32_s4",
    "generic_bt_64x64x16",
    "pipelined_bt_256x256x64_s2",
    "pipelined_256x256x32_s4_apair",
    "skinny_64x128_ring_k32_s4_splitk",
    "persistent_256x128x32_shortk",
    "pipelined_bt_256x256x32_s4_apair",
    "splitk_pipelined",
    "persistent_256x128x32_shortk_apair",
    "persistent_256x128x32_shortk_aresident",
    "persistent_128x256x32_shortk_roles",
};

// K-tile and stage count of each pipelined variant (0 for the others)
constexpr int kVariantBK[] = {0, 0, 64, 64, 32, 32, 32, 0, 0, 0, 32, 32, 0, 64, 32, 0, 32, 32, 0, 32, 32, 32};
constexpr int kVariantStages[] = {0, 0, 2, 2, 4, 5, 4, 0, 0, 0, 4, 4, 0, 2, 4, 0, 4, 4, 0, 4, 3, 4};
// which of them take K % BK != 0 (see pipelined_ok); filled below from the
// kernels' own layout
bool variant_tail(int v);


struct Call {
    int dtype;
    long long batch, M, N, K, lda, ldb, ldc, sA, sB, sC;
    const void* A;
    const void* B;
    void* C;
    int out_fp32;
    long long nb = 0;       // columns of B when it is a padded copy (0: N)
    int bt = 0;             // 1: B is given transposed, N x K with ldb >= K
    void* ws = nullptr;     // workspace granted to the call (nullptr: none; the
                            // split paths then run unsplit, the repack route
                            // falls back to the guarded kernel)
};

constexpr long long kI31 = (1LL << 31) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Does the pipelined kernel with this tile give the partial last K-tile a
// stage of its own (ring + one stage fit in LDS)?
template <int BM, int BN, int BK, int STAGES>
constexpr bool kTail = bpt::PipelinedGemm<_Float16, BM, BN, BK, STAGES, 2, 2, _Float16>::TAIL;

// Can a pipelined variant with K-tile BK and STAGES ring stages take this
// call?  The prologue fills every stage, so K must span at least STAGES full
// tiles; a partial last tile needs the tail stage (`tail`) and K % 8 == 0
// (A chunks of 8 k values are wholly inside K or wholly past it).  Column
// chunks of B are 8 wide and must not straddle B's width: N % 8 == 0, or
// for a padded copy of B its width (c.nb) % 8 == 0.
bool pipelined_ok(const Call& c, int BK, int STAGES, bool tail) {
    const long long nb = c.nb > 0 ? c.nb : c.N;
    if (c.K <= 0 || c.K / BK < STAGES) return false;
    if (c.K % BK != 0 && !(tail && c.K % 8 == 0)) return false;
    if (nb % 8 != 0 || nb < c.N || nb > c.ldb) return false;
    if (!aligned16(c.A) || !aligned16(c.B)) return false;
    if (c.lda % 8 != 0 || c.ldb % 8 != 0) return false;
    if (c.sA % 8 != 0 || c.sB % 8 != 0) return false;
    // buffer offsets are 32-bit: each operand's extent (plus one tile of
    // rows past M) must stay below 2^31 bytes
    long long extA = ((c.M + 256) * c.lda + c.K) * 2;
    long long extB = (c.K * c.ldb + nb + 256) * 2;
    if (extA > kI31 || extB > kI31) return false;
    return true;
}

// the skinny kernel: 4 waves split K, 64-deep chunks, 4 B stages and 3 A
// slots per wave (the fastest of the measured ring shapes on 64 x 8192 x 8192)
constexpr int kSkWaves = 4, kSkChunk = 64, kSkStages = 4, kSkSlots = 3;

// operand requirements shared by both skinny kernels
bool skinny_operands_ok(const Call& c) {
    if (c.N % 8 != 0) return false;
    if (!aligned16(c.A) || !aligned16(c.B)) return false;
    if (c.lda % 8 != 0 || c.ldb % 8 != 0 || c.sA % 8 != 0 || c.sB % 8 != 0) return false;
    long long extA = ((c.M + 64) * c.lda + c.K) * 2;
    long long extB = (c.K * c.ldb + c.N + 64) * 2;
    return extA <= kI31 && extB <= kI31;
}

bool skinny_ok(const Call& c) {
    if (c.K <= 0 || c.K % (kSkWaves * kSkChunk) != 0) return false;
    if (c.K / (kSkWaves * kSkChunk) < kSkStages) return false;
    return skinny_operands_ok(c);
}

// the wide skinny kernel: 128-column blocks (256-byte B row pieces), 4 waves,
// 32-deep chunks, 4 B stages and 2 A slots per wave, K split over `splits`
// workgroups per block
constexpr int kSwWaves = 4, kSwChunk = 32, kSwStages = 4, kSwSlots = 2, kSwBN = 128;
constexpr long long kWorkspaceMax = 256LL << 20;   // bytes of split partials per call

long long wide_blocks_per_launch(const Call& c) {
    long long nb = c.batch < 65535 ? c.batch : 65535;
    return (c.N + kSwBN - 1) / kSwBN * ((c.M + 63) / 64) * nb;
}

bool wide_split_fits(const Call& c, int S) {
    const long long per = (long long)S * kSwWaves * kSwChunk;
    return c.K % per == 0 && c.K / per >= kSwStages;
}

// the shared-ring skinny kernel: same blocks and workspace, 32-deep K
// chunks, a 4-stage ring for the workgroup (48 KiB; 3, 6, 8 and 12 stages
// and 64-deep chunks measured slower on 64 x 8192 x 8192); any whole number
// of chunks per split
constexpr int kSrChunk = 32, kSrStages = 4;

bool ring_split_fits(const Call& c, int S) {
    return c.K % ((long long)S * kSrChunk) == 0;
}

// Splits for the split-K skinny kernels: the fewest that give one
// workgroup per CU (256), else the most that K allows, within the workspace
// limit; 0 when the kernel cannot take the call.
int skinny_splits(const Call& c, bool (*fits)(const Call&, int), long long target = 256) {
    if (c.K <= 0 || !skinny_operands_ok(c) || !fits(c, 1)) return 0;
    const long long blocks = wide_blocks_per_launch(c);
    int best = 1;
    for (int S = 2; S <= 64; S *= 2) {
        if (!fits(c, S)) break;
        if (blocks * S * 64 * kSwBN * 4 > kWorkspaceMax) break;
        if (blocks * best >= target) break;
        best = S;
    }
    return best;
}

int wide_splits(const Call& c) { return skinny_splits(c, wide_split_fits); }
int ring_splits(const Call& c) { return skinny_splits(c, ring_split_fits); }

// ---- workspace ----------------------------------------------------------------
// The fp32 partials of the split-K paths and the padded copies of the repack
// route live in device buffers from a pool per device.  Each buffer carries
// an event recorded on the caller's stream after the last kernel that used
// it, and a call that takes a buffer whose event has not completed makes its
// stream wait for that event first (hipStreamWaitEvent).  So calls on
// different streams -- hipStreamPerThread from several host threads, a new
// stream that received a destroyed one's handle while its kernels still ran
// -- never use a buffer at the same time, whatever their handles.
//
// A buffer is allocated when no pooled one is free and large enough (the
// first such call on the device, a call needing more than before, or calls
// in flight on more streams than the pool holds).  A grown-out buffer is
// kept, not freed, until the process ends: hipFree synchronises the device.
// Per device: at most kPoolSlots buffers (more only while more host threads
// are between taking and returning one), each at most the largest single
// request (split partials <= 256 MiB, repack copies <= 1 GiB), plus the
// grown-out ones, whose total stays below the final sizes (each replacement
// is at least twice the size it replaces).  A call made while its stream is
// being captured into a graph gets no buffer (a graph must not hold the
// address of a buffer a later call could outgrow) and runs its kernel
// unsplit, or the guarded kernel instead of the repack.
constexpr int kPoolSlots = 4;

struct WsSlot {
    void* ptr = nullptr;
    long long bytes = 0;
    hipEvent_t done = nullptr;       // recorded after the last kernel that used ptr
    hipStream_t last = nullptr;      // the stream handle it was recorded on
    bool recorded = false;
    bool busy = false;               // taken by a call that has not yet recorded `done`
};

struct WsPool {
    std::mutex mu;
    std::vector<std::unique_ptr<WsSlot>> slots;
    long long retired_bytes = 0;     // grown-out buffers, kept until exit
};

WsPool& pool_of(int dev) {
    static std::mutex mu;
    static std::map<int, std::unique_ptr<WsPool>> pools;
    std::lock_guard<std::mutex> lock(mu);
    auto& p = pools[dev];
    if (!p) p = std::make_unique<WsPool>();
    return *p;
}

}  // namespace

// Which pooled buffer a call takes (the pure policy; no HIP calls).  For
// slot i: bytes[i], busy[i] (0/1: taken by a call in progress), state[i] (0:
// never used, 1: its last use has completed, 2: its last use may still
// run), same[i] (1: that last use was recorded on the caller's stream
// handle).  Returns the slot to take, or n for a new buffer; *wait = 1 when
// the caller's stream must first wait for the slot's last use (every slot
// in state 2, the caller's own handle included), *grow = 1 when the slot is
// too small and gets a new buffer (the old one is kept and not waited for).
// Preference: an idle buffer; one last used on the caller's handle (a wait
// within one stream); a new buffer while the pool has fewer than `cap`;
// one busy with another stream's work (the wait orders the two); growing an
// idle-sized one; a new buffer beyond `cap`.
extern "C" int bpt_ws_choose(int n, const long long* bytes, const int* busy, const int* state, const int* same,
                             long long need, int cap, int* wait, int* grow) {
    *wait = 0;
    *grow = 0;
    for (int i = 0; i < n; ++i)
        if (!busy[i] && bytes[i] >= need && state[i] != 2) return i;
    for (int i = 0; i < n; ++i)
        if (!busy[i] && bytes[i] >= need && same[i]) {
            *wait = 1;
            return i;
        }
    if (n < cap) return n;
    for (int i = 0; i < n; ++i)
        if (!busy[i] && bytes[i] >= need) {
            *wait = 1;
            return i;
        }
    for (int i = 0; i < n; ++i)
        if (!busy[i]) {
            *grow = 1;
            return i;
        }
    return n;
}

namespace {

// A pooled buffer taken by one call: ptr is nullptr when the call gets none.
struct WsLease {
    WsPool* pool = nullptr;
    WsSlot* slot = nullptr;
    void* ptr = nullptr;
};

long long ws_size_for(long long need, long long old) {
    long long want = 1LL << 20;
    while (want < need) want *= 2;
    if (want < 2 * old) want = 2 * old;
    if (want > (1LL << 30)) want = need > (1LL << 30) ? need : (1LL << 30);
    return want;
}

WsLease ws_acquire(long long bytes, hipStream_t stream) {
    WsLease L;
    if (bytes <= 0) return L;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) {
        (void)hipGetLastError();
        return L;
    }
    if (cap != hipStreamCaptureStatusNone) return L;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return L;
    }
    WsPool& P = pool_of(dev);
    std::lock_guard<std::mutex> lock(P.mu);
    const int n = (int)P.slots.size();
    std::vector<long long> by(n);
    std::vector<int> busy(n), state(n), same(n);
    for (int i = 0; i < n; ++i) {
        const WsSlot& s = *P.slots[i];
        by[i] = s.bytes;
        busy[i] = s.busy;
        same[i] = s.recorded && s.last == stream;
        state[i] = 0;
        if (s.recorded) {
            const hipError_t q = hipEventQuery(s.done);
            if (q != hipSuccess) (void)hipGetLastError();      // hipErrorNotReady
            state[i] = q == hipSuccess ? 1 : 2;
        }
    }
    int wait = 0, grow = 0;
    const int i = bpt_ws_choose(n, by.data(), busy.data(), state.data(), same.data(), bytes, kPoolSlots, &wait,
                                &grow);
    WsSlot* s;
    if (i == n) {
        auto fresh = std::make_unique<WsSlot>();
        if (hipEventCreateWithFlags(&fresh->done, hipEventDisableTiming) != hipSuccess) {
            (void)hipGetLastError();
            return L;
        }
        P.slots.push_back(std::move(fresh));
        s = P.slots.back().get();
    } else {
        s = P.slots[i].get();
    }
    if (grow || s->ptr == nullptr) {
        void* p = nullptr;
        const long long want = ws_size_for(bytes, s->bytes);
        // relaxed capture mode for this thread around the allocation: in the
        // default (global) mode, an allocation while another thread captures
        // a stream in global mode could invalidate that capture
        hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
        const bool swapped = hipThreadExchangeStreamCaptureMode(&mode) == hipSuccess;
        const hipError_t e = hipMalloc(&p, (size_t)want);
        if (swapped) (void)hipThreadExchangeStreamCaptureMode(&mode);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return L;                    // the call runs without a workspace
        }
        P.retired_bytes += s->bytes;     // the old buffer (if any) is kept
        s->ptr = p;
        s->bytes = want;
        // a new buffer has no earlier use to wait for; `done` still marks the
        // old buffer's last use, which the new one does not share
        wait = 0;
    }
    if (wait && hipStreamWaitEvent(stream, s->done, 0) != hipSuccess) {
        (void)hipGetLastError();
        return L;
    }
    s->busy = true;
    L.pool = &P;
    L.slot = s;
    L.ptr = s->ptr;
    return L;
}

// Record the buffer's last use on the stream the call's kernels went to.
void ws_release(WsLease& L, hipStream_t stream) {
    if (L.slot == nullptr) return;
    std::lock_guard<std::mutex> lock(L.pool->mu);
    WsSlot* s = L.slot;
    if (hipEventRecord(s->done, stream) == hipSuccess) {
        s->recorded = true;
        s->last = stream;
    } else {
        // its last use cannot be ordered against later calls: keep the
        // buffer out of the pool for good
        (void)hipGetLastError();
        L.pool->retired_bytes += s->bytes;
        s->ptr = nullptr;
        s->bytes = 0;
        s->recorded = false;
    }
    s->busy = false;
    L.slot = nullptr;
}

// B given transposed: its tiles are K-contiguous like A's, so the same rules
// as for A apply and N needs no alignment (rows past N read as zero).
template <int BM, int BN, int BK, int STAGES>
constexpr bool kTailBt = bpt::PipelinedGemm<_Float16, BM, BN, BK, STAGES, 2, 2, _Float16, true>::TAIL;

bool pipelined_bt_ok(const Call& c, int BK, int STAGES, bool tail) {
    if (c.K <= 0 || c.K / BK < STAGES) return false;
    if (c.K % BK != 0 && !(tail && c.K % 8 == 0)) return false;
    if (!aligned16(c.A) || !aligned16(c.B)) return false;
    if (c.lda % 8 != 0 || c.ldb % 8 != 0 || c.sA % 8 != 0 || c.sB % 8 != 0) return false;
    long long extA = ((c.M + 256) * c.lda + c.K) * 2;
    long long extB = ((c.N + 256) * c.ldb + c.K) * 2;
    return extA <= kI31 && extB <= kI31;
}

// With B given transposed both operands are copied as rows of K, BK halves
// each: 64-wide K-tiles move 128-byte segments (whole cache lines) where
// 32-wide ones move half lines; measured 1143 against 948 TFLOP/s on the
// 4096 x 4096 x 16384 bf16 shape, 987 against 970 on 4096^3.  The A-pair
// kernel's BT form (A in whole-line pairs, B^T in 32-wide stages) goes
// further: 4096^3 1160 -> 1276, the long-K shape 1249 -> 1268, against the
// 64-wide 2-stage kernel.
bool apair_bt_ok(const Call& c) {
    return c.K % 64 == 0 && c.K >= 192 && pipelined_bt_ok(c, 32, 4, false);
}

int choose_bt(const Call& c) {
    const long long tiles256 = ((c.M + 255) / 256) * ((c.N + 255) / 256) * c.batch;
    if (tiles256 >= 128 && apair_bt_ok(c)) return V_BT_256_K32_S4_AP;
    if (tiles256 >= 128 && pipelined_bt_ok(c, 64, 2, kTailBt<256, 256, 64, 2>)) return V_BT_256_K64_S2;
    if (tiles256 >= 128 && pipelined_bt_ok(c, 32, 4, kTailBt<256, 256, 32, 4>)) return V_BT_256_K32_S4;
    if (pipelined_bt_ok(c, 32, 4, kTailBt<128, 128, 32, 4>)) return V_BT_128_K32_S4;
    return V_BT_GENERIC;
}

// the pipelined variant for a call one of them accepts in place (or for its
// repacked form); V_GENERIC when none does
// The A-pair variant reads A in 64-wide K pairs: K a multiple of 64 with at
// least 6 K-tiles (the 4-stage B ring plus a pair), no K tail; otherwise the
// requirements of the 32-wide 4-stage kernel.
bool apair_ok(const Call& c) {
    return c.K % 64 == 0 && c.K >= 192 && pipelined_ok(c, 32, 4, false);
}

// the persistent short-K kernel: whole 256 x 128 tiles only, K = 128 or
// 256, 16-bit C, and at least one tile per CU
bool persist_ok(const Call& c) {
    if (c.bt || c.out_fp32 || (c.K != 128 && c.K != 256) || c.M % 256 != 0 || c.N % 128 != 0) return false;
    if (!pipelined_ok(c, 32, 4, false)) return false;
    // C is stored in 8- and 16-byte pieces without edge checks
    if (!aligned16(c.C) || (c.ldc * 2) % 16 != 0 || (c.sC * 2) % 16 != 0) return false;
    const long long total = (c.M / 256) * (c.N / 128) * c.batch;
    return total >= 256 && total <= kI31;
}

// the persistent kernel with wave roles: whole 128 x 256 tiles, K = 128 or
// 256, 16-bit C, and at least one row block per CU
bool persist_roles_ok(const Call& c) {
    if (c.bt || c.out_fp32 || (c.K != 128 && c.K != 256) || c.M % 128 != 0 || c.N % 256 != 0) return false;
    if (!pipelined_ok(c, 32, 4, false)) return false;
    if (!aligned16(c.C) || (c.ldc * 2) % 16 != 0 || (c.sC * 2) % 16 != 0) return false;
    const long long groups = (c.M / 128) * c.batch;
    return groups >= 256 && groups * (c.N / 256) <= kI31;
}

int choose_pipelined(const Call& c) {
    const long long tiles256 = ((c.M + 255) / 256) * ((c.N + 255) / 256) * c.batch;
    const bool big = tiles256 >= 128;
    // short K over many tiles (8 or more per CU): the persistent kernel
    // stores each tile's C during the next tile's K-loop; 64 x 4096^2 x 256
    // 1.17 -> 1.03 ms, K = 128 0.58 -> 0.49 ms on one machine, and even at 4
    // tiles per CU it was 4% slower.  A copied in K-tile pairs (whole
    // 128-byte lines, half the A copy instructions): 64 x 4096^2 x 256
    // 0.860 -> 0.810 ms against the half-line copies on one machine
    // With K = 128 the kernel that keeps each row block's A panel in LDS and
    // streams only B: 64 x 4096^2 x 128 0.493 -> 0.466 ms; with K = 256 its
    // 3-stage ring leaves the stores no room and it is slower (0.90 ms)
    // Wave roles (compute, copy and store waves, the A panel in LDS): the
    // copies' waits no longer count stores; on one machine, alternating,
    // 64 x 4096^2 x 256 0.690 -> 0.611 ms against the A-pair kernel,
    // K = 128 0.455 -> 0.396 ms against the A-resident one, and 7-30% on
    // six other batched shapes of 4096 to 8192 tiles
    if (persist_roles_ok(c) && (c.M / 128) * (c.N / 256) * c.batch >= 2048) return V_PERSIST_RL;
    if (persist_ok(c) && (c.M / 256) * (c.N / 128) * c.batch >= 2048) return c.K == 128 ? V_PERSIST_AR : V_PERSIST_AP;
    // whole-line A copies: 4096^3 1230 -> 1270 TFLOP/s, 4096 x 4096 x 16384
    // 1393 -> 1417 against the 32-wide 4-stage kernel on the same machine
    if (big && apair_ok(c)) return V_PIPE_256_K32_S4_AP;
    if (big && pipelined_ok(c, 32, 4, variant_tail(V_PIPE_256_K32_S4))) return V_PIPE_256_K32_S4;
    if (pipelined_ok(c, 32, 4, variant_tail(V_PIPE_128_K32_S4))) return V_PIPE_128_K32_S4;
    if (big && pipelined_ok(c, 64, 2, variant_tail(V_PIPE_256_K64_S2))) return V_PIPE_256_K64_S2;
    if (pipelined_ok(c, 64, 2, variant_tail(V_PIPE_128_K64_S2))) return V_PIPE_128_K64_S2;
    return V_GENERIC;
}

// ---- repack route ------------------------------------------------------------
// A call no fast path reads in place (odd N or K, leading dimensions or bases
// not 16-byte aligned) is copied into zero-padded, aligned A' (M x K') and
// B' (K' x N'), K' and N' rounded up to 8, and the pipelined kernel runs on
// the copies, storing C at its true N.  Worth it when the product is large
// enough for the copies (each operand read and written once) to be small
// against the guarded kernel's time; limited by the workspace.
constexpr long long kRepackMax = 1LL << 30;        // bytes of padded copies per call

long long round8(long long x) { return (x + 7) / 8 * 8; }

// Which operands need the copy.  With K % 8 == 0 an operand whose base,
// leading dimension and batch stride are 16-byte granular (and, for B,
// whose N is a multiple of 8) is read in place; K % 8 != 0 pads both.
bool repack_a(const Call& c) {
    return c.K % 8 != 0 || !aligned16(c.A) || c.lda % 8 != 0 || c.sA % 8 != 0;
}
bool repack_b(const Call& c) {
    return c.K % 8 != 0 || !aligned16(c.B) || c.ldb % 8 != 0 || c.sB % 8 != 0 || c.N % 8 != 0;
}

long long repack_a_bytes(const Call& c) {
    return repack_a(c) ? (c.batch * c.M * round8(c.K) * 2 + 255) / 256 * 256 : 0;
}

long long repack_bytes(const Call& c) {
    return repack_a_bytes(c) + (repack_b(c) ? c.batch * round8(c.K) * round8(c.N) * 2 : 0);
}

Call repacked_call(const Call& c, void* ws) {
    const long long Kp = round8(c.K), Np = round8(c.N);
    Call r = c;
    r.K = Kp;
    if (repack_a(c)) {
        r.lda = Kp;
        r.sA = c.batch > 1 ? c.M * Kp : 0;
        r.A = ws;
    }
    if (repack_b(c)) {
        r.ldb = Np;
        r.sB = c.batch > 1 ? Kp * Np : 0;
        r.nb = Np;
        r.B = static_cast<char*>(ws) + repack_a_bytes(c);
    }
    return r;
}

// would the repacked call run on a pipelined variant (within the workspace
// limit)?
bool repack_feasible(const Call& c) {
    if (c.K <= 0 || c.M <= 0 || c.N <= 0 || c.batch <= 0) return false;
    if (repack_bytes(c) > kRepackMax) return false;
    alignas(256) static char probe[256];           // stands in for the 256-byte aligned workspace
    return choose_pipelined(repacked_call(c, probe)) != V_GENERIC;
}

// ... and is the product large enough (16 M multiply-adds) to pay for it?
bool repack_ok(const Call& c) {
    return (double)c.batch * c.M * c.N * c.K >= (double)(1 << 24) && repack_feasible(c);
}

// ---- split-K for the pipelined kernels ----------------------------------------
// An output of at most 128 tiles of 128 x 128 (fewer than half the CUs get
// a workgroup) is computed as S K-ranges at once: the pipelined kernel runs
// with the ranges as its batch (A advanced by K/S columns, B by K/S rows per
// entry) into fp32 partials in the call's workspace, and splitk_sum_kernel
// adds them in split order.  S is the largest power of two (at most 64) that
// keeps the tiles within one workgroup per CU, with K/S a multiple of 64 and
// at least 256.  With B given transposed, entry s reads Bt from column
// s*K/S (batch stride K/S).
Call splitk_call(const Call& c, int S, void* ws) {
    Call p = c;
    p.batch = S;
    p.K = c.K / S;
    p.sA = p.K;
    p.sB = c.bt ? p.K : p.K * c.ldb;
    p.C = ws;
    p.ldc = c.N;
    p.sC = c.M * c.N;
    p.out_fp32 = 1;
    return p;
}

// the pipelined variant for a call in either layout (the plain one when none)
int choose_layout(const Call& c) { return c.bt ? choose_bt(c) : choose_pipelined(c); }
bool is_generic(int v) { return v == V_GENERIC || v == V_BT_GENERIC; }

int splitk_splits(const Call& c) {
    if (c.batch != 1 || c.M <= 128 || c.K <= 0 || c.N % 8 != 0) return 0;
    const long long tiles = ((c.M + 127) / 128) * ((c.N + 127) / 128);
    alignas(256) static char probe[256];           // stands in for the workspace
    int best = 0;
    for (int S = 2; S <= 64; S *= 2) {
        if (tiles * S > 256) break;
        if (c.K % (64LL * S) != 0 || c.K / S < 256) break;
        if ((long long)S * c.M * c.N * 4 > kWorkspaceMax) break;
        if (is_generic(choose_layout(splitk_call(c, S, probe)))) break;
        best = S;
    }
    return best;
}

bool variant_tail(int v) {
    switch (v) {
        case V_PIPE_256_K64_S2: return kTail<256, 256, 64, 2>;
        case V_PIPE_128_K64_S2: return kTail<128, 128, 64, 2>;
        case V_PIPE_256_K32_S4: return kTail<256, 256, 32, 4>;
        case V_PIPE_256_K32_S5: return kTail<256, 256, 32, 5>;
        case V_PIPE_128_K32_S4: return kTail<128, 128, 32, 4>;
        default: return false;
    }
}

int choose(const Call& c) {
    if (c.bt) {
        const int v = choose_bt(c);
        return v != V_BT_GENERIC && splitk_splits(c) > 1 ? V_SPLITK : v;
    }
    // few rows of A: stream B once with a skinny kernel when that yields at
    // least half a workgroup per CU; the 128-column ones read B in 256-byte
    // row pieces, which stream faster than the narrow one's 64-byte pieces,
    // and the shared-ring one of them streams fastest and takes any K that
    // is a multiple of 32
    if (c.M <= 128) {
        const int S = ring_splits(c);
        const long long ring_wgs = S > 0 ? wide_blocks_per_launch(c) * S : 0;
        const long long tiles128 = (c.M + 127) / 128 * ((c.N + 127) / 128) * c.batch;
        if (c.M <= 64) {
            if (ring_wgs >= 128) return V_SKINNY_RING;
            if ((c.N + 31) / 32 * c.batch >= 128 && skinny_ok(c)) return V_SKINNY;
        } else if (tiles128 < 256 && ring_wgs >= 128) {
            // two row blocks of the ring kernel (B streamed once per block)
            // beat 128 x 128 tiles that give fewer than one workgroup per
            // CU: 128 x 8192^2 0.0627 -> 0.0393 ms, 96 x 8192^2 0.0539 ->
            // 0.0371, 128 x 4096^2 0.0315 -> 0.0152 on one machine; at 192
            // and 256 rows the two were even
            return V_SKINNY_RING;
        }
        // narrow outputs over long K: too few workgroups either way, but the
        // ring's K splits give more of them than the output tiles do (64 x
        // 512 x 65536: 32 against 4, 0.354 -> 0.058 ms; 64 x 256 x 8192
        // 0.0464 -> 0.0123 ms)
        if (tiles128 < 256 && ring_wgs > tiles128) return V_SKINNY_RING;
    }
    const int v = choose_pipelined(c);
    if (v != V_GENERIC) return splitk_splits(c) > 1 ? V_SPLITK : v;
    if (repack_ok(c)) return V_REPACK;
    return V_GENERIC;
}

template <typename T, typename OutT, int BM, int BN, int BK, int STAGES, bool BT = false>
hipError_t launch_pipelined(const Call& c, hipStream_t stream) {
    bpt::GemmArgs a;
    a.M = (int)c.M; a.N = (int)c.N; a.K = (int)c.K;
    a.lda = (int)c.lda; a.ldb = (int)c.ldb; a.ldc = (int)c.ldc;
    a.strideA = c.sA; a.strideB = c.sB; a.strideC = c.sC;
    a.tiles_m = (int)((c.M + BM - 1) / BM);
    a.tiles_n = (int)((c.N + BN - 1) / BN);
    a.group_m = 4;
    const long long ob = (long long)sizeof(OutT);
    a.c_vec = aligned16(c.C) && (c.ldc * ob) % 16 == 0 && (c.sC * ob) % 16 == 0;
    a.nb = (int)(c.nb > 0 ? c.nb : c.N);
    const long long tiles = (long long)a.tiles_m * a.tiles_n;
    for (long long b0 = 0; b0 < c.batch; b0 += 65535) {
        long long nb = c.batch - b0 < 65535 ? c.batch - b0 : 65535;
        a.A = static_cast<const T*>(c.A) + b0 * c.sA;
        a.B = static_cast<const T*>(c.B) + b0 * c.sB;
        a.C = static_cast<OutT*>(c.C) + b0 * c.sC;
        hipLaunchKernelGGL((bpt::gemm_pipelined_kernel<T, BM, BN, BK, STAGES, 2, 2, OutT, BT>),
                           dim3((unsigned)tiles, (unsigned)nb), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

template <typename T, typename OutT, bool BT = false>
hipError_t launch_apair(const Call& c, hipStream_t stream) {
    bpt::GemmArgs a;
    a.M = (int)c.M; a.N = (int)c.N; a.K = (int)c.K;
    a.lda = (int)c.lda; a.ldb = (int)c.ldb; a.ldc = (int)c.ldc;
    a.strideA = c.sA; a.strideB = c.sB; a.strideC = c.sC;
    a.tiles_m = (int)((c.M + 255) / 256);
    a.tiles_n = (int)((c.N + 255) / 256);
    a.group_m = 4;
    const long long ob = (long long)sizeof(OutT);
    a.c_vec = aligned16(c.C) && (c.ldc * ob) % 16 == 0 && (c.sC * ob) % 16 == 0;
    a.nb = (int)(c.nb > 0 ? c.nb : c.N);
    const long long tiles = (long long)a.tiles_m * a.tiles_n;
    for (long long b0 = 0; b0 < c.batch; b0 += 65535) {
        long long nb = c.batch - b0 < 65535 ? c.batch - b0 : 65535;
        a.A = static_cast<const T*>(c.A) + b0 * c.sA;
        a.B = static_cast<const T*>(c.B) + b0 * c.sB;
        a.C = static_cast<OutT*>(c.C) + b0 * c.sC;
        hipLaunchKernelGGL((bpt::gemm_apair_kernel<T, OutT, BT>), dim3((unsigned)tiles, (unsigned)nb), dim3(256), 0,
                           stream, a);
    }
    return hipGetLastError();
}

template <typename T, typename OutT, bool APAIR = false>
hipError_t launch_persist(const Call& c, hipStream_t stream) {
    bpt::GemmArgs a;
    a.A = c.A; a.B = c.B; a.C = c.C;
    a.M = (int)c.M; a.N = (int)c.N; a.K = (int)c.K;
    a.lda = (int)c.lda; a.ldb = (int)c.ldb; a.ldc = (int)c.ldc;
    a.strideA = c.sA; a.strideB = c.sB; a.strideC = c.sC;
    a.tiles_m = (int)(c.M / 256);
    a.tiles_n = (int)(c.N / 128);
    a.group_m = 4;
    a.c_vec = 1;
    a.nb = (int)c.N;
    const int total = (int)((long long)a.tiles_m * a.tiles_n * c.batch);
    const int grid = total < 256 ? total : 256;            // one workgroup per CU
    if constexpr (APAIR) {
        if (c.K == 256)
            hipLaunchKernelGGL((bpt::gemm_persist_apair_kernel<T, OutT, 8>), dim3((unsigned)grid), dim3(256), 0, stream,
                               a, total);
        else
            hipLaunchKernelGGL((bpt::gemm_persist_apair_kernel<T, OutT, 4>), dim3((unsigned)grid), dim3(256), 0, stream,
                               a, total);
    } else {
        if (c.K == 256)
            hipLaunchKernelGGL((bpt::gemm_persist_kernel<T, OutT, 8>), dim3((unsigned)grid), dim3(256), 0, stream, a,
                               total);
        else
            hipLaunchKernelGGL((bpt::gemm_persist_kernel<T, OutT, 4>), dim3((unsigned)grid), dim3(256), 0, stream, a,
                               total);
    }
    return hipGetLastError();
}

// The A-resident persistent kernel walks groups of gn column tiles of one
// row block.  The columns of a row block are split into nsplit ranges, the
// largest power of two with tiles_m * nsplit <= 32 that divides tiles_n:
// then the 32 workgroups of one XCD hold the groups of about one batch
// entry at a time (16 row blocks x 2 ranges for 4096 x 4096), and its L2
// holds that entry's B once.
template <typename T, typename OutT>
hipError_t launch_persist_ares(const Call& c, hipStream_t stream) {
    bpt::GemmArgs a;
    a.A = c.A; a.B = c.B; a.C = c.C;
    a.M = (int)c.M; a.N = (int)c.N; a.K = (int)c.K;
    a.lda = (int)c.lda; a.ldb = (int)c.ldb; a.ldc = (int)c.ldc;
    a.strideA = c.sA; a.strideB = c.sB; a.strideC = c.sC;
    a.tiles_m = (int)(c.M / 256);
    a.tiles_n = (int)(c.N / 128);
    a.group_m = 1;
    a.c_vec = 1;
    a.nb = (int)c.N;
    int nsplit = 1;
    while (nsplit * 2 * a.tiles_m <= 32 && a.tiles_n % (nsplit * 2) == 0) nsplit *= 2;
    const int gn = a.tiles_n / nsplit;
    const int ngroups = (int)((long long)a.tiles_m * nsplit * c.batch);
    const int grid = ngroups < 256 ? ngroups : 256;        // one workgroup per CU
    if (c.K == 256)
        hipLaunchKernelGGL((bpt::gemm_persist_ares_kernel<T, OutT, 8>), dim3((unsigned)grid), dim3(256), 0, stream, a,
                           ngroups, gn, nsplit);
    else
        hipLaunchKernelGGL((bpt::gemm_persist_ares_kernel<T, OutT, 4>), dim3((unsigned)grid), dim3(256), 0, stream, a,
                           ngroups, gn, nsplit);
    return hipGetLastError();
}

// Groups are whole row blocks (128 rows, all N / 256 column tiles); one
// workgroup of 8 waves per CU.
template <typename T, typename OutT>
hipError_t launch_persist_roles(const Call& c, hipStream_t stream) {
    bpt::GemmArgs a;
    a.A = c.A; a.B = c.B; a.C = c.C;
    a.M = (int)c.M; a.N = (int)c.N; a.K = (int)c.K;
    a.lda = (int)c.lda; a.ldb = (int)c.ldb; a.ldc = (int)c.ldc;
    a.strideA = c.sA; a.strideB = c.sB; a.strideC = c.sC;
    a.tiles_m = (int)(c.M / 128);
    a.tiles_n = (int)(c.N / 256);
    a.group_m = 1;
    a.c_vec = 1;
    a.nb = (int)c.N;
    const int ngroups = (int)((long long)a.tiles_m * c.batch);
    const int grid = 256;                                  // persist_roles_ok: ngroups >= 256
    if (c.K == 256)
        hipLaunchKernelGGL((bpt::gemm_persist_roles_kernel<T, OutT, 8>), dim3((unsigned)grid), dim3(512), 0, stream, a,
                           ngroups, a.tiles_n);
    else
        hipLaunchKernelGGL((bpt::gemm_persist_roles_kernel<T, OutT, 4>), dim3((unsigned)grid), dim3(512), 0, stream, a,
                           ngroups, a.tiles_n);
    return hipGetLastError();
}

template <typename T, typename OutT>
hipError_t launch_skinny(const Call& c, hipStream_t stream) {
    bpt::SkinnyArgs a;
    a.M = (int)c.M; a.N = (int)c.N; a.K = (int)c.K;
    a.lda = (int)c.lda; a.ldb = (int)c.ldb; a.ldc = (int)c.ldc;
    a.strideA = c.sA; a.strideB = c.sB; a.strideC = c.sC;
    a.tiles_n = (int)((c.N + 31) / 32);
    a.splits = 1;
    a.partial = nullptr;
    const long long tm = (c.M + 63) / 64;
    for (long long b0 = 0; b0 < c.batch; b0 += 65535) {
        long long nb = c.batch - b0 < 65535 ? c.batch - b0 : 65535;
        a.A = static_cast<const T*>(c.A) + b0 * c.sA;
        a.B = static_cast<const T*>(c.B) + b0 * c.sB;
        a.C = static_cast<OutT*>(c.C) + b0 * c.sC;
        hipLaunchKernelGGL((bpt::gemm_skinny_kernel<T, kSkWaves, kSkChunk, kSkStages, kSkSlots, 1, OutT>),
                           dim3((unsigned)a.tiles_n, (unsigned)tm, (unsigned)nb), dim3(kSkWaves * 64), 0, stream, a);
    }
    return hipGetLastError();
}

template <typename OutT>
void launch_split_sum(const bpt::SkinnySumArgs& a, int S, hipStream_t stream) {
    const long long threads = a.blocks * 64 * kSwBN / 8;
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (S == 2) hipLaunchKernelGGL((bpt::skinny_sum_kernel<kSwBN, 2, OutT>), grid, dim3(256), 0, stream, a);
    else if (S == 4) hipLaunchKernelGGL((bpt::skinny_sum_kernel<kSwBN, 4, OutT>), grid, dim3(256), 0, stream, a);
    else if (S == 8) hipLaunchKernelGGL((bpt::skinny_sum_kernel<kSwBN, 8, OutT>), grid, dim3(256), 0, stream, a);
    else if (S == 16) hipLaunchKernelGGL((bpt::skinny_sum_kernel<kSwBN, 16, OutT>), grid, dim3(256), 0, stream, a);
    else if (S == 32) hipLaunchKernelGGL((bpt::skinny_sum_kernel<kSwBN, 32, OutT>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((bpt::skinny_sum_kernel<kSwBN, 64, OutT>), grid, dim3(256), 0, stream, a);
}

template <typename T, typename OutT, bool RING = false>
hipError_t launch_skinny_wide(const Call& c, hipStream_t stream) {
    int S = RING ? ring_splits(c) : wide_splits(c);
    float* ws = static_cast<float*>(c.ws);
    if (ws == nullptr) S = 1;           // S > 1 fits K, so S = 1 does too
    bpt::SkinnyArgs a;
    a.M = (int)c.M; a.N = (int)c.N; a.K = (int)c.K;
    a.lda = (int)c.lda; a.ldb = (int)c.ldb; a.ldc = (int)c.ldc;
    a.strideA = c.sA; a.strideB = c.sB; a.strideC = c.sC;
    a.tiles_n = (int)((c.N + kSwBN - 1) / kSwBN);
    a.splits = S;
    a.partial = ws;
    const long long tm = (c.M + 63) / 64;
    bpt::SkinnySumArgs r;
    r.partial = ws;
    r.M = (int)c.M; r.N = (int)c.N; r.ldc = (int)c.ldc;
    r.strideC = c.sC;
    r.tiles_n = a.tiles_n; r.tiles_m = (int)tm;
    const long long ob = (long long)sizeof(OutT);
    r.c_vec = aligned16(c.C) && (c.ldc * ob) % 16 == 0 && (c.sC * ob) % 16 == 0;
    for (long long b0 = 0; b0 < c.batch; b0 += 65535) {
        long long nb = c.batch - b0 < 65535 ? c.batch - b0 : 65535;
        a.A = static_cast<const T*>(c.A) + b0 * c.sA;
        a.B = static_cast<const T*>(c.B) + b0 * c.sB;
        a.C = static_cast<OutT*>(c.C) + b0 * c.sC;
        const dim3 grid((unsigned)(a.tiles_n * S), (unsigned)tm, (unsigned)nb);
        if constexpr (RING)
            hipLaunchKernelGGL((bpt::gemm_skinny_ring_kernel<T, kSrChunk, kSrStages, OutT>), grid, dim3(256), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((bpt::gemm_skinny_kernel<T, kSwWaves, kSwChunk, kSwStages, kSwSlots, 4, OutT>), grid,
                               dim3(kSwWaves * 64), 0, stream, a);
        if (S > 1) {
            r.C = a.C;
            r.blocks = a.tiles_n * tm * nb;
            launch_split_sum<OutT>(r, S, stream);
        }
    }
    return hipGetLastError();
}

template <typename T, typename OutT, bool BT = false>
hipError_t launch_generic(const Call& c, hipStream_t stream) {
    bpt::GenericArgs a;
    a.M = c.M; a.N = c.N; a.K = c.K;
    a.lda = c.lda; a.ldb = c.ldb; a.ldc = c.ldc;
    a.strideA = c.sA; a.strideB = c.sB; a.strideC = c.sC;
    const long long tm = (c.M + 63) / 64, tn = (c.N + 63) / 64;
    a.tiles_n = (int)tn;
    for (long long b0 = 0; b0 < c.batch; b0 += 65535) {
        long long nb = c.batch - b0 < 65535 ? c.batch - b0 : 65535;
        a.A = static_cast<const T*>(c.A) + b0 * c.sA;
        a.B = static_cast<const T*>(c.B) + b0 * c.sB;
        a.C = static_cast<OutT*>(c.C) + b0 * c.sC;
        hipLaunchKernelGGL((bpt::gemm_generic_kernel<T, OutT, BT>), dim3((unsigned)(tm * tn), (unsigned)nb),
                           dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

template <typename OutT>
hipError_t launch_zero(const Call& c, hipStream_t stream) {
    long long total = c.M * c.N;
    long long blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    for (long long b0 = 0; b0 < c.batch; b0 += 65535) {
        long long nb = c.batch - b0 < 65535 ? c.batch - b0 : 65535;
        hipLaunchKernelGGL((bpt::fill_zero_kernel<OutT>), dim3((unsigned)blocks, (unsigned)nb), dim3(256), 0,
                           stream, static_cast<OutT*>(c.C) + b0 * c.sC, c.M, c.N, c.ldc, c.sC);
    }
    return hipGetLastError();
}

template <typename T, typename OutT>
hipError_t dispatch_typed(const Call& c, int v, hipStream_t stream);

void launch_repack_copy(const void* src, long long ld, long long stride, void* dst, long long ldd, long long strided,
                        long long batch, long long rows, long long cols, long long rows_p, long long cols_p,
                        hipStream_t stream) {
    bpt::RepackArgs a;
    a.src = src; a.dst = dst;
    a.ld = ld; a.stride = stride; a.ldd = ldd; a.strided = strided;
    a.rows = (int)rows; a.cols = (int)cols; a.rows_p = (int)rows_p; a.cols_p = (int)cols_p;
    a.total8 = batch * rows_p * cols_p / 8;
    long long blocks = (a.total8 + 255) / 256;
    if (blocks > 16384) blocks = 16384;            // grid-stride loop covers the rest
    if (blocks > 0)
        hipLaunchKernelGGL(bpt::repack_pad_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
}

// Split-K for few output tiles: the K ranges run as one batched call of a
// pipelined variant into fp32 partials in the call's workspace, then the
// in-order sum kernel writes C.  Without a workspace the call runs unsplit.
template <typename T, typename OutT>
hipError_t launch_splitk(const Call& c, hipStream_t stream) {
    const int S = splitk_splits(c);
    float* ws = S > 1 ? static_cast<float*>(c.ws) : nullptr;
    if (ws == nullptr) {                // e.g. graph capture
        Call u = c;
        u.ws = nullptr;
        return dispatch_typed<T, OutT>(u, choose_layout(u), stream);
    }
    Call p = splitk_call(c, S, ws);
    p.ws = nullptr;                     // the partial products need none
    hipError_t e = dispatch_typed<T, float>(p, choose_layout(p), stream);
    if (e != hipSuccess) return e;
    bpt::SplitSumArgs a;
    a.partial = ws;
    a.C = c.C;
    a.M = c.M; a.N = c.N; a.ldc = c.ldc;
    a.splits = S;
    a.c_vec = aligned16(c.C) && (c.ldc * (long long)sizeof(OutT)) % 16 == 0;
    const long long threads = c.M * c.N / 8;
    hipLaunchKernelGGL((bpt::splitk_sum_kernel<OutT>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                       a);
    return hipGetLastError();
}

// Copy A and B into the call's workspace, zero-padded and aligned, then run
// the pipelined kernel on the copies.  Without a workspace (graph capture,
// allocation failure) the guarded kernel takes the call as it is.
template <typename T, typename OutT>
hipError_t launch_repack(const Call& c, hipStream_t stream) {
    if (repack_bytes(c) == 0) return dispatch_typed<T, OutT>(c, choose_pipelined(c), stream);   // nothing to copy
    void* ws = c.ws;
    if (ws == nullptr) return launch_generic<T, OutT>(c, stream);
    Call r = repacked_call(c, ws);
    r.ws = nullptr;
    if (repack_a(c))
        launch_repack_copy(c.A, c.lda, c.sA, const_cast<void*>(r.A), r.lda, c.M * r.lda, c.batch, c.M, c.K, c.M,
                           r.K, stream);
    if (repack_b(c))
        launch_repack_copy(c.B, c.ldb, c.sB, const_cast<void*>(r.B), r.ldb, r.K * r.ldb, c.batch, c.K, c.N, r.K,
                           r.nb, stream);
    return dispatch_typed<T, OutT>(r, choose_pipelined(r), stream);
}

template <typename T, typename OutT>
hipError_t dispatch_typed(const Call& c, int v, hipStream_t stream) {
    if (c.K == 0) return launch_zero<OutT>(c, stream);
    switch (v) {
        case V_PIPE_256_K64_S2: return launch_pipelined<T, OutT, 256, 256, 64, 2>(c, stream);
        case V_PIPE_128_K64_S2: return launch_pipelined<T, OutT, 128, 128, 64, 2>(c, stream);
        case V_PIPE_256_K32_S4: return launch_pipelined<T, OutT, 256, 256, 32, 4>(c, stream);
        case V_PIPE_256_K32_S5: return launch_pipelined<T, OutT, 256, 256, 32, 5>(c, stream);
        case V_PIPE_128_K32_S4: return launch_pipelined<T, OutT, 128, 128, 32, 4>(c, stream);
        case V_SKINNY: return launch_skinny<T, OutT>(c, stream);
        case V_SKINNY_WIDE: return launch_skinny_wide<T, OutT>(c, stream);
        case V_SKINNY_RING: return launch_skinny_wide<T, OutT, true>(c, stream);
        case V_REPACK: return launch_repack<T, OutT>(c, stream);
        case V_SPLITK: return launch_splitk<T, OutT>(c, stream);
        case V_BT_256_K32_S4: return launch_pipelined<T, OutT, 256, 256, 32, 4, true>(c, stream);
        case V_BT_128_K32_S4: return launch_pipelined<T, OutT, 128, 128, 32, 4, true>(c, stream);
        case V_BT_GENERIC: return launch_generic<T, OutT, true>(c, stream);
        case V_BT_256_K64_S2: return launch_pipelined<T, OutT, 256, 256, 64, 2, true>(c, stream);
        case V_PIPE_256_K32_S4_AP: return launch_apair<T, OutT>(c, stream);
        case V_BT_256_K32_S4_AP: return launch_apair<T, OutT, true>(c, stream);
        case V_PERSIST:
            if constexpr (sizeof(OutT) == 2) return launch_persist<T, OutT>(c, stream);
            return hipErrorInvalidValue;                      // persist_ok: 16-bit C only
        case V_PERSIST_AP:
            if constexpr (sizeof(OutT) == 2) return launch_persist<T, OutT, true>(c, stream);
            return hipErrorInvalidValue;
        case V_PERSIST_AR:
            if constexpr (sizeof(OutT) == 2) return launch_persist_ares<T, OutT>(c, stream);
            return hipErrorInvalidValue;
        case V_PERSIST_RL:
            if constexpr (sizeof(OutT) == 2) return launch_persist_roles<T, OutT>(c, stream);
            return hipErrorInvalidValue;
        default: return launch_generic<T, OutT>(c, stream);
    }
}

bpt_status validate(const Call& c) {
    if (c.dtype != 0 && c.dtype != 1) return fail(BPT_ERR_INVALID_ARG, "dtype must be 0 (fp16) or 1 (bf16), got %d", c.dtype);
    if (c.out_fp32 != 0 && c.out_fp32 != 1) return fail(BPT_ERR_INVALID_ARG, "out_fp32 must be 0 or 1, got %d", c.out_fp32);
    if (c.batch < 0 || c.M < 0 || c.N < 0 || c.K < 0)
        return fail(BPT_ERR_INVALID_ARG, "negative size: batch=%lld M=%lld N=%lld K=%lld", c.batch, c.M, c.N, c.K);
    if (c.lda < (c.K > 1 ? c.K : 1)) return fail(BPT_ERR_INVALID_ARG, "lda=%lld < max(1, K=%lld)", c.lda, c.K);
    if (c.bt) {
        if (c.ldb < (c.K > 1 ? c.K : 1)) return fail(BPT_ERR_INVALID_ARG, "ldbt=%lld < max(1, K=%lld)", c.ldb, c.K);
    } else if (c.ldb < (c.N > 1 ? c.N : 1)) {
        return fail(BPT_ERR_INVALID_ARG, "ldb=%lld < max(1, N=%lld)", c.ldb, c.N);
    }
    if (c.ldc < (c.N > 1 ? c.N : 1)) return fail(BPT_ERR_INVALID_ARG, "ldc=%lld < max(1, N=%lld)", c.ldc, c.N);
    if (c.sA < 0 || c.sB < 0 || c.sC < 0)
        return fail(BPT_ERR_INVALID_ARG, "negative batch stride: %lld %lld %lld", c.sA, c.sB, c.sC);
    const bool nonempty = c.batch > 0 && c.M > 0 && c.N > 0;
    if (nonempty) {
        if (c.C == nullptr) return fail(BPT_ERR_INVALID_ARG, "C is NULL");
        if (c.K > 0 && (c.A == nullptr || c.B == nullptr)) return fail(BPT_ERR_INVALID_ARG, "A or B is NULL");
    }
    if (c.M > kI31 || c.N > kI31 || c.K > kI31 || c.lda > kI31 || c.ldb > kI31 || c.ldc > kI31)
        return fail(BPT_ERR_UNSUPPORTED, "a dimension or leading dimension exceeds 2^31-1");
    return BPT_OK;
}

bool variant_accepts(const Call& c, int v) {
    // each layout has its own variants; split-K runs either layout's
    if (v != V_SPLITK && is_bt_variant(v) != (c.bt != 0)) return false;
    switch (v) {
        case V_BT_256_K32_S4: return pipelined_bt_ok(c, 32, 4, kTailBt<256, 256, 32, 4>);
        case V_BT_128_K32_S4: return pipelined_bt_ok(c, 32, 4, kTailBt<128, 128, 32, 4>);
        case V_BT_GENERIC: return true;
        case V_BT_256_K64_S2: return pipelined_bt_ok(c, 64, 2, kTailBt<256, 256, 64, 2>);
        case V_BT_256_K32_S4_AP: return apair_bt_ok(c);
        case V_GENERIC: return true;
        case V_SKINNY: return skinny_ok(c);
        case V_SKINNY_WIDE: return wide_splits(c) > 0;
        case V_SKINNY_RING: return ring_splits(c) > 0;
        case V_REPACK: return repack_feasible(c);
        case V_SPLITK: return splitk_splits(c) > 1;
        case V_PIPE_256_K32_S4_AP: return apair_ok(c);
        case V_PERSIST:
        case V_PERSIST_AP:
        case V_PERSIST_AR: return persist_ok(c);
        case V_PERSIST_RL: return persist_roles_ok(c);
        default:
            if (v > V_GENERIC && v < V_SKINNY) return pipelined_ok(c, kVariantBK[v], kVariantStages[v], variant_tail(v));
            return false;
    }
}

// Bytes of workspace the launch of variant v for this call would use (0:
// none): the fp32 partials of the split-K paths, the padded copies of the
// repack route.
long long workspace_need(const Call& c, int v) {
    if (c.K <= 0) return 0;
    switch (v) {
        case V_SKINNY_WIDE:
        case V_SKINNY_RING: {
            const int S = v == V_SKINNY_RING ? ring_splits(c) : wide_splits(c);
            return S > 1 ? wide_blocks_per_launch(c) * S * 64 * kSwBN * 4 : 0;
        }
        case V_SPLITK: {
            const int S = splitk_splits(c);
            return S > 1 ? (long long)S * c.M * c.N * 4 : 0;
        }
        case V_REPACK: return repack_bytes(c);
        default: return 0;
    }
}

bpt_status run(const Call& c, int variant, hipStream_t stream) {
    bpt_status s = validate(c);
    if (s != BPT_OK) return s;
    if (variant < 0 || variant > V_COUNT) return fail(BPT_ERR_INVALID_ARG, "no variant %d", variant);
    if (c.batch == 0 || c.M == 0 || c.N == 0) return BPT_OK;
    int v = variant == V_AUTO ? choose(c) : variant;
    if (c.K > 0 && !variant_accepts(c, v))
        return fail(BPT_ERR_UNSUPPORTED, "variant %s cannot take M=%lld N=%lld K=%lld lda=%lld ldb=%lld",
                    kVariantNames[v], c.M, c.N, c.K, c.lda, c.ldb);
    Call cw = c;
    WsLease lease = ws_acquire(workspace_need(c, v), stream);
    cw.ws = lease.ptr;
    hipError_t e;
    if (c.dtype == 0)
        e = c.out_fp32 ? dispatch_typed<_Float16, float>(cw, v, stream) : dispatch_typed<_Float16, _Float16>(cw, v, stream);
    else
        e = c.out_fp32 ? dispatch_typed<__bf16, float>(cw, v, stream) : dispatch_typed<__bf16, __bf16>(cw, v, stream);
    ws_release(lease, stream);
    if (e != hipSuccess) return fail(BPT_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
    return BPT_OK;
}

// ---- the no-allocation entry point (gemm_ex_noalloc) -------------------------
// For callers that cannot allocate (code under graph capture, loops that must
// not call hipMalloc): the split-K partials and repack copies go into one
// file-scope device array instead of the pool.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address on the current
// GPU comes from hipGetSymbolAddress, taken once per device on the first call
// there and kept; only that address is ever handed to a kernel.
constexpr long long kScratchBytes = 32LL << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

void* scratch_on_device(int dev) {
    static std::mutex mu;
    static std::map<int, void*> ptrs;
    std::lock_guard<std::mutex> lock(mu);
    auto it = ptrs.find(dev);
    if (it != ptrs.end()) return it->second;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        return nullptr;
    }
    ptrs[dev] = ptr;
    return ptr;
}

bpt_status run_noalloc(const Call& c, int variant, hipStream_t stream) {
    bpt_status s = validate(c);
    if (s != BPT_OK) return s;
    if (variant < 0 || variant > V_COUNT) return fail(BPT_ERR_INVALID_ARG, "no variant %d", variant);
    if (c.batch == 0 || c.M == 0 || c.N == 0) return BPT_OK;
    int v = variant == V_AUTO ? choose(c) : variant;
    if (c.K > 0 && !variant_accepts(c, v))
        return fail(BPT_ERR_UNSUPPORTED, "variant %s cannot take M=%lld N=%lld K=%lld lda=%lld ldb=%lld",
                    kVariantNames[v], c.M, c.N, c.K, c.lda, c.ldb);
    const long long need = workspace_need(c, v);
    if (need > kScratchBytes)
        return fail(BPT_ERR_UNSUPPORTED,
                    "variant %s needs %lld bytes of scratch for M=%lld N=%lld K=%lld batch=%lld; the "
                    "no-allocation entry point has %lld (use gemm_ex, or split the call)",
                    kVariantNames[v], need, c.M, c.N, c.K, c.batch, kScratchBytes);
    Call cw = c;
    if (need > 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(BPT_ERR_HIP, "hipGetDevice failed");
        }
        cw.ws = scratch_on_device(dev);
        if (cw.ws == nullptr) return fail(BPT_ERR_HIP, "hipGetSymbolAddress of the scratch array failed");
    }
    hipError_t e;
    if (c.dtype == 0)
        e = c.out_fp32 ? dispatch_typed<_Float16, float>(cw, v, stream) : dispatch_typed<_Float16, _Float16>(cw, v, stream);
    else
        e = c.out_fp32 ? dispatch_typed<__bf16, float>(cw, v, stream) : dispatch_typed<__bf16, __bf16>(cw, v, stream);
    if (e != hipSuccess) return fail(BPT_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
    return BPT_OK;
}

// ---------------------------------------------------------------------------
// attention: O = softmax(scale Q K^T) V
// ---------------------------------------------------------------------------

struct AttnCall {
    int dtype;
    long long BH, Sq, Skv, D;
    const void *Q, *K, *V;
    void* O;
    long long ldq, ldk, ldv, ldo, sQ, sK, sV, sO;
    float scale;
    int out_fp32;
};

// Workgroup shape per head dimension: waves (32 query rows each, two per
// SIMD so that one wave's softmax overlaps the other's matrix products), keys
// per block, ring stages.  Measured on 64 heads x 4096 x 4096: D = 256 at
// 1.03 ms with (8, 32, 4) against 1.24 ms with (4, 64, 2) (32-key blocks keep
// a wave within the 256 registers two waves per SIMD leave; (8, 64, 2) spills
// and took 1.78 ms); D = 128 at 0.539 ms with (8, 64, 2) against 0.557 ms.
// Shifting the two waves of a SIMD half a block apart (a stage refilled two
// blocks after its use, one stage more) measured slower: D = 256 1.003 ms
// against 0.967 with the waves in step, D = 128 0.542 against 0.513.
constexpr int kAttnWaves256 = 8, kAttnBlock256 = 32, kAttnStages256 = 4;
constexpr int kAttnWaves128 = 8, kAttnBlock128 = 64, kAttnStages128 = 2;

template <typename T, typename OutT>
hipError_t launch_attention(const AttnCall& c, hipStream_t stream) {
    bpt::AttnArgs a;
    a.Q = c.Q; a.K = c.K; a.V = c.V; a.O = c.O;
    a.Sq = (int)c.Sq; a.Skv = (int)c.Skv;
    a.ldq = (int)c.ldq; a.ldk = (int)c.ldk; a.ldv = (int)c.ldv; a.ldo = (int)c.ldo;
    a.sQ = c.sQ; a.sK = c.sK; a.sV = c.sV; a.sO = c.sO;
    a.c2 = (float)((double)c.scale * 1.4426950408889634);     // scale * log2(e)
    const bool pos = c.scale >= 0.f;
    auto go = [&](auto kernel, int waves) {
        a.q_tiles = (int)((c.Sq + 32 * waves - 1) / (32 * waves));
        hipLaunchKernelGGL(kernel, dim3((unsigned)(a.q_tiles * c.BH)), dim3(64 * waves), 0, stream, a);
    };
    constexpr int W256 = kAttnWaves256, B256 = kAttnBlock256, S256 = kAttnStages256;
    constexpr int W128 = kAttnWaves128, B128 = kAttnBlock128, S128 = kAttnStages128;
    // the instance with a masked last block only when Skv leaves one
    if (c.D == 256) {
        const bool ragged = c.Skv % B256 != 0;
        if (pos && ragged) go(bpt::attention_fwd_kernel<T, 256, OutT, true, W256, B256, S256, true>, W256);
        else if (pos) go(bpt::attention_fwd_kernel<T, 256, OutT, true, W256, B256, S256, false>, W256);
        else if (ragged) go(bpt::attention_fwd_kernel<T, 256, OutT, false, W256, B256, S256, true>, W256);
        else go(bpt::attention_fwd_kernel<T, 256, OutT, false, W256, B256, S256, false>, W256);
    } else {
        const bool ragged = c.Skv % B128 != 0;
        if (pos && ragged) go(bpt::attention_fwd_kernel<T, 128, OutT, true, W128, B128, S128, true>, W128);
        else if (pos) go(bpt::attention_fwd_kernel<T, 128, OutT, true, W128, B128, S128, false>, W128);
        else if (ragged) go(bpt::attention_fwd_kernel<T, 128, OutT, false, W128, B128, S128, true>, W128);
        else go(bpt::attention_fwd_kernel<T, 128, OutT, false, W128, B128, S128, false>, W128);
    }
    return hipGetLastError();
}

bpt_status attention_run(const AttnCall& c, hipStream_t stream) {
    if (c.dtype != 0 && c.dtype != 1) return fail(BPT_ERR_INVALID_ARG, "dtype must be 0 (fp16) or 1 (bf16), got %d", c.dtype);
    if (c.out_fp32 != 0 && c.out_fp32 != 1) return fail(BPT_ERR_INVALID_ARG, "out_fp32 must be 0 or 1, got %d", c.out_fp32);
    if (c.BH < 0 || c.Sq < 0 || c.Skv < 0 || c.D < 1)
        return fail(BPT_ERR_INVALID_ARG, "bad size: batch_heads=%lld seq_q=%lld seq_kv=%lld head_dim=%lld",
                    c.BH, c.Sq, c.Skv, c.D);
    if (c.ldq < c.D || c.ldk < c.D || c.ldv < c.D || c.ldo < c.D)
        return fail(BPT_ERR_INVALID_ARG, "a leading dimension is below head_dim=%lld (ldq=%lld ldk=%lld ldv=%lld ldo=%lld)",
                    c.D, c.ldq, c.ldk, c.ldv, c.ldo);
    if (c.sQ < 0 || c.sK < 0 || c.sV < 0 || c.sO < 0)
        return fail(BPT_ERR_INVALID_ARG, "negative stride: %lld %lld %lld %lld", c.sQ, c.sK, c.sV, c.sO);
    if (!std::isfinite(c.scale)) return fail(BPT_ERR_INVALID_ARG, "scale is not finite");
    if (c.BH == 0 || c.Sq == 0) return BPT_OK;
    if (c.Q == nullptr || c.O == nullptr) return fail(BPT_ERR_INVALID_ARG, "Q or O is NULL");
    if (c.Skv > 0 && (c.K == nullptr || c.V == nullptr)) return fail(BPT_ERR_INVALID_ARG, "K or V is NULL");
    if (c.D != 128 && c.D != 256) return fail(BPT_ERR_UNSUPPORTED, "head_dim %lld: only 128 and 256 are built", c.D);
    if (!aligned16(c.Q) || !aligned16(c.K) || !aligned16(c.V) || !aligned16(c.O) ||
        c.ldq % 8 || c.ldk % 8 || c.ldv % 8 || c.ldo % 8 || c.sQ % 8 || c.sK % 8 || c.sV % 8 || c.sO % 8)
        return fail(BPT_ERR_UNSUPPORTED, "attention needs 16-byte aligned bases and leading dimensions and "
                                         "strides that are multiples of 8 elements");
    const long long q_tiles = (c.Sq + 127) / 128;
    if ((c.Sq + 128) * c.ldq * 2 > kI31 || (c.Skv + 64) * c.ldk * 2 > kI31 || (c.Skv + 64) * c.ldv * 2 > kI31 ||
        c.Sq * c.ldo > kI31 || q_tiles * c.BH > kI31)
        return fail(BPT_ERR_UNSUPPORTED, "a head's Q, K, V or O extent, or the workgroup count, exceeds 2^31-1");
    hipError_t e;
    if (c.dtype == 0)
        e = c.out_fp32 ? launch_attention<_Float16, float>(c, stream) : launch_attention<_Float16, _Float16>(c, stream);
    else
        e = c.out_fp32 ? launch_attention<__bf16, float>(c, stream) : launch_attention<__bf16, __bf16>(c, stream);
    if (e != hipSuccess) return fail(BPT_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
    return BPT_OK;
}

}  // namespace

extern "C" {

bpt_status attention_fwd(int dtype, int64_t batch_heads, int64_t seq_q, int64_t seq_kv, int64_t head_dim,
                         const void* Q, int64_t ldq, int64_t strideQ,
                         const void* K, int64_t ldk, int64_t strideK,
                         const void* V, int64_t ldv, int64_t strideV,
                         void* O, int64_t ldo, int64_t strideO,
                         float scale, int out_fp32, struct ihipStream_t* stream) {
    AttnCall c{dtype, batch_heads, seq_q, seq_kv, head_dim, Q, K, V, O,
               ldq, ldk, ldv, ldo, strideQ, strideK, strideV, strideO, scale, out_fp32};
    return attention_run(c, reinterpret_cast<hipStream_t>(stream));
}

bpt_status gemm_ex(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                   const void* A, int64_t lda, int64_t strideA,
                   const void* B, int64_t ldb, int64_t strideB,
                   void* C, int64_t ldc, int64_t strideC,
                   int out_fp32, int variant, struct ihipStream_t* stream) {
    Call c{dtype, batch, M, N, K, lda, ldb, ldc, strideA, strideB, strideC, A, B, C, out_fp32};
    return run(c, variant, reinterpret_cast<hipStream_t>(stream));
}

bpt_status gemm_ex_noalloc(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                           const void* A, int64_t lda, int64_t strideA,
                           const void* B, int64_t ldb, int64_t strideB,
                           void* C, int64_t ldc, int64_t strideC,
                           int out_fp32, int variant, struct ihipStream_t* stream) {
    Call c{dtype, batch, M, N, K, lda, ldb, ldc, strideA, strideB, strideC, A, B, C, out_fp32};
    return run_noalloc(c, variant, reinterpret_cast<hipStream_t>(stream));
}

int64_t bpt_noalloc_scratch_bytes(void) { return kScratchBytes; }

bpt_status gemm_ex_bt(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                      const void* A, int64_t lda, int64_t strideA,
                      const void* Bt, int64_t ldbt, int64_t strideBt,
                      void* C, int64_t ldc, int64_t strideC,
                      int out_fp32, int variant, struct ihipStream_t* stream) {
    Call c{dtype, batch, M, N, K, lda, ldbt, ldc, strideA, strideBt, strideC, A, Bt, C, out_fp32};
    c.bt = 1;
    return run(c, variant, reinterpret_cast<hipStream_t>(stream));
}

bpt_status gemm_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                    void* C, int64_t ldc, int out_fp32, struct ihipStream_t* stream) {
    return gemm_ex(0, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, out_fp32, V_AUTO, stream);
}

bpt_status gemm_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                     void* C, int64_t ldc, int out_fp32, struct ihipStream_t* stream) {
    return gemm_ex(1, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, out_fp32, V_AUTO, stream);
}

bpt_status gemm_batched_f16(int64_t batch, int64_t M, int64_t N, int64_t K,
                            const void* A, int64_t lda, int64_t strideA,
                            const void* B, int64_t ldb, int64_t strideB,
                            void* C, int64_t ldc, int64_t strideC,
                            int out_fp32, struct ihipStream_t* stream) {
    return gemm_ex(0, batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, out_fp32, V_AUTO, stream);
}

int bpt_select_variant(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t lda, const void* B, int64_t ldb, int out_fp32) {
    Call c{dtype, batch, M, N, K, lda, ldb, N > 1 ? N : 1, 0, 0, 0, A, B, (void*)16, out_fp32};
    if (validate(c) != BPT_OK) return 0;
    if (batch == 0 || M == 0 || N == 0 || K == 0) return 0;
    return choose(c);
}

int bpt_select_variant_bt(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                          const void* A, int64_t lda, const void* Bt, int64_t ldbt, int out_fp32) {
    Call c{dtype, batch, M, N, K, lda, ldbt, N > 1 ? N : 1, 0, 0, 0, A, Bt, (void*)16, out_fp32};
    c.bt = 1;
    if (validate(c) != BPT_OK) return 0;
    if (batch == 0 || M == 0 || N == 0 || K == 0) return 0;
    return choose(c);
}

int bpt_variant_count(void) { return V_COUNT; }

const char* bpt_variant_name(int v) {
    if (v < 1 || v > V_COUNT) return nullptr;
    return kVariantNames[v];
}

const char* bpt_status_string(bpt_status s) {
    switch (s) {
        case BPT_OK: return "BPT_OK";
        case BPT_ERR_INVALID_ARG: return "BPT_ERR_INVALID_ARG";
        case BPT_ERR_UNSUPPORTED: return "BPT_ERR_UNSUPPORTED";
        case BPT_ERR_HIP: return "BPT_ERR_HIP";
    }
    return "unknown status";
}

const char* bpt_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
