// device_common.hpp -- gfx950 (CDNA4) building blocks shared by the GEMM
// kernels: vector types, buffer resource descriptors, LDS-DMA loads, the
// explicit wait/barrier primitives and the MFMA wrappers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpt {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));

#define BPT_LDS __attribute__((address_space(3)))

typedef int int4_t __attribute__((ext_vector_type(4)));

// Word 3 of a gfx9-family raw buffer resource: 32-bit data format, no
// swizzle, no stride, so num_records counts bytes and any access at or past
// num_records returns zero instead of touching memory.
constexpr int kBufferWord3 = 0x00020000;

// 128-bit buffer resource for `bytes` bytes starting at `base` (wave-uniform).
__device__ inline int4_t make_rsrc(const void* base, uint32_t bytes) {
    uint64_t p = reinterpret_cast<uint64_t>(base);
    int4_t r;
    r[0] = (int)(uint32_t)p;
    r[1] = (int)((p >> 32) & 0xffff);     // stride 0, no swizzle
    r[2] = (int)bytes;
    r[3] = kBufferWord3;
    return r;
}

// s_waitcnt immediate for "vmcnt(0)" alone (expcnt and lgkmcnt at their
// maxima, i.e. not waited for), for __builtin_amdgcn_s_waitcnt, which the
// compiler's own wait insertion takes into account (an inline-asm wait is
// opaque to it).
constexpr int kWaitVmcnt0 = 0x0F70;

// Wait until at most N of this wave's vector memory operations are
// outstanding (loads and LDS-DMA copies complete in issue order).
template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// 32-bit LDS address of a pointer into LDS.
__device__ inline uint32_t lds_addr(const BPT_LDS void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

#ifdef BPT_LDS_POISON
// Race-detection build (libbpt_gemm_poison.so): right before a copy is
// issued, its KiB of LDS is filled with 0x7fc0 halves, a NaN both as fp16 and
// as bf16, and the write is waited for.  A read of a ring stage that is not
// ordered after the copy's landing, or a copy issued while some wave still
// reads the stage's previous contents, then turns into NaN in the result
// instead of stale but plausible values.  The fill runs where the copy does,
// after the same publish, so it adds no ordering of its own.
__device__ inline void lds_poison_1k(uint32_t lds) {
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int4_t nan4 = {0x7fc07fc0, 0x7fc07fc0, 0x7fc07fc0, 0x7fc07fc0};
    asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(lds + 16u * lane), "v"(nan4) : "memory");
}
#endif

// One wave-wide 16-byte-per-lane global->LDS copy (LDS-DMA).  Lane p's 16
// bytes come from rsrc.base + voff + soff and land at lds + 16*p, i.e. one
// contiguous KiB per wave.  The copy is counted by this wave's vmcnt and has
// reached LDS once vmcnt has dropped past it.
//
// Written as inline asm on purpose: the compiler cannot prove that a DMA
// into one ring stage does not alias the reads of another stage, and for
// the builtin form it inserts a vmcnt(0) before every later LDS read, which
// serialises the pipeline.  Hidden from the compiler, these copies are
// accounted for only by the explicit publish<>() waits below.
__device__ inline void dma16(int4_t rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
#ifdef BPT_LDS_POISON
    lds_poison_1k(lds);
#endif
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// Publish a ring stage: wait until at most N of this wave's copies are still
// in flight (so the stage's copies of this wave have landed: the "bytes
// pending" half of a stage-ready condition), wait for this wave's LDS reads,
// then one s_barrier (the "all arrivals" half).  Every wave executes the same
// sequence of publish calls.  The memory clobber keeps the compiler from
// moving LDS reads across it.
template <int N>
__device__ inline void publish() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Lanes of one wave hand data to each other through LDS (write by one lane,
// read by another).  The hardware runs a wave's LDS instructions in order,
// but the compiler sees unsynchronised accesses of different lanes and may
// reorder them; this fence orders them at wave scope (no instruction is
// emitted for it).
__device__ inline void wave_lds_handoff() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

template <typename T>
struct Mfma;

template <>
struct Mfma<_Float16> {
    typedef _Float16 elem_t;
    typedef half8_t frag_t;
    __device__ static inline float16_t mma32(frag_t a, frag_t b, float16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    // acc + x + y in one v_dot2 (the pair dotted with (1, 1), fp32 sum)
    __device__ static inline float dot2(elem_t x, elem_t y, float acc) {
        typedef _Float16 pair_t __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2(pair_t{x, y}, pair_t{(_Float16)1.0f, (_Float16)1.0f}, acc, false);
    }
};

template <>
struct Mfma<__bf16> {
    typedef __bf16 elem_t;
    typedef bf16x8_t frag_t;
    __device__ static inline float16_t mma32(frag_t a, frag_t b, float16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline float dot2(elem_t x, elem_t y, float acc) {
        typedef __bf16 pair_t __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(pair_t{x, y}, pair_t{(__bf16)1.0f, (__bf16)1.0f}, acc, false);
    }
};

// Output conversions, round to nearest even.
template <typename OutT>
__device__ inline OutT cvt_out(float x);
template <>
__device__ inline float cvt_out<float>(float x) { return x; }
template <>
__device__ inline _Float16 cvt_out<_Float16>(float x) { return (_Float16)x; }
template <>
__device__ inline __bf16 cvt_out<__bf16>(float x) { return (__bf16)x; }

}  // namespace bpt
