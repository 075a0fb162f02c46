// Device helpers shared by the gfx950 attention kernels: vector types, MFMA
// wrappers, bf16 / fp16 packing, wave reductions and the direct global->LDS
// copy.
//
// 16-bit element types: the kernels carry 16-bit operands as bit containers
// (bf16x8, u32x4, u32x2) whatever the element type; only the MFMA opcode and
// the fp32 -> 16-bit rounding depend on it.  Kernels templated on
// `bool F16` read IEEE half inputs when F16 is true and bfloat16 otherwise,
// through the *_t<F16> wrappers below.
//
// MFMA lane layouts used throughout (wave64, 16x16 output tiles):
//   C/D  (f32x4): lane l holds C[4*(l/16) + i][l % 16], i = 0..3.
//   A/B of v_mfma_f32_16x16x32_bf16 (8 bf16 per lane): lane l holds
//        A[l % 16][k] / B[k][l % 16] for the 8 k of lane group g = l/16.
//   A/B of v_mfma_f32_16x16x16_bf16 (4 bf16 per lane): the 4 k of group g.
//   v_mfma_f32_32x32x16_bf16: A/B lane l holds row/column l % 32 and 8 k of
//        lane half l/32; C (f32x16): accumulator i of lane l is
//        C[8*(i/4) + 4*(l/32) + i%4][l % 32].
// The kernels only rely on A and B sharing one (group, slot) -> k map, so a
// contraction pairs A slot j of group g with B slot j of group g.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// MI355X (gfx950) has 8 XCDs of 32 compute units, each XCD with its own L2;
// the dispatcher deals workgroups to the XCDs round-robin by flat index.
// Only locality depends on this value, never correctness.
constexpr int kNumXcd = 8;
// Lazy rescaling: the running row maximum used for exponentiation is only
// raised when a new score exceeds it by more than this many log2 units, so
// probabilities stay below 2^kRescaleSlack and the accumulator rescale is
// rare.  Exact: numerator and denominator share the same reference maximum.
constexpr float kRescaleSlack = 8.0f;

// 24 wait states: more than any MFMA result needs before a VALU or
// v_accvgpr_read may read it
__device__ __forceinline__ void mfma_acc_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// acc *= alpha for an accumulator tile that lives in AGPRs, one register at
// a time through a temporary VGPR.  Written out so that the rare rescale of
// the output accumulators does not make the compiler move them into VGPRs.
__device__ __forceinline__ void scale_acc(f32x16& acc, float alpha) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float t;
        asm volatile(
            "v_accvgpr_read_b32 %1, %0\n\t"
            "v_mul_f32 %1, %1, %2\n\t"
            "v_accvgpr_write_b32 %0, %1"
            : "+a"(acc[i]), "=&v"(t)
            : "v"(alpha));
    }
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// MFMAs for either 16-bit element type (operands as bit containers).
template <bool F16>
__device__ __forceinline__ f32x16 mfma_32x32x16_t(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                      0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// The 32x32x16 MFMA with the accumulator pinned to AGPRs (srcC = dst =
// acc).  Used for the large O^T accumulators so that the register allocator
// keeps them in AGPRs and the score accumulators in VGPRs.  The compiler
// does not know this is an MFMA, so it inserts no wait states after it:
// every accumulator is used again only several MFMAs later, and code that
// reads the accumulators otherwise must first call mfma_acc_drain().
template <bool F16>
__device__ __forceinline__ void mfma_32x32x16_acc_t(const bf16x8& a, const bf16x8& b, f32x16& acc) {
    if constexpr (F16)
        asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <bool F16>
__device__ __forceinline__ f32x4 mfma_16x16x32_t(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                      0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
template <bool F16>
__device__ __forceinline__ f32x4 mfma_16x16x16_t(const u32x2& a, const u32x2& b, const f32x4& c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0,
                                                     0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                         c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// two floats -> two IEEE halves (round to nearest even)
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), f16x2));
}
template <bool F16>
__device__ __forceinline__ uint32_t pack2_t(float lo, float hi) {
    if constexpr (F16) return pack_f16x2(lo, hi);
    else return pack_bf16x2(lo, hi);
}
// acc + lo + hi of a packed pair of 16-bit values (one v_dot2c against
// ones; the products are exact)
template <bool F16>
__device__ __forceinline__ float add_pair_t(uint32_t packed, float acc) {
    if constexpr (F16) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, packed), h2{(_Float16)1.f, (_Float16)1.f}, acc, false);
    } else {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, packed), b2{(__bf16)1.f, (__bf16)1.f}, acc,
                                               false);
    }
}
template <bool F16>
__device__ __forceinline__ bf16x8 pack8_t(const f32x4& lo, const f32x4& hi) {
    u32x4 u;
    u.x = pack2_t<F16>(lo.x, lo.y);
    u.y = pack2_t<F16>(lo.z, lo.w);
    u.z = pack2_t<F16>(hi.x, hi.y);
    u.w = pack2_t<F16>(hi.z, hi.w);
    return __builtin_bit_cast(bf16x8, u);
}

// Byte permute: bytes 0-3 come from `lo`, 4-7 from `hi`.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}
constexpr uint32_t kSelLoHalves = 0x05040100u;  // {lo.h0, hi.h0}
constexpr uint32_t kSelHiHalves = 0x07060302u;  // {lo.h1, hi.h1}

// Max / sum over the two lane halves l, l^32 (the two halves holding one
// output column of a 32x32 MFMA tile).
// max of three floats in one v_max3_f32 (fmaxf chains also emit a NaN-
// quieting max per operand; scores here are never NaN)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// v_permlane32_swap with both operands = v leaves, in every lane, v of that
// lane and of its partner l ^ 32 in the two results (no LDS round trip).
__device__ __forceinline__ float max_over_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_over_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (the four lane groups
// that share one MFMA output column).
__device__ __forceinline__ float max_over_groups(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
__device__ __forceinline__ float sum_over_groups(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// 4s + a loads 4 bf16 (8 bytes); lane i receives element i % 4 of the load
// of lane 4s + i / 4 in slot s.  With lanes 4s..4s+3 reading 16 consecutive
// columns of row s of a row-major block, lane i gets column i of rows 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }
// Streaming 16-byte load (non-temporal hint): data read once, e.g. a KV cache.
__device__ __forceinline__ u32x4 ldg16_stream(const void* p) { return __builtin_nontemporal_load((const u32x4*)p); }
__device__ __forceinline__ bf16x8 ldg_bf16x8_stream(const void* p) {
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)p));
}
__device__ __forceinline__ bf16x8 ldg_bf16x8(const void* p) { return *(const bf16x8*)p; }

// Global -> LDS copies (global_load_lds_dwordx4: every lane supplies its own
// global address, lane i's 16 bytes land at M0 + instruction offset + 16 i;
// completion is tracked by vmcnt) are issued only from the inline asm below,
// which takes the LDS byte address as an operand constrained to M0: the
// compiler writes M0 itself and knows it is live, so no value it keeps in
// M0 is lost across these blocks.
// Inline asm (not the builtin) because the compiler stops tracking LDS
// reads precisely while it sees an LDS DMA in flight and waits for all of
// them (lgkmcnt(0)) before every use.  The asm has no register outputs;
// callers wait with wait_vmcnt<0>() and a barrier before reading the
// destination.  The leading s_nop covers a VALU->SGPR->VMEM read hazard on
// the base and the M0 write right before the copy.

// base (wave-uniform, SGPR pair) + voff (per lane) -> LDS byte address
// lds_byte + 16*lane.
__device__ __forceinline__ void copy16_to_lds_async(const void* base, uint32_t voff, uint32_t lds_byte) {
    asm volatile(
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(base), "{m0}"(lds_byte)
        : "memory");
}

// Four 1 KB copies S bytes apart (global base + S k -> LDS lds_byte + S k,
// k = 0..3) under one M0 value: the instruction offset moves both the
// global and the LDS address.
template <int S>
__device__ __forceinline__ void copy4_to_lds_async(const void* base, uint32_t voff, uint32_t lds_byte) {
    static_assert(S >= 1024 && 3 * S < 4096, "offset field");
    asm volatile(
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %0, %1\n\t"
        "global_load_lds_dwordx4 %0, %1 offset:%3\n\t"
        "global_load_lds_dwordx4 %0, %1 offset:%4\n\t"
        "global_load_lds_dwordx4 %0, %1 offset:%5"
        :
        : "v"(voff), "s"(base), "{m0}"(lds_byte), "n"(S), "n"(2 * S), "n"(3 * S)
        : "memory");
}

// The same copy with the non-temporal hint, for data read exactly once
// (an MLA latent cache streamed through LDS).
__device__ __forceinline__ void copy16_to_lds_async_stream(const void* base, uint32_t voff, uint32_t lds_byte) {
    asm volatile(
        "s_nop 4\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(voff), "s"(base), "{m0}"(lds_byte)
        : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform n known to be one of {0, A, B, A+B}.
template <int A, int B>
__device__ __forceinline__ void wait_vmcnt_of(int n) {
    if (n == A + B) wait_vmcnt<A + B>();
    else if (n == B) wait_vmcnt<B>();
    else if (n == A) wait_vmcnt<A>();
    else wait_vmcnt<0>();
}

// 32-bit LDS byte address of a __shared__ object
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(const char*)p;
}

// Scheduling hints: ask the compiler to place `first` LDS reads, then
// alternate one MFMA with one LDS read `steps` times (keeps reads running
// `first` operands ahead of the MFMA that consumes them).
template <int FIRST, int STEPS>
__device__ __forceinline__ void sched_reads_ahead() {
    __builtin_amdgcn_sched_group_barrier(0x100, FIRST, 0);
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
}


__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

}  // namespace mqa
