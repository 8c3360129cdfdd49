// device.h -- device-side helpers shared by the HIP kernels: element
// conversions, the FP32 -> 16-bit narrowing epilogue, batch decoding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace mm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));

// FP32 -> BF16, round to nearest, ties to even; NaN stays a (quiet) NaN,
// values beyond the largest finite BF16 round to infinity.  gfx950 converts
// in hardware (v_cvt_pk_bf16_f32), one instruction and no branches.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    const __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// FP32 -> FP16 with the hardware conversion (IEEE round to nearest even,
// overflow to infinity, subnormals kept).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Element traits by ONNX type code.
template <int DT>
struct Elem;

template <>
struct Elem<MM_FLOAT> {
    using S = float;
    static constexpr int kVE = 4;  // elements per 16 bytes
    __device__ static __forceinline__ float to_f32(S x) { return x; }
    __device__ static __forceinline__ S from_f32(float x) { return x; }
};

template <>
struct Elem<MM_FLOAT16> {
    using S = uint16_t;
    static constexpr int kVE = 8;
    __device__ static __forceinline__ float to_f32(S x) { return f16_to_f32(x); }
    __device__ static __forceinline__ S from_f32(float x) { return f32_to_f16(x); }
    // Two narrowed values in one word, `lo` in the low half.
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
};

template <>
struct Elem<MM_BFLOAT16> {
    using S = uint16_t;
    static constexpr int kVE = 8;
    __device__ static __forceinline__ float to_f32(S x) { return bf16_to_f32(x); }
    __device__ static __forceinline__ S from_f32(float x) { return f32_to_bf16(x); }
    // Two narrowed values in one word, `lo` in the low half (one v_cvt_pk_bf16_f32).
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        const b2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
};

// MatMulInteger operands (fed to the signed INT8 matrix cores; see KArgs).
template <>
struct Elem<MM_INT8> {
    using S = int8_t;
    static constexpr int kVE = 16;
    __device__ static __forceinline__ float to_f32(S x) { return (float)x; }
    __device__ static __forceinline__ S from_f32(float x) { return (S)x; }
    __device__ static __forceinline__ uint32_t pack2(float, float) { return 0u; }
};

// ---- direct global-to-LDS loads (gfx950 buffer loads with the LDS destination)

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr uint32_t kOutOfRange = 0x80000000u;  // beyond every buffer range used here: the load returns zeros

// Raw buffer resource: 48-bit base, stride 0, 2^31 - 1 bytes of range.
__device__ __forceinline__ i32x4 buffer_rsrc(const void *base) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32) & 0xffff);
    r[2] = 0x7fffffff;
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from global into LDS at lds_base + 16 * lane.  The
// load takes its LDS address from M0.  The compiler reserves M0 and ignores
// it in a clobber list, so the asm cannot declare the write; the kernels
// that use this helper must compile to code that uses M0 for nothing else,
// and the build disassembles every such kernel and fails if the compiler
// writes or reads M0 anywhere in it (m0check.py).  Saving and restoring M0
// around each load cost 2-3 % on the DMA-bound tiles; the compiler-owned
// builtin for this load makes the compiler wait for all outstanding LDS
// loads before the next LDS read, which serialises the stage pipeline.
__device__ __forceinline__ void load_to_lds16(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(rsrc)
                 : "memory");
}

// s_waitcnt vmcnt(N), other counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Gemm epilogue for output (m, n): alpha * acc + beta * C(m, n), C read in
// its broadcast layout (scalar, per column n, per row m, or full); without C
// the result is alpha * acc.  Positions outside the output read nothing.
template <typename E>
__device__ __forceinline__ float gemm_epilogue(const KArgs &a, float acc, int64_t m, int64_t n) {
    if (a.c_mode == kBiasNone) return a.alpha * acc;
    float c = 0.0f;
    if (m < a.M && n < a.N) {
        const typename E::S *C = (const typename E::S *)a.C;
        const int64_t idx = a.c_mode == kBiasScalar ? 0 : a.c_mode == kBiasRow ? n : a.c_mode == kBiasCol ? m : m * a.ldc + n;
        c = E::to_f32(C[idx]);
    }
    return a.alpha * acc + a.beta * c;
}

// MatMulInteger: zero point minus the INT8 offset of a UINT8 operand, as a
// 32-bit value (modulo 2^32): mode 0 none, 1 scalar, 2 one per index i.
__device__ __forceinline__ uint32_t int_zp(const void *zp, int mode, int is_signed, int64_t i) {
    int32_t z = 0;
    if (mode != 0) {
        const int64_t at = mode == 1 ? 0 : i;
        z = is_signed ? (int32_t)((const int8_t *)zp)[at] : (int32_t)((const uint8_t *)zp)[at];
    }
    return (uint32_t)(z - (is_signed ? 0 : 128));
}

// Element offsets of the A and B matrices used by output batch `b`.
__device__ __forceinline__ void batch_offsets(const BatchDesc &bd, int64_t b, int64_t &oa, int64_t &ob) {
    oa = 0;
    ob = 0;
    for (int d = bd.nb - 1; d >= 0; --d) {
        int64_t n = bd.dim[d];
        int64_t i = b % n;
        b /= n;
        oa += i * bd.sa[d];
        ob += i * bd.sb[d];
    }
}

// Workgroups are dealt to the XCDs round-robin by their linear id.  Remap so
// that each XCD receives a contiguous range of logical tile ids (neighbouring
// tiles then share that XCD's L2).  Bijective on [0, n).
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t n) {
    const int64_t per = n / kNumXCDs, rem = n % kNumXCDs;
    const int64_t xcd = bid % kNumXCDs, local = bid / kNumXCDs;
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

}  // namespace mm
