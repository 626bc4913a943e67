// Device-side building blocks shared by the batch-invariant GEMM and
// attention kernels for gfx950 (CDNA4): element types, exact conversions,
// and the single MFMA instruction used per input dtype.
//
// Everything here is arithmetic-neutral except the MFMA step itself and the
// rounding helpers; both are used identically by every kernel configuration,
// which is what keeps results independent of tile choice.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Dt : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

template <int dt> struct Elem;
template <> struct Elem<DT_F32> { using T = float; static constexpr int bytes = 4; };
template <> struct Elem<DT_F16> { using T = uint16_t; static constexpr int bytes = 2; };
template <> struct Elem<DT_BF16> { using T = uint16_t; static constexpr int bytes = 2; };

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// Round to nearest even; NaN stays a (quiet) NaN; overflow goes to +-Inf.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
// v_cvt_f16_f32 in the default round-to-nearest-even mode, of the value f as an fp32 number.  The empty asm
// hides where f came from: the compiler would otherwise fuse an fmaf producing f with this conversion into
// one v_fma_mixlo_f16, which rounds the exact sum once to fp16 instead of to fp32 and then to fp16, and
// does so in some kernels and not in others (their outputs then differ in rare elements).
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
    asm("" : "+v"(f));
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int dt> __device__ __forceinline__ float load_as_f32(const void *p, int64_t idx);
template <> __device__ __forceinline__ float load_as_f32<DT_F32>(const void *p, int64_t idx) {
    return static_cast<const float *>(p)[idx];
}
template <> __device__ __forceinline__ float load_as_f32<DT_BF16>(const void *p, int64_t idx) {
    return bf16_to_f32(static_cast<const uint16_t *>(p)[idx]);
}
template <> __device__ __forceinline__ float load_as_f32<DT_F16>(const void *p, int64_t idx) {
    return f16_to_f32(static_cast<const uint16_t *>(p)[idx]);
}

template <int dt> __device__ __forceinline__ void store_from_f32(void *p, int64_t idx, float v);
template <> __device__ __forceinline__ void store_from_f32<DT_F32>(void *p, int64_t idx, float v) {
    static_cast<float *>(p)[idx] = v;
}
template <> __device__ __forceinline__ void store_from_f32<DT_BF16>(void *p, int64_t idx, float v) {
    static_cast<uint16_t *>(p)[idx] = (uint16_t)f32_to_bf16(v);
}
template <> __device__ __forceinline__ void store_from_f32<DT_F16>(void *p, int64_t idx, float v) {
    static_cast<uint16_t *>(p)[idx] = (uint16_t)f32_to_f16(v);
}

// Pack two fp32 values into one dword of two 16-bit elements (low = a).
template <int dt> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<DT_BF16>(float a, float b) {
    return f32_to_bf16(a) | (f32_to_bf16(b) << 16);
}
template <> __device__ __forceinline__ uint32_t pack2<DT_F16>(float a, float b) {
    return f32_to_f16(a) | (f32_to_f16(b) << 16);
}

// ---------------------------------------------------------------- the MFMA step
// One 16x16 output-fragment instruction per input dtype, used by every GEMM
// and attention kernel:
//   bf16 / fp16 : v_mfma_f32_16x16x32_{bf16,f16}; a lane holds 8 consecutive
//                 k of one row (A) or one column (B): lane l covers row /
//                 column l % 16 and k slots 8*(l/16) .. 8*(l/16)+7.
//   fp32        : v_mfma_f32_16x16x4_f32; lane l holds k slot l/16.
// The 16x16 fp32 result: lane l, register i holds row 4*(l/16)+i, column l%16.
template <int dt> struct Mfma;
template <> struct Mfma<DT_BF16> {
    static constexpr int KG = 32;
    using Frag = u32x4;
    static __device__ __forceinline__ f32x4 step(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<DT_F16> {
    static constexpr int KG = 32;
    using Frag = u32x4;
    static __device__ __forceinline__ f32x4 step(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<DT_F32> {
    static constexpr int KG = 4;
    using Frag = float;
    static __device__ __forceinline__ f32x4 step(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ u32x4 zero_u4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ u32x4 ldg16(const void *p) { return *static_cast<const u32x4 *>(p); }

#define BI_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]; expcnt and lgkmcnt left at max).
#define BI_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N) & 0xF) | (((N) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

}  // namespace bi
