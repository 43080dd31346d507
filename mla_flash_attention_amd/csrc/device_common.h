// device_common.h -- small device helpers shared by the attention kernels (gfx950).
// Internal; included by attn.hip and mha.hip inside their anonymous namespaces.
#pragma once

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef _Float16 f16x8 __attribute__((__vector_size__(16)));
typedef float f32x4 __attribute__((__vector_size__(16)));
typedef short s16x4 __attribute__((__vector_size__(8)));
typedef unsigned u32x4 __attribute__((__vector_size__(16)));
typedef unsigned u32x2 __attribute__((__vector_size__(8)));

#define LDS_PTR(T) __attribute__((address_space(3))) T *

constexpr float kLog2e = 1.4426950408889634f;

template <typename T> __device__ __forceinline__ T bitcast_to(u32x4 v) {
    return __builtin_bit_cast(T, v);
}

template <int KIND>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (KIND == KV_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast_to<bf16x8>(a), bitcast_to<bf16x8>(b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast_to<f16x8>(a), bitcast_to<f16x8>(b),
                                                      c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(unsigned b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ unsigned f32_to_bf16_bits(float x) {   // nearest even
    return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)x);
}

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// two floats -> two f16 (nearest even) in one register: one v_cvt_pk_f16_f32
__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2v){lo, hi}, f16x2v));
}
// two floats -> two bf16 (nearest even) in one register: one v_cvt_pk_bf16_f32
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2v){lo, hi}, bf16x2v));
}

// Clamp to the finite f16 range [-65504, 65504]: a value past it then converts to the
// largest finite f16 instead of to infinity (NaN inputs are not defined for the path).
__device__ __forceinline__ float sat_f16(float x) { return __builtin_fminf(__builtin_fmaxf(x, -65504.f), 65504.f); }
__device__ __forceinline__ f16x2v sat_f16x2(f16x2v x) {
    const f16x2v hi = {(_Float16)65504.f, (_Float16)65504.f};
    return __builtin_elementwise_max(__builtin_elementwise_min(x, hi), -hi);
}

__device__ __forceinline__ float f16_bits_to_f32(unsigned short b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

template <int KIND> __device__ __forceinline__ unsigned pack_p(float lo, float hi) {
    if constexpr (KIND == KV_BF16)
        return pack_bf16x2(lo, hi);
    else
        return pack_f16x2(lo, hi);
}

__device__ __forceinline__ float wave_max_groups(float x) {
    // max over the four 16-lane groups (lanes l, l^16, l^32, l^48)
    auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}

__device__ __forceinline__ float wave_sum_groups(float x) {
    auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
    auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
}

// max over the 16 lanes of this lane's 16-lane group (DPP row rotations: VALU only)
__device__ __forceinline__ float group16_max(float x) {
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));  // row_ror:8
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));  // row_ror:4
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));  // row_ror:2
    return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));  // row_ror:1
}

// Exponent e of a split partial's half: max |value| < 2^e (0 for an all-zero half; at
// least -100, so that the scale 2^(15 - e) stays a normal float).
__device__ __forceinline__ int partial_exp(float mx) {
    const int e = mx > 0.f ? __builtin_amdgcn_frexp_expf(mx) : 0;
    return e < -100 ? -100 : e;
}

__device__ __forceinline__ int shfl_int(int v, int src_lane) {
    return __builtin_amdgcn_ds_bpermute(src_lane << 2, v);
}
__device__ __forceinline__ float shfl_f(float v, int src_lane) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(v)));
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt untouched): gfx9 encoding, vmcnt bits 3:0 and
// 15:14 (6 bits: at most 63 vector memory operations are counted per wave)
template <int N> __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vm0() { wait_vm<0>(); }

// Workgroup barrier over LDS only: this wave's LDS operations complete, then s_barrier.
// Outstanding global -> LDS copies are not waited for (a full __syncthreads would).
// The empty asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0); vmcnt, expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

