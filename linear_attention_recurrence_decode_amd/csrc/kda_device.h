// kda_device.h -- device helpers shared by the KDA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Storage type of bf16 activations: the raw 16 bits.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Activation load/store: element access and 4-wide vector access.
template <typename ACT> struct Act;

template <> struct Act<float> {
    static constexpr int kBytes = 4;
    using raw = float;     // as loaded, before conversion
    __device__ __forceinline__ static raw ld_raw(const float* p) { return *p; }
    __device__ __forceinline__ static float cvt(raw r) { return r; }
    using raw4 = float4;
    __device__ __forceinline__ static raw4 ld4_raw(const float* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ static float4 cvt4(raw4 r) { return r; }
    __device__ __forceinline__ static float ld(const float* p) { return *p; }
    __device__ __forceinline__ static void st(float* p, float x) { *p = x; }
    __device__ __forceinline__ static float4 ld4(const float* p) {
        return *reinterpret_cast<const float4*>(p);
    }
    __device__ __forceinline__ static void st4(float* p, float4 x) {
        *reinterpret_cast<float4*>(p) = x;
    }
};

template <> struct Act<bf16_t> {
    static constexpr int kBytes = 2;
    using raw = uint16_t;
    __device__ __forceinline__ static raw ld_raw(const bf16_t* p) { return p->bits; }
    __device__ __forceinline__ static float cvt(raw r) { return bf16_to_f32(r); }
    using raw4 = uint2;
    __device__ __forceinline__ static raw4 ld4_raw(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ static float4 cvt4(raw4 r) {
        return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                           __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
    }
    __device__ __forceinline__ static float ld(const bf16_t* p) { return bf16_to_f32(p->bits); }
    __device__ __forceinline__ static void st(bf16_t* p, float x) { p->bits = f32_to_bf16(x); }
    __device__ __forceinline__ static float4 ld4(const bf16_t* p) {
        uint2 r = *reinterpret_cast<const uint2*>(p);
        return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                           __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
    }
    __device__ __forceinline__ static void st4(bf16_t* p, float4 x) {
        uint2 r;
        r.x = static_cast<uint32_t>(f32_to_bf16(x.x)) | (static_cast<uint32_t>(f32_to_bf16(x.y)) << 16);
        r.y = static_cast<uint32_t>(f32_to_bf16(x.z)) | (static_cast<uint32_t>(f32_to_bf16(x.w)) << 16);
        *reinterpret_cast<uint2*>(p) = r;
    }
};

// SiLU and the logistic function with the hardware reciprocal (about 1 ulp)
// instead of an IEEE division sequence.  For y -> -inf, 1 + exp(-y) -> inf and
// the reciprocal -> 0, so both go to 0 without NaN.
__device__ __forceinline__ float sigmoid(float y) { return __builtin_amdgcn_rcpf(1.0f + __expf(-y)); }
__device__ __forceinline__ float silu(float y) { return y * sigmoid(y); }

// One causal conv tap sum over a 4-token window a, b, c, d (oldest first;
// w.w multiplies the newest).  The prefill and the projection's conv front
// end both use this order, so they form the same fp32 value.
__device__ __forceinline__ float conv4(const float4& w, float a, float b, float c, float d) {
    float y = w.x * a;
    y = fmaf(w.y, b, y);
    y = fmaf(w.z, c, y);
    return fmaf(w.w, d, y);
}

// Sum over aligned groups of G lanes (G = 1, 2, 4, 8 or 16) with DPP lane
// moves: swap neighbours, swap pairs, mirror within 8, mirror within 16.
// Every lane of a group ends with the group's sum.
template <int G>
__device__ __forceinline__ float dpp_group_sum(float x) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group of 1..16 lanes");
    if constexpr (G >= 2) x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
    if constexpr (G >= 4) x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
    if constexpr (G >= 8) x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
    if constexpr (G >= 16) x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));
    return x;
}

// x plus the value of lane l ^ 8: each row of 16 lanes rotated by 8 (DPP).
__device__ __forceinline__ float add_lane_xor8(float x) {
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}

// x plus the value of lane l ^ 16, and of lane l ^ 32: the gfx950 row swaps
// exchange odd rows of 16 (halves of 32) of one operand with even rows
// (halves) of the other; with x in both, one holds the even row's value and
// the other the odd row's in every lane, so both lanes of a pair add the same
// two values in the same order.
__device__ __forceinline__ float add_lane_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_lane_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned groups of G lanes (G = 8, 16, 32 or 64); every lane of a
// group ends with the same bits.  No LDS traffic and no index registers.
template <int G>
__device__ __forceinline__ float lane_sum_below(float x) {
    static_assert(G == 8 || G == 16 || G == 32 || G == 64, "groups of 8 to 64 lanes");
    x = dpp_group_sum<(G < 16 ? G : 16)>(x);
    if constexpr (G >= 32) x = add_lane_xor16(x);
    if constexpr (G >= 64) x = add_lane_xor32(x);
    return x;
}

// Sum over the lanes of a wave64 whose ids differ only in the bits from LO
// up (LO = 8, 16, 32 or 64; 64 is the identity): e.g. LO = 32 adds lanes l
// and l ^ 32.
template <int LO>
__device__ __forceinline__ float lane_sum_from(float x) {
    static_assert(LO == 8 || LO == 16 || LO == 32 || LO == 64, "lane bits from 8, 16, 32 or 64");
    if constexpr (LO <= 8) x = add_lane_xor8(x);
    if constexpr (LO <= 16) x = add_lane_xor16(x);
    if constexpr (LO <= 32) x = add_lane_xor32(x);
    return x;
}

__device__ __forceinline__ float nan_f32() { return __uint_as_float(0x7fc00000u); }

// Raw buffer access: a 128-bit resource (base, size in bytes) in scalar
// registers, a per-lane byte offset and a uniform byte offset.  Accesses past
// `bytes` read zero and drop writes.  The third descriptor word is the gfx9
// family's raw-buffer format.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ float4 buf_ld4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 0);
    return make_float4(__int_as_float(v.x), __int_as_float(v.y), __int_as_float(v.z), __int_as_float(v.w));
}

__device__ __forceinline__ float buf_ldf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), static_cast<int>(soff), 0));
}

__device__ __forceinline__ uint16_t buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(voff), static_cast<int>(soff), 0);
}

__device__ __forceinline__ void buf_stf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(x), r, static_cast<int>(voff), static_cast<int>(soff), 0);
}

__device__ __forceinline__ void buf_st16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint16_t x) {
    __builtin_amdgcn_raw_buffer_store_b16(x, r, static_cast<int>(voff), static_cast<int>(soff), 0);
}

// 16-byte buffer store with the whole offset in the per-lane VGPR and a literal
// zero soffset.  The compiler pads a VALU write to a store-data register that
// follows a >64-bit buffer store with a wait state only when soffset is not a
// register; with a register soffset it issued the write right after the store
// and the store occasionally wrote the new value (seen as corrupted state
// entries in a few lanes).  So wide buffer stores never take an soffset here.
__device__ __forceinline__ void buf_st4(__amdgpu_buffer_rsrc_t r, uint32_t voff, float4 x) {
    i32x4 v;
    v.x = __float_as_int(x.x);
    v.y = __float_as_int(x.y);
    v.z = __float_as_int(x.z);
    v.w = __float_as_int(x.w);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(voff), 0, 0);
}

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 8-byte buffer load / store (literal zero soffset, as for the wide stores).
__device__ __forceinline__ uint2 buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    const i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(voff), 0, 0);
    return make_uint2(static_cast<uint32_t>(v.x), static_cast<uint32_t>(v.y));
}
__device__ __forceinline__ void buf_st8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint2 x) {
    i32x2 v;
    v.x = static_cast<int>(x.x);
    v.y = static_cast<int>(x.y);
    __builtin_amdgcn_raw_buffer_store_b64(v, r, static_cast<int>(voff), 0, 0);
}

// Four bf16 values (two 32-bit words, lower element in the low half) to fp32.
__device__ __forceinline__ float4 bf16x4_to_f32(uint2 w) {
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

// Four fp32 values to bf16, round to nearest even (packed hardware conversion).
__device__ __forceinline__ uint2 f32_to_bf16x4(float4 x) {
    const bf16x2_t a = __builtin_convertvector(f32x2_t{x.x, x.y}, bf16x2_t);
    const bf16x2_t b = __builtin_convertvector(f32x2_t{x.z, x.w}, bf16x2_t);
    return make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
}

}  // namespace kda
