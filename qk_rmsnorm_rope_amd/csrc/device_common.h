// device_common.h -- gfx950 device helpers shared by the two operator kernels:
// 16-byte vector loads/stores, storage <-> fp32 conversion, the cache
// encoders (int8 round-half-even + clamp, FP8 E4M3FN round-to-nearest-even
// with saturation) and wavefront sum reductions built on DPP.
//
// All arithmetic is fp32. Rounding to a storage type happens once per output
// element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qknr {

// ---------------------------------------------------------------------------
// storage types
// ---------------------------------------------------------------------------

struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_hw __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    f32x2 v = {a, b};
    bf16x2_hw h = __builtin_convertvector(v, bf16x2_hw);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float lo_f16(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float hi_f16(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
// Two fp32 -> packed f16x2, round to nearest even (not the round-toward-zero pkrtz form).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    f32x2 v = {a, b};
    f16x2_hw h = __builtin_convertvector(v, f16x2_hw);
    return __builtin_bit_cast(uint32_t, h);
}

// Elements of storage type T per 32-bit word and their decode/encode.
template <typename T> struct Storage;

template <> struct Storage<float> {
    static constexpr int kPerWord = 1;
    __device__ __forceinline__ static void decode(uint32_t w, float *out) { out[0] = __uint_as_float(w); }
    __device__ __forceinline__ static uint32_t encode(const float *in) { return __float_as_uint(in[0]); }
};
template <> struct Storage<bf16_t> {
    static constexpr int kPerWord = 2;
    __device__ __forceinline__ static void decode(uint32_t w, float *out) { out[0] = lo_bf16(w); out[1] = hi_bf16(w); }
    __device__ __forceinline__ static uint32_t encode(const float *in) { return pack_bf16(in[0], in[1]); }
};
template <> struct Storage<f16_t> {
    static constexpr int kPerWord = 2;
    __device__ __forceinline__ static void decode(uint32_t w, float *out) { out[0] = lo_f16(w); out[1] = hi_f16(w); }
    __device__ __forceinline__ static uint32_t encode(const float *in) { return pack_f16(in[0], in[1]); }
};

// ---------------------------------------------------------------------------
// vector memory access: N 32-bit words at a naturally aligned address
// ---------------------------------------------------------------------------

template <int WORDS> struct Words { uint32_t w[WORDS]; };

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) accesses: data read or written exactly once is
// marked so that it does not displace reused lines (gammas, tables, scales)
// in the caches.
template <int WORDS>
__device__ __forceinline__ Words<WORDS> load_words_nt(const void *p) {
    Words<WORDS> r;
    if constexpr (WORDS == 4) {
        u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else if constexpr (WORDS == 2) {
        u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
        r.w[0] = v.x; r.w[1] = v.y;
    } else {
        r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
    }
    return r;
}

template <int WORDS>
__device__ __forceinline__ void store_words_nt(void *p, const Words<WORDS> &r) {
    if constexpr (WORDS == 4) {
        u32x4_t v = {r.w[0], r.w[1], r.w[2], r.w[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(p));
    } else if constexpr (WORDS == 2) {
        u32x2_t v = {r.w[0], r.w[1]};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t *>(p));
    } else {
        __builtin_nontemporal_store(r.w[0], reinterpret_cast<uint32_t *>(p));
    }
}

template <int WORDS>
__device__ __forceinline__ Words<WORDS> load_words(const void *p) {
    Words<WORDS> r;
    if constexpr (WORDS == 4) {
        uint4 v = *reinterpret_cast<const uint4 *>(p);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else if constexpr (WORDS == 2) {
        uint2 v = *reinterpret_cast<const uint2 *>(p);
        r.w[0] = v.x; r.w[1] = v.y;
    } else {
        static_assert(WORDS == 1, "1, 2 or 4 words");
        r.w[0] = *reinterpret_cast<const uint32_t *>(p);
    }
    return r;
}

template <int WORDS>
__device__ __forceinline__ void store_words(void *p, const Words<WORDS> &r) {
    if constexpr (WORDS == 4) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
    } else if constexpr (WORDS == 2) {
        *reinterpret_cast<uint2 *>(p) = make_uint2(r.w[0], r.w[1]);
    } else {
        *reinterpret_cast<uint32_t *>(p) = r.w[0];
    }
}

// LDS accesses through pointers typed for the LDS address space, so that
// they always compile to ds_read / ds_write: whatever form the global
// accesses above take (cache-policy bits, inline assembly), an LDS address
// can never reach a global store.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

template <int WORDS>
__device__ __forceinline__ void lds_store_words(lds_u8 *p, const Words<WORDS> &r) {
    if constexpr (WORDS == 4) {
        u32x4_t v = {r.w[0], r.w[1], r.w[2], r.w[3]};
        *reinterpret_cast<lds_u32x4 *>(p) = v;
    } else if constexpr (WORDS == 2) {
        u32x2_t v = {r.w[0], r.w[1]};
        *reinterpret_cast<lds_u32x2 *>(p) = v;
    } else {
        static_assert(WORDS == 1, "1, 2 or 4 words");
        *reinterpret_cast<lds_u32 *>(p) = r.w[0];
    }
}

template <int WORDS>
__device__ __forceinline__ Words<WORDS> lds_load_words(const lds_u8 *p) {
    Words<WORDS> r;
    if constexpr (WORDS == 4) {
        const u32x4_t v = *reinterpret_cast<const lds_u32x4 *>(p);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else if constexpr (WORDS == 2) {
        const u32x2_t v = *reinterpret_cast<const lds_u32x2 *>(p);
        r.w[0] = v.x; r.w[1] = v.y;
    } else {
        static_assert(WORDS == 1, "1, 2 or 4 words");
        r.w[0] = *reinterpret_cast<const lds_u32 *>(p);
    }
    return r;
}

// VEC elements of T held as raw 32-bit words (VEC * sizeof(T) in {4, 8, 16}
// bytes): loaded and stored with one naturally aligned vector access and
// decoded to fp32 only where an element is used, which keeps registers
// packed while loads are in flight.
template <typename T, int VEC>
struct Chunk {
    static constexpr int kWords = VEC * (int)sizeof(T) / 4;
    static_assert(kWords == 1 || kWords == 2 || kWords == 4, "4, 8 or 16 bytes per chunk");
    uint32_t w[kWords];

    __device__ __forceinline__ void load(const T *p) {
        Words<kWords> r = load_words<kWords>(p);
#pragma unroll
        for (int i = 0; i < kWords; i++) w[i] = r.w[i];
    }
    __device__ __forceinline__ void load_nt(const T *p) {
        Words<kWords> r = load_words_nt<kWords>(p);
#pragma unroll
        for (int i = 0; i < kWords; i++) w[i] = r.w[i];
    }
    __device__ __forceinline__ void store_nt(T *p) const {
        Words<kWords> r;
#pragma unroll
        for (int i = 0; i < kWords; i++) r.w[i] = w[i];
        store_words_nt<kWords>(p, r);
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < kWords; i++) w[i] = 0u;
    }
    // all VEC elements as fp32
    __device__ __forceinline__ void decode(float *out) const {
#pragma unroll
        for (int i = 0; i < kWords; i++) Storage<T>::decode(w[i], out + i * Storage<T>::kPerWord);
    }
    // sum of squares of the elements, accumulated in fp32
    __device__ __forceinline__ float sumsq(float acc) const;
};

template <>
__device__ __forceinline__ float Chunk<float, 4>::sumsq(float acc) const {
#pragma unroll
    for (int i = 0; i < 4; i++) acc = fmaf(__uint_as_float(w[i]), __uint_as_float(w[i]), acc);
    return acc;
}
template <>
__device__ __forceinline__ float Chunk<float, 1>::sumsq(float acc) const {
    return fmaf(__uint_as_float(w[0]), __uint_as_float(w[0]), acc);
}
// bf16 / f16 pairs: one v_dot2 per word (products of 16-bit values are exact in fp32)
template <int VEC>
__device__ __forceinline__ float sumsq_bf16_words(const uint32_t *w, float acc) {
#pragma unroll
    for (int i = 0; i < VEC / 2; i++) {
        bf16x2_hw v = __builtin_bit_cast(bf16x2_hw, w[i]);
        acc = __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
    }
    return acc;
}
template <int VEC>
__device__ __forceinline__ float sumsq_f16_words(const uint32_t *w, float acc) {
#pragma unroll
    for (int i = 0; i < VEC / 2; i++) {
        f16x2_hw v = __builtin_bit_cast(f16x2_hw, w[i]);
        acc = __builtin_amdgcn_fdot2(v, v, acc, false);
    }
    return acc;
}
template <> __device__ __forceinline__ float Chunk<bf16_t, 8>::sumsq(float acc) const { return sumsq_bf16_words<8>(w, acc); }
template <> __device__ __forceinline__ float Chunk<bf16_t, 4>::sumsq(float acc) const { return sumsq_bf16_words<4>(w, acc); }
template <> __device__ __forceinline__ float Chunk<bf16_t, 2>::sumsq(float acc) const { return sumsq_bf16_words<2>(w, acc); }
template <> __device__ __forceinline__ float Chunk<f16_t, 8>::sumsq(float acc) const { return sumsq_f16_words<8>(w, acc); }
template <> __device__ __forceinline__ float Chunk<f16_t, 4>::sumsq(float acc) const { return sumsq_f16_words<4>(w, acc); }
template <> __device__ __forceinline__ float Chunk<f16_t, 2>::sumsq(float acc) const { return sumsq_f16_words<2>(w, acc); }

template <typename T, int VEC>
__device__ __forceinline__ void load_vec(const T *p, float *out) {
    Chunk<T, VEC> c;
    c.load(p);
    c.decode(out);
}

template <typename T, int VEC>
__device__ __forceinline__ void store_vec(T *p, const float *in) {
    constexpr int W = VEC * (int)sizeof(T) / 4;
    Words<W> r;
#pragma unroll
    for (int i = 0; i < W; i++) r.w[i] = Storage<T>::encode(in + i * Storage<T>::kPerWord);
    store_words<W>(p, r);
}

template <typename T, int VEC>
__device__ __forceinline__ void store_vec_nt(T *p, const float *in) {
    constexpr int W = VEC * (int)sizeof(T) / 4;
    Words<W> r;
#pragma unroll
    for (int i = 0; i < W; i++) r.w[i] = Storage<T>::encode(in + i * Storage<T>::kPerWord);
    store_words_nt<W>(p, r);
}

// ---------------------------------------------------------------------------
// cache encoders
// ---------------------------------------------------------------------------

// Every encoder returns the code in bits 0..7 of its result; the higher bits
// are unspecified (the packers take byte 0 only). All three are branch-free.

// INT8: clamp to [-128, 127], then round half to even by adding 1.5 * 2^23:
// the sum lies in [2^23, 2^24), where fp32 spacing is 1, so the add rounds
// the value to an integer (ties to even, as 1.5 * 2^23 is even) and the low
// mantissa bits hold that integer in two's complement. Clamping first gives
// the same code as rounding first because both bounds are integers. NaN
// clamps to -128.
__device__ __forceinline__ uint32_t enc_int8(float t) {
    const float c = fminf(fmaxf(t, -128.0f), 127.0f);
    return __float_as_uint(c + 12582912.0f);
}

// The subnormal field of an FP8 code: rint(|t| * 2^k) for |t| below the
// smallest normal 2^-m (k = m + mantissa bits), computed as the low bits of
// fma(min(|t|, 2^-m), 2^k, 2^23): the product is exact (a power-of-two
// scaling), and the one rounding of the fma to spacing 1 is round half to even.
__device__ __forceinline__ uint32_t fp8_subnormal_field(float af, float smallest_normal, float scale) {
    return __float_as_uint(fmaf(fminf(af, smallest_normal), scale, 8388608.0f)) - 0x4B000000u;
}

// FP8 E4M3FN (OCP): bias 7, 3 mantissa bits, largest finite 448, no
// infinities. Round to nearest even; magnitudes at or above 448 saturate to
// 448; NaN maps to the NaN code. Bit-level construction from the fp32 value:
//   below 2^-6 the format is subnormal with spacing 2^-9, so the code is the
//   integer rint(|t| * 2^9) (0..8; 8 is the smallest normal, code 0x08);
//   otherwise drop 20 mantissa bits with round-to-nearest-even and rebias the
//   exponent from 127 to 7. Every case is computed and the right one selected.
__device__ __forceinline__ uint32_t enc_e4m3fn(float t) {
    const uint32_t u = __float_as_uint(t);
    const uint32_t a = u & 0x7FFFFFFFu;
    const float af = __uint_as_float(a);
    const uint32_t nrm = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);   // RNE at bit 20, rebias
    const uint32_t sub = fp8_subnormal_field(af, 0.015625f, 512.0f);
    uint32_t code = af < 0.015625f ? sub : nrm;
    code = af >= 448.0f ? 0x7Eu : code;                  // saturate (inf included)
    code = a > 0x7F800000u ? 0x7Fu : code;               // NaN
    return ((u >> 24) & 0x80u) | code;
}

// OCP FP8 E5M2 (bias 15, 2 mantissa bits, largest finite 57344 = 0x7B, inf and
// NaN at exponent 31), round to nearest even, saturating at +-57344:
//   |t| >= 57344 -> 0x7B (everything that would round past it, and inf);
//   |t| < 2^-14 (below the smallest normal) -> the subnormal field, the
//   integer rint(|t| * 2^16) (0..4; 4 is the smallest normal, code 0x04);
//   otherwise drop 21 mantissa bits with round-to-nearest-even and rebias the
//   exponent from 127 to 15.
__device__ __forceinline__ uint32_t enc_e5m2(float t) {
    const uint32_t u = __float_as_uint(t);
    const uint32_t a = u & 0x7FFFFFFFu;
    const float af = __uint_as_float(a);
    const uint32_t nrm = ((a + 0xFFFFFu + ((a >> 21) & 1u)) >> 21) - (112u << 2);   // RNE at bit 21, rebias
    const uint32_t sub = fp8_subnormal_field(af, 6.103515625e-05f, 65536.0f);
    uint32_t code = af < 6.103515625e-05f ? sub : nrm;
    code = af >= 57344.0f ? 0x7Bu : code;
    code = a > 0x7F800000u ? 0x7Fu : code;
    return ((u >> 24) & 0x80u) | code;
}

// Byte 0 of each of four words -> one word (b0 lowest), with v_perm_b32.
__device__ __forceinline__ uint32_t pack_bytes4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u);   // [b0, b1, 0, 0]
    const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0C0C0400u);   // [b2, b3, 0, 0]
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);               // [b0, b1, b2, b3]
}
__device__ __forceinline__ uint32_t pack_bytes2(uint32_t b0, uint32_t b1) {
    return __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u);
}

// ---------------------------------------------------------------------------
// wavefront reductions (wave64). Every lane of a group ends with the same
// bits: each step adds a lane's value to its partner's, and both partners
// compute the same commutative sum.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float dpp_quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_row_half_mirror(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_row_mirror(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));
}
__device__ __forceinline__ float swizzle_xor16(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}

// Sum over aligned groups of G consecutive lanes (G in 8, 16, 32, 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group size");
    v += dpp_quad_xor1(v);
    v += dpp_quad_xor2(v);
    if constexpr (G >= 8) v += dpp_row_half_mirror(v);   // lane i <-> 7-i inside 8
    if constexpr (G >= 16) v += dpp_row_mirror(v);       // lane i <-> 15-i inside 16
    if constexpr (G >= 32) v += swizzle_xor16(v);        // lane i <-> i^16 inside 32
    if constexpr (G >= 64) {
        float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
        float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
        v = a + b;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

}  // namespace qknr
