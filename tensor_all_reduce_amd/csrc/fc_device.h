// fc_device.h -- device helpers for the gfx950 kernels: number formats, wavefront DPP reductions, and the
// per-lane group quantizer / dequantizer.  Compiled with -ffp-contract=off: every float expression below
// is exactly the sequence of IEEE operations written, except where __builtin_fmaf is spelled out.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fc {

// ---- bit casts and formats ------------------------------------------------------------------------
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// bf16 held in the low / high half of a 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return u2f(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (a in the low half), round to nearest even (native gfx950 conversion).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2 v = {a, b};
    bf2 r = __builtin_convertvector(v, bf2);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t f16_rne(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// Largest fp16 <= v: nearest-even conversion, then one step toward -inf if it landed above v.  A step is
// needed only when v < 0 or the result is positive: for a negative result (-0 included: -0 + 1 is the
// negative subnormal 0x8001) the step is the next bit pattern up, for a positive one the next down; +0
// never lands above v (a negative v converts to -0 or below).
__device__ __forceinline__ uint32_t f16_rd(float v) {
    const uint32_t h = f16_rne(v);
    return f16_to_f32(h) > v ? ((h & 0x8000u) ? h + 1u : h - 1u) : h;
}
// Smallest fp16 >= v, for v >= 0 (the only use: a group's range over qmax).  The nearest-even result
// is then +0 or positive, and the next fp16 up is the next bit pattern (from +0, the smallest
// subnormal).
__device__ __forceinline__ uint32_t f16_ru_nonneg(float v) {
    const uint32_t h = f16_rne(v);
    return f16_to_f32(h) < v ? h + 1u : h;
}

// ---- wavefront reductions -------------------------------------------------------------------------
// DPP controls (GFX9 encoding): quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror.
// Applied in this sequence, the first k of them leave every lane of an aligned 2^k-lane group holding
// the reduction over that group.
enum : int { DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140 };

// bound_ctrl is set: every control used here reads a lane of the same row, so it never applies, and with it
// set the compiler folds the move into the VALU instruction that consumes it (v_min_f32_dpp etc.).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return u2f((uint32_t)__builtin_amdgcn_mov_dpp((int)f2u(v), CTRL, 0xF, 0xF, true));
}

template <int LANES>
__device__ __forceinline__ float group_min(float v) {
    if constexpr (LANES >= 2) v = fminf(v, dpp<DPP_XOR1>(v));
    if constexpr (LANES >= 4) v = fminf(v, dpp<DPP_XOR2>(v));
    if constexpr (LANES >= 8) v = fminf(v, dpp<DPP_HALF_MIRROR>(v));
    if constexpr (LANES >= 16) v = fminf(v, dpp<DPP_MIRROR>(v));
    if constexpr (LANES >= 32) v = fminf(v, __shfl_xor(v, 16, 64));
    static_assert(LANES <= 32, "a group spans at most half a wavefront");
    return v;
}
template <int LANES>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (LANES >= 2) v = fmaxf(v, dpp<DPP_XOR1>(v));
    if constexpr (LANES >= 4) v = fmaxf(v, dpp<DPP_XOR2>(v));
    if constexpr (LANES >= 8) v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
    if constexpr (LANES >= 16) v = fmaxf(v, dpp<DPP_MIRROR>(v));
    if constexpr (LANES >= 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
    return v;
}
// Sum over the whole wavefront; every lane gets the same bits (each step adds a commutative pair).
__device__ __forceinline__ float wave_sum(float v) {
    v = v + dpp<DPP_XOR1>(v);
    v = v + dpp<DPP_XOR2>(v);
    v = v + dpp<DPP_HALF_MIRROR>(v);
    v = v + dpp<DPP_MIRROR>(v);
    v = v + __shfl_xor(v, 16, 64);
    v = v + __shfl_xor(v, 32, 64);
    return v;
}

// ---- group quantizer --------------------------------------------------------------------------------
// A group spans LPG aligned consecutive lanes, each holding E consecutive elements.  The quantizer is
// split into its three steps so that a kernel can run the per-group step once for several groups:
//   lane_minmax + group_min/max   the group's min and max in every lane of the group;
//   group_params                  zero point, scale, reciprocal and meta word (scale | zero << 16);
//   encode_lane                   the lane's packed codes (E * BITS / 32 words).
// Non-finite inputs are outside the contract (the kernels are compiled assuming no NaN).
template <int E>
__device__ __forceinline__ void lane_minmax(const float (&v)[E], float& lo, float& hi) {
    lo = v[0];
    hi = v[0];
#pragma unroll
    for (int i = 1; i < E; ++i) {
        lo = fminf(lo, v[i]);
        hi = fmaxf(hi, v[i]);
    }
}

struct GroupQ {
    float z, inv;   // zero point and fp32 reciprocal of the scale (0 for a constant group)
    uint32_t meta;  // scale | zero << 16
};

// The quantizer's two quotients, correctly rounded (the IEEE results) without the division sequence: one
// fma correction of an approximate quotient rounds them exactly.  Both are checked exhaustively on the GPU
// against the IEEE division (the test-support library's self-check): div_by_qmax for every non-negative
// finite float x and qmax = 15 and 255; recip_fp16 for every positive finite fp16 value s.
template <int QMAX>
__device__ __forceinline__ float div_by_qmax(float x) {
    constexpr float r = 1.0f / (float)QMAX;  // RN(1 / qmax), folded at compile time
    const float q0 = x * r;
    return __builtin_fmaf(__builtin_fmaf(-q0, (float)QMAX, x), r, q0);
}
__device__ __forceinline__ float recip_fp16(float s) {
    const float r0 = __builtin_amdgcn_rcpf(s);  // within one ulp
    return __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
}

template <int BITS>
__device__ __forceinline__ GroupQ group_params(float lo, float hi) {
    constexpr int QMAX = (1 << BITS) - 1;
    lo = lo + 0.0f;  // -0 -> +0
    const uint32_t zb = f16_rd(lo);
    const float z = f16_to_f32(zb);
    const float diff = hi - z;
    // Without a branch: diff >= 0, and the scale comes out +0 exactly when diff is 0 (the round-up of a
    // positive quotient is at least the smallest subnormal); only the reciprocal needs the select.
    const uint32_t sb = f16_ru_nonneg(div_by_qmax<QMAX>(diff));  // RN(diff / qmax), rounded up to fp16
    const float inv = sb != 0 ? recip_fp16(f16_to_f32(sb)) : 0.0f;  // RN(1 / s) for a positive fp16 s
    return GroupQ{z, inv, sb | (zb << 16)};
}

// Codes: q = clamp(round-half-even((x - z) * inv), 0, qmax), the subtraction and the product each rounded
// (no contraction).  v_cvt_pk_u8_f32 converts a float to an unsigned byte with round-half-even and
// saturation to [0, 255], and inserts it into byte `sel` of a word, leaving the other bytes (checked on
// gfx950 against rint + clamp over ties, near-ties, negatives and values past 255).  For 8-bit codes that
// is exactly the definition's rounding and clamp.  For 4-bit codes the saturation is at 255, not 15: for
// in-contract inputs 0 <= v < qmax + 0.5 (z <= x, and s >= (max - z)/qmax up to the roundings of one
// division and one reciprocal, so v <= qmax*(1 + 2^-21)), so the clamp at qmax never changes a code; an
// out-of-contract input gives a wrong code but the masks below keep it out of its neighbour's nibble.
template <int BITS, int E>
__device__ __forceinline__ void encode_lane(const float (&v)[E], float z, float inv, uint32_t (&w)[E * BITS / 32]) {
    float q[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const float d = v[i] - z;
        q[i] = d * inv;
    }
#pragma unroll
    for (int k = 0; k < E * BITS / 32; ++k) {
        if constexpr (BITS == 8) {
            uint32_t x = __builtin_amdgcn_cvt_pk_u8_f32(q[4 * k], 0, 0u);
            x = __builtin_amdgcn_cvt_pk_u8_f32(q[4 * k + 1], 1, x);
            x = __builtin_amdgcn_cvt_pk_u8_f32(q[4 * k + 2], 2, x);
            w[k] = __builtin_amdgcn_cvt_pk_u8_f32(q[4 * k + 3], 3, x);
        } else {
            // byte j of ev / od = code 2j / 2j+1; the odd codes go to the high nibbles
            const float* qq = q + 8 * k;
            uint32_t ev = __builtin_amdgcn_cvt_pk_u8_f32(qq[0], 0, 0u);
            ev = __builtin_amdgcn_cvt_pk_u8_f32(qq[2], 1, ev);
            ev = __builtin_amdgcn_cvt_pk_u8_f32(qq[4], 2, ev);
            ev = __builtin_amdgcn_cvt_pk_u8_f32(qq[6], 3, ev);
            uint32_t od = __builtin_amdgcn_cvt_pk_u8_f32(qq[1], 0, 0u);
            od = __builtin_amdgcn_cvt_pk_u8_f32(qq[3], 1, od);
            od = __builtin_amdgcn_cvt_pk_u8_f32(qq[5], 2, od);
            od = __builtin_amdgcn_cvt_pk_u8_f32(qq[7], 3, od);
            w[k] = (ev & 0x0f0f0f0fu) | ((od << 4) & 0xf0f0f0f0u);
        }
    }
}

// All three steps for one group per lane.
template <int BITS, int E, int LPG>
__device__ __forceinline__ void quantize_lane(const float (&v)[E], uint32_t (&w)[E * BITS / 32], uint32_t& meta) {
    float lo, hi;
    lane_minmax<E>(v, lo, hi);
    const GroupQ q = group_params<BITS>(group_min<LPG>(lo), group_max<LPG>(hi));
    meta = q.meta;
    encode_lane<BITS, E>(v, q.z, q.inv, w);
}

// Value of lane J of the caller's LPG-lane group, in every lane of the group.  16-lane groups are DPP rows
// (row_newbcast, gfx90a and later), 4-lane groups are quads (quad_perm [J,J,J,J]); other widths go
// through ds_bpermute.
template <int LPG, int J>
__device__ __forceinline__ float group_bcast(float v, int lane) {
    static_assert(J < LPG, "source lane inside the group");
    if constexpr (LPG == 16) return dpp<0x150 + J>(v);
    else if constexpr (LPG == 4) return dpp<J | (J << 2) | (J << 4) | (J << 6)>(v);
    else return __shfl(v, (lane & ~(LPG - 1)) + J, 64);
}

// ---- dequantization of one packed code word -------------------------------------------------------
// fl(q*s + z): q*s is exact (at most 8 x 11 significant bits), so one fused multiply-add gives the same
// bits as the two separate operations.
template <int BITS>
struct Unpack;

template <>
struct Unpack<8> {
    static constexpr int PER_WORD = 4;
    __device__ __forceinline__ static void run(uint32_t w, float s, float z, float* out) {
        out[0] = __builtin_fmaf((float)(w & 0xffu), s, z);
        out[1] = __builtin_fmaf((float)((w >> 8) & 0xffu), s, z);
        out[2] = __builtin_fmaf((float)((w >> 16) & 0xffu), s, z);
        out[3] = __builtin_fmaf((float)(w >> 24), s, z);
    }
};

template <>
struct Unpack<4> {
    static constexpr int PER_WORD = 8;
    // Codes as fp16 subnormals: a half-word holding a code q (0..15) in bits 0..3 is the fp16 value
    // q * 2^-24, and in bits 4..7 the value q * 2^-20.  The mixed-precision fma converts either exactly, so
    // fma(q * 2^-24, s * 2^24, z) = fma(q * 2^-20, s * 2^20, z) = fl(q*s + z), with no int-to-float
    // conversion (s * 2^24 and s * 2^20 are exact).  Masks that keep one nibble per half-word isolate the
    // codes in pairs: w & 0x000f000f holds codes 0 and 4, w & 0x00f000f0 codes 1 and 5 (4 bits up), and
    // the same masks on w >> 8 codes 2, 6 and 3, 7.  This relies on fp16 subnormals being kept (the
    // kernels' floating-point mode flushes no fp16 or fp32 subnormals).
    __device__ __forceinline__ static void run(uint32_t w, float s, float z, float* out) {
        const float s24 = s * 16777216.0f, s20 = s * 1048576.0f;
        const uint32_t w8 = w >> 8;
        const uint32_t p[4] = {w & 0x000f000fu, w & 0x00f000f0u, w8 & 0x000f000fu, w8 & 0x00f000f0u};
#pragma unroll
        for (int k = 0; k < 4; ++k) {  // p[k]: code k in the low half-word, code k + 4 in the high one
            const float sk = (k & 1) ? s20 : s24;
            const _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(p[k] & 0xffffu));
            const _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(p[k] >> 16));
            out[k] = __builtin_fmaf((float)lo, sk, z);
            out[k + 4] = __builtin_fmaf((float)hi, sk, z);
        }
    }
};

__device__ __forceinline__ float meta_scale(uint32_t m) { return f16_to_f32(m & 0xffffu); }
__device__ __forceinline__ float meta_zero(uint32_t m) { return f16_to_f32(m >> 16); }

// ---- global memory access ------------------------------------------------------------------------
// Every kernel lays its data out so that one wavefront-wide memory instruction covers one contiguous
// span (lane i at base + i * width), so each instruction moves whole cache lines.  Data read or written
// exactly once is "streamed"; FC_STREAM_NT selects the non-temporal cache policy for it (reused data
// such as gamma always uses the default policy).
#ifndef FC_STREAM_NT
#define FC_STREAM_NT 1
#endif
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// base + a 32-bit byte offset: with a wavefront-uniform base the load or store takes the base in scalar
// registers and one 32-bit offset register per lane, where element-indexed pointer arithmetic would
// build a 64-bit address in two vector registers per access.
template <class T>
__device__ __forceinline__ T* at(T* base, uint32_t byte_off) {
    return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + byte_off);
}
template <class T>
__device__ __forceinline__ const T* at(const T* base, uint32_t byte_off) {
    return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint4 lds16(const void* p) {
#if FC_STREAM_NT
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
#else
    return *reinterpret_cast<const uint4*>(p);
#endif
}
__device__ __forceinline__ uint2 lds8(const void* p) {
#if FC_STREAM_NT
    const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
    return make_uint2(v.x, v.y);
#else
    return *reinterpret_cast<const uint2*>(p);
#endif
}
__device__ __forceinline__ uint32_t lds4(const void* p) {
#if FC_STREAM_NT
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
#else
    return *reinterpret_cast<const uint32_t*>(p);
#endif
}
__device__ __forceinline__ void sts16(void* p, uint4 v) {
#if FC_STREAM_NT
    const v4u w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<v4u*>(p));
#else
    *reinterpret_cast<uint4*>(p) = v;
#endif
}
__device__ __forceinline__ void sts8(void* p, uint2 v) {
#if FC_STREAM_NT
    const v2u w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<v2u*>(p));
#else
    *reinterpret_cast<uint2*>(p) = v;
#endif
}
__device__ __forceinline__ void sts4(void* p, uint32_t v) {
#if FC_STREAM_NT
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
#else
    *reinterpret_cast<uint32_t*>(p) = v;
#endif
}

// Quantized messages (the rank messages and the all-gather payload) are written with write-back stores:
// the next call of the step reads them, and at the 70B prefill size (142 MB of rank messages, 35 MB of
// payload) they stay in the 256 MB memory-side cache between the calls, which streamed stores bypass.
// Same-process A/B on the prefill step: 181.5 -> 174.2 us (the quantize alone 108.5 -> 107.3 us).
__device__ __forceinline__ void stm16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ void stm8(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }
__device__ __forceinline__ void stm4(void* p, uint32_t v) { *reinterpret_cast<uint32_t*>(p) = v; }

}  // namespace fc
