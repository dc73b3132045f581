// Per-element arithmetic of the vector-wise quantization, shared by every
// kernel that quantizes or scans activations, so that all of them take the
// same decisions bit for bit.
//
//   scale   s = fl32(absmax / 127)
//   code    q = round half to even of fl32(x / s), in [-127, 127]
// (tqpw.cn/news/5683, section 2.1, the absmax procedure and its worked
// example; lowentro.cn quantization notes, Q2 and Q11.)
//
// Magnitudes of binary16 values are compared as integers: for a finite h,
// |h| is monotone in (h & 0x7fff), which also gives the exact absmax.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace li8 {

typedef unsigned short li8_us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Quotient fl32(x / s) without a per-element division: with r = fl32(1/s)
// computed once per vector, q0 = fl32(x*r), the residual e = x - q0*s is
// exact as an fma, and fl32(q0 + e*r) is the correctly rounded quotient.
// This is Markstein's correction step; for these inputs (s = fl32(a/127)
// for a binary16 absmax a, x binary16 with |x| <= a) it has been checked
// bit-exact against IEEE division over every such pair.
__device__ __forceinline__ float quotient(float x, float s, float r)
{
    // q0 = fl32(x*r) as an fma with a zero the compiler cannot see through,
    // so that it folds the binary16 -> fp32 conversion of x into one
    // mixed-precision fma (v_fma_mix_f32) instead of a convert and a
    // multiply.  The +0 addend can only turn a -0 product into +0, i.e.
    // only for x = 0, whose code is 0 either way.
    float zero;
    asm("v_mov_b32 %0, 0" : "=v"(zero));
    const float q0 = fmaf(x, r, zero);
    const float e = fmaf(-q0, s, x);
    return fmaf(e, r, q0);
}

// Code of one value for a scale s > 0 with r = fl32(1/s): round half to
// even of the fp32 quotient, clamped to [-127, 127].
__device__ __forceinline__ int code_of(uint32_t h, float s, float r)
{
    float q = rintf(quotient(h2f(h), s, r));
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    return (int)q;
}

// Code byte of one value for a row scale s > 0 (r = fl32(1/s)), in the low
// byte of the result.  Adding 1.5 * 2^23 rounds the quotient half-to-even
// to an integer held in the low mantissa bits (two's complement), and
// |code| <= 127 holds for every |x| <= absmax, so no clamp is needed; both
// facts, like the quotient itself, are checked over every possible input.
__device__ __forceinline__ uint32_t code_bits(uint32_t h, float s, float r)
{
    return __builtin_bit_cast(uint32_t, quotient(h2f(h), s, r) + 12582912.0f);
}

// Two fp32 values rounded to binary16 (nearest even) and packed, a in the
// low half: one v_cvt_pk_f16_f32, which rounds as the scalar conversion
// does (checked over every fp32 bit pattern apart from NaN payloads).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b)
{
    typedef float li8_f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 li8_h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((li8_f2){a, b}, li8_h2));
}

// Low bytes of four words packed into one (v_perm_b32 byte selects).
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    return __builtin_amdgcn_perm(b, a, 0x0c0c0400u) | __builtin_amdgcn_perm(d, c, 0x04000c0cu);
}

// Codes of the 8 values of a 16-byte chunk of a token row with scale s > 0;
// positions set in `skip` (outlier columns) get code 0.
__device__ __forceinline__ uint2 token_codes8(uint4 v, uint32_t skip, float s, float r)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t c[8];
#pragma unroll
    for (int e = 0; e < 8; e++)
        c[e] = code_bits((w[e >> 1] >> (16 * (e & 1))) & 0xffffu, s, r);
    if (skip) {
#pragma unroll
        for (int e = 0; e < 8; e++)
            if ((skip >> e) & 1u)
                c[e] = 0u;
    }
    return make_uint2(pack_low_bytes(c[0], c[1], c[2], c[3]), pack_low_bytes(c[4], c[5], c[6], c[7]));
}

// Byte masks for the 8 codes of a chunk: byte e of the result (x: bytes
// 0-3, y: bytes 4-7) is 0xff when bit e of `skip` is clear and 0 when it is
// set.  (Multiplying a 4-bit value by 0x00204081 places its bit b at bit
// 8b with no carries; the mask keeps those bits and *0xff widens them.)
__device__ __forceinline__ uint2 keep_bytes8(uint32_t skip)
{
    const uint32_t lo = ((skip & 0xfu) * 0x00204081u) & 0x01010101u;
    const uint32_t hi = (((skip >> 4) & 0xfu) * 0x00204081u) & 0x01010101u;
    return make_uint2(~(lo * 0xffu), ~(hi * 0xffu));
}

// Codes of a chunk as token_codes8, with the outlier positions cleared by
// byte masks from keep_bytes8 (for a caller that quantizes several tokens
// over the same columns and builds the masks once).
__device__ __forceinline__ uint2 token_codes8_keep(uint4 v, uint2 keep, float s, float r)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t c[8];
#pragma unroll
    for (int e = 0; e < 8; e++)
        c[e] = code_bits((w[e >> 1] >> (16 * (e & 1))) & 0xffffu, s, r);
    return make_uint2(pack_low_bytes(c[0], c[1], c[2], c[3]) & keep.x,
                      pack_low_bytes(c[4], c[5], c[6], c[7]) & keep.y);
}

// Max magnitude of the 8 binary16 values in v whose bit in `skip` is clear.
__device__ __forceinline__ uint32_t masked_max8(uint4 v, uint32_t skip)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
        if (!((skip >> (2 * i)) & 1u))
            m = max(m, lo);
        if (!((skip >> (2 * i + 1)) & 1u))
            m = max(m, hi);
    }
    return m;
}

// Max magnitude of the 8 values of a chunk, skipping positions set in skip.
__device__ __forceinline__ uint32_t chunk_max(uint4 v, uint32_t skip)
{
    if (skip)
        return masked_max8(v, skip);
    li8_us2 m = __builtin_elementwise_max(__builtin_bit_cast(li8_us2, v.x & 0x7fff7fffu),
                                          __builtin_bit_cast(li8_us2, v.y & 0x7fff7fffu));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(li8_us2, v.z & 0x7fff7fffu));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(li8_us2, v.w & 0x7fff7fffu));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

// Per-column magnitude max of a chunk folded into m (4 packed pairs).
__device__ __forceinline__ void column_max8(li8_us2 m[4], uint4 v)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++)
        m[i] = __builtin_elementwise_max(m[i], __builtin_bit_cast(li8_us2, w[i] & 0x7fff7fffu));
}

// Outlier flags of the 8 columns of a chunk from their magnitude maxima:
// bit e set iff column e's max exceeds the threshold pattern.
__device__ __forceinline__ uint32_t outlier_flags8(const li8_us2 m[4], uint32_t thr_mag)
{
    uint32_t f = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        f |= ((uint32_t)m[i].x > thr_mag ? 1u : 0u) << (2 * i);
        f |= ((uint32_t)m[i].y > thr_mag ? 1u : 0u) << (2 * i + 1);
    }
    return f;
}

// Max over the 64 lanes of a wave (every lane active), in every lane.
// DPP moves within each row of 16 lanes (swap neighbours, swap pairs, the
// half-row mirror, the row mirror), then the gfx950 lane swaps combine
// rows 0/1 and 2/3, then the two halves: plain VALU work with no LDS round
// trip, so that independent reductions overlap.
__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
    const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max((uint32_t)r16[0], (uint32_t)r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max((uint32_t)r32[0], (uint32_t)r32[1]);
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() is
// also a release fence, which makes every wave wait for all of its global
// loads still in flight; this one waits for the wave's LDS operations
// (lgkmcnt) and nothing else, so prefetched global data keeps streaming in
// across it.  Use it only where the barrier guards LDS data.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

} // namespace li8
