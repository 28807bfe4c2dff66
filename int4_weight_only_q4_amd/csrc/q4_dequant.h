// Device routines shared by the int4 matvec kernels of libq4 (gfx950).
//
// Format (Zero TVM Documentation, "Q4F16 quantization format"): eight 4-bit
// codes per uint32, element i of a word in bits 4i..4i+3, one binary16 scale
// per 32-element group, value (code - 7) * scale.
//
// Unpack without conversions (see group_dot): codes are masked straight into
// subnormal binary16 pairs that v_dot2_f32_f16 multiplies exactly. The
// activation is staged with each 8-element chunk stored as the pairs (x0,x4)
// (x1,x5) (x2,x6) (x3,x7), which line up with the masks, and with each 32-value
// group's sum beside it.
#pragma once

#include "q4_common.h"

namespace q4 {

// Weight and scale loads. Weights are read once per token, so they use
// non-temporal loads (they do not displace the activation or the published
// vectors in the caches), through global (not flat) addressing so that they
// count only against the vector-memory counter. A scale is returned in a
// 32-bit register of its own: two 16-bit scales packed into one register make
// the compiler wait for the first load before it can issue the next, which
// serialises the whole load sequence.
typedef uint32_t q4_v4u32 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const q4_v4u32 q4_global_v4u32;
typedef __attribute__((address_space(1))) const uint16_t q4_global_u16;

__device__ __forceinline__ uint4 load_weights(const uint4 *p)
{
    const q4_v4u32 v = __builtin_nontemporal_load((q4_global_v4u32 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t load_scale(const uint16_t *p)
{
    return __builtin_nontemporal_load((q4_global_u16 *)p);
}

// Sum over one group (four words, 32 codes) of (c - 7) * x.
//
// A code c kept in mantissa bits 0..3 of a binary16 whose exponent field is
// zero is the exact subnormal c * 2^-24; kept in bits 4..7 it is c * 2^-20. So
// for a word w, (w & 0x000F000F) holds the codes of elements 0 and 4 as such a
// pair, (w & 0x00F000F0) those of 1 and 5, and the same masks on w >> 8 those
// of 2, 6 and 3, 7: one shift and four ANDs per word, no conversion. The
// activation chunk is staged as the matching pairs (x0,x4) (x1,x5) (x2,x6)
// (x3,x7). v_dot2_f32_f16 multiplies exactly (f16 denormals are kept) and
// accumulates in f32; lo gathers the 2^-24-scaled pairs, hi the 2^-20-scaled
// ones, and sum (c - 7) x = 2^24 lo + 2^20 hi - 7 sum(x), with sum(x) staged
// beside the activation. A one-hot x therefore gives (c - 7) exactly.
// Position in the staged activation of quarter q (chunk 4 g + q) of group g.
// The four 16-byte quarters of a group are rotated by g / 2: lanes that read
// the same quarter of consecutive groups (64 bytes apart) would otherwise hit
// the same LDS banks; rotated, 8 such lanes cover 8 distinct 16-byte bank
// groups.
__device__ __forceinline__ int staged_index(int g, int q) { return 4 * g + ((q + (g >> 1)) & 3); }

// lo (the 2^-24-scaled pairs) and hi (the 2^-20-scaled ones) of the 32 codes
// of wv against staged group g, accumulated onto the values passed in.
__device__ __forceinline__ void group_dot_parts(uint4 wv, const uint4 *xs, int g, float &lo,
                                                float &hi)
{
    const uint32_t m0 = 0x000F000Fu, m1 = 0x00F000F0u;
    const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 xq = xs[staged_index(g, q)];
        const uint32_t t = w[q] >> 8;
        lo = __builtin_amdgcn_fdot2(as_h2(w[q] & m0), as_h2(xq.x), lo, false);
        hi = __builtin_amdgcn_fdot2(as_h2(w[q] & m1), as_h2(xq.y), hi, false);
        lo = __builtin_amdgcn_fdot2(as_h2(t & m0), as_h2(xq.z), lo, false);
        hi = __builtin_amdgcn_fdot2(as_h2(t & m1), as_h2(xq.w), hi, false);
    }
}

// sum over the group of (c - 7) x; sx = the staged sum of x over the group.
__device__ __forceinline__ float group_dot(uint4 wv, const uint4 *xs, int g, float sx)
{
    float lo = 0.f, hi = 0.f;
    group_dot_parts(wv, xs, g, lo, hi);
    return fmaf(0x1p24f, lo, fmaf(0x1p20f, hi, -7.f * sx));
}

// sum over the group of c x (the unsigned codes of the affine format).
__device__ __forceinline__ float group_dot_unsigned(uint4 wv, const uint4 *xs, int g)
{
    float lo = 0.f, hi = 0.f;
    group_dot_parts(wv, xs, g, lo, hi);
    return fmaf(0x1p24f, lo, 0x1p20f * hi);
}

// Stage x[K] (K % 32 == 0) into LDS: xs[K/8] pair-interleaved chunks and
// cs[K/32] = group sums. Must be called by all 256 threads.
__device__ __forceinline__ void stage_activation(const uint16_t *__restrict__ x, int K, uint4 *xs, float *cs)
{
    const int chunks = K >> 3;
    for (int base = 0; base < chunks; base += 256) {
        const int c = base + threadIdx.x;
        float sum = 0.f;
        if (c < chunks) {
            const uint4 v = reinterpret_cast<const uint4 *>(x)[c];
            uint4 p;
            p.x = (v.x & 0xFFFFu) | (v.z << 16);
            p.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
            p.z = (v.y & 0xFFFFu) | (v.w << 16);
            p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
            xs[staged_index(c >> 2, c & 3)] = p;
            sum = ((h2f(v.x & 0xFFFF) + h2f(v.x >> 16)) + (h2f(v.y & 0xFFFF) + h2f(v.y >> 16))) +
                  ((h2f(v.z & 0xFFFF) + h2f(v.z >> 16)) + (h2f(v.w & 0xFFFF) + h2f(v.w >> 16)));
        }
        sum = quad_sum(sum);
        if (c < chunks && (c & 3) == 0)
            cs[c >> 2] = sum;
    }
}

// The 8 binary16 values of a chunk, in order, as floats.
__device__ __forceinline__ void chunk_to_float(uint4 v, float f[8])
{
    f[0] = h2f(v.x & 0xFFFF); f[1] = h2f(v.x >> 16);
    f[2] = h2f(v.y & 0xFFFF); f[3] = h2f(v.y >> 16);
    f[4] = h2f(v.z & 0xFFFF); f[5] = h2f(v.z >> 16);
    f[6] = h2f(v.w & 0xFFFF); f[7] = h2f(v.w >> 16);
}

// Write one staged chunk (thread-held, chunk index c of a K-vector) into LDS in
// the pair-interleaved order, and the group sum for every 4th chunk. All
// 256 threads must call it together (for every j), since it shuffles.
__device__ __forceinline__ void put_chunk(uint4 v, int c, bool valid, uint4 *xs, float *cs)
{
    float sum = 0.f;
    if (valid) {
        uint4 p;
        p.x = (v.x & 0xFFFFu) | (v.z << 16);
        p.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
        p.z = (v.y & 0xFFFFu) | (v.w << 16);
        p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
        xs[staged_index(c >> 2, c & 3)] = p;
        sum = ((h2f(v.x & 0xFFFF) + h2f(v.x >> 16)) + (h2f(v.y & 0xFFFF) + h2f(v.y >> 16))) +
              ((h2f(v.z & 0xFFFF) + h2f(v.z >> 16)) + (h2f(v.w & 0xFFFF) + h2f(v.w >> 16)));
    }
    sum = quad_sum(sum);
    if (valid && (c & 3) == 0)
        cs[c >> 2] = sum;
}

}  // namespace q4
