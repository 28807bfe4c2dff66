// Packing, add+RMSNorm and split-SiLU-multiply kernels for gfx950.
//
//  * pack / unpack: Zero TVM Documentation, "Q4F16 quantization format"
//    (element i of a word in bits 4i..4i+3).
//  * add + RMSNorm: shaders 2 and 7 of "WGSL Kernel Roles" (residual_out = A + B,
//    then x / sqrt(mean(x^2) + eps) * gamma), one workgroup per row. The sum of
//    squares uses the canonical visiting order that the matvec's normalising
//    prologue also follows, so the two give identical bits; rows of up to 8192
//    values with 16-byte-aligned vectors are held in registers.
//  * SiLU-multiply: RESEARCH.md "1. Dispatch profile" (gate split + SiLU +
//    elementwise multiply), gate first.
#include "q4_common.h"

namespace q4 {
namespace {

// One thread per packed word: 8 codes -> 1 word.
__global__ __launch_bounds__(256) void k_pack(const uint8_t *__restrict__ codes,
                                              uint32_t *__restrict__ packed, int64_t words)
{
    const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (w >= words)
        return;
    const uint8_t *c = codes + w * 8;
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v |= (uint32_t)(c[i] & 0xF) << (4 * i);
    packed[w] = v;
}

__global__ __launch_bounds__(256) void k_unpack(const uint32_t *__restrict__ packed,
                                                uint8_t *__restrict__ codes, int64_t words)
{
    const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (w >= words)
        return;
    const uint32_t v = packed[w];
    uint8_t *c = codes + w * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        c[i] = (uint8_t)((v >> (4 * i)) & 0xF);
}

// One workgroup per row, the canonical summation order (see q4_common.h).
// res_out may be null (the residual is then not stored; a == null and
// res_out == null normalises res_in as it is).
__global__ __launch_bounds__(256) void k_add_rmsnorm(const uint16_t *__restrict__ a,
                                                     const uint16_t *__restrict__ res_in,
                                                     const uint16_t *__restrict__ gamma,
                                                     uint16_t *__restrict__ out,
                                                     uint16_t *__restrict__ res_out, int D,
                                                     float eps)
{
    __shared__ float red[4];
    const int64_t base = (int64_t)blockIdx.x * D;
    const uint16_t *r = res_in + base;
    float ss = 0.f;
    for (int c = threadIdx.x; c * 8 < D; c += 256)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = 8 * c + e;
            if (i < D) {
                const uint16_t v16 = a ? f2h(h2f(a[base + i]) + h2f(r[i])) : r[i];
                if (res_out)
                    res_out[base + i] = v16;
                const float v = h2f(v16);
                ss = fmaf(v, v, ss);
            }
        }
    ss = block_sum_256(ss, red);
    const float inv = rms_inv(ss, D, eps);
    for (int c = threadIdx.x; c * 8 < D; c += 256)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = 8 * c + e;
            if (i < D) {
                const uint16_t v16 = a ? f2h(h2f(a[base + i]) + h2f(r[i])) : r[i];
                out[base + i] = f2h(h2f(v16) * inv * h2f(gamma[i]));
            }
        }
}

// The same row normalisation with the row held in registers: CH 16-byte
// chunks per thread (D % 8 == 0, every vector 16-byte aligned), loaded once
// with 16-byte loads; per thread the same chunks and element order as
// k_add_rmsnorm, so the same bits.
template <int CH>
__global__ __launch_bounds__(256) void k_add_rmsnorm_vec(const uint16_t *__restrict__ a,
                                                         const uint16_t *__restrict__ res_in,
                                                         const uint16_t *__restrict__ gamma,
                                                         uint16_t *__restrict__ out,
                                                         uint16_t *__restrict__ res_out, int D,
                                                         float eps)
{
    __shared__ float red[4];
    const int64_t base = (int64_t)blockIdx.x * D;
    const int chunks = D >> 3;
    const uint4 *r4 = reinterpret_cast<const uint4 *>(res_in + base);
    const uint4 *a4 = a ? reinterpret_cast<const uint4 *>(a + base) : nullptr;
    uint4 rv[CH], av[CH], gv[CH];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        const int c = threadIdx.x + 256 * q;
        if (c < chunks) {
            rv[q] = r4[c];
            if (a4)
                av[q] = a4[c];
            gv[q] = reinterpret_cast<const uint4 *>(gamma)[c];
        }
    }
    uint32_t h[CH][8];
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        const int c = threadIdx.x + 256 * q;
        if (c < chunks) {
            const uint32_t rw[4] = {rv[q].x, rv[q].y, rv[q].z, rv[q].w};
            const uint32_t aw[4] = {a4 ? av[q].x : 0u, a4 ? av[q].y : 0u, a4 ? av[q].z : 0u,
                                    a4 ? av[q].w : 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint16_t r16 = (uint16_t)(rw[e >> 1] >> (16 * (e & 1)));
                const uint16_t a16 = (uint16_t)(aw[e >> 1] >> (16 * (e & 1)));
                const uint16_t v16 = a4 ? f2h(h2f(a16) + h2f(r16)) : r16;
                h[q][e] = v16;
                const float v = h2f(v16);
                ss = fmaf(v, v, ss);
            }
            if (res_out)
                reinterpret_cast<uint4 *>(res_out + base)[c] =
                    make_uint4(h[q][0] | (h[q][1] << 16), h[q][2] | (h[q][3] << 16),
                               h[q][4] | (h[q][5] << 16), h[q][6] | (h[q][7] << 16));
        }
    }
    ss = block_sum_256(ss, red);
    const float inv = rms_inv(ss, D, eps);
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        const int c = threadIdx.x + 256 * q;
        if (c < chunks) {
            const uint32_t gw[4] = {gv[q].x, gv[q].y, gv[q].z, gv[q].w};
            uint32_t o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[e] = f2h(h2f((uint16_t)h[q][e]) * inv *
                           h2f((uint16_t)(gw[e >> 1] >> (16 * (e & 1)))));
            reinterpret_cast<uint4 *>(out + base)[c] =
                make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16),
                           o[6] | (o[7] << 16));
        }
    }
}

__global__ __launch_bounds__(256) void k_silu_mul(const uint16_t *__restrict__ gu,
                                                  uint16_t *__restrict__ out, int F, int64_t total)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= total)
        return;
    const int64_t m = t / F, i = t % F;
    const uint16_t *row = gu + m * 2 * F;
    out[t] = f2h(silu_mul_f(h2f(row[i]), h2f(row[F + i])));
}

}  // namespace

q4_status launch_pack(const uint8_t *codes, uint32_t *packed, int64_t words, hipStream_t st)
{
    const int64_t blocks = (words + 255) / 256;
    hipLaunchKernelGGL(k_pack, dim3((unsigned)blocks), dim3(256), 0, st, codes, packed, words);
    return check_launch("k_pack");
}

q4_status launch_unpack(const uint32_t *packed, uint8_t *codes, int64_t words, hipStream_t st)
{
    const int64_t blocks = (words + 255) / 256;
    hipLaunchKernelGGL(k_unpack, dim3((unsigned)blocks), dim3(256), 0, st, packed, codes, words);
    return check_launch("k_unpack");
}

q4_status launch_add_rmsnorm(const uint16_t *a, const uint16_t *res_in, const uint16_t *gamma,
                             uint16_t *out, uint16_t *res_out, int D, int M, float eps,
                             hipStream_t st)
{
    auto al16 = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    const int ch = (D / 8 + 255) / 256;  // 16-byte chunks per thread
    if (D % 8 == 0 && ch <= 4 && al16(a) && al16(res_in) && al16(gamma) && al16(out) &&
        al16(res_out)) {
        switch (ch) {
        case 1: hipLaunchKernelGGL(k_add_rmsnorm_vec<1>, dim3(M), dim3(256), 0, st, a, res_in, gamma, out, res_out, D, eps); break;
        case 2: hipLaunchKernelGGL(k_add_rmsnorm_vec<2>, dim3(M), dim3(256), 0, st, a, res_in, gamma, out, res_out, D, eps); break;
        case 3: hipLaunchKernelGGL(k_add_rmsnorm_vec<3>, dim3(M), dim3(256), 0, st, a, res_in, gamma, out, res_out, D, eps); break;
        default: hipLaunchKernelGGL(k_add_rmsnorm_vec<4>, dim3(M), dim3(256), 0, st, a, res_in, gamma, out, res_out, D, eps); break;
        }
        return check_launch("k_add_rmsnorm_vec");
    }
    hipLaunchKernelGGL(k_add_rmsnorm, dim3(M), dim3(256), 0, st, a, res_in, gamma, out, res_out,
                       D, eps);
    return check_launch("k_add_rmsnorm");
}

q4_status launch_silu_mul(const uint16_t *gu, uint16_t *out, int F, int M, hipStream_t st)
{
    const int64_t total = (int64_t)F * M;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_silu_mul, dim3((unsigned)blocks), dim3(256), 0, st, gu, out, F, total);
    return check_launch("k_silu_mul");
}

}  // namespace q4
