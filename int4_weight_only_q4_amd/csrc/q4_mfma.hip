// Batched int4 x f16 matvec on the gfx950 matrix cores: M = 2..16 activation
// rows share one read of the weights (more rows: one launch per 16).
//
// What is computed is the group-quantised matvec of the Zero TVM Documentation
// ("Q4F16 quantization format"; the batched decode of "WGSL Kernel Roles"):
// y[m][n] = sum_g s[n][g] * sum_{k in g} (q[n][k] - 7) * x[m][k]. At M >= 2
// the shared weight read makes it a small dense contraction, so the inner sums
// run on v_mfma_f32_16x16x32_f16, one MFMA per quantisation group of 16
// weight rows and 16 activation rows:
//  * the B operand is the codes as the exact binary16 integers q - 7 and the
//    product with the f16 activation is exact; the group's f32 sum is then
//    multiplied by the group's scale in f32, as in the single-row matvec. No
//    dequantised weight is ever rounded to f16;
//  * the A operand is the activation, staged once per workgroup in LDS; rows
//    m >= M of the MFMA tile repeat row M - 1 and are never stored;
//  * a lane (row n = lane % 16, lane row kb = lane / 16) loads one 16-byte
//    group of its row per step (four consecutive groups per wave and step, 64
//    bytes contiguous per row); a 4 x 4 transpose across the lane rows
//    (permlane16/32 swaps) then gives each lane row one word of every group,
//    which is the B layout of an MFMA covering one group;
//  * about three workgroups per CU stay resident: each stages its activation
//    chunk once and its waves then take up to four 16-row tiles each, a
//    tile's 4 KB of weights in flight per wave;
//  * K is split into chunks of 512 values (the staged activation);
//    the f32 partials are summed by a second kernel in a fixed order, so
//    results are identical run to run.
#include <algorithm>

#include "q4_dequant.h"
#include "q4_moe_route.h"

namespace q4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
// native vector (HIP's uint4 is a struct, whose private arrays the compiler
// keeps in scratch memory instead of registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;            // 16 weight rows per wave
constexpr int kDepth = 4;            // steps (4 groups each) of one tile's weight loads
constexpr int kGroupsPerSplit = 4 * kDepth;  // K chunk per workgroup: 512 values
constexpr int kMTile = 16;           // activation rows per launch
constexpr int kXq = (kMTile * kGroupsPerSplit * 4 + 255) / 256;  // x chunks per thread
constexpr int kMaxTilesPerWave = 4;  // finished tiles wait in LDS until the last is done
// k_moe_finish modes (the per-slot mode is the remaining one, 0)
constexpr int kMoeSilu = 1, kMoeCombine = 2;

// The 8 codes of word w as the exact binary16 integers q - 7, in the pair
// order (e0, e4) (e1, e5) (e2, e6) (e3, e7): (w >> 4i) & 0x000F000F puts codes i
// and i + 4 in the two halves, the exponent pattern 0x6400 makes them 1024 + q
// and subtracting 1031 is exact. The activation is staged in the same order.
// (UNSIGNED: the codes q themselves, the 1024 of the exponent pattern removed.)
template <bool UNSIGNED = false>
__device__ __forceinline__ half8 codes_minus7(uint32_t w, uint32_t mask)
{
    const _Float16 off = UNSIGNED ? (_Float16)1024.0f : (_Float16)1031.0f;
    const half2v c1031 = {off, off};
    half8 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // (mask & (w >> 4i)) | (~mask & 0x64006400) in one bitfield insert
        // (mask = 0x000F000F sits in a register: an instruction of this
        // encoding takes at most one constant)
        uint32_t bits;
        asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(bits) : "v"(mask), "v"(w >> (4 * i)), "s"(0x64006400u));
        const half2v q = __builtin_bit_cast(half2v, bits) - c1031;
        out[2 * i] = q[0];
        out[2 * i + 1] = q[1];
    }
    return out;
}

// 4 x 4 transpose over (lane row, register): afterwards r[t] in row q holds
// what r[q] held in row t.
__device__ __forceinline__ void transpose_rows(uint32_t (&r)[4])
{
    swap32(r[0], r[2]);
    swap32(r[1], r[3]);
    swap16(r[0], r[1]);
    swap16(r[2], r[3]);
}

// Row broadcast: afterwards out[t] in every row holds what v held in row t.
__device__ __forceinline__ void broadcast_rows(uint32_t v, uint32_t (&out)[4])
{
    uint32_t p = v, q = v;
    swap16(p, q);  // p: rows 0, 0, 2, 2; q: rows 1, 1, 3, 3
    uint32_t p2 = p, q2 = q;
    swap32(p, p2);  // p: row 0 everywhere; p2: row 2
    swap32(q, q2);  // q: row 1; q2: row 3
    out[0] = p;
    out[1] = q;
    out[2] = p2;
    out[3] = q2;
}

// A 16-byte chunk of 8 activations x0..x7 in the pair order of codes_minus7.
__device__ __forceinline__ u32x4 pair_order(u32x4 v)
{
    return u32x4{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                 __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                 __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                 __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
}

// The loads of one 16-row weight tile of a split: lane (n, kb) holds group
// 4p + kb of row n (16 bytes) and its scale for step p = 0..kDepth-1.
struct TileRegs {
    uint4 w[kDepth];
    uint32_t s[kDepth];
    uint32_t b[kDepth];  // affine format: biases
};

// The work of one workgroup for one split ks of K (groups [ks * gc, min(G,
// (ks + 1) * gc)), gc = kGroupsPerSplit) and M <= 16 activation rows:
// row_ptr(m) gives activation row m; wave w takes the 16-row weight tiles
// tile0(w), + tstride, ... (at most kMaxTilesPerWave), and emit(m, n, value)
// receives every finished f32 result.
// AFF: the MLX affine format (unsigned codes, w = s * q + b per 64 codes, scales
// and biases [N][G/2]): each group's MFMA sum is scaled, and the bias times the
// group's sum of x (staged per row) added.
template <bool AFF, typename RowPtr, typename Emit>
__device__ __forceinline__ void mfma_rows(const uint4 *__restrict__ W,
                                          const uint16_t *__restrict__ S,
                                          const uint16_t *__restrict__ Bias, int N, int G, int M,
                                          int gc, int ks, int tile0, int tstride, RowPtr row_ptr,
                                          Emit emit)
{
    extern __shared__ uint4 smem[];
    const int t = threadIdx.x, l = t & 63;
    const int g0 = ks * gc, gn = min(gc, G - g0);  // groups of this split, >= 1
    const int xstride = gc * 32 + 8;  // staged row: the chunk plus 16 bytes against bank conflicts
    // LDS: the activation chunk, M rows; affine: then the groups' sums of x,
    // [group of the split][16 rows]
    _Float16 *xs = reinterpret_cast<_Float16 *>(smem);
    float *xsum = reinterpret_cast<float *>(xs + M * xstride);
    const int cpr = gn * 4;           // 16-byte chunks per staged row

    // the tiles of this wave (a wave-uniform count: the guards below are
    // scalar branches)
    tile0 = __builtin_amdgcn_readfirstlane(tile0);
    const int ntiles = (N + 15) >> 4;
    const int my_tiles = tile0 < ntiles ? (ntiles - 1 - tile0) / tstride + 1 : 0;
    const int n = l & 15, kb = l >> 4;
    const int m = l & 15;
    // this lane's A operand row: rows past M repeat row M - 1 (they only feed
    // MFMA output rows that are never emitted)
    const _Float16 *xrow = xs + min(m, M - 1) * xstride + 8 * kb;
    const uint32_t mask = 0x000F000Fu;

    // step p of a tile covers groups 4p .. 4p + 3 of the split; lane (n, kb)
    // loads group 4p + kb of row n and its scale (branch-free: past the split
    // it re-reads the last group, which gets scale 0 below)
    auto load_tile = [&](TileRegs &r, int j) __attribute__((always_inline)) {
        const size_t rb = (size_t)min((tile0 + j * tstride) * 16 + n, N - 1) * G + g0;
#pragma unroll
        for (int p = 0; p < kDepth; ++p) {
            const int gi = min(4 * p + kb, gn - 1);
            r.w[p] = load_weights(W + rb + gi);
            if (AFF) {
                const size_t sb = (size_t)min((tile0 + j * tstride) * 16 + n, N - 1) * (G >> 1) +
                                  ((g0 + gi) >> 1);
                r.s[p] = load_scale(S + sb);
                r.b[p] = load_scale(Bias + sb);
            } else {
                r.s[p] = load_scale(S + rb + gi);
            }
        }
    };
    // Step p covers groups 4p .. 4p + 3 of the split, loaded by lane rows
    // 0..3. After a transpose, lane (n, kb) holds word kb of group 4p + t in
    // register t, so MFMA t takes exactly group 4p + t of the 16 rows: its B
    // operand is the exact integers q - 7 and its f32 result, the group's sum
    // of (q - 7) x, is scaled by that group's scale (broadcast from lane row t;
    // 0 past the split).
    auto compute_tile = [&](const TileRegs &r) __attribute__((always_inline)) {
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
        floatx4 acc = zero;
#pragma unroll
        for (int p = 0; p < kDepth; ++p) {
            half8 a[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)  // the four activation reads first
                a[tt] = *reinterpret_cast<const half8 *>(xrow + min(4 * p + tt, gn - 1) * 32);
            uint32_t sc[4], bc[4];
            broadcast_rows(4 * p + kb < gn ? r.s[p] : 0u, sc);
            if (AFF)
                broadcast_rows(4 * p + kb < gn ? r.b[p] : 0u, bc);
            uint32_t w[4] = {r.w[p].x, r.w[p].y, r.w[p].z, r.w[p].w};
            transpose_rows(w);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    a[tt], codes_minus7<AFF>(w[tt], mask), zero, 0, 0, 0);
                const float sf = h2f((uint16_t)sc[tt]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[e] = fmaf(sf, d[e], acc[e]);
                if (AFF) {  // + bias * (sum of x over the group) of rows 4 kb .. 4 kb + 3
                    const floatx4 sx = *reinterpret_cast<const floatx4 *>(
                        xsum + min(4 * p + tt, gn - 1) * 16 + 4 * kb);
                    const float bf = h2f((uint16_t)bc[tt]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[e] = fmaf(bf, sx[e], acc[e]);
                }
            }
        }
        return acc;
    };

    // 1. the activation chunk (all loads issued together, then stored in the
    //    pair order); affine: rows M .. 15 of the group sums are zero
    if (AFF) {
        for (int i = t; i < gc * 16; i += 256)
            xsum[i] = 0.f;
        __syncthreads();
    }
    u32x4 xr[kXq];
#pragma unroll
    for (int q = 0; q < kXq; ++q) {
        const int c = min(t + 256 * q, M * cpr - 1);  // branch-free: the tail re-reads
        const int mm = c / cpr, jj = c - mm * cpr;
        xr[q] = *reinterpret_cast<const u32x4 *>(row_ptr(mm) + (int64_t)g0 * 32 + 8 * jj);
    }
#pragma unroll
    for (int q = 0; q < kXq; ++q) {
        const int c = min(t + 256 * q, M * cpr - 1);  // the tail rewrites the last chunk
        const int mm = c / cpr, jj = c - mm * cpr;
        *reinterpret_cast<u32x4 *>(xs + mm * xstride + 8 * jj) = pair_order(xr[q]);
        if (AFF) {
            // the group's sum: 8 values in order, then the four 16-byte pieces
            // of the group, held by four consecutive lanes (chunk rows are
            // whole groups, so a quad of lanes never mixes groups or rows;
            // the tail's clamped lanes form quads of their own and do not write)
            const uint32_t u[4] = {xr[q].x, xr[q].y, xr[q].z, xr[q].w};
            float sm = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm = (sm + h2f((uint16_t)(u[e] & 0xFFFF))) + h2f((uint16_t)(u[e] >> 16));
            sm = quad_sum(sm);
            if ((jj & 3) == 0 && t + 256 * q < M * cpr)
                xsum[(jj >> 2) * 16 + mm] = sm;
        }
    }
    __syncthreads();

    // 2. the wave's tiles, one after another: a tile's loads are issued
    //    together and consumed in the same step (loads kept in flight across
    //    steps make the compiler copy, and so wait for, them); the resident
    //    waves of the CU overlap one another. Finished tiles stay in registers
    //    (a global store here would count against the loads in flight).
    floatx4 res[kMaxTilesPerWave];
#pragma unroll
    for (int j = 0; j < kMaxTilesPerWave; ++j)
        if (j < my_tiles) {
            TileRegs r;
            load_tile(r, j);
            res[j] = compute_tile(r);
        }

    // 3. emit: lane holds D[4 * (l / 16) + r][l % 16] of each tile
#pragma unroll
    for (int j = 0; j < kMaxTilesPerWave; ++j) {
        const int col = (tile0 + j * tstride) * 16 + n;
        if (j < my_tiles && col < N)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int mr = 4 * kb + r;
                if (mr < M)
                    emit(mr, col, res[j][r]);
            }
    }
}

// Batched matvec: grid (P, KS), 256 threads; wave w of workgroup b takes the
// tiles b * 4 + w, + 4 P, ... KS == 1: the f32 result written to yf when set,
// else rounded to y; KS > 1: f32 partials part[ks][m][n] for k_combine.
// (at most 128 registers: four waves per SIMD)
template <bool AFF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_gemv_mfma(const uint4 *__restrict__ W,
                                                   const uint16_t *__restrict__ S,
                                                   const uint16_t *__restrict__ Bias,
                                                   const uint16_t *__restrict__ x, int64_t ldx,
                                                   uint16_t *__restrict__ y,
                                                   float *__restrict__ yf, int64_t ldy,
                                                   float *__restrict__ part, int N, int G, int M,
                                                   int gc)
{
    const int ks = blockIdx.y, KS = gridDim.y;
    mfma_rows<AFF>(
        W, S, Bias, N, G, M, gc, ks, blockIdx.x * kWaves + (threadIdx.x >> 6), gridDim.x * kWaves,
        [&](int m) { return x + m * ldx; },
        [&](int mr, int col, float v) {
            if (KS > 1)
                part[((size_t)ks * M + mr) * N + col] = v;
            else if (yf)
                yf[mr * ldy + col] = v;
            else
                y[mr * ldy + col] = f2h(v);
        });
}

// MoE expert stage: grid (ceil(ntiles / 4), KS, slots); blockIdx.z is a
// distinct expert of the routing, whose pairs (token, slot) form the activation
// rows, 16 at a time. The routing comes from k_moe_route (meta), or, for few
// pairs and experts (meta == nullptr), from the workgroup itself. Per-pair f32
// results go to part[ks][pair][n].
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void k_moe_mfma(
    const uint4 *__restrict__ Wall, const uint16_t *__restrict__ Sall,
    const int32_t *__restrict__ ids, int E, const int32_t *__restrict__ meta, int P,
    const uint16_t *__restrict__ x, int64_t ldx, int64_t slot_stride, int TOPK,
    float *__restrict__ part, int N, int G, int gc)
{
    __shared__ int s_cnt[kFuseExperts];
    __shared__ int s_pairs[kFusePairs];
    __shared__ int s_np;
    const int d = blockIdx.z;
    int e, q0, q1;
    const int32_t *order;
    if (meta) {
        if (d >= meta[0])  // fewer distinct experts than slots: the whole workgroup leaves
            return;
        e = meta[1 + d];
        q0 = meta[1 + P + d];
        q1 = meta[1 + P + d + 1];
        order = meta + 2 + 2 * P;
    } else {
        e = route_in_workgroup(ids, P, E, d, kFusePairs, s_cnt, s_pairs, &s_np, &q0);
        if (e < 0)
            return;
        q1 = s_np;
        order = s_pairs;
    }
    const int ks = blockIdx.y;
    const uint4 *W = Wall + (size_t)e * N * G;
    const uint16_t *S = Sall + (size_t)e * N * G;
    for (int qa = q0; qa < q1; qa += kMTile) {
        if (qa > q0)
            __syncthreads();  // the previous rows' staged activation is still read
        mfma_rows<false>(
            W, S, nullptr, N, G, min(kMTile, q1 - qa), gc, ks, blockIdx.x * kWaves + (threadIdx.x >> 6),
            gridDim.x * kWaves,
            [&](int m) {
                const int pr = order[qa + m];
                return x + (int64_t)(pr / TOPK) * ldx + (int64_t)(pr % TOPK) * slot_stride;
            },
            [&](int mr, int col, float v) {
                part[((size_t)ks * P + order[qa + mr]) * N + col] = v;
            });
    }
}

// Per-pair results from the split partials (summed in split order), by mode:
//  MOE_PER_SLOT: y[p][n] = f16(r);  MOE_SILU: y[p][i] = f16(silu(f16(r_gate)) *
//  f16(r_up)) over the N / 2 gate and up rows;  MOE_COMBINE: y[t][n] =
//  f16(sum over slots s, in order, of route_w[t][s] * r[t * TOPK + s][n]).
// Pairs whose id is outside [0, E) get zeros (per-pair modes) or contribute
// nothing (combine).
__device__ __forceinline__ float moe_sum(const float *part, int KS, int P, int N, int p, int n)
{
    float v = 0.f;
    for (int k = 0; k < KS; ++k)
        v += part[((size_t)k * P + p) * N + n];
    return v;
}

__global__ __launch_bounds__(256) void k_moe_finish(int mode, const float *__restrict__ part,
                                                    int KS, int P, int N,
                                                    const int32_t *__restrict__ ids,
                                                    const uint16_t *__restrict__ route_w,
                                                    uint16_t *__restrict__ y, int E, int TOPK)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (mode == kMoeCombine) {
        const int T = P / TOPK;
        if (i >= (int64_t)T * N)
            return;
        const int t = (int)(i / N), n = (int)(i % N);
        float acc = 0.f;
        for (int s = 0; s < TOPK; ++s) {
            const int p = t * TOPK + s;
            const int e = ids[p];
            if (e >= 0 && e < E)
                acc = fmaf(h2f(route_w[p]), moe_sum(part, KS, P, N, p, n), acc);
        }
        y[(int64_t)t * N + n] = f2h(acc);
        return;
    }
    const int w = mode == kMoeSilu ? N / 2 : N;
    if (i >= (int64_t)P * w)
        return;
    const int p = (int)(i / w), c = (int)(i % w);
    const int e = ids[p];
    if (e < 0 || e >= E) {  // an invalid id contributes zeros
        y[(int64_t)p * w + c] = 0;
        return;
    }
    if (mode == kMoeSilu) {
        const float g = h2f(f2h(moe_sum(part, KS, P, N, p, c)));
        const float u = h2f(f2h(moe_sum(part, KS, P, N, p, w + c)));
        y[(int64_t)p * w + c] = f2h(silu_mul_f(g, u));
    } else {
        y[(int64_t)p * w + c] = f2h(moe_sum(part, KS, P, N, p, c));
    }
}

// sum over ks, in order, of part[ks][m][n]: to yf[m][n] when set, else
// rounded to y[m][n]
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ part, int KS, int M,
                                                 int N, uint16_t *__restrict__ y,
                                                 float *__restrict__ yf, int64_t ldy)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * N)
        return;
    const int mr = (int)(i / N), col = (int)(i % N);
    float s = 0.f;
    for (int k = 0; k < KS; ++k)
        s += part[((size_t)k * M + mr) * N + col];
    if (yf)
        yf[mr * ldy + col] = s;
    else
        y[mr * ldy + col] = f2h(s);
}


// ---------------------------------------------------------------------------
// Batched matvec for a few activation rows on the matrix cores with the
// single-row kernel's nibble unpack (k_gemv_mma).
//
// With y[m][n] = sum_g s[n][g] * (sum_{k in g} c[n][k] x[m][k] - 7 X_g[m]),
// X_g[m] the sum of activation row m over group g:
//  * the code sums take one MFMA per group and 16-row tile
//    (v_mfma_f32_16x16x32_f16, A = activation rows, B = weights). B holds the
//    codes as the exact binary16 subnormals the single-row kernel forms (one
//    shift and four ANDs per word): c * 2^-24 in the pairs (e0, e4) and
//    (e2, e6), c * 2^-20 in (e1, e5) and (e3, e7). A holds the activation in
//    the same pair order, the values that meet the 2^-20 pairs divided by 16
//    (exact for |x| >= 2^-10), so that each product is c * x * 2^-24. The lane
//    adds the group's f32 sum times the row's scale to its accumulator;
//  * the zero-point term sum_g s[n][g] X_g[m] is itself a contraction over the
//    groups: one v_mfma_f32_16x16x4_f32 per four groups and tile, A = the
//    activation's group sums (f32), B = the scales;
//  * y = 2^24 * (code part) - 7 * (zero-point part).
// For a one-hot activation both parts are exact (c s and 7 s, at most 15
// significant bits) and so is their difference: the result is (q - 7) * s
// exactly, as with the other matvecs. A-operand rows m >= M repeat row M - 1
// and are never stored.
// AFF (the MLX affine format, w = s q + b per 64 values, scales and biases
// [N][G/2]): the code part is the same with each 64-value group's scale on
// both of its 32-value halves, and the second contraction takes the biases in
// place of the scales: y = 2^24 * (code part) + (bias part).
//
// Work split. One workgroup of kMmaWaves waves per CU stages the activation
// once in LDS (pair order, odd positions / 16, group sums) and keeps it for
// the whole launch. A unit of work is one 16-row tile times one of KP equal
// parts of K (SK = 2 SK2 steps of four groups); wave w takes part w % KP of
// the tiles blockIdx.x + gridDim.x * (w / KP + (kMmaWaves / KP) * round), one
// unit per round (waves from (kMmaWaves / KP) * KP on, when KP does not
// divide kMmaWaves, take none). A wave issues all loads of a unit at once, in
// whole memory lines: the unit's scales as a row-major block (64 consecutive
// scales, or pairs of them, per load), then its weights as 8 rows x 128 bytes per load
// (a pair of steps per two loads). The scales go to a per-wave LDS block, each
// pair of steps' weights to a per-wave LDS tile from which every lane reads
// the words of its MFMA lane (word kb of each group of row n): no exchanges
// across lanes in registers. The KP parts of a tile meet in an LDS slot
// without a barrier, so the waves of a CU drift apart and one wave's loads
// overlap another's arithmetic: the last of the KP waves to arrive (an LDS
// counter) adds the parts in K order, stores, and frees the slot for its use
// two rounds later. A wave stops at its first tile past the last one; the KP
// waves of a tile slot share their tiles, so they stop together. Where the
// staged rows of the whole of K exceed the LDS (PH), the launch has one round
// and K runs in NPH phases of KPH groups: the workgroup stages one phase's
// activation at a time (a barrier before each restaging), and each wave adds
// its part of every phase into the same sums before the parts meet.
constexpr int kMmaWaves = 12;   // three waves per SIMD
constexpr int kMmaMaxPairs = 6;  // steps per unit <= 12 (7 pairs spill registers)
constexpr int kMmaXq = 8;       // activation chunks per thread held in registers
constexpr int kMmaTileStride = 9;  // 16-byte slots per row of the weight tile (8 + 1 against conflicts)

// The subnormal codes of word w as a B operand, pairs (e0,e4) (e1,e5) (e2,e6)
// (e3,e7).
__device__ __forceinline__ half8 codes_subnormal(uint32_t w)
{
    const uint32_t m0 = 0x000F000Fu, m1 = 0x00F000F0u, t = w >> 8;
    const u32x4 v = {w & m0, w & m1, t & m0, t & m1};
    return __builtin_bit_cast(half8, v);
}

struct MmaArgs {
    const uint4 *W;
    const uint16_t *S;
    const uint16_t *B;  // AFF: the biases [N][G/2]
    const uint16_t *x;
    int64_t ldx;
    uint16_t *y;  // f16 results, or
    float *yf;    // f32 results
    int64_t ldy;
    // when set: the workgroup's largest argmax_key of each of its rows' results,
    // cand[m * gridDim.x + blockIdx.x]
    unsigned long long *cand;
    int N, G, M;
    int KP, rounds;  // K parts, rounds
    int NPH, KPH;    // K phases and groups per phase (one phase: 1 and G)
};

// LDS bytes of one wave's scale block (AFF: scale and bias per group, 4
// bytes) and weight tile
constexpr int mma_wave_lds(int SK2, bool AFF = false)
{
    return 16 * 8 * SK2 * (AFF ? 4 : 2) + 16 * kMmaTileStride * 16;
}

template <int SK2, bool SP, bool AFF, bool PH>
__global__ __launch_bounds__(64 * kMmaWaves) void k_gemv_mma(MmaArgs a)
{
    static_assert(!(AFF && SP), "affine scales are loaded one per group");
    constexpr int SK = 2 * SK2;  // steps per unit
    constexpr int GU = 4 * SK;   // groups per unit
    // short units: the first unit's loads go out before the activation is
    // staged (behind its loads); with long units, the whole matrix at once
    // would hold the activation's loads back in the memory queues
    constexpr bool kEarly = SK2 <= 3;
    extern __shared__ uint4 smem[];
    __shared__ unsigned long long s_cand[16];  // (cand) each row's largest key so far
    const int G = a.G, M = a.M, N = a.N;
    // PH: K in NPH phases of KPH groups, the activation staged one phase at a
    // time (one round: each wave's unit accumulates over the phases)
    const int KPH = PH ? a.KPH : G, NPH = PH ? a.NPH : 1;
    const int xstride = KPH * 32 + 8;  // staged row: 16 bytes of padding against bank conflicts
    const int t = threadIdx.x, l = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int n = l & 15, kb = l >> 4;
    // LDS: per wave a scale block [16][GU] and a weight tile [16][9] x 16 B;
    // the waves' parts [2][kMmaWaves][64 lanes][4] f32; arrival counters and
    // use counts [2][kMmaWaves] u32 each; the staged rows [M][xstride]
    // binary16; the group sums [KPH][16] f32
    char *wbase = reinterpret_cast<char *>(smem) + (size_t)wave * mma_wave_lds(SK2, AFF);
    uint16_t *sblk = reinterpret_cast<uint16_t *>(wbase);  // AFF: uint32 (scale | bias << 16)
    uint4 *wtile = reinterpret_cast<uint4 *>(wbase + 16 * GU * (AFF ? 4 : 2));
    float *red = reinterpret_cast<float *>(reinterpret_cast<char *>(smem) +
                                           (size_t)kMmaWaves * mma_wave_lds(SK2, AFF));
    uint32_t *arrived = reinterpret_cast<uint32_t *>(red + 2 * kMmaWaves * 256);
    uint32_t *uses = arrived + 2 * kMmaWaves;
    _Float16 *xs = reinterpret_cast<_Float16 *>(uses + 2 * kMmaWaves);
    float *xsum = reinterpret_cast<float *>(xs + M * xstride);

    const int KP = a.KP, rounds = a.rounds;
    const int kp = wave % KP, tslot = wave / KP, tpr = kMmaWaves / KP;
    const int ntiles = (N + 15) >> 4;
    // waves past tpr * KP (KP not dividing kMmaWaves) take no tiles
    const bool working = tslot < tpr;
    const int gp0 = kp * GU;  // first group of this wave's part of K (of the phase)
    auto tile_of = [&](int r) { return (int)blockIdx.x + (int)gridDim.x * (tslot + tpr * r); };

    // the loads of unit r over groups [gbase, gend) (branch-free: groups past
    // gend re-read group gend - 1 and are zeroed at use; rows past N re-read
    // row N - 1): its scales as elements e = 64 j + l of the row-major block
    // [16][GU], then its weights, pair q and half i as lane l reading group
    // gbase + gp0 + 8 q + (l & 7) of row 8 i + (l >> 3): 8 rows x 128 bytes
    // per load
    // (SP, G even: the scales in pairs, elements 2 (64 j + l) and the next, one
    // 4-byte load each: a pair never straddles a row and is 4-byte aligned;
    // AFF: element e holds its 64-value group's scale and bias, s | b << 16)
    constexpr int NSL = SP ? SK2 : SK;  // scale loads per unit
    struct Unit {
        uint32_t sl[NSL];
        uint4 wl[SK2][2];
    };
    auto load_unit = [&](int r, Unit &u, int gbase, int gend) __attribute__((always_inline)) {
        const int row0 = min(tile_of(r), ntiles - 1) * 16;
#pragma unroll
        for (int j = 0; j < NSL; ++j) {
            const int e = SP ? 2 * (64 * j + l) : 64 * j + l;
            const int rr = e / GU, cc = e - rr * GU;
            if (AFF) {
                const size_t off = (size_t)min(row0 + rr, N - 1) * (G >> 1) +
                                   (min(gbase + gp0 + cc, gend - 1) >> 1);
                u.sl[j] = load_scale(a.S + off) | (load_scale(a.B + off) << 16);
                continue;
            }
            const size_t off = (size_t)min(row0 + rr, N - 1) * G +
                               min(gbase + gp0 + cc, gend - (SP ? 2 : 1));
            if (SP)
                u.sl[j] = __builtin_nontemporal_load(
                    (__attribute__((address_space(1))) const uint32_t *)(a.S + off));
            else
                u.sl[j] = load_scale(a.S + off);
        }
#pragma unroll
        for (int q = 0; q < SK2; ++q)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int rr = min(row0 + 8 * i + (l >> 3), N - 1);
                u.wl[q][i] = load_weights(a.W + (size_t)rr * G +
                                          min(gbase + gp0 + 8 * q + (l & 7), gend - 1));
            }
    };

    Unit ua;
    // 2. the units' arithmetic (the rounds follow the staging below)
    unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};  // (cand) rows 4 kb + e
    const int mrow = min(n, M - 1);  // A row m = n
    const _Float16 *xrow = xs + mrow * xstride + 8 * kb;
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    // the unit's products over groups [gbase, gend) (the staged activation's
    // first group is gbase) added to acc (code part) and acc0 (second
    // contraction)
    auto accumulate = [&](const Unit &u, floatx4 &acc, floatx4 &acc0, int gbase, int gend)
                          __attribute__((always_inline)) {
        // the scales into the wave's block (a wave's LDS accesses complete in
        // order: the previous unit's reads are done)
#pragma unroll
        for (int j = 0; j < NSL; ++j) {
            if (SP || AFF)
                reinterpret_cast<uint32_t *>(sblk)[64 * j + l] = u.sl[j];
            else
                sblk[64 * j + l] = (uint16_t)u.sl[j];
        }
#pragma unroll
        for (int q = 0; q < SK2; ++q) {
            // the pair's weights into the wave's tile: row 8 i + (l >> 3), slot
            // l & 7 (the previous pair's reads are done)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                wtile[(8 * i + (l >> 3)) * kMmaTileStride + (l & 7)] = u.wl[q][i];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int p = 2 * q + h;
                const int gb = gbase + gp0 + 4 * p;  // the step's first group (uniform)
                half8 av[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    av[tt] = *reinterpret_cast<const half8 *>(
                        xrow + (min(gb + tt, gend - 1) - gbase) * 32);
                const float a0 = xsum[(min(gb + kb, gend - 1) - gbase) * 16 + mrow];
                // word kb of group 4 h + tt of row n
                uint32_t w[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    w[tt] = reinterpret_cast<const uint32_t *>(
                        &wtile[n * kMmaTileStride + 4 * h + tt])[kb];
                // the step's four scales of row n (zero past G), and the
                // second contraction's operand for group gb + kb: its scale
                // (AFF: its bias)
                uint32_t sc[4], sk;
                if (AFF) {
                    const uint4 sb = *reinterpret_cast<const uint4 *>(
                        &reinterpret_cast<const uint32_t *>(sblk)[n * GU + 4 * p]);
                    sc[0] = sb.x & 0xFFFFu;
                    sc[1] = sb.y & 0xFFFFu;
                    sc[2] = sb.z & 0xFFFFu;
                    sc[3] = sb.w & 0xFFFFu;
                    const uint32_t bk = (kb & 2) ? ((kb & 1) ? sb.w : sb.z) : ((kb & 1) ? sb.y : sb.x);
                    sk = gb + kb < gend ? bk >> 16 : 0u;
                } else {
                    const uint2 s4 = *reinterpret_cast<const uint2 *>(&sblk[n * GU + 4 * p]);
                    sc[0] = s4.x & 0xFFFFu;
                    sc[1] = s4.x >> 16;
                    sc[2] = s4.y & 0xFFFFu;
                    sc[3] = s4.y >> 16;
                    const uint32_t hs = (kb & 2) ? s4.y : s4.x;
                    sk = gb + kb < gend ? ((kb & 1) ? hs >> 16 : hs & 0xFFFFu) : 0u;
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    if (gb + tt >= gend)
                        sc[tt] = 0u;
                acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, h2f((uint16_t)sk), acc0, 0, 0, 0);
                floatx4 d[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    d[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[tt], codes_subnormal(w[tt]),
                                                                   zero, 0, 0, 0);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    // the f16 scale converted inside the FMA (v_fma_mix_f32)
                    const float sf = h2f((uint16_t)sc[tt]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[e] = fmaf(sf, d[tt][e], acc[e]);
                }
                // the step's products are accumulated here, not deferred to
                // the end of the unrolled steps (which would keep every
                // step's MFMA results live at once)
                asm volatile("" : "+v"(acc));
            }
        }
    };
    // the wave's part of tile_of(r) from its sums, then the meeting and store
    auto finish = [&](int r, floatx4 acc, const floatx4 &acc0) __attribute__((always_inline)) {
        // this wave's part: 2^24 * code part - 7 * zero-point part (AFF:
        // + bias part)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc[e] = fmaf(AFF ? 1.0f : -7.0f, acc0[e], acc[e] * 0x1p24f);
        // the KP parts of the tile meet in LDS slot r & 1 without a barrier:
        // each wave waits until the slot's previous use (round r - 2) has
        // been read, writes its part, and counts itself in; the last to
        // arrive adds the parts in K order, stores, and releases the slot.
        // Lane (n, kb) holds rows m = 4 kb .. 4 kb + 3 of column n.
        const int tile = tile_of(r);
        bool last = true;
        floatx4 v = acc;
        if (KP > 1) {
            const int sl = (r & 1) * kMmaWaves + tslot;
            float *slot = red + (size_t)(r & 1) * kMmaWaves * 256;
            const uint32_t want = (uint32_t)(r >> 1);
            // (bounded: the reader of round r - 2 depends on no other wave)
            for (int spin = 0; spin < (1 << 22); ++spin) {
                const uint32_t u =
                    __hip_atomic_load(&uses[sl], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (__builtin_amdgcn_readfirstlane(u) == want)
                    break;
                __builtin_amdgcn_s_sleep(2);
            }
            *reinterpret_cast<floatx4 *>(slot + (wave * 64 + l) * 4) = acc;
            uint32_t before = 0;
            if (l == 0)
                before = __hip_atomic_fetch_add(&arrived[sl], 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_WORKGROUP);
            last = __builtin_amdgcn_readfirstlane(before) == (uint32_t)(KP - 1);
            if (last) {
                const int w0 = tslot * KP;  // the tile's kp = 0 wave
                v = *reinterpret_cast<const floatx4 *>(slot + (w0 * 64 + l) * 4);
                for (int qq = 1; qq < KP; ++qq) {
                    const floatx4 o = *reinterpret_cast<const floatx4 *>(slot + ((w0 + qq) * 64 + l) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] += o[e];
                }
                if (l == 0) {
                    __hip_atomic_store(&arrived[sl], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    __hip_atomic_store(&uses[sl], want + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
                }
            }
        }
        if (last && tile < ntiles) {
            const int col = tile * 16 + n;
            if (col < N)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = 4 * kb + e;
                    if (m < M) {
                        if (a.yf)
                            a.yf[m * a.ldy + col] = v[e];
                        else
                            a.y[m * a.ldy + col] = f2h(v[e]);
                        if (a.cand) {
                            const unsigned long long key = argmax_key(v[e], (uint32_t)col);
                            best[e] = key > best[e] ? key : best[e];
                        }
                    }
                }
        }
    };
    // 3. the activation's chunks of groups [gbase, gend) (up to kMmaXq per
    //    thread) into registers, then into LDS: the pair order, the odd
    //    positions x1 x3 x5 x7 (the high halves of the words, which meet the
    //    2^-20 pairs) divided by 16, and each group's sum of the unscaled
    //    values (a quad of lanes holds the four chunks of a group: cpr and the
    //    thread count are multiples of 4, so quads never mix rows). early: the
    //    first unit's loads go out between the two.
    //    Staged once (PH: phase by phase, each wave adding its unit's part of
    //    the phase into pacc / pacc0), then the rounds.
    const bool mine = PH && working && tile_of(0) < ntiles;  // PH: one round
    floatx4 pacc = zero, pacc0 = zero;
    for (int ph = 0; ph < NPH; ++ph) {
        const int gbase = ph * KPH, gend = min(G, gbase + KPH);
        if (ph > 0)
            __syncthreads();  // the previous phase's activation reads are done
        {
            const int cpr = (gend - gbase) * 4;
            const int total = M * cpr;  // a multiple of 4
            constexpr int kThreads = 64 * kMmaWaves;
            const half2v odd16 = {(_Float16)1.0f, (_Float16)0.0625f};
            const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
            // chunk c = i * kThreads + t of the phase as (row m, chunk j of
            // the row): one division per thread, then steps of kThreads chunks
            // (c < total exactly when m < M; cpr and kThreads are multiples of
            // 4, so j & 3 is the chunk's place in its quad)
            struct Pos {
                int m, j;
            };
            const int dm = kThreads / cpr, dj = kThreads - dm * cpr;  // uniform
            auto step = [&](Pos q) __attribute__((always_inline)) {
                q.m += dm;
                q.j += dj;
                if (q.j >= cpr) {
                    q.j -= cpr;
                    ++q.m;
                }
                return q;
            };
            auto chunk = [&](Pos q) __attribute__((always_inline)) {
                // a quad past the end re-reads the last group and stores nothing
                if (q.m >= M)
                    q = Pos{M - 1, cpr - 4 + (q.j & 3)};
                return *reinterpret_cast<const u32x4 *>(a.x + q.m * a.ldx + 8 * (4 * gbase + q.j));
            };
            auto stage = [&](Pos q, u32x4 v) __attribute__((always_inline)) {
                float sum = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // through a scalar: this compiler's bit_cast of a vector
                    // element reads element 0
                    const uint32_t h = v[e];
                    sum = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, h), ones, sum, false);
                    v[e] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, h) * odd16);
                }
                sum = quad_sum(sum);
                if (q.m < M) {
                    *reinterpret_cast<u32x4 *>(xs + q.m * xstride + 8 * q.j) = pair_order(v);
                    if ((q.j & 3) == 0)
                        xsum[(q.j >> 2) * 16 + q.m] = sum;
                }
            };
            const Pos p0 = {t / cpr, t - (t / cpr) * cpr};
            const int xq = min((total + kThreads - 1) / kThreads, kMmaXq);  // uniform
            u32x4 xr[kMmaXq];
            // PH: every register chunk is loaded (those past the end re-read
            // the last quad): loads under the uniform guard, in the phase
            // loop, leave the compiler waiting on each before the next issues
            Pos q = p0;
#pragma unroll
            for (int i = 0; i < kMmaXq; ++i) {
                if (PH || i < xq)
                    xr[i] = chunk(q);
                q = step(q);
            }
            if (PH ? kEarly && mine : kEarly)
                load_unit(0, ua, gbase, gend);
            q = p0;
#pragma unroll
            for (int i = 0; i < kMmaXq; ++i) {
                if (i < xq)
                    stage(q, xr[i]);
                q = step(q);
            }
            // more chunks than the registers hold: the rest one by one
            for (int c0 = kMmaXq * kThreads; c0 < total; c0 += kThreads) {
                stage(q, chunk(q));
                q = step(q);
            }
        }
        if (ph == 0) {
            if (t < 4 * kMmaWaves)
                arrived[t] = 0u;  // and uses[]
            if (t < 16)
                s_cand[t] = 0ull;
        }
        __syncthreads();
        if (mine) {
            if (!kEarly)
                load_unit(0, ua, gbase, gend);
            accumulate(ua, pacc, pacc0, gbase, gend);
        }
    }
    if (!PH) {
        for (int r = 0; working && r < rounds; ++r) {
            // tiles grow with the round: a wave stops at its first tile past
            // the last, and every wave of its tile slot (the KP parts that
            // meet in LDS) stops at the same round
            if (tile_of(r) >= ntiles)
                break;
            if (!kEarly || r > 0)
                load_unit(r, ua, 0, G);
            floatx4 acc = zero, acc0 = zero;
            accumulate(ua, acc, acc0, 0, G);
            finish(r, acc, acc0);
        }
    } else if (mine) {
        finish(0, pacc, pacc0);
    }
    if (a.cand) {
        // the lane row's largest keys over its 16 lanes (rows 4 kb + e), into
        // the workgroup's, and once every wave is done, out
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int off = 1; off < 16; off <<= 1)
            {
                const unsigned long long o = __shfl_xor(best[e], off);
                best[e] = o > best[e] ? o : best[e];
            }
            if (n == 0 && 4 * kb + e < M)
                __hip_atomic_fetch_max(&s_cand[4 * kb + e], best[e], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        __syncthreads();
        if (t < M)
            a.cand[(size_t)t * gridDim.x + blockIdx.x] = s_cand[t];
    }
}

}  // namespace

int mfma_splits(int K)
{
    return (K / 32 + kGroupsPerSplit - 1) / kGroupsPerSplit;
}

size_t mfma_part_bytes(int N, int K)
{
    const int KS = mfma_splits(K);
    return KS > 1 ? (size_t)KS * kMTile * N * sizeof(float) : 0;
}

q4_status launch_mfma_rows(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                           uint16_t *y, float *yf, int64_t ldy, int N, int K, int mt,
                           float *part, hipStream_t stream, const uint16_t *bias)
{
    const int G = K / 32;
    // K splits of kGroupsPerSplit groups (the last may be shorter)
    const int gc = kGroupsPerSplit;
    const int KS = mfma_splits(K);
    const int ntiles = (N + 15) / 16;
    // about three resident workgroups per CU, each looping over its tiles (at
    // most kMaxTilesPerWave per wave)
    const int P = std::max({1, (ntiles + kWaves * kMaxTilesPerWave - 1) / (kWaves * kMaxTilesPerWave),
                            std::min((ntiles + kWaves - 1) / kWaves, (3 * cu_count() + KS - 1) / KS)});
    const size_t lds = (size_t)mt * (gc * 32 + 8) * 2 +          // staged rows
                       (bias ? (size_t)gc * 16 * sizeof(float) : 0);  // affine: group sums
    if (bias)
        Q4_LAUNCH_MATVEC(k_gemv_mfma<true>, dim3(P, KS), dim3(256), lds, stream,
                         reinterpret_cast<const uint4 *>(W), S, bias, x, ldx, yf ? nullptr : y, yf,
                         ldy, part, N, G, mt, gc);
    else
        Q4_LAUNCH_MATVEC(k_gemv_mfma<false>, dim3(P, KS), dim3(256), lds, stream,
                         reinterpret_cast<const uint4 *>(W), S, nullptr, x, ldx,
                         yf ? nullptr : y, yf, ldy, part, N, G, mt, gc);
    return check_launch("k_gemv_mfma");
}

namespace {
// The launch of k_gemv_mma for an N x K matrix and mt <= 16 activation rows:
// the K parts per tile, the rounds, workgroups and LDS bytes. Among the part
// counts KP = 1..12 whose part fits a unit (at most 2 max_pairs steps), whose
// last part is not empty and whose LDS fits the CU, the plan takes the fewest
// rounds (each round adds a wave's load latency and the meeting of the parts:
// measured, more rounds of shorter units are slower), then the least
// occupancy of the workgroup's waves (working waves x rounds x steps per unit,
// the padding of a short last part included; counting only the steps of the
// tiles that exist would favour long units on few waves). lds is SIZE_MAX
// when no part count fits.
struct MmaPlan {
    int KP, SK2, rounds, blocks;
    int NPH, KPH;  // K phases (the activation staged one phase at a time) and groups per phase
    size_t lds;
};

constexpr size_t kMmaLdsLimit = 160 * 1024;
constexpr int kMmaMaxPhases = 4;

MmaPlan mma_plan(int N, int K, int mt, bool aff)
{
    MmaPlan pl;
    const int G = K / 32, ntiles = (N + 15) / 16;
    // (6 pairs with single scales, G odd or affine, spill registers)
    const int max_pairs = G % 2 == 0 && !aff ? kMmaMaxPairs : kMmaMaxPairs - 1;
    pl.blocks = std::min(cu_count(), ntiles);
    pl.KP = 0;
    pl.lds = SIZE_MAX;
    // the fewest K phases that fit the CU's LDS (several phases only with one
    // round: a wave's unit then accumulates over the phases)
    for (int nph = 1; nph <= kMmaMaxPhases && !pl.KP; ++nph) {
        int kph = (G + nph - 1) / nph;
        kph += nph > 1 ? (kph & 1) : 0;  // even: pairs of scales stay in one phase
        if (nph > 1 && (int64_t)kph * (nph - 1) >= G)
            break;  // the last phase would be empty
        const int steps = (kph + 3) / 4;  // steps of four groups over a phase
        int64_t best_work = 0;
        for (int c = 1; c <= kMmaWaves; ++c) {
            const int sk2 = ((steps + c - 1) / c + 1) / 2;
            if (sk2 > max_pairs || (c > 1 && (c - 1) * 2 * sk2 >= steps))
                continue;  // a unit of too many steps, or an empty last part
            const size_t lds = (size_t)kMmaWaves * mma_wave_lds(sk2, aff) +
                               (size_t)2 * kMmaWaves * 256 * sizeof(float) +
                               (size_t)4 * kMmaWaves * sizeof(uint32_t) +
                               (size_t)mt * (kph * 32 + 8) * 2 + (size_t)kph * 16 * sizeof(float);
            if (lds > kMmaLdsLimit)
                continue;
            const int tpr = kMmaWaves / c;
            const int rounds = (ntiles + pl.blocks * tpr - 1) / (pl.blocks * tpr);
            if (nph > 1 && rounds > 1)
                continue;
            const int64_t work = (int64_t)tpr * c * rounds * 2 * sk2;
            if (!pl.KP || rounds < pl.rounds || (rounds == pl.rounds && work < best_work)) {
                pl.KP = c;
                pl.SK2 = sk2;
                pl.rounds = rounds;
                pl.NPH = nph;
                pl.KPH = kph;
                pl.lds = lds;
                best_work = work;
            }
        }
    }
    return pl;
}

template <int SK2, bool PH>
q4_status run_mma(const MmaArgs &args, const MmaPlan &pl, hipStream_t stream)
{
    if (args.B)
        Q4_LAUNCH_MATVEC((k_gemv_mma<SK2, false, true, PH>), dim3(pl.blocks),
                         dim3(64 * kMmaWaves), pl.lds, stream, args);
    else if (args.G % 2 == 0 && (reinterpret_cast<uintptr_t>(args.S) & 3) == 0)
        Q4_LAUNCH_MATVEC((k_gemv_mma<SK2, true, false, PH>), dim3(pl.blocks),
                         dim3(64 * kMmaWaves), pl.lds, stream, args);
    else
        Q4_LAUNCH_MATVEC((k_gemv_mma<SK2, false, false, PH>), dim3(pl.blocks),
                         dim3(64 * kMmaWaves), pl.lds, stream, args);
    return check_launch("k_gemv_mma");
}
}  // namespace

bool mma_fits(int N, int K, int M, bool aff)
{
    return mma_plan(N, K, std::min(M, kMTile), aff).lds <= kMmaLdsLimit;
}

int mma_blocks(int N) { return std::min(cu_count(), (N + 15) / 16); }

q4_status launch_gemv_mma(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                          uint16_t *y, float *yf, int64_t ldy, int N, int K, int M,
                          hipStream_t stream, unsigned long long *cand, const uint16_t *bias)
{
    for (int m0 = 0; m0 < M; m0 += kMTile) {
        const int mt = std::min(kMTile, M - m0);
        const MmaPlan pl = mma_plan(N, K, mt, bias != nullptr);
        if (pl.lds > kMmaLdsLimit)
            return fail(Q4_ERANGE, "internal: the batched matrix-core kernel does not fit K = %d", K);
        MmaArgs args;
        args.W = reinterpret_cast<const uint4 *>(W);
        args.S = S;
        args.B = bias;
        args.x = x + m0 * ldx;
        args.ldx = ldx;
        args.y = yf ? nullptr : y + m0 * ldy;
        args.yf = yf ? yf + m0 * ldy : nullptr;
        args.ldy = ldy;
        args.cand = cand ? cand + (size_t)m0 * pl.blocks : nullptr;
        args.N = N;
        args.G = K / 32;
        args.M = mt;
        args.KP = pl.KP;
        args.rounds = pl.rounds;
        args.NPH = pl.NPH;
        args.KPH = pl.KPH;
        q4_status st;
        switch (pl.SK2) {
#define Q4_MMA_CASE(d)                                                                            \
    case d:                                                                                       \
        st = pl.NPH > 1 ? run_mma<d, true>(args, pl, stream) : run_mma<d, false>(args, pl, stream); \
        break;
            Q4_MMA_CASE(1) Q4_MMA_CASE(2) Q4_MMA_CASE(3) Q4_MMA_CASE(4) Q4_MMA_CASE(5) Q4_MMA_CASE(6)
#undef Q4_MMA_CASE
        default: return fail(Q4_ERANGE, "internal: %d step pairs for the batched matrix-core kernel", pl.SK2);
        }
        if (st != Q4_OK)
            return st;
    }
    return Q4_OK;
}

size_t ws_rows(int N, int K, int M)
{
    // single-row, few-row and workgroup-reduced kernels, or no K split, for
    // both formats (the affine call checks the few-row kernel without N, and
    // its workgroup-reduced kernel needs more LDS)
    if (M <= 1 || mfma_splits(K) <= 1 || mma_fits(N, K, M, true) ||
        (gemv_rows_fits(M, K, N) && gemv_rows_fits(M, K)))
        return 0;
    return kWsHeader + mfma_part_bytes(N, K);
}

q4_status launch_gemv_mfma(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                           uint16_t *y, float *yf, int64_t ldy, int N, int K, int M,
                           hipStream_t stream, const uint16_t *bias)
{
    if (mma_fits(N, K, M, bias != nullptr))
        return launch_gemv_mma(W, S, x, ldx, y, yf, ldy, N, K, M, stream, nullptr, bias);
    const int KS = mfma_splits(K);
    float *part = nullptr;
    if (KS > 1) {
        char *ws = static_cast<char *>(workspace(stream, ws_rows(N, K, M)));
        if (!ws)
            return workspace_status();
        part = reinterpret_cast<float *>(ws + kWsHeader);
    }
    for (int m0 = 0; m0 < M; m0 += kMTile) {
        const int mt = std::min(kMTile, M - m0);
        q4_status st = launch_mfma_rows(W, S, x + m0 * ldx, ldx, yf ? nullptr : y + m0 * ldy,
                                        yf ? yf + m0 * ldy : nullptr, ldy, N, K, mt, part,
                                        stream, bias);
        if (st != Q4_OK)
            return st;
        if (KS > 1) {
            const int64_t total = (int64_t)mt * N;
            hipLaunchKernelGGL(k_combine, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                               stream, part, KS, mt, N, yf ? nullptr : y + m0 * ldy,
                               yf ? yf + m0 * ldy : nullptr, ldy);
            if ((st = check_launch("k_combine")) != Q4_OK)
                return st;
        }
    }
    return Q4_OK;
}

q4_status launch_moe_mfma(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                          const int32_t *meta, const uint16_t *route_w, const uint16_t *x,
                          int64_t ldx, int64_t x_slot_stride, uint16_t *y, float *part, int E,
                          int N, int K, int T, int TOPK, int mode, hipStream_t stream)
{
    const int P = T * TOPK, G = K / 32;
    const int gc = kGroupsPerSplit, KS = (G + gc - 1) / gc;
    const int ntiles = (N + 15) / 16;
    const dim3 grid((ntiles + kWaves - 1) / kWaves, KS, std::min(P, E));
    const size_t lds = (size_t)kMTile * (gc * 32 + 8) * 2;  // staged rows
    Q4_LAUNCH_MATVEC(k_moe_mfma, grid, dim3(256), lds, stream, reinterpret_cast<const uint4 *>(W),
                     S, ids, E, meta, P, x, ldx, x_slot_stride, TOPK, part, N, G, gc);
    q4_status st = check_launch("k_moe_mfma");
    if (st != Q4_OK)
        return st;
    return launch_moe_finish(mode, part, KS, P, N, ids, route_w, y, E, T, TOPK, stream);
}

q4_status launch_moe_finish(int mode, const float *part, int KS, int P, int N,
                            const int32_t *ids, const uint16_t *route_w, uint16_t *y, int E,
                            int T, int TOPK, hipStream_t stream)
{
    const int64_t total = mode == kMoeCombine ? (int64_t)T * N
                                              : (int64_t)P * (mode == kMoeSilu ? N / 2 : N);
    hipLaunchKernelGGL(k_moe_finish, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       mode, part, KS, P, N, ids, route_w, y, E, TOPK);
    return check_launch("k_moe_finish");
}

bool moe_routes_in_kernel(int P, int E) { return P <= kFusePairs && E <= kFuseExperts; }

size_t moe_part_bytes(int N, int K, int P)
{
    const int G = K / 32, KS = (G + kGroupsPerSplit - 1) / kGroupsPerSplit;
    return (size_t)KS * P * N * sizeof(float);
}

}  // namespace q4
