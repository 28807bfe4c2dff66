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

size_t ws_rows(int N, int K, int M)
{
    if (M <= 1 || gemv_rows_fits(M, K) || mfma_splits(K) <= 1)
        return 0;  // single-row and few-row kernels, or no K split
    return kWsHeader + mfma_part_bytes(N, K);
}

q4_status launch_gemv_mfma(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                           uint16_t *y, float *yf, int64_t ldy, int N, int K, int M,
                           hipStream_t stream, const uint16_t *bias)
{
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
