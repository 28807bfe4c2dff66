// Batched int4 x f16 matvec on the gfx950 matrix cores: M = 2..16 activation
// rows share one read of the weights (more rows: one launch per 16).
//
// What is computed is the group-quantised matvec of the Zero TVM Documentation
// ("Q4F16 quantization format"; the batched decode of "WGSL Kernel Roles"):
// y[m][n] = sum_k (q[n][k] - 7) * s[n][k/32] * x[m][k]. At M >= 2 the shared
// weight read makes it a small dense contraction, so it runs on
// v_mfma_f32_16x16x32_f16 (one MFMA = 16 activation rows x 16 weight rows x
// one 32-element quantisation group):
//  * the B operand is the weights w = (q - 7) * s, dequantised in registers as
//    two binary16 vectors hi + lo whose sum is exact (dequant_split), each
//    multiplied by the activation on the matrix core with f32 accumulation:
//    no dequantised weight is rounded;
//  * the A operand is the activation, staged once per workgroup in LDS; rows
//    m >= M of the MFMA tile are never stored;
//  * a lane (row n = lane % 16, k-block kb = lane / 16) loads one 16-byte
//    group of its row per step (four consecutive groups per wave and step, 64
//    bytes contiguous per row), and MFMA t of the step takes word t of that
//    group: lane (., kb) of both operands then covers k = 32 (g0 + kb) + 8 t +
//    0..7, so A and B agree on every k and each 16-byte load feeds four MFMA
//    pairs;
//  * about three workgroups per CU stay resident: each stages its activation
//    chunk once and its waves then loop over 16-row tiles, a tile's 8 KB of
//    weights in flight per wave (an activation staging per tile would queue
//    behind the other workgroups' weight loads on the CU);
//  * K is split into chunks of 1024 values (the staged activation);
//    the f32 partials are summed by a second kernel in a fixed order, so
//    results are identical run to run.
#include <algorithm>

#include "q4_dequant.h"

namespace q4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
// native vector (HIP's uint4 is a struct, whose private arrays the compiler
// keeps in scratch memory instead of registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;            // 16 weight rows per wave
constexpr int kRowsPerWg = 16 * kWaves;
constexpr int kDepth = 8;            // steps (4 groups each) of weight loads issued together
constexpr int kGroupsPerSplit = 32;  // K chunk per workgroup: 1024 values
constexpr int kBatches = kGroupsPerSplit / (4 * kDepth);  // load batches per tile
constexpr int kMTile = 16;           // activation rows per launch
constexpr int kXq = (kMTile * kGroupsPerSplit * 4 + 255) / 256;  // x chunks per thread
constexpr int kMaxTilesPerWave = 4;  // finished tiles wait in LDS until the loop ends
constexpr int kMoePerSlot = 0, kMoeSilu = 1, kMoeCombine = 2;

// The 8 weights of word w, w = (q - 7) * s, as two binary16 vectors whose sum
// is exact: hi = f16((q - 7) * s) and lo = (q - 7) * s - hi. Codes become
// exact binary16 integers 1024 + q through the exponent pattern 0x6400 and
// 1031 is subtracted exactly; the product of a 4-bit integer and a binary16
// scale has at most 15 significant bits, so its rounding residual has at most
// 4 and lies on the product's own grid (no finer than 2^-18 for scales above
// 2^-8): it is exactly representable (as a subnormal if small) and a fused
// multiply-add with one rounding returns it exactly.
__device__ __forceinline__ void dequant_split(uint32_t w, half2v s2, half8 &hi, half8 &lo)
{
    const half2v c1031 = {(_Float16)1031.0f, (_Float16)1031.0f};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t u = w >> (8 * p);
        const uint32_t bits = (u & 0xFu) | ((u & 0xF0u) << 12) | 0x64006400u;
        const half2v q = __builtin_bit_cast(half2v, bits) - c1031;
        const half2v h = q * s2;
        const half2v r = __builtin_elementwise_fma(q, s2, -h);
        hi[2 * p] = h[0];
        hi[2 * p + 1] = h[1];
        lo[2 * p] = r[0];
        lo[2 * p + 1] = r[1];
    }
}

__device__ __forceinline__ uint32_t word(const uint4 &v, int t)
{
    return t == 0 ? v.x : (t == 1 ? v.y : (t == 2 ? v.z : v.w));
}

// The work of one workgroup for one split ks of K (groups [ks * gc, min(G,
// (ks + 1) * gc)), gc = kGroupsPerSplit) and M <= 16 activation rows:
// row_ptr(m) gives activation row m; its chunk is staged once, then wave w
// takes the 16-row weight tiles tile0(w), + tstride, ... one after another,
// and emit(m, n, value) receives every finished f32 result.
template <typename RowPtr, typename Emit>
__device__ __forceinline__ void mfma_rows(const uint4 *__restrict__ W,
                                          const uint16_t *__restrict__ S, int N, int G, int M,
                                          int gc, int ks, int tile0, int tstride, RowPtr row_ptr,
                                          Emit emit)
{
    extern __shared__ uint4 smem[];
    const int t = threadIdx.x, l = t & 63, wave = t >> 6;
    const int g0 = ks * gc, gn = min(gc, G - g0);  // groups of this split, >= 1
    const int xstride = gc * 32 + 8;  // staged row: the chunk plus 16 bytes against bank conflicts
    // LDS: finished tiles [kWaves][kMaxTilesPerWave][64 lanes] float4, then the activation
    floatx4 *obuf = reinterpret_cast<floatx4 *>(smem);
    _Float16 *xs = reinterpret_cast<_Float16 *>(smem + kWaves * kMaxTilesPerWave * 64);
    const int cpr = gn * 4;           // 16-byte chunks per staged row

    // 1. the activation chunk (all loads issued together, then stored)
    u32x4 xr[kXq];
#pragma unroll
    for (int q = 0; q < kXq; ++q) {
        const int c = min(t + 256 * q, M * cpr - 1);  // branch-free: the tail re-reads
        const int m = c / cpr, j = c - m * cpr;
        xr[q] = *reinterpret_cast<const u32x4 *>(row_ptr(m) + (int64_t)g0 * 32 + 8 * j);
    }
#pragma unroll
    for (int q = 0; q < kXq; ++q) {
        const int c = min(t + 256 * q, M * cpr - 1);  // the tail rewrites the last chunk
        const int m = c / cpr, j = c - m * cpr;
        *reinterpret_cast<u32x4 *>(xs + m * xstride + 8 * j) = xr[q];
    }
    __syncthreads();

    // 2. this wave's tiles, one after another, each in kBatches batches whose
    //    loads (20 per lane) are issued together and consumed in the same
    //    iteration; the resident waves of the CU (16) overlap one another's
    //    loads. (Loads kept in flight across iterations make the compiler copy,
    //    and so wait for, them at the loop edge.)
    const int ntiles = (N + 15) >> 4;
    const int my_tiles = tile0 < ntiles ? (ntiles - 1 - tile0) / tstride + 1 : 0;
    const int n = l & 15, kb = l >> 4;
    const int m = l & 15;
    const bool mok = m < M;
    for (int j = 0; j < my_tiles; ++j) {
        const size_t rb = (size_t)min((tile0 + j * tstride) * 16 + n, N - 1) * G + g0;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1  // one batch's loads at a time (unrolled, the batches' loads overlap)
        for (int bt = 0; bt < kBatches; ++bt) {
            // step p of batch bt covers groups g = 4 kDepth bt + 4p .. + 3 of the
            // split; lane (n, kb) loads group g + kb of row n (16 bytes) and its
            // scale; MFMA t of the step takes word t of that group, so lane
            // (., kb) of both operands covers k = 32 (g + kb) + 8 t + 0..7
            const int gb = 4 * kDepth * bt;
            uint4 wq[kDepth];
            uint32_t sq[kDepth];
#pragma unroll
            for (int p = 0; p < kDepth; ++p) {
                const int gi = min(gb + 4 * p + kb, gn - 1);
                wq[p] = load_weights(W + rb + gi);
                sq[p] = load_scale(S + rb + gi);
            }
#pragma unroll
            for (int p = 0; p < kDepth; ++p) {
                const int gi = gb + 4 * p + kb;
                const _Float16 *xa = xs + m * xstride + min(gi, gn - 1) * 32;
                half8 a[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)  // the four activation reads first
                    a[tt] = mok ? *reinterpret_cast<const half8 *>(xa + 8 * tt) : half8{};
                // groups past the split get scale 0
                const uint16_t s16 = gi < gn ? (uint16_t)sq[p] : (uint16_t)0;
                const _Float16 sh = __builtin_bit_cast(_Float16, s16);
                const half2v s2 = {sh, sh};
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    half8 bh, bl;
                    dequant_split(word(wq[p], tt), s2, bh, bl);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[tt], bh, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[tt], bl, acc, 0, 0, 0);
                }
            }
        }
        // park the finished tile in LDS: a global store here would count
        // against the next tile's weight loads
        obuf[(wave * kMaxTilesPerWave + j) * 64 + l] = acc;
    }

    // 3. emit this wave's tiles: lane holds D[4 * (l / 16) + r][l % 16]
    for (int j = 0; j < my_tiles; ++j) {
        const floatx4 d = obuf[(wave * kMaxTilesPerWave + j) * 64 + l];
        const int col = (tile0 + j * tstride) * 16 + n;
        if (col < N)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int mr = 4 * kb + r;
                if (mr < M)
                    emit(mr, col, d[r]);
            }
    }
}

// Batched matvec: grid (P, KS), 256 threads; wave w of workgroup b takes the
// tiles b * 4 + w, + 4 P, ... KS == 1: the f32 result written to yf when set,
// else rounded to y; KS > 1: f32 partials part[ks][m][n] for k_combine.
__global__ __launch_bounds__(256) void k_gemv_mfma(const uint4 *__restrict__ W,
                                                   const uint16_t *__restrict__ S,
                                                   const uint16_t *__restrict__ x, int64_t ldx,
                                                   uint16_t *__restrict__ y,
                                                   float *__restrict__ yf, int64_t ldy,
                                                   float *__restrict__ part, int N, int G, int M,
                                                   int gc)
{
    const int ks = blockIdx.y, KS = gridDim.y;
    mfma_rows(
        W, S, N, G, M, gc, ks, blockIdx.x * kWaves + (threadIdx.x >> 6), gridDim.x * kWaves,
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
// distinct expert of the routing (meta from k_moe_route), whose pairs (token,
// slot) form the activation rows, 16 at a time. Per-pair f32 results go to
// part[ks][pair][n].
__global__ __launch_bounds__(256) void k_moe_mfma(const uint4 *__restrict__ Wall,
                                                  const uint16_t *__restrict__ Sall,
                                                  const int32_t *__restrict__ meta, int P,
                                                  const uint16_t *__restrict__ x, int64_t ldx,
                                                  int64_t slot_stride, int TOPK,
                                                  float *__restrict__ part, int N, int G, int gc)
{
    const int d = blockIdx.z;
    if (d >= meta[0])  // fewer distinct experts than slots: the whole workgroup leaves
        return;
    const int e = meta[1 + d];
    const int q0 = meta[1 + P + d], q1 = meta[1 + P + d + 1];
    const int32_t *order = meta + 2 + 2 * P;
    const int ks = blockIdx.y;
    const uint4 *W = Wall + (size_t)e * N * G;
    const uint16_t *S = Sall + (size_t)e * N * G;
    for (int qa = q0; qa < q1; qa += kMTile) {
        if (qa > q0)
            __syncthreads();  // the previous rows' staged activation is still read
        mfma_rows(
            W, S, N, G, min(kMTile, q1 - qa), gc, ks, blockIdx.x * kWaves + (threadIdx.x >> 6),
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
// Pairs whose id is outside [0, E) were zeroed by k_moe_route (per-pair modes)
// or contribute nothing (combine).
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
    if (e < 0 || e >= E)
        return;
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

int cus()
{
    static int n[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (!n[dev]) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            c = 256;
        n[dev] = c;
    }
    return n[dev];
}

}  // namespace

q4_status launch_gemv_mfma(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                           uint16_t *y, float *yf, int64_t ldy, int N, int K, int M,
                           hipStream_t stream)
{
    const int G = K / 32;
    // K splits of kGroupsPerSplit groups (the last may be shorter)
    const int gc = kGroupsPerSplit;
    const int KS = (G + gc - 1) / gc;
    const int ntiles = (N + 15) / 16;
    // about three resident workgroups per CU, each looping over its tiles (at
    // most kMaxTilesPerWave per wave)
    const int P = std::max({1, (ntiles + kWaves * kMaxTilesPerWave - 1) / (kWaves * kMaxTilesPerWave),
                            std::min((ntiles + kWaves - 1) / kWaves, (3 * cus() + KS - 1) / KS)});
    float *part = nullptr;
    for (int m0 = 0; m0 < M; m0 += kMTile) {
        const int mt = std::min(kMTile, M - m0);
        const size_t lds = (size_t)kWaves * kMaxTilesPerWave * 64 * 16 +  // finished tiles
                           (size_t)mt * (gc * 32 + 8) * 2;  // staged rows of this launch
        if (KS > 1 && !part) {
            char *ws = static_cast<char *>(
                workspace(stream, kWsHeader + (size_t)KS * kMTile * N * sizeof(float)));
            if (!ws)
                return Q4_EHIP;
            part = reinterpret_cast<float *>(ws + kWsHeader);
        }
        Q4_LAUNCH_MATVEC(k_gemv_mfma, dim3(P, KS), dim3(256), lds, stream,
                         reinterpret_cast<const uint4 *>(W), S, x + m0 * ldx, ldx,
                         yf ? nullptr : y + m0 * ldy, yf ? yf + m0 * ldy : nullptr, ldy, part, N,
                         G, mt, gc);
        q4_status st = check_launch("k_gemv_mfma");
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
    const size_t lds = (size_t)kWaves * kMaxTilesPerWave * 64 * 16 + (size_t)kMTile * (gc * 32 + 8) * 2;
    Q4_LAUNCH_MATVEC(k_moe_mfma, grid, dim3(256), lds, stream, reinterpret_cast<const uint4 *>(W),
                     S, meta, P, x, ldx, x_slot_stride, TOPK, part, N, G, gc);
    q4_status st = check_launch("k_moe_mfma");
    if (st != Q4_OK)
        return st;
    const int64_t total = mode == kMoeCombine ? (int64_t)T * N
                                              : (int64_t)P * (mode == kMoeSilu ? N / 2 : N);
    hipLaunchKernelGGL(k_moe_finish, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       mode, part, KS, P, N, ids, route_w, y, E, TOPK);
    return check_launch("k_moe_finish");
}

size_t moe_part_bytes(int N, int K, int P)
{
    const int G = K / 32, KS = (G + kGroupsPerSplit - 1) / kGroupsPerSplit;
    return (size_t)KS * P * N * sizeof(float);
}

}  // namespace q4
