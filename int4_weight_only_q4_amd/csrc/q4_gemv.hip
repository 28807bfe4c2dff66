// Dequantising int4 x f16 matvec for gfx950 (single token, M = 1), with the
// SiLU-multiply and add+RMSNorm epilogues.
//
// What is computed follows the Zero TVM Documentation ("Q4F16 quantization
// format"; "WGSL Kernel Roles", shaders 5, 6 and 7): y[n] = sum_k (q - 7) * s * x.
// How it is computed is designed for CDNA4 rather than taken from the pages'
// WGSL:
//  * One quantisation group (32 codes = four uint32 = 16 bytes) is one 128-bit
//    load per lane. A row is spread over LPR consecutive lanes (a "segment"),
//    lane j taking groups j, j + LPR, ...; one wave covers 64 / LPR rows, so a
//    wave-wide load instruction reads LPR * 16 contiguous bytes of each row.
//  * Every weight and scale load of a lane is issued before the activation is
//    staged, so the whole tile is in flight at once.
//  * The activation vector is staged once per workgroup in LDS, with each
//    8-element chunk stored as the pairs (x0,x4) (x1,x5) (x2,x6) (x3,x7) that
//    line up with the in-register nibble unpack, plus 7 * (group sum).
//  * Nibble unpack without conversions (q4_dequant.h): codes are masked into
//    exact subnormal binary16 pairs for v_dot2_f32_f16 (1 shift + 4 ANDs +
//    4 dot2 per word), and the group's sum of (c - 7) x is applied with its
//    scale in f32. A one-hot x therefore reproduces (c - 7) * s exactly.
//  * The LPR partial sums of a row are combined in a fixed order by DPP and
//    permlane steps (no LDS round trips), so results are identical run to run.
#include <algorithm>

#include "q4_dequant.h"
#include "q4_moe_route.h"

namespace q4 {
namespace {

constexpr int kWaves = 4;  // 256 threads per workgroup
constexpr int kMaxRowsDot = 4;  // batched rows handled by the dot2 kernel
// pairs from which the dot2 expert kernel takes twice the single-row kernel's
// rows per workgroup: each workgroup routes and stages its pairs' activations
// once, for more weight rows (measured on 128 experts, top 8: 32 pairs and
// up gain, 8 pairs need the workgroups)
constexpr int kMoeWideRowsPairs = 32;
// the token-by-token down kernel: activation chunks per thread held in
// registers, 64-lane weight units per wave, output rows per workgroup
constexpr int kMoeTokXq = 4;
constexpr int kMoeTokCpt = 8;
constexpr int kMoeTokRows = 8;
constexpr int kMoeTokMaxPairs = 32;  // pairs from which experts chosen twice cost too much

enum { PRO_X = 0, PRO_NORM = 1 };
enum { EPI_NONE_ = 0, EPI_SILU = 1, EPI_RESID = 2, EPI_LOGITS = 3, EPI_ROPE = 4 };

struct GemvParams {
    const uint4 *W;     // [N][G] groups of 16 bytes
    const uint16_t *S;  // [N][G]; affine: [N][G/2] (one scale per 64 codes)
    const uint16_t *Bias;  // affine: biases [N][G/2]
    int N, G;
    // prologue: PRO_X reads x; PRO_NORM stages f16(RMSNorm(src) * gamma)
    const uint16_t *x;  // [K], 16-byte aligned (PRO_X) or the residual (PRO_NORM)
    const uint16_t *pro_gamma;
    float pro_eps;
    // epilogue
    uint16_t *y;              // NONE: [N]; SILU: [N/2]
    const uint16_t *res_in;   // RESID: res_out[n] = f16(f16(y[n]) + res_in[n])
    uint16_t *res_out;
    float *yf;                 // LOGITS: yf[n] = acc
    unsigned long long *cand;  // LOGITS: this workgroup's largest argmax_key, or null
    RopeArgs rope;             // ROPE: geometry, position, cache and q_out
};

// AFF: the MLX affine format (unsigned codes, w = s * q + b per 64 codes): a
// 16-byte load is half a group, its scale and bias are those of group g / 2.
template <int LPR, int NG, int RPS, int EPI, int PRO, bool AFF = false>
__global__ __launch_bounds__(256) void k_gemv(GemvParams a)
{
    constexpr int SPW = 64 / LPR;             // segments (rows) per wave
    constexpr int RB = kWaves * SPW * RPS;    // rows per workgroup
    constexpr int XCH = (LPR * NG + 63) / 64; // activation chunks (8 values) per thread
    extern __shared__ uint4 smem[];
    __shared__ float red[4];
    __shared__ float vals[(EPI == EPI_SILU || EPI == EPI_ROPE) ? RB : 1];
    __shared__ unsigned long long wkey;  // LOGITS: the workgroup's best key so far
    __shared__ uint32_t wdone;           // LOGITS: waves that have added theirs

    const int G = a.G;
    const int K = G * 32;
    const int chunks = K >> 3;
    uint4 *xs = smem;
    float *cs = reinterpret_cast<float *>(smem + chunks);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = lane / LPR, j = lane % LPR;
    const int half = a.N >> 1;

    // 0. this thread's activation chunks (issued first: waiting for them must
    //    not wait for the weight loads behind them)
    uint4 xr[XCH];
    uint4 gr[PRO == PRO_NORM ? XCH : 1];
#pragma unroll
    for (int q = 0; q < XCH; ++q) {
        const int c = tid + 256 * q;
        if (c < chunks) {
            xr[q] = reinterpret_cast<const uint4 *>(a.x)[c];
            if (PRO == PRO_NORM)
                gr[q] = reinterpret_cast<const uint4 *>(a.pro_gamma)[c];
        }
    }

    int row[RPS], li[RPS];
    bool ok[RPS];
#pragma unroll
    for (int r = 0; r < RPS; ++r) {
        li[r] = (wave * SPW + seg) * RPS + r;
        int rr;
        if (EPI == EPI_SILU) {
            const int gi = blockIdx.x * (RB / 2) + (li[r] % (RB / 2));
            ok[r] = gi < half;
            rr = li[r] < RB / 2 ? gi : half + gi;
        } else if (EPI == EPI_ROPE) {
            // local rows [0, RB/2) are the first rows of RoPE pairs, the rest
            // their partners (head_dim / 2 further on)
            const int hh = a.rope.head_dim >> 1;
            const int pi = blockIdx.x * (RB / 2) + (li[r] % (RB / 2));
            ok[r] = pi < half;
            const int head = pi / hh;
            rr = head * a.rope.head_dim + (pi - head * hh) + (li[r] < RB / 2 ? 0 : hh);
        } else {
            rr = blockIdx.x * RB + li[r];
            ok[r] = rr < a.N;
        }
        row[r] = ok[r] ? rr : 0;
    }

    // ROPE: the step's position behind the activation (a wave-uniform load
    // the epilogue's angle and cache page wait for)
    const int rope_pos = EPI == EPI_ROPE ? *a.rope.pos : 0;

    // 1. weight and scale loads, in the order they are consumed (group-major)
    uint4 wv[NG][RPS];
    uint32_t sv[NG][RPS];
    uint32_t bv[AFF ? NG : 1][AFF ? RPS : 1];
    // (branch-free: a lane past the last group re-reads group G - 1, which the
    // accumulation skips; a conditional load would let the compiler convert the
    // scale inside the branch and wait for it there)
#pragma unroll
    for (int i = 0; i < NG; ++i)
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
            const int g = min(j + LPR * i, G - 1);
            const size_t off = (size_t)row[r] * G + g;
            wv[i][r] = load_weights(a.W + off);
            if (AFF) {
                const size_t soff = (size_t)row[r] * (G >> 1) + (g >> 1);
                sv[i][r] = load_scale(a.S + soff);
                bv[i][r] = load_scale(a.Bias + soff);
            } else {
                sv[i][r] = load_scale(a.S + off);
            }
        }
    // ROPE: this thread's pair (threads RB / 2 .. repeat the last one), its
    // angle and cache slot while the weights stream (in the epilogue they
    // would add two memory round trips after the sums)
    RopePair rp;
    if (EPI == EPI_ROPE)
        rp = rope_pair_prepare(a.rope, min(blockIdx.x * (RB / 2) + min(tid, RB / 2 - 1), half - 1),
                               rope_pos);
    // RESID: the residual rows behind the weights (consumed in the epilogue;
    // loaded there, they would add a memory round trip after the sums)
    uint16_t rin[EPI == EPI_RESID ? RPS : 1];
    if (EPI == EPI_RESID)
#pragma unroll
        for (int r = 0; r < RPS; ++r)
            rin[r] = a.res_in[row[r]];

    // 2. activation into LDS (after an RMSNorm of the residual for PRO_NORM)
    if (PRO == PRO_NORM) {
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < XCH; ++q)
            if (tid + 256 * q < chunks) {
                float f[8];
                chunk_to_float(xr[q], f);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    ss = fmaf(f[e], f[e], ss);
            }
        ss = block_sum_256(ss, red);
        const float inv = rms_inv(ss, K, a.pro_eps);
#pragma unroll
        for (int q = 0; q < XCH; ++q)
            if (tid + 256 * q < chunks) {
                float f[8], g8[8];
                chunk_to_float(xr[q], f);
                chunk_to_float(gr[q], g8);
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    h[e] = f2h(f[e] * inv * g8[e]);
                xr[q] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                   h[6] | (h[7] << 16));
            }
    }
#pragma unroll
    for (int q = 0; q < XCH; ++q) {
        const int c = tid + 256 * q;
        put_chunk(xr[q], c, c < chunks, xs, cs);
    }
    if (EPI == EPI_LOGITS && tid == 0) {
        wkey = 0;
        wdone = 0;
    }
    __syncthreads();

    // 3. dequantise and accumulate, in load order
    float acc[RPS];
#pragma unroll
    for (int r = 0; r < RPS; ++r)
        acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = j + LPR * i;
        if (g < G) {
            const float sx = cs[g];
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                if (AFF) {
                    acc[r] = fmaf(h2f(sv[i][r]), group_dot_unsigned(wv[i][r], xs, g), acc[r]);
                    acc[r] = fmaf(h2f(bv[i][r]), sx, acc[r]);
                } else {
                    acc[r] = fmaf(h2f(sv[i][r]), group_dot(wv[i][r], xs, g, sx), acc[r]);
                }
            }
        }
    }

    // 4. combine the LPR lanes of each row
#pragma unroll
    for (int r = 0; r < RPS; ++r)
        acc[r] = segment_sum(acc[r], LPR);

    // 5. epilogue
    if (EPI == EPI_NONE_) {
        if (j == 0)
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                if (ok[r])
                    a.y[row[r]] = f2h(acc[r]);
    } else if (EPI == EPI_SILU) {
        if (j == 0)
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                vals[li[r]] = h2f(f2h(acc[r]));  // as stored by an unfused matvec
        __syncthreads();
        if (tid < RB / 2) {
            const int gi = blockIdx.x * (RB / 2) + tid;
            if (gi < half)
                a.y[gi] = f2h(silu_mul_f(vals[tid], vals[tid + RB / 2]));
        }
    } else if (EPI == EPI_ROPE) {  // RoPE of the pairs, Q out, K and V into the cache
        if (j == 0)
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                vals[li[r]] = h2f(f2h(acc[r]));  // as stored by an unfused matvec
        __syncthreads();
        if (tid < RB / 2) {
            const int pi = blockIdx.x * (RB / 2) + tid;
            if (pi < half)
                rope_pair_finish(rp, vals[tid], vals[tid + RB / 2]);
        }
    } else if (EPI == EPI_LOGITS) {  // f32 logits and this workgroup's argmax candidate
        unsigned long long key = 0;
        if (j == 0)
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                if (ok[r]) {
                    a.yf[row[r]] = acc[r];
                    const unsigned long long k = argmax_key(acc[r], (uint32_t)row[r]);
                    key = k > key ? k : key;
                }
        if (a.cand) {
            // only the segment leaders (lanes 0, LPR, 2 LPR, ...) hold rows
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) {
                const unsigned long long o = __shfl_xor(key, off, 64);
                key = o > key ? o : key;
            }
            // the wave's key into LDS; the last wave to arrive stores the
            // workgroup's (no barrier: the other waves leave at once)
            if (lane == 0) {
                __hip_atomic_fetch_max(&wkey, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                const uint32_t before = __hip_atomic_fetch_add(&wdone, 1u, __ATOMIC_ACQ_REL,
                                                               __HIP_MEMORY_SCOPE_WORKGROUP);
                if (before == kWaves - 1)
                    a.cand[blockIdx.x] =
                        __hip_atomic_load(&wkey, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    } else {  // EPI_RESID: the residual add of an add+RMSNorm, row by row
        if (j == 0)
#pragma unroll
            for (int r = 0; r < RPS; ++r)
                if (ok[r]) {
                    const float t = h2f(f2h(acc[r]));  // as stored by an unfused matvec
                    a.res_out[row[r]] = f2h(t + h2f(rin[r]));
                }
    }
}

// MR activation rows (2..4) against the same weights, f16 outputs
// y[m * ldy + n] (or f32 ones in yf when set): the single-row kernel's loads, unpack and arithmetic per
// activation row (each nibble pair's dot2 issued once per row), so every row's
// result equals the single-row matvec of that row bit for bit. The MR rows are
// staged one after another in LDS (pair order, group sums). AFF: the MLX
// affine format, as in k_gemv.
template <int LPR, int NG, int RPS, int MR, bool AFF>
__global__ __launch_bounds__(256) void k_gemv_rows(GemvParams a, int64_t ldx, int64_t ldy)
{
    constexpr int SPW = 64 / LPR;
    constexpr int RB = kWaves * SPW * RPS;
    constexpr int XCH = (LPR * NG + 63) / 64;
    extern __shared__ uint4 smem[];
    const int G = a.G, K = G * 32, chunks = K >> 3;
    // row m: xs at smem + m * stride, its group sums after the chunks
    const int stride = chunks + G / 4 + 1;  // uint4 units (G floats rounded up)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = lane / LPR, j = lane % LPR;

    uint4 xr[MR][XCH];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int q = 0; q < XCH; ++q) {
            const int c = tid + 256 * q;
            if (c < chunks)
                xr[m][q] = reinterpret_cast<const uint4 *>(a.x + m * ldx)[c];
        }
    int row[RPS];
    bool ok[RPS];
#pragma unroll
    for (int r = 0; r < RPS; ++r) {
        const int rr = blockIdx.x * RB + (wave * SPW + seg) * RPS + r;
        ok[r] = rr < a.N;
        row[r] = ok[r] ? rr : 0;
    }
    uint4 wv[NG][RPS];
    uint32_t sv[NG][RPS];
    uint32_t bv[AFF ? NG : 1][AFF ? RPS : 1];
#pragma unroll
    for (int i = 0; i < NG; ++i)
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
            const int g = min(j + LPR * i, G - 1);
            const size_t off = (size_t)row[r] * G + g;
            wv[i][r] = load_weights(a.W + off);
            if (AFF) {
                const size_t soff = (size_t)row[r] * (G >> 1) + (g >> 1);
                sv[i][r] = load_scale(a.S + soff);
                bv[i][r] = load_scale(a.Bias + soff);
            } else {
                sv[i][r] = load_scale(a.S + off);
            }
        }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        uint4 *xs = smem + m * stride;
        float *cs = reinterpret_cast<float *>(xs + chunks);
#pragma unroll
        for (int q = 0; q < XCH; ++q) {
            const int c = tid + 256 * q;
            put_chunk(xr[m][q], c, c < chunks, xs, cs);
        }
    }
    __syncthreads();

    float acc[RPS][MR];
#pragma unroll
    for (int r = 0; r < RPS; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m)
            acc[r][m] = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = j + LPR * i;
        if (g < G) {
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const float s = h2f(sv[i][r]);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    const uint4 *xs = smem + m * stride;
                    const float sx = reinterpret_cast<const float *>(xs + chunks)[g];
                    if (AFF) {
                        acc[r][m] = fmaf(s, group_dot_unsigned(wv[i][r], xs, g), acc[r][m]);
                        acc[r][m] = fmaf(h2f(bv[i][r]), sx, acc[r][m]);
                    } else {
                        acc[r][m] = fmaf(s, group_dot(wv[i][r], xs, g, sx), acc[r][m]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RPS; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m)
            acc[r][m] = segment_sum(acc[r][m], LPR);
    if (j == 0)
#pragma unroll
        for (int r = 0; r < RPS; ++r)
            if (ok[r])
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    if (a.yf)  // f32 outputs (the LM head's logits)
                        a.yf[m * ldy + row[r]] = acc[r][m];
                    else
                        a.y[m * ldy + row[r]] = f2h(acc[r][m]);
                }
}

// Outputs of k_moe_rows: f32 per-pair results for k_moe_finish (the down
// stage's routing-weighted sum), f16 per-pair outputs, or the SiLU-multiply
// of each pair's gate and up halves.
enum : int { kMoeOutPart = 0, kMoeOutSlot = 1, kMoeOutSilu = 2 };

// One unit of k_moe_rows: the nr <= MR pairs pairs[0 .. nr) of expert e
// through this workgroup's rows (MR activation rows staged in LDS, missing
// ones repeating the last pair; results stored for the nr pairs). SILU: local
// rows [0, RB/2) are gate rows, [RB/2, RB) the matching up rows (as k_gemv's
// SiLU epilogue), and vals is MR * RB floats of LDS.
template <int LPR, int NG, int RPS, int MR, bool SILU>
__device__ __forceinline__ void moe_rows_unit(const uint4 *__restrict__ Wall,
                                              const uint16_t *__restrict__ Sall, int e,
                                              const int32_t *pairs, int nr,
                                              const uint16_t *__restrict__ x, int64_t ldx,
                                              int64_t slot_stride, int TOPK, int out,
                                              float *__restrict__ part, uint16_t *__restrict__ y,
                                              float *vals, int N, int G)
{
    constexpr int SPW = 64 / LPR;
    constexpr int RB = kWaves * SPW * RPS;
    constexpr int XCH = (LPR * NG + 63) / 64;
    extern __shared__ uint4 smem[];
    const int K = G * 32, chunks = K >> 3;
    const int stride = chunks + G / 4 + 1;  // uint4 units per staged row
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = lane / LPR, j = lane % LPR;
    const int half = N >> 1;
    const uint4 *W = Wall + (size_t)e * N * G;
    const uint16_t *S = Sall + (size_t)e * N * G;

    // activation rows first (the pairs' rows; missing ones repeat the last)
    uint4 xr[MR][XCH];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const int pr = pairs[min(m, nr - 1)];
        const uint16_t *xp = x + (int64_t)(pr / TOPK) * ldx + (int64_t)(pr % TOPK) * slot_stride;
#pragma unroll
        for (int q = 0; q < XCH; ++q) {
            const int c = tid + 256 * q;
            if (c < chunks)
                xr[m][q] = reinterpret_cast<const uint4 *>(xp)[c];
        }
    }
    int row[RPS], li[RPS];
    bool ok[RPS];
#pragma unroll
    for (int r = 0; r < RPS; ++r) {
        li[r] = (wave * SPW + seg) * RPS + r;
        int rr;
        if (SILU) {
            const int gi = blockIdx.x * (RB / 2) + (li[r] % (RB / 2));
            ok[r] = gi < half;
            rr = li[r] < RB / 2 ? gi : half + gi;
        } else {
            rr = blockIdx.x * RB + li[r];
            ok[r] = rr < N;
        }
        row[r] = ok[r] ? rr : 0;
    }
    uint4 wv[NG][RPS];
    uint32_t sv[NG][RPS];
#pragma unroll
    for (int i = 0; i < NG; ++i)
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
            const int g = min(j + LPR * i, G - 1);
            const size_t off = (size_t)row[r] * G + g;
            wv[i][r] = load_weights(W + off);
            sv[i][r] = load_scale(S + off);
        }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        uint4 *xs = smem + m * stride;
        float *cs = reinterpret_cast<float *>(xs + chunks);
#pragma unroll
        for (int q = 0; q < XCH; ++q) {
            const int c = tid + 256 * q;
            put_chunk(xr[m][q], c, c < chunks, xs, cs);
        }
    }
    __syncthreads();

    float acc[RPS][MR];
#pragma unroll
    for (int r = 0; r < RPS; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m)
            acc[r][m] = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = j + LPR * i;
        if (g < G) {
#pragma unroll
            for (int r = 0; r < RPS; ++r) {
                const float s = h2f(sv[i][r]);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    const uint4 *xs = smem + m * stride;
                    const float sx = reinterpret_cast<const float *>(xs + chunks)[g];
                    acc[r][m] = fmaf(s, group_dot(wv[i][r], xs, g, sx), acc[r][m]);
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RPS; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m)
            acc[r][m] = segment_sum(acc[r][m], LPR);
    if (SILU) {
        if (j == 0)
#pragma unroll
            for (int r = 0; r < RPS; ++r)
#pragma unroll
                for (int m = 0; m < MR; ++m)
                    vals[m * RB + li[r]] = h2f(f2h(acc[r][m]));  // as a stored gate_up output
        __syncthreads();
        if (tid < RB / 2) {
            const int gi = blockIdx.x * (RB / 2) + tid;
            if (gi < half)
#pragma unroll
                for (int m = 0; m < MR; ++m)
                    if (m < nr)
                        y[(int64_t)pairs[m] * half + gi] =
                            f2h(silu_mul_f(vals[m * RB + tid], vals[m * RB + tid + RB / 2]));
        }
    } else if (j == 0) {
#pragma unroll
        for (int r = 0; r < RPS; ++r)
            if (ok[r])
#pragma unroll
                for (int m = 0; m < MR; ++m)
                    if (m < nr) {
                        if (out == kMoeOutSlot)
                            y[(int64_t)pairs[m] * N + row[r]] = f2h(acc[r][m]);
                        else
                            part[(size_t)pairs[m] * N + row[r]] = acc[r][m];
                    }
    }
}

// MoE expert stage with the single-row arithmetic per (token, slot) pair:
// grid (row blocks, 1, P), P <= 256. The distinct experts of the routing
// (k_moe_route's meta, or each workgroup's own when meta == nullptr) own
// ceil(pairs / MR) units of at most MR of their pairs; blockIdx.z is a unit
// (P bounds their number). The workgroup runs its unit's pairs through its
// rows of the expert, each pair with k_gemv_rows' arithmetic (activations
// staged in LDS), and writes by `out`: the per-pair f32 results part[pair][n]
// for k_moe_finish, the f16 outputs y[pair][n], or (SILU) y[pair][i] =
// f16(silu(f16(gate_i)) * f16(up_i)) over the N / 2 gate and up rows, as
// k_moe_finish would form them. In the last two forms the slice z = 0 also
// writes zeros for the pairs whose id is outside [0, E) (they have no unit).
template <int LPR, int NG, int RPS, bool SILU>
__global__ __launch_bounds__(256) void k_moe_rows(const uint4 *__restrict__ Wall,
                                                  const uint16_t *__restrict__ Sall,
                                                  const int32_t *__restrict__ ids, int E,
                                                  const int32_t *__restrict__ meta, int P,
                                                  const uint16_t *__restrict__ x, int64_t ldx,
                                                  int64_t slot_stride, int TOPK, int out,
                                                  float *__restrict__ part,
                                                  uint16_t *__restrict__ y, int N, int G)
{
    constexpr int MR = kMaxRowsDot;
    constexpr int RB = kWaves * (64 / LPR) * RPS;
    __shared__ float s_vals[SILU ? MR * RB : 1];
    if (out != kMoeOutPart && blockIdx.z == 0) {
        // zeros for the pairs routed nowhere, over this workgroup's outputs
        // (thread t checks pair t, P <= 256; nothing to do when all are valid)
        const int id_t = (int)threadIdx.x < P ? ids[threadIdx.x] : 0;
        const bool bad = (int)threadIdx.x < P && (id_t < 0 || id_t >= E);
        if (__syncthreads_or(bad)) {
            const int width = SILU ? RB / 2 : RB, ncol = SILU ? N / 2 : N;
            const int c0 = blockIdx.x * width;
            for (int i = threadIdx.x; i < P * width; i += 256) {
                const int p = i / width, c = c0 + i % width;
                const int id = ids[p];
                if ((id < 0 || id >= E) && c < ncol)
                    y[(int64_t)p * ncol + c] = 0;
            }
        }
    }
    __shared__ int s_cnt[kFuseExperts];
    __shared__ int s_pairs[kFusePairs];
    __shared__ int s_np;
    const int u = blockIdx.z;
    int e, q0, q1;
    const int32_t *order;
    if (meta) {
        // the unit's expert: thread k holds listed expert k's unit count (at
        // most P <= 256 experts are listed), a block scan places unit u
        __shared__ int s_red[4], s_k, s_first;
        const int nd = meta[0], t = threadIdx.x;
        const int uk = t < nd ? (meta[1 + P + t + 1] - meta[1 + P + t] + MR - 1) / MR : 0;
        if (t == 0)
            s_k = -1;
        int total;
        const int before = block_exclusive_scan(uk, s_red, &total);
        if (u >= before && u < before + uk) {
            s_k = t;
            s_first = (u - before) * MR;
        }
        __syncthreads();
        const int k = s_k;
        if (k < 0)  // fewer units than slots: the whole workgroup leaves
            return;
        e = meta[1 + k];
        q0 = meta[1 + P + k] + s_first;
        q1 = min(q0 + MR, meta[1 + P + k + 1]);
        order = meta + 2 + 2 * P;
    } else {
        e = route_in_workgroup(ids, P, E, u, MR, s_cnt, s_pairs, &s_np, &q0);
        if (e < 0)
            return;
        q1 = min(q0 + MR, s_np);
        order = s_pairs;
    }
    const int nr = q1 - q0;  // 1..MR pairs
    // as many activation rows as the unit has pairs (1, 2 or 4)
    if (nr == 1)
        moe_rows_unit<LPR, NG, RPS, 1, SILU>(Wall, Sall, e, order + q0, nr, x, ldx, slot_stride,
                                             TOPK, out, part, y, s_vals, N, G);
    else if (nr == 2)
        moe_rows_unit<LPR, NG, RPS, 2, SILU>(Wall, Sall, e, order + q0, nr, x, ldx, slot_stride,
                                             TOPK, out, part, y, s_vals, N, G);
    else
        moe_rows_unit<LPR, NG, RPS, MR, SILU>(Wall, Sall, e, order + q0, nr, x, ldx, slot_stride,
                                              TOPK, out, part, y, s_vals, N, G);
}

// MoE down stage with the routing-weighted combine, token by token, for few
// pairs: grid (row blocks, T). Workgroup (b, t) runs block b of rows of each
// of token t's TOPK experts against the slot's activation row, with the
// single-row group arithmetic, and stores y[t][n] = f16(sum_s route_w[t][s]
// v_s[n]) over the slots with a valid id, in slot order, as k_moe_finish
// forms it: the combine without per-pair results, a routing step or a second
// kernel. An expert chosen by several tokens is read once per token (the
// expert-grouped kernels read it once), so the host takes this path for few
// pairs.
// Work split: each slot's rows * G weight chunks (one contiguous block of its
// expert's matrix: row-major, rows of G chunks) are cut into segs units of 64
// lanes; wave w takes units w, w + 4, ..., so every unit's slot, and with it
// the expert id, is the same for the whole wave (a scalar load). Each chunk's
// scaled group sum goes to LDS; 8 lanes per (slot, row) add the G sums.
template <int CPT>
__global__ __launch_bounds__(256) void k_moe_tokens(const uint4 *__restrict__ Wall,
                                                    const uint16_t *__restrict__ Sall,
                                                    const int32_t *__restrict__ ids,
                                                    const uint16_t *__restrict__ route_w,
                                                    const uint16_t *__restrict__ x, int64_t ldx,
                                                    int64_t slot_stride, uint16_t *__restrict__ y,
                                                    int E, int N, int G, int TOPK, int rows,
                                                    int segs)
{
    extern __shared__ uint4 smem[];
    const int K = G * 32, chunks = K >> 3;
    const int stride = chunks + G / 4 + 1;  // uint4 units per staged activation row
    const int nx = slot_stride ? TOPK : 1;  // staged activation rows (one when all slots share it)
    const int t = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int per_slot = rows * G, units = TOPK * segs, nrow = TOPK * rows;
    float *part = reinterpret_cast<float *>(smem + nx * stride);  // [TOPK][rows][G]
    float *vrow = part + TOPK * per_slot;                         // [TOPK][rows]
    float *s_w = vrow + nrow;                                     // [TOPK] routing weights
    int *s_ok = reinterpret_cast<int *>(s_w + TOPK);              // [TOPK] id in [0, E)
    // matrix row of local row r, or -1 past the matrix
    auto row_of = [&](int r) {
        const int n = blockIdx.x * rows + r;
        return n < N ? n : -1;
    };

    // 1. the slots' validity and weights, and the activation rows
    //    (kMoeTokXq chunks per thread at most) into registers
    if (tid < TOPK) {
        const int e = ids[t * TOPK + tid];
        s_ok[tid] = e >= 0 && e < E;
        s_w[tid] = h2f(route_w[t * TOPK + tid]);
    }
    const int xtot = nx * chunks;
    uint4 xr[kMoeTokXq];
#pragma unroll
    for (int i = 0; i < kMoeTokXq; ++i) {
        const int c = tid + 256 * i;
        xr[i] = make_uint4(0u, 0u, 0u, 0u);
        if (c < xtot) {
            const int sl = c / chunks, j = c - sl * chunks;
            xr[i] = reinterpret_cast<const uint4 *>(x + (int64_t)t * ldx + (int64_t)sl * slot_stride)[j];
        }
    }
    // 2. the weight chunks, unit wave + 4 i (branch-free: units and chunks
    //    past the end re-read the last one, an invalid id reads expert 0, a
    //    row past the matrix reads row 0; none of these is used)
    uint4 wv[CPT];
    uint32_t sv[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int u = min(wave + 4 * i, units - 1);  // uniform
        const int sl = u / segs;
        const int cs = min((u - sl * segs) * 64 + lane, per_slot - 1);
        const int r = cs / G, g = cs - r * G;
        const int e = ids[t * TOPK + sl];  // uniform
        const size_t off = ((size_t)(e >= 0 && e < E ? e : 0) * N + max(row_of(r), 0)) * G + g;
        wv[i] = load_weights(Wall + off);
        sv[i] = load_scale(Sall + off);
    }
    // 3. the activation rows into LDS (pair order and group sums)
#pragma unroll
    for (int i = 0; i < kMoeTokXq; ++i) {
        const int c = tid + 256 * i;
        const bool live = c < xtot;
        const int sl = live ? c / chunks : 0, j = live ? c - sl * chunks : 0;
        uint4 *xs = smem + sl * stride;
        put_chunk(xr[i], j, live, xs, reinterpret_cast<float *>(xs + chunks));
    }
    __syncthreads();
    // 4. every chunk's scaled group sum
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int u = wave + 4 * i;
        const int sl = u / segs, cs = (u - sl * segs) * 64 + lane;
        if (u < units && cs < per_slot) {
            const int g = cs % G;
            const uint4 *xs = smem + (slot_stride ? sl : 0) * stride;
            const float sx = reinterpret_cast<const float *>(xs + chunks)[g];
            part[sl * per_slot + cs] = h2f(sv[i]) * group_dot(wv[i], xs, g, sx);
        }
    }
    __syncthreads();
    // 5. each (slot, row): its G group sums, 8 lanes in a fixed order
    for (int q0 = 0; q0 < nrow; q0 += 32) {
        const int q = q0 + (tid >> 3), k = tid & 7;
        float v = 0.f;
        if (q < nrow)
            for (int g = k; g < G; g += 8)
                v += part[q * G + g];
        v = segment_sum(v, 8);
        if (k == 0 && q < nrow)
            vrow[q] = v;
    }
    __syncthreads();
    // 6. each row: the valid slots in order, by routing weight
    const int n = tid < rows ? row_of(tid) : -1;
    if (n >= 0) {
        float acc = 0.f;
        for (int sl = 0; sl < TOPK; ++sl)
            if (s_ok[sl])
                acc = fmaf(s_w[sl], vrow[sl * rows + tid], acc);
        y[(int64_t)t * N + n] = f2h(acc);
    }
}

struct Cfg {
    int lpr, ng;
};

int max_ng(int lpr) { return lpr == 64 ? 12 : 8; }

// rows (segments) per lane group: fewer groups per lane, more rows per lane
constexpr int rows_per_segment(int ng) { return ng <= 2 ? 4 : (ng <= 4 ? 2 : 1); }

Cfg choose_cfg(int G)
{
    Cfg best{0, 0};
    int best_waste = 1 << 30;
    for (int lpr : {64, 32, 16, 8}) {
        const int ng = (G + lpr - 1) / lpr;
        if (ng > max_ng(lpr))
            continue;
        const int waste = ng * lpr - G;
        if (waste < best_waste) {
            best_waste = waste;
            best = {lpr, ng};
        }
    }
    return best;
}

template <int LPR, int NG, int EPI, int PRO, bool AFF>
q4_status run_gemv(const GemvParams &p, hipStream_t st)
{
    // residual-epilogue launches at three or four groups per lane (the O and
    // down projections, 3072 x 3072 and 3072 x 8192) take one row per segment:
    // twice the workgroups of matrices with few rows (measured: 0.5 % and
    // 1.2 % off a decode token; the norm-prologue QKV launch loses with it)
    constexpr int RPS = (EPI == EPI_RESID && (NG == 3 || NG == 4)) ? 1 : rows_per_segment(NG);
    constexpr int RB = kWaves * (64 / LPR) * RPS;
    const bool paired = EPI == EPI_SILU || EPI == EPI_ROPE;
    const int rows = paired ? p.N / 2 : p.N;
    const int rb = paired ? RB / 2 : RB;
    const int blocks = (rows + rb - 1) / rb;
    const size_t lds = (size_t)p.G * 32 * 2 + (size_t)p.G * 4;
    Q4_LAUNCH_MATVEC((k_gemv<LPR, NG, RPS, EPI, PRO, AFF>), dim3(blocks), dim3(256), lds, st, p);
    return check_launch("k_gemv");
}

template <int LPR, int EPI, int PRO, bool AFF = false>
q4_status dispatch_ng(int ng, const GemvParams &p, hipStream_t st)
{
    switch (ng) {
    case 1: return run_gemv<LPR, 1, EPI, PRO, AFF>(p, st);
    case 2: return run_gemv<LPR, 2, EPI, PRO, AFF>(p, st);
    case 3: return run_gemv<LPR, 3, EPI, PRO, AFF>(p, st);
    case 4: return run_gemv<LPR, 4, EPI, PRO, AFF>(p, st);
    case 5: return run_gemv<LPR, 5, EPI, PRO, AFF>(p, st);
    case 6: return run_gemv<LPR, 6, EPI, PRO, AFF>(p, st);
    case 7: return run_gemv<LPR, 7, EPI, PRO, AFF>(p, st);
    case 8: return run_gemv<LPR, 8, EPI, PRO, AFF>(p, st);
    default: break;
    }
    if constexpr (LPR == 64) {
        switch (ng) {
        case 9: return run_gemv<64, 9, EPI, PRO, AFF>(p, st);
        case 10: return run_gemv<64, 10, EPI, PRO, AFF>(p, st);
        case 11: return run_gemv<64, 11, EPI, PRO, AFF>(p, st);
        case 12: return run_gemv<64, 12, EPI, PRO, AFF>(p, st);
        default: break;
        }
    }
    return fail(Q4_ERANGE, "no matvec configuration for %d groups per lane", ng);
}

template <int EPI, int PRO, bool AFF = false>
q4_status dispatch_lpr(const Cfg &c, const GemvParams &p, hipStream_t st)
{
    switch (c.lpr) {
    case 64: return dispatch_ng<64, EPI, PRO, AFF>(c.ng, p, st);
    case 32: return dispatch_ng<32, EPI, PRO, AFF>(c.ng, p, st);
    case 16: return dispatch_ng<16, EPI, PRO, AFF>(c.ng, p, st);
    case 8: return dispatch_ng<8, EPI, PRO, AFF>(c.ng, p, st);
    default: return fail(Q4_ERANGE, "no matvec configuration for K = %d", p.G * 32);
    }
}

template <int LPR, int NG, int MR>
q4_status run_gemv_rows(const GemvParams &p, int64_t ldx, int64_t ldy, hipStream_t st)
{
    constexpr int RPS = rows_per_segment(NG);
    constexpr int RB = kWaves * (64 / LPR) * RPS;
    const int blocks = (p.N + RB - 1) / RB;
    const int chunks = p.G * 4;
    const size_t lds = (size_t)MR * (chunks + p.G / 4 + 1) * 16;
    if (p.Bias)
        Q4_LAUNCH_MATVEC((k_gemv_rows<LPR, NG, RPS, MR, true>), dim3(blocks), dim3(256), lds, st,
                         p, ldx, ldy);
    else
        Q4_LAUNCH_MATVEC((k_gemv_rows<LPR, NG, RPS, MR, false>), dim3(blocks), dim3(256), lds, st,
                         p, ldx, ldy);
    return check_launch("k_gemv_rows");
}

template <int LPR, int MR>
q4_status rows_ng(int ng, const GemvParams &p, int64_t ldx, int64_t ldy, hipStream_t st)
{
    switch (ng) {
    case 1: return run_gemv_rows<LPR, 1, MR>(p, ldx, ldy, st);
    case 2: return run_gemv_rows<LPR, 2, MR>(p, ldx, ldy, st);
    case 3: return run_gemv_rows<LPR, 3, MR>(p, ldx, ldy, st);
    case 4: return run_gemv_rows<LPR, 4, MR>(p, ldx, ldy, st);
    case 5: return run_gemv_rows<LPR, 5, MR>(p, ldx, ldy, st);
    case 6: return run_gemv_rows<LPR, 6, MR>(p, ldx, ldy, st);
    case 7: return run_gemv_rows<LPR, 7, MR>(p, ldx, ldy, st);
    case 8: return run_gemv_rows<LPR, 8, MR>(p, ldx, ldy, st);
    default: break;
    }
    if constexpr (LPR == 64) {
        switch (ng) {
        case 9: return run_gemv_rows<64, 9, MR>(p, ldx, ldy, st);
        case 10: return run_gemv_rows<64, 10, MR>(p, ldx, ldy, st);
        case 11: return run_gemv_rows<64, 11, MR>(p, ldx, ldy, st);
        case 12: return run_gemv_rows<64, 12, MR>(p, ldx, ldy, st);
        default: break;
        }
    }
    return fail(Q4_ERANGE, "no matvec configuration for %d groups per lane", ng);
}

template <int MR>
q4_status rows_lpr(const Cfg &c, const GemvParams &p, int64_t ldx, int64_t ldy, hipStream_t st)
{
    switch (c.lpr) {
    case 64: return rows_ng<64, MR>(c.ng, p, ldx, ldy, st);
    case 32: return rows_ng<32, MR>(c.ng, p, ldx, ldy, st);
    case 16: return rows_ng<16, MR>(c.ng, p, ldx, ldy, st);
    case 8: return rows_ng<8, MR>(c.ng, p, ldx, ldy, st);
    default: return fail(Q4_ERANGE, "no matvec configuration for K = %d", p.G * 32);
    }
}

struct MoeRowsArgs {
    const uint4 *W;
    const uint16_t *S;
    const int32_t *ids, *meta;
    const uint16_t *x;
    int64_t ldx, slot_stride;
    float *part;
    uint16_t *y;
    int out, E, N, G, P, TOPK, slots;
};

template <int LPR, int NG, int SC = 1>
q4_status run_moe_rows(const MoeRowsArgs &a, hipStream_t st)
{
    if (a.P >= kMoeWideRowsPairs && SC == 1)
        return run_moe_rows<LPR, NG, 2>(a, st);
    constexpr int RPS = SC * rows_per_segment(NG);
    constexpr int RB = kWaves * (64 / LPR) * RPS;
    const size_t lds = (size_t)kMaxRowsDot * (a.G * 4 + a.G / 4 + 1) * 16;
    if (a.out == kMoeOutSilu)
        Q4_LAUNCH_MATVEC((k_moe_rows<LPR, NG, RPS, true>),
                         dim3((a.N / 2 + RB / 2 - 1) / (RB / 2), 1, a.slots), dim3(256), lds, st,
                         a.W, a.S, a.ids, a.E, a.meta, a.P, a.x, a.ldx, a.slot_stride, a.TOPK,
                         a.out, a.part, a.y, a.N, a.G);
    else
        Q4_LAUNCH_MATVEC((k_moe_rows<LPR, NG, RPS, false>), dim3((a.N + RB - 1) / RB, 1, a.slots),
                         dim3(256), lds, st, a.W, a.S, a.ids, a.E, a.meta, a.P, a.x, a.ldx,
                         a.slot_stride, a.TOPK, a.out, a.part, a.y, a.N, a.G);
    return check_launch("k_moe_rows");
}

template <int LPR>
q4_status moe_rows_ng(int ng, const MoeRowsArgs &a, hipStream_t st)
{
    switch (ng) {
    case 1: return run_moe_rows<LPR, 1>(a, st);
    case 2: return run_moe_rows<LPR, 2>(a, st);
    case 3: return run_moe_rows<LPR, 3>(a, st);
    case 4: return run_moe_rows<LPR, 4>(a, st);
    case 5: return run_moe_rows<LPR, 5>(a, st);
    case 6: return run_moe_rows<LPR, 6>(a, st);
    case 7: return run_moe_rows<LPR, 7>(a, st);
    case 8: return run_moe_rows<LPR, 8>(a, st);
    default: break;
    }
    if constexpr (LPR == 64) {
        switch (ng) {
        case 9: return run_moe_rows<64, 9>(a, st);
        case 10: return run_moe_rows<64, 10>(a, st);
        case 11: return run_moe_rows<64, 11>(a, st);
        case 12: return run_moe_rows<64, 12>(a, st);
        default: break;
        }
    }
    return fail(Q4_ERANGE, "no matvec configuration for %d groups per lane", ng);
}

}  // namespace

q4_status launch_moe_rows(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                          const int32_t *meta, const uint16_t *x, int64_t ldx,
                          int64_t x_slot_stride, int out, float *part, uint16_t *y, int E, int N,
                          int K, int T, int TOPK, hipStream_t stream)
{
    MoeRowsArgs a;
    a.out = out;
    a.y = y;
    a.W = reinterpret_cast<const uint4 *>(W);
    a.S = S;
    a.ids = ids;
    a.meta = meta;
    a.x = x;
    a.ldx = ldx;
    a.slot_stride = x_slot_stride;
    a.part = part;
    a.E = E;
    a.N = N;
    a.G = K / 32;
    a.P = T * TOPK;
    a.TOPK = TOPK;
    if (a.P > kFusePairs)
        return fail(Q4_ERANGE, "the dot2 expert kernel takes at most %d pairs (got %d)",
                    kFusePairs, a.P);
    a.slots = a.P;  // units of at most kMaxRowsDot pairs: never more than the pairs
    const Cfg c = choose_cfg(a.G);
    switch (c.lpr) {
    case 64: return moe_rows_ng<64>(c.ng, a, stream);
    case 32: return moe_rows_ng<32>(c.ng, a, stream);
    case 16: return moe_rows_ng<16>(c.ng, a, stream);
    case 8: return moe_rows_ng<8>(c.ng, a, stream);
    default: return fail(Q4_ERANGE, "no matvec configuration for K = %d", K);
    }
}

namespace {
// Rows per workgroup of the token-wise down kernel: at most kMoeTokRows and
// within kMoeTokCpt units per wave; 0 if none fits. (The row count barely
// matters at one token on 128 experts, top 8: 1 to 8 rows measured within
// 0.5 us; the kernel waits on two memory round trips, ids then weights.)
int moe_tokens_rows(int TOPK, int K)
{
    const int G = K / 32;
    for (int rows = kMoeTokRows; rows >= 1; --rows)
        if (TOPK * ((rows * G + 63) / 64) <= 4 * kMoeTokCpt)
            return rows;
    return 0;
}
}  // namespace

bool moe_tokens_fits(int T, int TOPK, int K, bool shared_x)
{
    return T * TOPK <= kMoeTokMaxPairs && (shared_x ? 1 : TOPK) * (K / 8) <= 256 * kMoeTokXq &&
           moe_tokens_rows(TOPK, K) > 0;
}

q4_status launch_moe_tokens(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                            const uint16_t *route_w, const uint16_t *x, int64_t ldx,
                            int64_t x_slot_stride, uint16_t *y, int E, int N, int K, int T,
                            int TOPK, hipStream_t stream)
{
    const int G = K / 32, chunks = K / 8, stride = chunks + G / 4 + 1;
    const int rows = moe_tokens_rows(TOPK, K);
    if (rows == 0)
        return fail(Q4_ERANGE, "internal: no row block for the token-wise expert kernel");
    const int segs = (rows * G + 63) / 64, cpt = (TOPK * segs + 3) / 4;
    const int nx = x_slot_stride ? TOPK : 1;
    const size_t lds = (size_t)nx * stride * 16 + (size_t)TOPK * (segs * 64 + rows + 2) * 4;
    const dim3 grid((N + rows - 1) / rows, T);
    const uint4 *Wv = reinterpret_cast<const uint4 *>(W);
#define Q4_TOK_CASE(c)                                                                            \
    case c:                                                                                       \
        Q4_LAUNCH_MATVEC((k_moe_tokens<c>), grid, dim3(256), lds, stream, Wv, S, ids, route_w, x,  \
                         ldx, x_slot_stride, y, E, N, G, TOPK, rows, segs);                       \
        break;
    switch (cpt) {
        Q4_TOK_CASE(1) Q4_TOK_CASE(2) Q4_TOK_CASE(3) Q4_TOK_CASE(4) Q4_TOK_CASE(5) Q4_TOK_CASE(6)
        Q4_TOK_CASE(7) Q4_TOK_CASE(8)
    default: return fail(Q4_ERANGE, "internal: %d units per wave for the token-wise down kernel", cpt);
    }
#undef Q4_TOK_CASE
    return check_launch("k_moe_tokens");
}

int matvec_blocks(int N, int K)
{
    const Cfg c = choose_cfg(K / 32);
    if (!c.lpr)
        return 0;
    const int rb = kWaves * (64 / c.lpr) * rows_per_segment(c.ng);
    return (N + rb - 1) / rb;
}

q4_status launch_gemv_op(const GemvOp &op, hipStream_t stream)
{
    GemvParams p{};
    p.W = reinterpret_cast<const uint4 *>(op.W);
    p.S = op.S;
    p.N = op.N;
    p.G = op.K / 32;
    p.x = op.norm_src ? op.norm_src : op.x;
    p.pro_gamma = op.norm_gamma;
    p.pro_eps = op.norm_eps;
    p.y = op.y;
    p.res_in = op.res_in;
    p.res_out = op.res_out;
    p.yf = op.yf;
    p.cand = op.cand;
    p.rope = op.rope;
    p.Bias = op.bias;
    const Cfg c = choose_cfg(p.G);
    const bool norm = op.norm_src != nullptr;
    if (op.bias) {  // the affine format: plain output only
        if (norm || op.epi != GemvOp::NONE)
            return fail(Q4_EINVAL, "internal: the affine format has no prologue or epilogue");
        return dispatch_lpr<EPI_NONE_, PRO_X, true>(c, p, stream);
    }
    switch (op.epi) {
    case GemvOp::NONE:
        return norm ? dispatch_lpr<EPI_NONE_, PRO_NORM>(c, p, stream)
                    : dispatch_lpr<EPI_NONE_, PRO_X>(c, p, stream);
    case GemvOp::SILU:
        return norm ? dispatch_lpr<EPI_SILU, PRO_NORM>(c, p, stream)
                    : dispatch_lpr<EPI_SILU, PRO_X>(c, p, stream);
    case GemvOp::RESID:
        if (norm)
            return fail(Q4_EINVAL, "internal: normalising prologue with a residual epilogue");
        return dispatch_lpr<EPI_RESID, PRO_X>(c, p, stream);
    case GemvOp::LOGITS:
        if (norm)
            return fail(Q4_EINVAL, "internal: normalising prologue with the logits epilogue");
        return dispatch_lpr<EPI_LOGITS, PRO_X>(c, p, stream);
    case GemvOp::ROPE:
        return norm ? dispatch_lpr<EPI_ROPE, PRO_NORM>(c, p, stream)
                    : dispatch_lpr<EPI_ROPE, PRO_X>(c, p, stream);
    default:
        return fail(Q4_EINVAL, "internal: unknown matvec epilogue %d", op.epi);
    }
}

q4_status launch_gemv(const uint32_t *W, const uint16_t *S, const uint16_t *x, uint16_t *y,
                      int N, int K, const EpiArgs &epi, hipStream_t stream)
{
    GemvOp op;
    op.W = W;
    op.S = S;
    op.N = N;
    op.K = K;
    if (epi.norm_gamma) {
        op.norm_src = x;
        op.norm_gamma = epi.norm_gamma;
        op.norm_eps = epi.eps;
    } else {
        op.x = x;
    }
    switch (epi.kind) {
    case Q4_EPI_NONE:
        op.epi = GemvOp::NONE;
        op.y = y;
        return launch_gemv_op(op, stream);
    case Q4_EPI_SILU_MUL:
        op.epi = GemvOp::SILU;
        op.y = y;
        return launch_gemv_op(op, stream);
    case Q4_EPI_ADD_RMSNORM: {
        // residual rows in the matvec's epilogue, then one workgroup normalises
        // the stored row: no synchronisation between workgroups of a kernel
        op.epi = GemvOp::RESID;
        op.res_in = epi.res_in;
        op.res_out = epi.res_out;
        q4_status st = launch_gemv_op(op, stream);
        if (st != Q4_OK)
            return st;
        return launch_add_rmsnorm(nullptr, epi.res_out, epi.gamma, y, nullptr, N, 1, epi.eps,
                                  stream);
    }
    default:
        return fail(Q4_EINVAL, "unknown epilogue kind %d", epi.kind);
    }
}

// Batched matvec: M = 1 is the matvec above; M >= 2 rows share each weight
// read on the matrix cores (q4_mfma.hip).
bool gemv_rows_fits(int M, int K, int64_t N)
{
    if (M < 2 || M > kMaxRowsDot || M * K > 24576)
        return false;
    return !(M >= 3 && N * K >= (int64_t(1) << 26) && mma_fits((int)N, K, M));
}

q4_status launch_gemv_rows(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                           uint16_t *y, int64_t ldy, int N, int K, int M, hipStream_t stream,
                           const uint16_t *bias, float *yf)
{
    GemvParams p{};
    p.W = reinterpret_cast<const uint4 *>(W);
    p.S = S;
    p.Bias = bias;
    p.yf = yf;
    p.N = N;
    p.G = K / 32;
    p.x = x;
    p.y = y;
    const Cfg c = choose_cfg(p.G);
    switch (M) {
    case 2: return rows_lpr<2>(c, p, ldx, ldy, stream);
    case 3: return rows_lpr<3>(c, p, ldx, ldy, stream);
    case 4: return rows_lpr<4>(c, p, ldx, ldy, stream);
    default: return fail(Q4_EINVAL, "internal: %d rows for the dot2 batched matvec", M);
    }
}

q4_status launch_gemv_batched(const uint32_t *W, const uint16_t *S, const uint16_t *x,
                              int64_t ldx, uint16_t *y, int64_t ldy, int N, int K, int M,
                              hipStream_t stream)
{
    if (M == 1)  // a single row is the bandwidth-bound matvec
        return launch_gemv(W, S, x, y, N, K, EpiArgs{}, stream);
    if (gemv_rows_fits(M, K, N))  // a few rows: the single-row kernel's arithmetic per row
        return launch_gemv_rows(W, S, x, ldx, y, ldy, N, K, M, stream);
    return launch_gemv_mfma(W, S, x, ldx, y, nullptr, ldy, N, K, M, stream);
}

}  // namespace q4
