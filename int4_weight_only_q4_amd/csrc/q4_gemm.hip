// Prefill (many-token) int4 x f16 matmul on the gfx950 matrix cores.
//
// What is computed is the batched matmul of the q4f16_1 format (Zero TVM
// Documentation, "Q4F16 quantization format"; BENCH.md, "Tiled batched GEMM"
// and "Subgroup-matrix GEMM graduated"): Y[m][n] = f16( sum_k (q[n][k] - 7) *
// s[n][k/32] * X[m][k] ), f32 accumulation, for any number M of activation
// rows. The decode kernels stream the weights once for at most 16 rows; here
// each weight tile is dequantised once per 64 or 128 rows:
//  * workgroup tile: 64 activation rows x 128 weight rows (four waves, three
//    workgroups per CU) or 128 x 256 (eight waves, one per CU, two steps of
//    loads in flight); wave w owns weight rows [32 w, 32 w + 32) of the tile
//    (two 16-row matrix-core tiles) and all 16-row activation tiles, so each
//    dequantised weight feeds four or eight MFMAs;
//  * exact weights: the codes q - 7 (exact in binary16) enter the matrix
//    core, one MFMA per 32-value group gives the group's f32 sum over the
//    tile, and each lane (its output column is its weight row) adds s times
//    it into its accumulator with one f32 FMA per element, so no dequantised
//    weight is rounded (the page's matrix-unit kernel rounds the staged
//    weights to f16: the f16-weight mode, which multiplies f16((q - 7) s));
//  * a step covers four quantisation groups (128 values of K): lane (n, kb)
//    loads group 4 p + kb of its weight row (16 bytes), a 4 x 4 transpose over
//    the lane rows (permlane swaps) gives each lane row its word of every
//    group, and MFMA t of the step takes group t; the step's 64 x 128
//    activation values are staged in LDS in the pair order of the unpack;
//  * the next step's loads are in flight while the current step multiplies;
//  * tiles go to the XCDs in contiguous slabs of weight rows, activation tile
//    fastest, so an XCD's L2 keeps the weight tile for all its row blocks;
//  * rows past M or N are clamped on load and never stored; groups past K get
//    scale 0 and zero activations.
// The MLX affine format (w = s * q + b, q unsigned, s and b per 64 codes; Zero
// TVM Documentation, the Qwen3.6-35B-A3B entry; BENCH.md "Subgroup-matrix GEMM
// graduated", the _affine variants) runs through the same exact loop with
// unsigned codes and the scale of group g / 2 (applied per 32 values); its
// bias term sum_g b[n][g] * xs[m][g],
// xs[m][g] = the sum of row m's activations over group g, is a few more K steps
// of the same matrix product: A = xs split into binary16 hi and lo halves (a
// small kernel forms them), B = the binary16 biases.
#include <algorithm>
#include <type_traits>

#include "q4_dequant.h"

namespace q4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBNMax = 256;            // weight rows per workgroup: 32 per wave, up to 8 waves
constexpr int kStepK = 128;            // K values per step (four groups)
constexpr int kAStride = kStepK + 8;   // staged row in halves (16 bytes of padding)
constexpr int kXcds = 8;
constexpr int kMaxSplits = 16;   // K splits of one launch

// 4 x 4 transpose over (lane row, register): afterwards r[t] in lane row q
// holds what r[q] held in lane row t.
__device__ __forceinline__ void transpose_rows(uint32_t (&r)[4])
{
    swap32(r[0], r[2]);
    swap32(r[1], r[3]);
    swap16(r[0], r[1]);
    swap16(r[2], r[3]);
}

// Row broadcast: afterwards out[t] in every lane row holds v of lane row t.
__device__ __forceinline__ void broadcast_rows(uint32_t v, uint32_t (&out)[4])
{
    uint32_t p = v, q = v;
    swap16(p, q);
    uint32_t p2 = p, q2 = q;
    swap32(p, p2);
    swap32(q, q2);
    out[0] = p;
    out[1] = q;
    out[2] = p2;
    out[3] = q2;
}

// The 8 codes of word w as binary16 q - 7 (AFF: q), exact, in the pair order
// (e0, e4) (e1, e5) (e2, e6) (e3, e7). A nibble in mantissa bits 0..3 under
// exponent field 25 is the binary16 1024 + q; in bits 4..7 under exponent
// field 21 it is 64 + q, so one shift of the word by 8 reaches all four pairs.
template <bool AFF>
__device__ __forceinline__ half8 codes_of(uint32_t w)
{
    const half2v c1031 = {(_Float16)(AFF ? -1024.0f : -1031.0f), (_Float16)(AFF ? -1024.0f : -1031.0f)};
    const half2v c71 = {(_Float16)(AFF ? -64.0f : -71.0f), (_Float16)(AFF ? -64.0f : -71.0f)};
    const uint32_t w8 = w >> 8;
    uint32_t b[4];
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(b[0]) : "v"(0x000F000Fu), "v"(w), "s"(0x64006400u));
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(b[1]) : "v"(0x00F000F0u), "v"(w), "s"(0x54005400u));
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(b[2]) : "v"(0x000F000Fu), "v"(w8), "s"(0x64006400u));
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(b[3]) : "v"(0x00F000F0u), "v"(w8), "s"(0x54005400u));
    half8 q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2v v = __builtin_bit_cast(half2v, b[i]) + ((i & 1) ? c71 : c1031);
        q[2 * i] = v[0];
        q[2 * i + 1] = v[1];
    }
    return q;
}

// The 8 binary16 weights f16((q - 7) s) of word w, in the pair order of codes_of.
__device__ __forceinline__ half8 f16_weights_of(uint32_t w, half2v s2)
{
    const half8 q = codes_of<false>(w);
    half8 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2v p = half2v{q[2 * i], q[2 * i + 1]} * s2;
        h[2 * i] = p[0];
        h[2 * i + 1] = p[1];
    }
    return h;
}

// A 16-byte chunk of 8 activations in the pair order of codes_of.
__device__ __forceinline__ u32x4 pair_order(u32x4 v)
{
    return u32x4{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                 __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                 __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                 __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
}

// The buffers of one launch (sizes in bytes; an offset past the size reads 0).
struct Bufs {
    __amdgpu_buffer_rsrc_t w, s, x;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

constexpr uint32_t kOut = 0x80000000u;  // an offset beyond every buffer: loads return 0

// A thread's byte offsets at step 0, the same at every step but for the
// step's own scalar offset: its lane's word group and scale of the wave's two
// weight rows, and XP 16-byte pieces of the activation tile (piece q: row
// (t + NT q) / 16, eight values (t % 16) of the step, NT threads per
// workgroup). Rows past N or M read 0.
template <int XP>
struct Offsets {
    uint32_t w[2], s[2], x[XP];
};

// One step's loaded data of a thread.
template <int XP, bool S4>
struct StepLoads {
    u32x4 w[2];
    uint32_t s[2][S4 ? 2 : 1];
    u32x4 x[XP];
};

// (AFF: a step spans two 64-code groups, so its scales are 4 bytes on.) S4
// (G % 4 == 0): each lane loads all the scales of the step's groups of its row
// in one load (8 bytes, four scales; affine: 4 bytes, two scales of 64 codes);
// otherwise each of the row's four lanes loads one 2-byte scale and permlane
// swaps hand every lane the other three.
template <int XP, bool AFF, bool S4>
__device__ __forceinline__ void load_step(StepLoads<XP, S4> &L, const Bufs &B,
                                          const Offsets<XP> &O, int st)
{
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        L.w[ns] = __builtin_amdgcn_raw_buffer_load_b128(B.w, O.w[ns], st * 64, 0);
        if (S4 && AFF) {
            L.s[ns][0] = __builtin_amdgcn_raw_buffer_load_b32(B.s, O.s[ns], st * 4, 0);
        } else if (S4) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(B.s, O.s[ns], st * 8, 0);
            L.s[ns][0] = v[0];
            L.s[ns][S4 ? 1 : 0] = v[1];
        } else {
            L.s[ns][0] = __builtin_amdgcn_raw_buffer_load_b16(B.s, O.s[ns], st * (AFF ? 4 : 8), 0);
        }
    }
#pragma unroll
    for (int q = 0; q < XP; ++q)
        L.x[q] = __builtin_amdgcn_raw_buffer_load_b128(B.x, O.x[q], st * 256, 0);
}

// Weight words and scales of a step, rearranged for the matrix core:
// wt[ns][tt] is this lane row's word of group tt, s2[ns][tt] that group's
// scale (both halves). LAST: groups past K get scale 0.
struct StepWeights {
    uint32_t wt[2][4];
    half2v s2[2][4];
};

template <int XP, bool LAST, bool S4, bool AFF>
__device__ __forceinline__ void prepare(StepWeights &P, const StepLoads<XP, S4> &L, int gs,
                                        int kb, int G)
{
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        P.wt[ns][0] = L.w[ns].x;
        P.wt[ns][1] = L.w[ns].y;
        P.wt[ns][2] = L.w[ns].z;
        P.wt[ns][3] = L.w[ns].w;
        transpose_rows(P.wt[ns]);
        uint32_t sc[4];
        if (S4 && AFF) {
            // groups 0, 1 of the step share the first 64-code scale, 2, 3 the second
            sc[0] = sc[1] = L.s[ns][0] & 0xFFFFu;
            sc[2] = sc[3] = L.s[ns][0] >> 16;
        } else if (S4) {
            // (G % 4 == 0: a step never reaches past K)
            sc[0] = L.s[ns][0] & 0xFFFFu;
            sc[1] = L.s[ns][0] >> 16;
            sc[2] = L.s[ns][S4 ? 1 : 0] & 0xFFFFu;
            sc[3] = L.s[ns][S4 ? 1 : 0] >> 16;
        } else {
            uint32_t s = L.s[ns][0];
            if (LAST && gs + kb >= G)
                s = 0;
            broadcast_rows(s, sc);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
            P.s2[ns][tt] = __builtin_bit_cast(half2v, sc[tt] * 0x10001u);
    }
}

// Stores a step's activation pieces into an LDS buffer in pair order. LAST:
// values past K are zero.
template <int XP, bool LAST, int NT, bool S4>
__device__ __forceinline__ void stage(_Float16 *buf, const StepLoads<XP, S4> &L, int gs, int G,
                                      int t)
{
#pragma unroll
    for (int q = 0; q < XP; ++q) {
        const int c = t + NT * q;
        u32x4 v = pair_order(L.x[q]);
        if (LAST && gs * 32 + 8 * (c & 15) >= G * 32)
            v = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(buf + (c >> 4) * kAStride + 8 * (c & 15)) = v;
    }
}

// Weight modes: binary16 weights f16((q - 7) s) (kWF16), or exact products
// (kWGroup): the codes q - 7 enter the matrix core as they are, one MFMA per
// 32-value group gives that group's sum over the tile in f32, and the lane
// (whose output column is its weight row) adds s times it into the
// accumulator with one f32 FMA per element.
enum : int { kWF16 = 0, kWGroup = 1 };

template <int MS, int MODE, bool AFF>
__device__ __forceinline__ void multiply(floatx4 (&acc)[MS][2], const _Float16 *cur,
                                         const StepWeights &P, int n, int kb)
{
    if constexpr (MODE == kWGroup) {
        // each group sum is scaled into its accumulator after the next MFMA
        // has been issued (read right after its own MFMA, it would wait out
        // the MFMA's latency)
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
        floatx4 prev = zero;
        float sprev = 0.f;
        int pm = 0, pn = 0;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            half8 a[MS], bq[2];
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
                a[ms] = *reinterpret_cast<const half8 *>(cur + (16 * ms + n) * kAStride + 8 * kb +
                                                         32 * tt);
#pragma unroll
            for (int ns = 0; ns < 2; ++ns)
                bq[ns] = codes_of<AFF>(P.wt[ns][tt]);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    const floatx4 gsum =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ms], bq[ns], zero, 0, 0, 0);
                    if (tt > 0 || ms > 0 || ns > 0)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[pm][pn][i] = fmaf(sprev, prev[i], acc[pm][pn][i]);
                    prev = gsum;
                    sprev = (float)P.s2[ns][tt][0];
                    pm = ms;
                    pn = ns;
                }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[pm][pn][i] = fmaf(sprev, prev[i], acc[pm][pn][i]);
        return;
    }
    // kWF16 (symmetric codes only)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        half8 a[MS], bh[2];
        __builtin_amdgcn_iglp_opt(1);  // interleave the matrix-core and LDS work
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
            a[ms] = *reinterpret_cast<const half8 *>(cur + (16 * ms + n) * kAStride + 8 * kb +
                                                     32 * tt);
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
            bh[ns] = f16_weights_of(P.wt[ns][tt], P.s2[ns][tt]);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int ns = 0; ns < 2; ++ns)
                acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ms], bh[ns], acc[ms][ns],
                                                                     0, 0, 0);
    }
}

// The affine bias term as extra K steps: step bs covers entries [128 bs,
// 128 bs + 128) of the group-sum rows xs[m][0 .. 2 GP) (hi halves of groups
// 0..GP-1, then the lo halves; entries of groups past G64 are 0) against
// B[j][n] = bias[n][j mod GP] (0 past G64), in natural order (no pair order
// on either side). The caller has passed the last barrier of the main loop.
// Bias steps [b0, b1); bvec: the bias rows allow 16-byte loads (G64 % 8 == 0,
// Bias 16-byte aligned).
template <int MS, int XP, int NT>
__device__ __forceinline__ void bias_steps(floatx4 (&acc)[MS][2], _Float16 *buf,
                                           const uint16_t *__restrict__ XS, int M, int m0,
                                           const uint16_t *__restrict__ Bias, int N, int n0,
                                           int G64, int GP, int b0, int b1, bool bvec, int t,
                                           int n, int kb)
{
    const int ld = 2 * GP;
    const __amdgpu_buffer_rsrc_t rx = rsrc(XS, (uint32_t)((int64_t)M * ld * 2));
    const __amdgpu_buffer_rsrc_t rb = rsrc(Bias, (uint32_t)N * (uint32_t)G64 * 2u);
    for (int bs = b0; bs < b1; ++bs) {
        __syncthreads();  // the buffer's previous contents are no longer read
#pragma unroll
        for (int q = 0; q < XP; ++q) {
            const int c = t + NT * q, row = m0 + (c >> 4);
            const uint32_t off = row < M ? (uint32_t)((row * ld + 128 * bs + 8 * (c & 15)) * 2) : kOut;
            *reinterpret_cast<u32x4 *>(buf + (c >> 4) * kAStride + 8 * (c & 15)) =
                __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
        }
        __syncthreads();
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int j0 = 128 * bs + 32 * tt + 8 * kb;  // this lane row's 8 K entries
            const int g0 = j0 < GP ? j0 : j0 - GP;
            half8 bb[2];
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const int row = n0 + 16 * ns + n;
                if (bvec) {  // eight biases of one group range in one load (0 past G64)
                    const uint32_t off = row < N && g0 < G64 ? (uint32_t)(row * G64 + g0) * 2u : kOut;
                    bb[ns] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t off = row < N && g0 + e < G64 ? (uint32_t)(row * G64 + g0 + e) * 2u : kOut;
                        bb[ns][e] = __builtin_bit_cast(_Float16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rb, off, 0, 0));
                    }
                }
            }
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                const half8 a = *reinterpret_cast<const half8 *>(buf + (16 * ms + n) * kAStride + 8 * kb + 32 * tt);
#pragma unroll
                for (int ns = 0; ns < 2; ++ns)
                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bb[ns], acc[ms][ns], 0, 0, 0);
            }
        }
    }
}

// Group sums of the activation rows for the affine bias: xs[m][g] = hi and
// xs[m][GP + g] = lo with s = the f32 sum over x[m][64 g .. 64 g + 63], hi =
// f16(s), lo = f16(s - hi); 0 for g >= G64. One thread per 8-value chunk sums
// its chunk in order; the 8 chunks of a group (8 consecutive lanes) are added
// by segment_sum, in one fixed order.
__global__ __launch_bounds__(256) void k_group_sums(const uint16_t *__restrict__ X, int64_t ldx,
                                                    uint16_t *__restrict__ XS, int M, int G64,
                                                    int GP)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // chunk index
    const int64_t gi = i >> 3;                                     // (m, g)
    const bool live = gi < (int64_t)M * GP;
    const int m = live ? (int)(gi / GP) : 0, g = live ? (int)(gi % GP) : 0;
    float s = 0.f;
    if (live && g < G64) {
        float f[8];
        chunk_to_float(*reinterpret_cast<const uint4 *>(X + (int64_t)m * ldx + 64 * g +
                                                        8 * (int)(i & 7)),
                       f);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            s += f[e];
    }
    s = segment_sum(s, 8);  // all lanes take part
    if (live && (i & 7) == 0) {
        const uint16_t hi = f2h(s);
        XS[(int64_t)m * 2 * GP + g] = hi;
        XS[(int64_t)m * 2 * GP + GP + g] = f2h(s - h2f(hi));
    }
}

// Grid: one workgroup per (16 MS-row activation tile, 32 NW-row weight tile),
// NW waves; wave w owns weight rows [32 w, 32 w + 32) of the tile and all MS
// 16-row activation tiles. A thread stages XP pieces of the step's activation
// tile. Eight waves share each staged tile between twice the weight rows and
// keep two steps of loads in flight (register buffers used in turn); four
// waves keep one. Buffer sizes below 2^31 bytes (the launcher splits larger
// problems).
// AFF: the affine format; S and Bias [N][G / 2]; XS the group sums of X
// (k_group_sums, GP groups per half).
template <int MS, int MODE, bool AFF, int NW, bool S4>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : (MS == 8 ? 2 : 3)) void k_gemm_q4(
    const uint4 *__restrict__ W, const uint16_t *__restrict__ S, const uint16_t *__restrict__ X,
    int64_t ldx, uint16_t *__restrict__ Y, int64_t ldy, float *__restrict__ part, int M, int N,
    int G, int sps, const uint16_t *__restrict__ Bias, const uint16_t *__restrict__ XS, int GP,
    int bvec)
{
    constexpr int BM = 16 * MS, BN = 32 * NW, NT = 64 * NW, XP = 4 * MS / NW;
    constexpr int D = NW == 8 ? 2 : 1;  // steps of loads in flight
    __shared__ _Float16 xs[2][BM * kAStride];
    const int t = threadIdx.x, l = t & 63, wave = t >> 6;
    const int n = l & 15, kb = l >> 4;

    // XCD-aware tile order: workgroup b runs on XCD b % 8; XCD x takes the
    // contiguous tile range [start(x), start(x) + count(x)), activation tile fastest
    const int mtiles = (M + BM - 1) / BM, ntiles = (N + BN - 1) / BN;
    const int total = mtiles * ntiles, per = total / kXcds, rem = total % kXcds;
    const int b = blockIdx.x, x = b % kXcds;
    const int r = x * per + min(x, rem) + b / kXcds;
    const int m0 = (r % mtiles) * BM, n0 = (r / mtiles) * BN + 32 * wave;

    Bufs B;
    B.w = rsrc(W, (uint32_t)N * (uint32_t)G * 16u);
    B.s = rsrc(S, (uint32_t)N * (uint32_t)(AFF ? G / 2 : G) * 2u);
    B.x = rsrc(X, (uint32_t)(((int64_t)(M - 1) * ldx + G * 32) * 2));
    Offsets<XP> O;
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        const int row = n0 + 16 * ns + n;
        O.w[ns] = row < N ? (uint32_t)(row * G + kb) * 16u : kOut;
        O.s[ns] = row < N ? (uint32_t)(AFF ? row * (G / 2) + (S4 ? 0 : kb / 2)
                                           : row * G + (S4 ? 0 : kb)) * 2u
                          : kOut;
    }
#pragma unroll
    for (int q = 0; q < XP; ++q) {
        const int c = t + NT * q, row = m0 + (c >> 4);
        O.x[q] = row < M ? (uint32_t)((row * ldx + 8 * (c & 15)) * 2) : kOut;
    }

    floatx4 acc[MS][2];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
            acc[ms][ns] = floatx4{0.f, 0.f, 0.f, 0.f};

    // step st: groups [4 st, 4 st + 4); its loads are issued one step ahead.
    // K split z (grid y) takes the steps [z sps, min((z + 1) sps, total)); in
    // the affine format the bias steps follow the weight steps.
    const int steps = (G + 3) / 4, z = blockIdx.y;
    const int total_steps = steps + (AFF ? GP / 64 : 0);
    const int st0 = z * sps, st1 = min(steps, st0 + sps);
    const int bs1 = min(total_steps, st0 + sps);
    StepLoads<XP, S4> L[D];
    StepWeights P;
    // one step from register buffer Lr: stage its activation tile into LDS
    // buffer st & 1 and its weights into P, refill Lr with step `next` (LOAD;
    // the loads stay in flight D steps), then multiply once the tile is
    // staged. The LDS buffer was last read two steps before, ahead of the
    // previous step's barrier. LAST: groups past K (only the last step of the
    // last split). A refill past the split's last step re-reads that step
    // (unconditional loads keep the two buffers' registers apart).
    auto body = [&](StepLoads<XP, S4> &Lr, int st, int next, auto last, auto load)
                    __attribute__((always_inline)) {
        stage<XP, decltype(last)::value, NT, S4>(xs[st & 1], Lr, 4 * st, G, t);
        prepare<XP, decltype(last)::value, S4, AFF>(P, Lr, 4 * st, kb, G);
        if constexpr (decltype(load)::value)
            load_step<XP, AFF, S4>(Lr, B, O, next);
        __syncthreads();
        multiply<MS, MODE, AFF>(acc, xs[st & 1], P, n, kb);
    };
    const std::false_type no;
    const std::true_type yes;
    if (st0 < st1) {
#pragma unroll
        for (int d = 0; d < D; ++d)
            load_step<XP, AFF, S4>(L[d], B, O, min(st0 + d, st1 - 1));
        if constexpr (D == 1) {
            for (int st = st0; st < st1 - 1; ++st)
                body(L[0], st, st + 1, no, yes);
            body(L[0], st1 - 1, 0, yes, no);
        } else {
            int st = st0;
            for (; st + 2 < st1; st += 2) {
                body(L[0], st, st + 2, no, yes);
                body(L[1], st + 1, min(st + 3, st1 - 1), no, yes);
            }
            if (st + 1 < st1) {
                body(L[0], st, 0, no, no);
                body(L[1], st + 1, 0, yes, no);
            } else {
                body(L[0], st, 0, yes, no);
            }
        }
    }
    if (AFF && bs1 > steps)  // this split's share of the bias steps
        bias_steps<MS, XP, NT>(acc, xs[0], XS, M, m0, Bias, N, n0, G / 2, GP,
                               max(st0, steps) - steps, bs1 - steps, bvec != 0, t, n, kb);

    // lane (n, kb) holds D[4 kb + i][n] of each (activation, weight) tile:
    // rounded to Y, or with several K splits the f32 partial part[z][row][col]
    const bool split = gridDim.y > 1;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            const int col = n0 + 16 * ns + n;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + 16 * ms + 4 * kb + i;
                if (row < M && col < N) {
                    if (split)
                        part[((size_t)z * M + row) * N + col] = acc[ms][ns][i];
                    else
                        Y[(int64_t)row * ldy + col] = f2h(acc[ms][ns][i]);
                }
            }
        }
}

// Y[m][n] = f16(sum over z, in order, of part[z][m][n]); thread i takes the
// V consecutive outputs from V i (V = 4: N % 4 == 0 and Y rows 8-byte aligned).
template <int V>
__global__ __launch_bounds__(256) void k_gemm_combine(const float *__restrict__ part, int KS,
                                                      int M, int N, uint16_t *__restrict__ Y,
                                                      int64_t ldy)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
    const int64_t plane = (int64_t)M * N;
    if (i >= plane)
        return;
    const int row = (int)(i / N), col = (int)(i % N);
    if (V == 4) {
        float4 v[kMaxSplits];
#pragma unroll
        for (int z = 0; z < kMaxSplits; ++z)
            if (z < KS)
                v[z] = *reinterpret_cast<const float4 *>(part + z * plane + i);
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int z = 0; z < kMaxSplits; ++z)
            if (z < KS) {
                s.x += v[z].x;
                s.y += v[z].y;
                s.z += v[z].z;
                s.w += v[z].w;
            }
        const uint32_t lo = f2h(s.x) | (uint32_t)f2h(s.y) << 16;
        const uint32_t hi = f2h(s.z) | (uint32_t)f2h(s.w) << 16;
        *reinterpret_cast<uint2 *>(Y + (int64_t)row * ldy + col) = make_uint2(lo, hi);
    } else {
        float s = 0.f;
        for (int z = 0; z < KS; ++z)
            s += part[z * plane + i];
        Y[(int64_t)row * ldy + col] = f2h(s);
    }
}

// Launch shape of one chunk: activation rows per workgroup (16 MS), waves per
// workgroup (NW, 32 weight rows each) and the number of K splits. 128 x 256
// tiles (eight waves) run one workgroup per CU, 64 x 128 tiles (four waves)
// three at about kRound4 of the time per 128 x 256 tile; the shape with fewer
// estimated rounds wins. A grid that fills fewer than half the workgroup slots
// splits K (at least four steps per split, at most kMaxSplits) into f32
// partials that k_gemm_combine sums in split order.
struct GemmShape {
    int ms, nw, splits, sps;
};
constexpr double kRound4 = 0.72;  // measured: Phi-3 gate_up at M = 1024, exact weights

// (extra: steps after the weight steps, the affine bias steps)
GemmShape gemm_shape(int M, int N, int G, size_t max_part_bytes, int extra = 0)
{
    const int cus = cu_count(), steps = (G + 3) / 4 + extra;
    const int64_t t8 = (int64_t)((M + 127) / 128) * ((N + 255) / 256);
    const int64_t t4 = (int64_t)((M + 63) / 64) * ((N + 127) / 128);
    const double r8 = (double)((t8 + cus - 1) / cus);
    const double r4 = kRound4 * (double)((t4 + 3 * cus - 1) / (3 * cus));
    GemmShape g;
    g.ms = r4 < r8 ? 4 : 8;
    g.nw = g.ms == 4 ? 4 : 8;
    const int64_t tiles = g.ms == 4 ? t4 : t8, slots = (g.ms == 4 ? 3 : 1) * (int64_t)cus;
    int ks = 1;
    if (2 * tiles <= slots) {
        ks = (int)std::min<int64_t>({(slots + tiles - 1) / tiles, std::max(1, steps / 4), kMaxSplits});
        while (ks > 1 && (size_t)ks * M * N * sizeof(float) > max_part_bytes)
            --ks;
    }
    g.sps = (steps + ks - 1) / ks;
    g.splits = (steps + g.sps - 1) / g.sps;  // every split has at least one step
    return g;
}

template <int MS, int NW>
q4_status launch_tiles(bool exact, dim3 grid, hipStream_t stream, const uint4 *w, const uint16_t *s,
                       const uint16_t *x, int64_t ldx, uint16_t *y, int64_t ldy, float *part,
                       int M, int N, int G, int sps, const uint16_t *bias, const uint16_t *xsum,
                       int gp)
{
    const int bvec = bias && (G / 2) % 8 == 0 && reinterpret_cast<uintptr_t>(bias) % 16 == 0;
    if (!bias && G % 4 == 0) {  // four scales per lane in one load
        if (exact)
            Q4_LAUNCH_MATVEC((k_gemm_q4<MS, kWGroup, false, NW, true>), grid, dim3(64 * NW), 0, stream, w, s, x, ldx,
                             y, ldy, part, M, N, G, sps, nullptr, nullptr, 0, 0);
        else
            Q4_LAUNCH_MATVEC((k_gemm_q4<MS, kWF16, false, NW, true>), grid, dim3(64 * NW), 0, stream, w, s, x, ldx,
                             y, ldy, part, M, N, G, sps, nullptr, nullptr, 0, 0);
    } else if (bias && G % 4 == 0)
        Q4_LAUNCH_MATVEC((k_gemm_q4<MS, kWGroup, true, NW, true>), grid, dim3(64 * NW), 0, stream, w, s, x, ldx,
                         y, ldy, part, M, N, G, sps, bias, xsum, gp, bvec);
    else if (bias)
        Q4_LAUNCH_MATVEC((k_gemm_q4<MS, kWGroup, true, NW, false>), grid, dim3(64 * NW), 0, stream, w, s, x, ldx,
                         y, ldy, part, M, N, G, sps, bias, xsum, gp, bvec);
    else if (exact)
        Q4_LAUNCH_MATVEC((k_gemm_q4<MS, kWGroup, false, NW, false>), grid, dim3(64 * NW), 0, stream, w, s, x, ldx,
                         y, ldy, part, M, N, G, sps, nullptr, nullptr, 0, 0);
    else
        Q4_LAUNCH_MATVEC((k_gemm_q4<MS, kWF16, false, NW, false>), grid, dim3(64 * NW), 0, stream, w, s, x, ldx,
                         y, ldy, part, M, N, G, sps, nullptr, nullptr, 0, 0);
    return check_launch("k_gemm_q4");
}

}  // namespace

namespace {
constexpr size_t kMaxPart = size_t(256) << 20;  // f32 partials of a split launch

// The launches of one prefill call: weight rows in chunks of nchunk, activation
// rows in chunks of mchunk, so that every buffer of a launch stays under 2^31
// bytes (whole 128-row tiles).
struct GemmChunks {
    int nchunk, mchunk;
    GemmChunks(int K, int64_t ldx)
    {
        const int64_t wrow_bytes = (int64_t)(K / 32) * 16;
        nchunk = (int)std::max<int64_t>(kBNMax, ((int64_t(1) << 31) / wrow_bytes) / kBNMax * kBNMax);
        mchunk = (int)std::max<int64_t>(
            128, ((int64_t(1) << 31) / (2 * std::max<int64_t>(ldx, 1)) - 1) / 128 * 128);
    }
};

// f32 partials and (affine) group sums of the launch over mm x nn
void gemm_scratch(int mm, int nn, int G, bool affine, size_t *part_b, size_t *xsum_b)
{
    const int GP = (G / 2 + 63) / 64 * 64;
    const GemmShape g = gemm_shape(mm, nn, G, kMaxPart, affine ? GP / 64 : 0);
    *part_b = g.splits > 1 ? (size_t)g.splits * mm * nn * sizeof(float) : 0;
    *xsum_b = affine ? (size_t)mm * 2 * GP * sizeof(uint16_t) : 0;
}
}  // namespace

size_t ws_gemm(int N, int K, int M, bool affine, int64_t ldx)
{
    const GemmChunks c(K, ldx);
    size_t need = 0;
    for (int n0 = 0; n0 < N; n0 += c.nchunk)
        for (int m0 = 0; m0 < M; m0 += c.mchunk) {
            size_t part_b, xsum_b;
            gemm_scratch(std::min(c.mchunk, M - m0), std::min(c.nchunk, N - n0), K / 32, affine,
                         &part_b, &xsum_b);
            if (part_b + xsum_b)
                need = std::max(need, kWsHeader + part_b + xsum_b);
        }
    return need;
}

q4_status launch_gemm(const uint32_t *W, const uint16_t *S, const uint16_t *X, int64_t ldx,
                      uint16_t *Y, int64_t ldy, int N, int K, int M, bool exact,
                      hipStream_t stream, const uint16_t *bias)
{
    const int G = K / 32;
    // affine: scales and biases per 64 codes; group sums padded to GP groups
    const int G64 = G / 2, GP = (G64 + 63) / 64 * 64;
    const int sg = bias ? G64 : G;  // scales per weight row
    const GemmChunks c(K, ldx);
    const int nchunk = c.nchunk, mchunk = c.mchunk;
    for (int n0 = 0; n0 < N; n0 += nchunk)
        for (int m0 = 0; m0 < M; m0 += mchunk) {
            const int nn = std::min(nchunk, N - n0), mm = std::min(mchunk, M - m0);
            const GemmShape g = gemm_shape(mm, nn, G, kMaxPart, bias ? GP / 64 : 0);
            const int BM = 16 * g.ms, BN = 32 * g.nw;
            const int64_t tiles = (int64_t)((mm + BM - 1) / BM) * ((nn + BN - 1) / BN);
            const dim3 grid((unsigned)tiles, (unsigned)g.splits);
            const uint4 *w = reinterpret_cast<const uint4 *>(W) + (size_t)n0 * G;
            const uint16_t *s = S + (size_t)n0 * sg, *x = X + (size_t)m0 * ldx;
            uint16_t *y = Y + (size_t)m0 * ldy + n0;
            float *part = nullptr;
            uint16_t *xsum = nullptr;
            size_t part_b, xsum_b;
            gemm_scratch(mm, nn, G, bias != nullptr, &part_b, &xsum_b);
            if (part_b + xsum_b) {
                // the largest launch of the call: the workspace is sized once
                char *ws = static_cast<char *>(
                    workspace(stream, ws_gemm(N, K, M, bias != nullptr, ldx)));
                if (!ws)
                    return workspace_status();
                part = part_b ? reinterpret_cast<float *>(ws + kWsHeader) : nullptr;
                xsum = xsum_b ? reinterpret_cast<uint16_t *>(ws + kWsHeader + part_b) : nullptr;
            }
            if (bias) {
                const int64_t cnt = (int64_t)mm * GP * 8;  // one thread per 8-value chunk
                hipLaunchKernelGGL(k_group_sums, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0,
                                   stream, x, ldx, xsum, mm, G64, GP);
                q4_status st = check_launch("k_group_sums");
                if (st != Q4_OK)
                    return st;
            }
            const uint16_t *bz = bias ? bias + (size_t)n0 * G64 : nullptr;
            q4_status st = g.ms == 4
                               ? launch_tiles<4, 4>(exact, grid, stream, w, s, x, ldx, y, ldy, part,
                                                    mm, nn, G, g.sps, bz, xsum, GP)
                               : launch_tiles<8, 8>(exact, grid, stream, w, s, x, ldx, y, ldy, part,
                                                    mm, nn, G, g.sps, bz, xsum, GP);
            if (st != Q4_OK)
                return st;
            if (g.splits > 1) {
                const int64_t total = (int64_t)mm * nn;
                const bool vec = nn % 4 == 0 && ldy % 4 == 0 &&
                                 reinterpret_cast<uintptr_t>(y) % 8 == 0;
                if (vec)
                    hipLaunchKernelGGL(k_gemm_combine<4>, dim3((unsigned)((total / 4 + 255) / 256)),
                                       dim3(256), 0, stream, part, g.splits, mm, nn, y, ldy);
                else
                    hipLaunchKernelGGL(k_gemm_combine<1>, dim3((unsigned)((total + 255) / 256)),
                                       dim3(256), 0, stream, part, g.splits, mm, nn, y, ldy);
                if ((st = check_launch("k_gemm_combine")) != Q4_OK)
                    return st;
            }
        }
    return Q4_OK;
}

}  // namespace q4
