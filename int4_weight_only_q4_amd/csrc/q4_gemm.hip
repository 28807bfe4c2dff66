// Prefill (many-token) int4 x f16 matmul on the gfx950 matrix cores.
//
// What is computed is the batched matmul of the q4f16_1 format (Zero TVM
// Documentation, "Q4F16 quantization format"; BENCH.md, "Tiled batched GEMM"
// and "Subgroup-matrix GEMM graduated"): Y[m][n] = f16( sum_k (q[n][k] - 7) *
// s[n][k/32] * X[m][k] ), f32 accumulation, for any number M of activation
// rows. The decode kernels stream the weights once for at most 16 rows; here
// each weight tile is dequantised once per 64 rows:
//  * workgroup tile: 64 activation rows x 128 weight rows; wave w owns weight
//    rows [32 w, 32 w + 32) of the tile (two 16-row matrix-core tiles) and all
//    four 16-row activation tiles, so each dequantised weight feeds four MFMAs;
//  * the weights enter the matrix core exactly: w = (q - 7) * s is split into
//    binary16 hi = f16(w) and lo = w - hi (exact: the product of a 4-bit
//    integer and a binary16 scale has at most 15 significant bits), and both
//    are multiplied with f32 accumulation, so the accumulator runs over all of
//    K with no per-group arithmetic on the results (the page's matrix-unit
//    kernel rounds the staged weights to f16 instead);
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
#include <algorithm>

#include "q4_dequant.h"

namespace q4 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBN = 128;               // weight rows per workgroup (32 per wave)
constexpr int kStepK = 128;            // K values per step (four groups)
constexpr int kAStride = kStepK + 8;   // staged row in halves (16 bytes of padding)
constexpr int kXcds = 8;

__device__ __forceinline__ void swap16(uint32_t &a, uint32_t &b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

__device__ __forceinline__ void swap32(uint32_t &a, uint32_t &b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}

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

// The 8 weights of word w, w = (q - 7) * s, in the pair order (e0, e4) (e1,
// e5) (e2, e6) (e3, e7): EXACT gives binary16 hi = f16(w) and lo = w - hi,
// otherwise hi = f16(w) alone. A nibble in mantissa bits 0..3 under exponent
// field 25 is the binary16 1024 + q; in bits 4..7 under exponent field 21 it
// is 64 + q, so one shift of the word by 8 reaches all four pairs.
template <bool EXACT>
__device__ __forceinline__ void weights_of(uint32_t w, half2v s2, half8 &hi, half8 &lo)
{
    const half2v c1031 = {(_Float16)-1031.0f, (_Float16)-1031.0f};
    const half2v c71 = {(_Float16)-71.0f, (_Float16)-71.0f};
    const uint32_t w8 = w >> 8;
    uint32_t b[4];
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(b[0]) : "v"(0x000F000Fu), "v"(w), "s"(0x64006400u));
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(b[1]) : "v"(0x00F000F0u), "v"(w), "s"(0x54005400u));
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(b[2]) : "v"(0x000F000Fu), "v"(w8), "s"(0x64006400u));
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(b[3]) : "v"(0x00F000F0u), "v"(w8), "s"(0x54005400u));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2v q = __builtin_bit_cast(half2v, b[i]) + ((i & 1) ? c71 : c1031);  // exact q - 7
        const half2v h = q * s2;
        hi[2 * i] = h[0];
        hi[2 * i + 1] = h[1];
        if (EXACT) {
            const half2v r = __builtin_elementwise_fma(q, s2, -h);
            lo[2 * i] = r[0];
            lo[2 * i + 1] = r[1];
        }
    }
}

// A 16-byte chunk of 8 activations in the pair order of weights_of.
__device__ __forceinline__ u32x4 pair_order(u32x4 v)
{
    return u32x4{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                 __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                 __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                 __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
}

// One step's global loads of a thread: its lane's word group of the wave's
// two weight rows and their scales, and MS 16-byte pieces of the activation tile.
template <int MS>
struct StepLoads {
    uint4 w[2];
    uint32_t s[2];
    u32x4 x[MS];
};

template <int MS>
__device__ __forceinline__ void load_step(StepLoads<MS> &L, const uint4 *__restrict__ W,
                                          const uint16_t *__restrict__ S,
                                          const uint16_t *__restrict__ X, int64_t ldx,
                                          const size_t (&wrow)[2], int m0, int M, int G, int gs,
                                          int kb, int t)
{
    const int gi = min(gs + kb, G - 1);
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        L.w[ns] = load_weights(W + wrow[ns] + gi);
        L.s[ns] = load_scale(S + wrow[ns] + gi);
    }
#pragma unroll
    for (int q = 0; q < MS; ++q) {
        const int c = t + 256 * q;  // piece c: row c / 16, eight values c % 16 of the step
        const int mr = min(m0 + (c >> 4), M - 1);
        const int kk = min(gs * 32 + 8 * (c & 15), G * 32 - 8);
        L.x[q] = *reinterpret_cast<const u32x4 *>(X + (int64_t)mr * ldx + kk);
    }
}

// Weight words and scales of a step, rearranged for the matrix core:
// wt[ns][tt] is this lane row's word of group tt, s2[ns][tt] that group's
// scale (both halves).
struct StepWeights {
    uint32_t wt[2][4];
    half2v s2[2][4];
};

template <int MS>
__device__ __forceinline__ void prepare(StepWeights &P, const StepLoads<MS> &L, bool tail,
                                        int gs, int kb, int G)
{
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        P.wt[ns][0] = L.w[ns].x;
        P.wt[ns][1] = L.w[ns].y;
        P.wt[ns][2] = L.w[ns].z;
        P.wt[ns][3] = L.w[ns].w;
        transpose_rows(P.wt[ns]);
        uint32_t s = L.s[ns];
        if (tail && gs + kb >= G)
            s = 0;  // a group past K gets scale 0
        uint32_t sc[4];
        broadcast_rows(s, sc);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
            P.s2[ns][tt] = __builtin_bit_cast(half2v, sc[tt] * 0x10001u);
    }
}

// Stores a step's activation pieces into an LDS buffer (pair order; values
// past K zero in the tail step).
template <int MS>
__device__ __forceinline__ void stage(_Float16 *buf, const StepLoads<MS> &L, bool tail, int gs,
                                      int G, int t)
{
#pragma unroll
    for (int q = 0; q < MS; ++q) {
        const int c = t + 256 * q;
        u32x4 v = pair_order(L.x[q]);
        if (tail && gs * 32 + 8 * (c & 15) >= G * 32)
            v = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(buf + (c >> 4) * kAStride + 8 * (c & 15)) = v;
    }
}

// Grid: one workgroup per (16 MS-row activation tile, 128-row weight tile),
// 256 threads; wave w owns weight rows [32 w, 32 w + 32) of the tile and all
// MS 16-row activation tiles.
template <int MS, bool EXACT>
__global__ __launch_bounds__(256, 2) void k_gemm_q4(const uint4 *__restrict__ W,
                                                    const uint16_t *__restrict__ S,
                                                    const uint16_t *__restrict__ X, int64_t ldx,
                                                    uint16_t *__restrict__ Y, int64_t ldy, int M,
                                                    int N, int G)
{
    constexpr int BM = 16 * MS;
    __shared__ _Float16 xs[2][BM * kAStride];
    const int t = threadIdx.x, l = t & 63, wave = t >> 6;
    const int n = l & 15, kb = l >> 4;

    // XCD-aware tile order: workgroup b runs on XCD b % 8; XCD x takes the
    // contiguous tile range [start(x), start(x) + count(x)), activation tile fastest
    const int mtiles = (M + BM - 1) / BM, ntiles = (N + kBN - 1) / kBN;
    const int total = mtiles * ntiles, per = total / kXcds, rem = total % kXcds;
    const int b = blockIdx.x, x = b % kXcds;
    const int r = x * per + min(x, rem) + b / kXcds;
    const int m0 = (r % mtiles) * BM, n0 = (r / mtiles) * kBN + 32 * wave;

    size_t wrow[2];
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
        wrow[ns] = (size_t)min(n0 + 16 * ns + n, N - 1) * G;
    floatx4 acc[MS][2];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
            acc[ms][ns] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int steps = (G + 3) / 4;
    StepLoads<MS> L;
    StepWeights P;
    load_step<MS>(L, W, S, X, ldx, wrow, m0, M, G, 0, kb, t);
    stage<MS>(xs[0], L, G < 4, 0, G, t);
    prepare<MS>(P, L, G < 4, 0, kb, G);
    load_step<MS>(L, W, S, X, ldx, wrow, m0, M, G, min(4, 4 * (steps - 1)), kb, t);
    __syncthreads();
    for (int st = 0; st < steps; ++st) {
        const _Float16 *cur = xs[st & 1];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            half8 a[MS], bh[2], bl[2];
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
                a[ms] = *reinterpret_cast<const half8 *>(cur + (16 * ms + n) * kAStride + 8 * kb +
                                                         32 * tt);
#pragma unroll
            for (int ns = 0; ns < 2; ++ns)
                weights_of<EXACT>(P.wt[ns][tt], P.s2[ns][tt], bh[ns], bl[ns]);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int ns = 0; ns < 2; ++ns)
                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ms], bh[ns],
                                                                         acc[ms][ns], 0, 0, 0);
            if (EXACT) {
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                    for (int ns = 0; ns < 2; ++ns)
                        acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            a[ms], bl[ns], acc[ms][ns], 0, 0, 0);
            }
        }
        // the next step: its activation tile into the other buffer (last read
        // before the previous barrier), its weights rearranged, and the loads
        // of the step after it (the last steps re-read the final one, unused)
        const int gn = 4 * min(st + 1, steps - 1);
        const bool tail = gn + 4 > G;
        stage<MS>(xs[(st + 1) & 1], L, tail, gn, G, t);
        prepare<MS>(P, L, tail, gn, kb, G);
        load_step<MS>(L, W, S, X, ldx, wrow, m0, M, G, 4 * min(st + 2, steps - 1), kb, t);
        __syncthreads();
    }

    // lane (n, kb) holds D[4 kb + i][n] of each (activation, weight) tile
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            const int col = n0 + 16 * ns + n;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + 16 * ms + 4 * kb + i;
                if (row < M && col < N)
                    Y[(int64_t)row * ldy + col] = f2h(acc[ms][ns][i]);
            }
        }
}

}  // namespace

q4_status launch_gemm(const uint32_t *W, const uint16_t *S, const uint16_t *X, int64_t ldx,
                      uint16_t *Y, int64_t ldy, int N, int K, int M, bool exact,
                      hipStream_t stream)
{
    constexpr int MS = 8;
    const int64_t tiles = (int64_t)((M + 16 * MS - 1) / (16 * MS)) * ((N + kBN - 1) / kBN);
    if (exact)
        Q4_LAUNCH_MATVEC((k_gemm_q4<MS, true>), dim3((unsigned)tiles), dim3(256), 0, stream,
                         reinterpret_cast<const uint4 *>(W), S, X, ldx, Y, ldy, M, N, K / 32);
    else
        Q4_LAUNCH_MATVEC((k_gemm_q4<MS, false>), dim3((unsigned)tiles), dim3(256), 0, stream,
                         reinterpret_cast<const uint4 *>(W), S, X, ldx, Y, ldy, M, N, K / 32);
    return check_launch("k_gemm_q4");
}

}  // namespace q4
