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
// weight rows, and MS 16-byte pieces of the activation tile (piece q: row
// (t + 256 q) / 16, eight values (t % 16) of the step). Rows past N or M read 0.
template <int MS>
struct Offsets {
    uint32_t w[2], s[2], x[MS];
};

// One step's loaded data of a thread.
template <int MS>
struct StepLoads {
    u32x4 w[2];
    uint32_t s[2];
    u32x4 x[MS];
};

template <int MS>
__device__ __forceinline__ void load_step(StepLoads<MS> &L, const Bufs &B, const Offsets<MS> &O,
                                          int st)
{
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        L.w[ns] = __builtin_amdgcn_raw_buffer_load_b128(B.w, O.w[ns], st * 64, 0);
        L.s[ns] = __builtin_amdgcn_raw_buffer_load_b16(B.s, O.s[ns], st * 8, 0);
    }
#pragma unroll
    for (int q = 0; q < MS; ++q)
        L.x[q] = __builtin_amdgcn_raw_buffer_load_b128(B.x, O.x[q], st * 256, 0);
}

// Weight words and scales of a step, rearranged for the matrix core:
// wt[ns][tt] is this lane row's word of group tt, s2[ns][tt] that group's
// scale (both halves). LAST: groups past K get scale 0.
struct StepWeights {
    uint32_t wt[2][4];
    half2v s2[2][4];
};

template <int MS, bool LAST>
__device__ __forceinline__ void prepare(StepWeights &P, const StepLoads<MS> &L, int gs, int kb,
                                        int G)
{
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        P.wt[ns][0] = L.w[ns].x;
        P.wt[ns][1] = L.w[ns].y;
        P.wt[ns][2] = L.w[ns].z;
        P.wt[ns][3] = L.w[ns].w;
        transpose_rows(P.wt[ns]);
        uint32_t s = L.s[ns];
        if (LAST && gs + kb >= G)
            s = 0;
        uint32_t sc[4];
        broadcast_rows(s, sc);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
            P.s2[ns][tt] = __builtin_bit_cast(half2v, sc[tt] * 0x10001u);
    }
}

// Stores a step's activation pieces into an LDS buffer in pair order. LAST:
// values past K are zero.
template <int MS, bool LAST>
__device__ __forceinline__ void stage(_Float16 *buf, const StepLoads<MS> &L, int gs, int G, int t)
{
#pragma unroll
    for (int q = 0; q < MS; ++q) {
        const int c = t + 256 * q;
        u32x4 v = pair_order(L.x[q]);
        if (LAST && gs * 32 + 8 * (c & 15) >= G * 32)
            v = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(buf + (c >> 4) * kAStride + 8 * (c & 15)) = v;
    }
}

template <int MS, bool EXACT>
__device__ __forceinline__ void multiply(floatx4 (&acc)[MS][2], const _Float16 *cur,
                                         const StepWeights &P, int n, int kb)
{
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        half8 a[MS], bh[2], bl[2];
        __builtin_amdgcn_iglp_opt(1);  // interleave the matrix-core and LDS work
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
                acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ms], bh[ns], acc[ms][ns],
                                                                     0, 0, 0);
        if (EXACT) {
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int ns = 0; ns < 2; ++ns)
                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ms], bl[ns],
                                                                         acc[ms][ns], 0, 0, 0);
        }
    }
}

// Grid: one workgroup per (16 MS-row activation tile, 128-row weight tile),
// 256 threads; wave w owns weight rows [32 w, 32 w + 32) of the tile and all
// MS 16-row activation tiles. Buffer sizes below 2^31 bytes (the launcher
// splits larger problems).
template <int MS, bool EXACT>
__global__ __launch_bounds__(256, MS == 8 ? 2 : 3) void k_gemm_q4(
    const uint4 *__restrict__ W, const uint16_t *__restrict__ S, const uint16_t *__restrict__ X,
    int64_t ldx, uint16_t *__restrict__ Y, int64_t ldy, float *__restrict__ part, int M, int N,
    int G, int sps)
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

    Bufs B;
    B.w = rsrc(W, (uint32_t)N * (uint32_t)G * 16u);
    B.s = rsrc(S, (uint32_t)N * (uint32_t)G * 2u);
    B.x = rsrc(X, (uint32_t)(((int64_t)(M - 1) * ldx + G * 32) * 2));
    Offsets<MS> O;
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        const int row = n0 + 16 * ns + n;
        O.w[ns] = row < N ? (uint32_t)(row * G + kb) * 16u : kOut;
        O.s[ns] = row < N ? (uint32_t)(row * G + kb) * 2u : kOut;
    }
#pragma unroll
    for (int q = 0; q < MS; ++q) {
        const int c = t + 256 * q, row = m0 + (c >> 4);
        O.x[q] = row < M ? (uint32_t)((row * ldx + 8 * (c & 15)) * 2) : kOut;
    }

    floatx4 acc[MS][2];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
            acc[ms][ns] = floatx4{0.f, 0.f, 0.f, 0.f};

    // step st: groups [4 st, 4 st + 4); its loads are issued one step ahead.
    // K split z (grid y) takes the steps [z sps, min((z + 1) sps, steps)).
    const int steps = (G + 3) / 4, z = blockIdx.y;
    const int st0 = z * sps, st1 = min(steps, st0 + sps);
    StepLoads<MS> L;
    StepWeights P;
    load_step<MS>(L, B, O, st0);
    for (int st = st0; st < st1 - 1; ++st) {
        stage<MS, false>(xs[st & 1], L, 4 * st, G, t);
        prepare<MS, false>(P, L, 4 * st, kb, G);
        load_step<MS>(L, B, O, st + 1);
        __syncthreads();  // the tile is staged; the other buffer was last read before this
        multiply<MS, EXACT>(acc, xs[st & 1], P, n, kb);
    }
    {
        const int st = st1 - 1;  // groups past K only in the last step of the last split
        stage<MS, true>(xs[st & 1], L, 4 * st, G, t);
        prepare<MS, true>(P, L, 4 * st, kb, G);
        __syncthreads();
        multiply<MS, EXACT>(acc, xs[st & 1], P, n, kb);
    }

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

// Launch shape of one chunk: activation rows per workgroup (16 MS) and the
// number of K splits. 128-row tiles run two workgroups per CU, 64-row tiles
// three at about 0.74 of the time per tile; the shape with fewer estimated
// tile-rounds wins. A grid that fills fewer than half the workgroup slots
// splits K (at least four steps per split, at most kMaxSplits) into f32
// partials that k_gemm_combine sums in split order.
struct GemmShape {
    int ms, splits, sps;
};

GemmShape gemm_shape(int M, int N, int G, size_t max_part_bytes)
{
    const int cus = cu_count(), nt = (N + kBN - 1) / kBN, steps = (G + 3) / 4;
    const int64_t t8 = (int64_t)((M + 127) / 128) * nt, t4 = (int64_t)((M + 63) / 64) * nt;
    const double r8 = (double)((t8 + 2 * cus - 1) / (2 * cus));
    const double r4 = 0.74 * (double)((t4 + 3 * cus - 1) / (3 * cus));
    GemmShape g;
    g.ms = r4 < r8 ? 4 : 8;
    const int64_t tiles = g.ms == 4 ? t4 : t8, slots = (g.ms == 4 ? 3 : 2) * (int64_t)cus;
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

template <int MS>
q4_status launch_tiles(bool exact, dim3 grid, hipStream_t stream, const uint4 *w, const uint16_t *s,
                       const uint16_t *x, int64_t ldx, uint16_t *y, int64_t ldy, float *part,
                       int M, int N, int G, int sps)
{
    if (exact)
        Q4_LAUNCH_MATVEC((k_gemm_q4<MS, true>), grid, dim3(256), 0, stream, w, s, x, ldx, y, ldy,
                         part, M, N, G, sps);
    else
        Q4_LAUNCH_MATVEC((k_gemm_q4<MS, false>), grid, dim3(256), 0, stream, w, s, x, ldx, y,
                         ldy, part, M, N, G, sps);
    return check_launch("k_gemm_q4");
}

}  // namespace

q4_status launch_gemm(const uint32_t *W, const uint16_t *S, const uint16_t *X, int64_t ldx,
                      uint16_t *Y, int64_t ldy, int N, int K, int M, bool exact,
                      hipStream_t stream)
{
    constexpr size_t kMaxPart = size_t(256) << 20;  // f32 partials of a split launch
    const int G = K / 32;
    // every buffer of a launch under 2^31 bytes: chunks of weight rows (whole
    // 128-row tiles) and of activation rows (whole 128-row tiles)
    const int64_t wrow_bytes = (int64_t)G * 16;
    const int nchunk = (int)std::max<int64_t>(kBN, ((int64_t(1) << 31) / wrow_bytes) / kBN * kBN);
    const int mchunk = (int)std::max<int64_t>(
        128, ((int64_t(1) << 31) / (2 * std::max<int64_t>(ldx, 1)) - 1) / 128 * 128);
    for (int n0 = 0; n0 < N; n0 += nchunk)
        for (int m0 = 0; m0 < M; m0 += mchunk) {
            const int nn = std::min(nchunk, N - n0), mm = std::min(mchunk, M - m0);
            const GemmShape g = gemm_shape(mm, nn, G, kMaxPart);
            const int BM = 16 * g.ms;
            const int64_t tiles = (int64_t)((mm + BM - 1) / BM) * ((nn + kBN - 1) / kBN);
            const dim3 grid((unsigned)tiles, (unsigned)g.splits);
            float *part = nullptr;
            if (g.splits > 1) {
                char *ws = static_cast<char *>(
                    workspace(stream, kWsHeader + (size_t)g.splits * mm * nn * sizeof(float)));
                if (!ws)
                    return Q4_EHIP;
                part = reinterpret_cast<float *>(ws + kWsHeader);
            }
            const uint4 *w = reinterpret_cast<const uint4 *>(W) + (size_t)n0 * G;
            const uint16_t *s = S + (size_t)n0 * G, *x = X + (size_t)m0 * ldx;
            uint16_t *y = Y + (size_t)m0 * ldy + n0;
            q4_status st = g.ms == 4
                               ? launch_tiles<4>(exact, grid, stream, w, s, x, ldx, y, ldy, part,
                                                 mm, nn, G, g.sps)
                               : launch_tiles<8>(exact, grid, stream, w, s, x, ldx, y, ldy, part,
                                                 mm, nn, G, g.sps);
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
