// LM head and greedy sampling for gfx950.
//
// After the last layer the LM-head matmul writes the logits and the next token
// is their argmax (Zero TVM Documentation, "Decode loop"; shader 10, "Argmax
// Sampler"). The LM head is the f32-output variant of the int4 matmul, kept
// in f32 so the argmax is not decided by f16 rounding (RESEARCH.md, "Why Fewer
// Dispatches Matter", the per-decode dispatch table and the note below it).
//
// The pages reduce the 32,064 logits in one workgroup after the matmul. Here:
//  * M = 1: the matvec's own epilogue (k_gemv, LOGITS) writes the f32 logits
//    and one candidate per workgroup, the largest (value, index) key of its
//    rows; k_argmax_finish reduces the candidates in one workgroup. No logit
//    is read back and no atomics are used, so the token is deterministic.
//  * M = 2..4 on the few-row kernel: the f32 logits, then k_argmax_partial
//    and k_argmax_finish;
//  * M >= 2 on the workgroup-reduced matrix-core kernel (k_gemv_mma): as it
//    stores a tile it keeps each lane's largest key per row; at its end the
//    workgroup's per-row best (an LDS maximum, order-independent) goes to a
//    candidate array that k_argmax_finish reduces;
//  * otherwise the matrix-core matvec's split-K partials are summed by
//    k_combine_argmax, which writes the f32 logits and the first argmax pass's
//    candidates (k_argmax_partial when K is not split), then k_argmax_finish.
// Ties go to the smallest index, -0 equals +0 and a NaN ranks above every
// number (argmax_key); the pages leave these open.
#include <algorithm>

#include "q4_common.h"

namespace q4 {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 4096;      // logits per workgroup of k_argmax_partial
constexpr int kMaxPartial = 1024; // workgroups per row at most

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b)
{
    return a > b ? a : b;
}

// Block-wide maximum over 256 threads; `red` is kThreads / 64 keys of LDS.
__device__ __forceinline__ unsigned long long block_max(unsigned long long k,
                                                        unsigned long long *red)
{
    k = wave_max_u64(k);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = k;
    __syncthreads();
    unsigned long long m = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w)
        m = umax64(m, red[w]);
    return m;
}

// Row m = blockIdx.y: the largest key over v[m * ld + [b * chunk, (b + 1) *
// chunk) cut at n] goes to cand[m * gridDim.x + b]. Loads are issued kPer at
// a time and clamped to the last element of the range: a repeated element
// repeats its key, which leaves the maximum unchanged.
constexpr int kPer = 16;
__global__ __launch_bounds__(kThreads) void k_argmax_partial(const float *__restrict__ v,
                                                             int64_t ld, int n, int chunk,
                                                             unsigned long long *__restrict__ cand)
{
    __shared__ unsigned long long red[kThreads / 64];
    const float *row = v + (int64_t)blockIdx.y * ld;
    const int i0 = blockIdx.x * chunk, i1 = min(n, i0 + chunk);
    unsigned long long k = 0;
    if (i0 < i1) {
        for (int base = i0; base < i1; base += kPer * kThreads) {
            float f[kPer];
            int idx[kPer];
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                idx[u] = min(base + (int)threadIdx.x + u * kThreads, i1 - 1);
                f[u] = row[idx[u]];
            }
#pragma unroll
            for (int u = 0; u < kPer; ++u)
                k = umax64(k, argmax_key(f[u], (uint32_t)idx[u]));
        }
    }
    const unsigned long long m = block_max(k, red);
    if (threadIdx.x == 0)
        cand[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = m;
}

// Split-K matrix-core results: block (b, m) sums the KS f32 partials of row m,
// columns [b * kCombineChunk, (b + 1) * kCombineChunk) cut at n, in split
// order, writes them to yf[m * ldy ...] and hands the largest key to
// cand[m * gridDim.x + b]. Each thread's kCombinePer sums are independent, so
// their loads of one split are issued together.
constexpr int kCombinePer = 2;
constexpr int kCombineChunk = kCombinePer * kThreads;
__global__ __launch_bounds__(kThreads) void k_combine_argmax(const float *__restrict__ part,
                                                             int KS, int M, int n,
                                                             float *__restrict__ yf, int64_t ldy,
                                                             unsigned long long *__restrict__ cand)
{
    __shared__ unsigned long long red[kThreads / 64];
    const int mr = blockIdx.y;
    const int i0 = blockIdx.x * kCombineChunk;
    float s[kCombinePer];
    int idx[kCombinePer];
#pragma unroll
    for (int u = 0; u < kCombinePer; ++u) {
        idx[u] = min(i0 + (int)threadIdx.x + u * kThreads, n - 1);  // clamped: see above
        s[u] = 0.f;
    }
    for (int ks = 0; ks < KS; ++ks) {
        const float *p = part + ((size_t)ks * M + mr) * n;
#pragma unroll
        for (int u = 0; u < kCombinePer; ++u)
            s[u] += p[idx[u]];
    }
    unsigned long long k = 0;
#pragma unroll
    for (int u = 0; u < kCombinePer; ++u) {
        if (i0 + (int)threadIdx.x + u * kThreads < n)
            yf[mr * ldy + idx[u]] = s[u];
        k = umax64(k, argmax_key(s[u], (uint32_t)idx[u]));
    }
    const unsigned long long m = block_max(k, red);
    if (threadIdx.x == 0)
        cand[(int64_t)mr * gridDim.x + blockIdx.x] = m;
}

// Row m = blockIdx.x: index[m] = the index of the largest of the nc keys
// cand[m * nc ...] (clamped loads, as above).
constexpr int kFinishThreads = 1024;
__global__ __launch_bounds__(kFinishThreads) void k_argmax_finish(
    const unsigned long long *__restrict__ cand, int nc, int32_t *__restrict__ index)
{
    __shared__ unsigned long long red[kFinishThreads / 64];
    const unsigned long long *c = cand + (int64_t)blockIdx.x * nc;
    unsigned long long k = 0;
    for (int base = 0; base < nc; base += kPer * kFinishThreads) {
        unsigned long long v[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u)
            v[u] = c[min(base + (int)threadIdx.x + u * kFinishThreads, nc - 1)];
#pragma unroll
        for (int u = 0; u < kPer; ++u)
            k = umax64(k, v[u]);
    }
    k = wave_max_u64(k);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = k;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long m = red[0];
        for (int w = 1; w < kFinishThreads / 64; ++w)
            m = umax64(m, red[w]);
        index[blockIdx.x] = argmax_index(m);
    }
}

q4_status finish(const unsigned long long *cand, int nc, int M, int32_t *index,
                 hipStream_t stream)
{
    hipLaunchKernelGGL(k_argmax_finish, dim3(M), dim3(kFinishThreads), 0, stream, cand, nc,
                       index);
    return check_launch("k_argmax_finish");
}

}  // namespace

q4_status launch_gemv_f32(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                          float *y, int64_t ldy, int N, int K, int M, hipStream_t stream)
{
    if (M == 1) {
        GemvOp op;
        op.W = W;
        op.S = S;
        op.N = N;
        op.K = K;
        op.x = x;
        op.epi = GemvOp::LOGITS;
        op.yf = y;
        return launch_gemv_op(op, stream);
    }
    if (gemv_rows_fits(M, K, N))  // a few rows: the single-row arithmetic per row
        return launch_gemv_rows(W, S, x, ldx, nullptr, ldy, N, K, M, stream, nullptr, y);
    return launch_gemv_mfma(W, S, x, ldx, nullptr, y, ldy, N, K, M, stream);
}

namespace {
// Workgroups per row of the two-pass argmax, and the logits each covers
void partial_grid(int N, int *blocks, int *chunk)
{
    *blocks = std::min(kMaxPartial, (N + kChunk - 1) / kChunk);
    *chunk = (N + *blocks - 1) / *blocks;
}
}  // namespace

size_t ws_argmax(int N, int M)
{
    int blocks, chunk;
    partial_grid(N, &blocks, &chunk);
    return kWsHeader + (size_t)M * blocks * sizeof(unsigned long long);
}

namespace {
// M >= 2 rows on the matrix cores: argmax candidates per (row, block) and the
// K-split partials
int lm_head_mfma_blocks(int N, int K)
{
    int blocks, chunk;
    partial_grid(N, &blocks, &chunk);
    if (mfma_splits(K) > 1)
        blocks = (N + kCombineChunk - 1) / kCombineChunk;
    return blocks;
}
size_t lm_head_cand_bytes(int N, int K, int M)
{
    return ((size_t)M * lm_head_mfma_blocks(N, K) * sizeof(unsigned long long) + 255) / 256 * 256;
}
}  // namespace

size_t ws_lm_head(int N, int K, int M)
{
    if (M > 1 && gemv_rows_fits(M, K, N))
        return ws_argmax(N, M);
    if (M > 1 && mma_fits(N, K, M))
        return kWsHeader + (size_t)M * mma_blocks(N) * sizeof(unsigned long long);
    if (M > 1)
        return kWsHeader + lm_head_cand_bytes(N, K, M) + mfma_part_bytes(N, K);
    return kWsHeader + (size_t)matvec_blocks(N, K) * sizeof(unsigned long long);
}

q4_status launch_argmax(const float *v, int64_t ld, int N, int M, int32_t *index,
                        hipStream_t stream)
{
    int blocks, chunk;
    partial_grid(N, &blocks, &chunk);
    char *ws = static_cast<char *>(workspace(stream, ws_argmax(N, M)));
    if (!ws)
        return workspace_status();
    auto *cand = reinterpret_cast<unsigned long long *>(ws + kWsHeader);
    hipLaunchKernelGGL(k_argmax_partial, dim3(blocks, M), dim3(kThreads), 0, stream, v, ld, N,
                       chunk, cand);
    q4_status st = check_launch("k_argmax_partial");
    if (st != Q4_OK)
        return st;
    return finish(cand, blocks, M, index, stream);
}

q4_status launch_lm_head_argmax(const uint32_t *W, const uint16_t *S, const uint16_t *x,
                                int64_t ldx, float *logits, int64_t ldl, int32_t *tokens, int N,
                                int K, int M, hipStream_t stream)
{
    if (M > 1 && gemv_rows_fits(M, K, N)) {
        // a few rows: the f32 logits by M single-row matvecs, then the argmax
        q4_status st = launch_gemv_f32(W, S, x, ldx, logits, ldl, N, K, M, stream);
        if (st != Q4_OK)
            return st;
        return launch_argmax(logits, ldl, N, M, tokens, stream);
    }
    if (M > 1 && mma_fits(N, K, M)) {
        // the workgroup-reduced matrix-core kernel writes the f32 logits and
        // each workgroup's best key per row; one finish reduces them
        char *ws = static_cast<char *>(workspace(stream, ws_lm_head(N, K, M)));
        if (!ws)
            return workspace_status();
        auto *cand = reinterpret_cast<unsigned long long *>(ws + kWsHeader);
        q4_status st = launch_gemv_mma(W, S, x, ldx, nullptr, logits, ldl, N, K, M, stream, cand);
        if (st != Q4_OK)
            return st;
        return finish(cand, mma_blocks(N), M, tokens, stream);
    }
    if (M > 1) {
        // per launch of up to 16 rows: the matrix-core partials, then their sum
        // in split order fused with the first argmax pass (or, without a K
        // split, the first pass over the written logits); one finish for all
        const int KS = mfma_splits(K);
        int blocks, chunk;
        partial_grid(N, &blocks, &chunk);
        blocks = lm_head_mfma_blocks(N, K);
        const size_t cand_b = lm_head_cand_bytes(N, K, M);
        char *ws = static_cast<char *>(workspace(stream, ws_lm_head(N, K, M)));
        if (!ws)
            return workspace_status();
        auto *cand = reinterpret_cast<unsigned long long *>(ws + kWsHeader);
        float *part = reinterpret_cast<float *>(ws + kWsHeader + cand_b);
        for (int m0 = 0; m0 < M; m0 += 16) {
            const int mt = std::min(16, M - m0);
            q4_status st = launch_mfma_rows(W, S, x + m0 * ldx, ldx, nullptr, logits + m0 * ldl,
                                            ldl, N, K, mt, KS > 1 ? part : nullptr, stream);
            if (st != Q4_OK)
                return st;
            if (KS > 1) {
                hipLaunchKernelGGL(k_combine_argmax, dim3(blocks, mt), dim3(kThreads), 0, stream,
                                   part, KS, mt, N, logits + m0 * ldl, ldl,
                                   cand + (size_t)m0 * blocks);
                st = check_launch("k_combine_argmax");
            } else {
                hipLaunchKernelGGL(k_argmax_partial, dim3(blocks, mt), dim3(kThreads), 0, stream,
                                   logits + m0 * ldl, ldl, N, chunk, cand + (size_t)m0 * blocks);
                st = check_launch("k_argmax_partial");
            }
            if (st != Q4_OK)
                return st;
        }
        return finish(cand, blocks, M, tokens, stream);
    }
    const int blocks = matvec_blocks(N, K);
    if (blocks <= 0)
        return fail(Q4_ERANGE, "no matvec configuration for K = %d", K);
    char *ws = static_cast<char *>(workspace(stream, ws_lm_head(N, K, 1)));
    if (!ws)
        return workspace_status();
    GemvOp op;
    op.W = W;
    op.S = S;
    op.N = N;
    op.K = K;
    op.x = x;
    op.epi = GemvOp::LOGITS;
    op.yf = logits;
    op.cand = reinterpret_cast<unsigned long long *>(ws + kWsHeader);
    q4_status st = launch_gemv_op(op, stream);
    if (st != Q4_OK)
        return st;
    return finish(op.cand, blocks, 1, tokens, stream);
}

}  // namespace q4
