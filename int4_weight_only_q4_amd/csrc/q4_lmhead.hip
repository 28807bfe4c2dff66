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
//  * M >= 2: the matrix-core matvec writes f32 logits, then k_argmax_partial
//    (many workgroups per row) and k_argmax_finish.
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
// chunk) cut at n] goes to cand[m * gridDim.x + b].
__global__ __launch_bounds__(kThreads) void k_argmax_partial(const float *__restrict__ v,
                                                             int64_t ld, int n, int chunk,
                                                             unsigned long long *__restrict__ cand)
{
    __shared__ unsigned long long red[kThreads / 64];
    const float *row = v + (int64_t)blockIdx.y * ld;
    const int i0 = blockIdx.x * chunk, i1 = min(n, i0 + chunk);
    unsigned long long k0 = 0, k1 = 0, k2 = 0, k3 = 0;
    int i = i0 + threadIdx.x;
    for (; i + 3 * kThreads < i1; i += 4 * kThreads) {  // four independent loads
        const float a = row[i], b = row[i + kThreads];
        const float c = row[i + 2 * kThreads], d = row[i + 3 * kThreads];
        k0 = umax64(k0, argmax_key(a, (uint32_t)i));
        k1 = umax64(k1, argmax_key(b, (uint32_t)(i + kThreads)));
        k2 = umax64(k2, argmax_key(c, (uint32_t)(i + 2 * kThreads)));
        k3 = umax64(k3, argmax_key(d, (uint32_t)(i + 3 * kThreads)));
    }
    for (; i < i1; i += kThreads)
        k0 = umax64(k0, argmax_key(row[i], (uint32_t)i));
    const unsigned long long m = block_max(umax64(umax64(k0, k1), umax64(k2, k3)), red);
    if (threadIdx.x == 0)
        cand[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = m;
}

// Row m = blockIdx.x: index[m] = the index of the largest of the nc keys
// cand[m * nc ...].
__global__ __launch_bounds__(kThreads) void k_argmax_finish(
    const unsigned long long *__restrict__ cand, int nc, int32_t *__restrict__ index)
{
    __shared__ unsigned long long red[kThreads / 64];
    const unsigned long long *c = cand + (int64_t)blockIdx.x * nc;
    unsigned long long k0 = 0, k1 = 0, k2 = 0, k3 = 0;
    int i = threadIdx.x;
    for (; i + 3 * kThreads < nc; i += 4 * kThreads) {
        k0 = umax64(k0, c[i]);
        k1 = umax64(k1, c[i + kThreads]);
        k2 = umax64(k2, c[i + 2 * kThreads]);
        k3 = umax64(k3, c[i + 3 * kThreads]);
    }
    for (; i < nc; i += kThreads)
        k0 = umax64(k0, c[i]);
    const unsigned long long m = block_max(umax64(umax64(k0, k1), umax64(k2, k3)), red);
    if (threadIdx.x == 0)
        index[blockIdx.x] = argmax_index(m);
}

q4_status finish(const unsigned long long *cand, int nc, int M, int32_t *index,
                 hipStream_t stream)
{
    hipLaunchKernelGGL(k_argmax_finish, dim3(M), dim3(kThreads), 0, stream, cand, nc, index);
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
    return launch_gemv_mfma(W, S, x, ldx, nullptr, y, ldy, N, K, M, stream);
}

q4_status launch_argmax(const float *v, int64_t ld, int N, int M, int32_t *index,
                        hipStream_t stream)
{
    const int blocks = std::min(kMaxPartial, (N + kChunk - 1) / kChunk);
    const int chunk = (N + blocks - 1) / blocks;
    char *ws = static_cast<char *>(
        workspace(stream, kWsHeader + (size_t)M * blocks * sizeof(unsigned long long)));
    if (!ws)
        return Q4_EHIP;
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
    if (M > 1) {
        q4_status st = launch_gemv_mfma(W, S, x, ldx, nullptr, logits, ldl, N, K, M, stream);
        if (st != Q4_OK)
            return st;
        return launch_argmax(logits, ldl, N, M, tokens, stream);
    }
    const int blocks = matvec_blocks(N, K);
    if (blocks <= 0)
        return fail(Q4_ERANGE, "no matvec configuration for K = %d", K);
    char *ws = static_cast<char *>(
        workspace(stream, kWsHeader + (size_t)blocks * sizeof(unsigned long long)));
    if (!ws)
        return Q4_EHIP;
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
