// RoPE + paged-KV append and decode attention for gfx950.
//
// What is computed follows the Zero TVM Documentation: "KV cache" (16-slot
// pages behind a page table), shader 3 (the QKV matmul with RoPE of Q and K
// and the K/V write fused, decode), shader 4 (paged attention with an online
// softmax, one workgroup per head), shaders 8 and 9 (the unfused KV append and
// RoPE), and BENCH.md's split-K attention (the positions split over several
// workgroups, then a combine step).
//
// The fused QKV step is an epilogue of the matvec (q4_gemv.hip, EPI_ROPE);
// this file holds the unfused RoPE + append (same device function, so the
// same bits) and the attention:
//  * k_attn: workgroup (head h, split s) walks its positions in blocks of 256,
//    one position per thread for the scores (the key row, head_dim f16, all
//    its loads in flight) and (8-dim chunk, position group) threads for the
//    probability-weighted values (all of a thread's loads in flight, their
//    rows located in the score phase); an online softmax across blocks
//    (running maximum and sum, earlier partial sums rescaled); the partial state
//    (maximum, sum, head_dim weighted sums) goes to a workspace, or, with one
//    split, the normalised output straight to out;
//  * k_attn_combine merges the splits of a head in split order.
// No atomics: results are identical run to run.
#include <algorithm>
#include <cmath>

#include "q4_common.h"

namespace q4 {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kMaxHeadDim = 256;
constexpr int kMaxSplits = 32;
constexpr int kSplitGrain = 64;  // positions: a split covers whole pieces of this size

// One thread per RoPE pair of a stored f16 qkv vector.
__global__ __launch_bounds__(256) void k_rope_append(const uint16_t *__restrict__ qkv, RopeArgs r,
                                                     int pairs)
{
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= pairs)
        return;
    const int half = r.head_dim >> 1;
    const int head = p / half, i = p - head * half;
    const size_t row = (size_t)head * r.head_dim + i;
    rope_pair_store(r, p, h2f(qkv[row]), h2f(qkv[row + half]));
}

// Offset (in f16 elements) of the cache row of position t of key/value head
// kvh for K (add the K-to-V distance for V), or -1 when the position's page
// is outside the table or the cache.
__device__ __forceinline__ int64_t cache_row(const RopeArgs &r, int t, int kvh)
{
    const int lp = t / r.page_size, slot = t - lp * r.page_size;
    if (lp >= r.max_pages)
        return -1;
    const int pp = r.page_table[lp];
    if (pp < 0 || pp >= r.n_pages)
        return -1;
    return (((int64_t)pp * 2) * r.n_kv + kvh) * r.page_size * r.head_dim +
           (int64_t)slot * r.head_dim;
}

__device__ __forceinline__ float block_reduce(float v, float *red, bool is_max)
{
    v = is_max ? segment_max(v, 64) : segment_sum(v, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        red[wave] = v;
    __syncthreads();
    float t = red[0];
#pragma unroll
    for (int w = 1; w < kAttnThreads / 64; ++w)
        t = is_max ? fmaxf(t, red[w]) : t + red[w];
    __syncthreads();
    return t;
}

__device__ __forceinline__ void fma8(float (&o)[8], float p, uint4 w)
{
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o[2 * e] = fmaf(p, h2f((uint16_t)(u[e] & 0xFFFF)), o[2 * e]);
        o[2 * e + 1] = fmaf(p, h2f((uint16_t)(u[e] >> 16)), o[2 * e + 1]);
    }
}

// Workgroup (head, split): partial softmax state of the split's positions,
// in blocks of PB positions (256, or 64 or 128 where every split is at most
// that long: the value phase then loads and adds only the chunks of those
// positions; the ones it drops are past the block, with weight 0).
// part layout: [n_heads][splits][2 + head_dim] = (max, sum, weighted values).
// NC = head_dim / 8 (16-byte chunks of a cache row).
template <int NC, int PB>
__global__ __launch_bounds__(kAttnThreads) void k_attn(const uint16_t *__restrict__ q,
                                                       const uint16_t *__restrict__ kv,
                                                       RopeArgs r, float scale,
                                                       float *__restrict__ part,
                                                       uint16_t *__restrict__ out)
{
    constexpr int D = 8 * NC;
    static_assert(PB == 64 || PB == 128 || PB == kAttnThreads, "positions per block");
    constexpr int groups = kAttnThreads / NC;      // position groups of the value phase
    constexpr int U = (PB + groups - 1) / groups;  // positions per value thread
    __shared__ float qs[D];
    __shared__ float ps[PB];
    __shared__ int64_t vofs[PB];
    __shared__ float red[kAttnThreads / 64];
    __shared__ float osum[groups * D];

    const int h = blockIdx.x, s = blockIdx.y, NS = gridDim.y;
    const int tid = threadIdx.x;
    const int kvh = h / (r.n_heads / r.n_kv);
    const int64_t kv_dist = (int64_t)r.n_kv * r.page_size * D;  // K row -> V row
    const int cap = r.max_pages * r.page_size;
    const int L = min(max(*r.pos + 1, 0), cap);
    // splits of whole kSplitGrain-position pieces
    const int npc = (L + kSplitGrain - 1) / kSplitGrain;
    const int chunk = kSplitGrain * ((npc + NS - 1) / NS);
    const int t0 = s * chunk, t1 = min(L, t0 + chunk);

    for (int d = tid; d < D; d += kAttnThreads)
        qs[d] = h2f(q[(size_t)h * D + d]);
    __syncthreads();

    const int dc = tid % NC, tg = tid / NC;
    const bool pv_thread = tg < groups;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    for (int tb = t0; tb < t1; tb += PB) {
        const int nb = min(PB, t1 - tb);
        // scores: one position per thread, its key row's loads all in flight;
        // the row's value offset goes to LDS for the value phase
        const int64_t koff = tid < nb ? cache_row(r, tb + tid, kvh) : -1;
        float sc = -INFINITY;
        if (koff >= 0) {
            const uint4 *krow = reinterpret_cast<const uint4 *>(kv + koff);
            uint4 w[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c)
                w[c] = krow[c];
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const uint32_t uu[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dot = fmaf(qs[8 * c + 2 * e], h2f((uint16_t)(uu[e] & 0xFFFF)), dot);
                    dot = fmaf(qs[8 * c + 2 * e + 1], h2f((uint16_t)(uu[e] >> 16)), dot);
                }
            }
            sc = dot * scale;
        }
        if (tid < PB)
            vofs[tid] = koff < 0 ? -1 : koff + kv_dist;
        const float m_blk = block_reduce(sc, red, true);
        const float m_new = fmaxf(m_run, m_blk);
        // with no valid position yet there is nothing to rescale or add
        const float alpha = m_new == -INFINITY ? 1.f : expf(m_run - m_new);
        const float p = sc == -INFINITY ? 0.f : expf(sc - m_new);
        if (tid < PB)
            ps[tid] = p;
        const float l_blk = block_reduce(p, red, false);  // its barrier publishes ps, vofs
        l_run = l_run * alpha + l_blk;
        m_run = m_new;
        if (pv_thread) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[e] *= alpha;
            // every value load of this thread in flight, then the sums
            // (positions without a row, or past the block, add nothing)
            uint4 vw[U];
            float pj[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = min(tg + u * groups, PB - 1);
                const int64_t vo = vofs[j];
                pj[u] = (tg + u * groups < PB && vo >= 0) ? ps[j] : 0.f;
                vw[u] = reinterpret_cast<const uint4 *>(kv + (vo >= 0 ? vo : 0))[dc];
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                fma8(o, pj[u], vw[u]);
        }
        __syncthreads();  // ps and vofs are rewritten by the next block
    }

    // the position groups' sums of each dimension, added in group order
    if (pv_thread)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            osum[tg * D + 8 * dc + e] = o[e];
    __syncthreads();
    for (int d = tid; d < D; d += kAttnThreads) {
        float v = 0.f;
        for (int g = 0; g < groups; ++g)
            v += osum[g * D + d];
        if (NS == 1) {
            out[(size_t)h * D + d] = f2h(l_run > 0.f ? v / l_run : 0.f);
        } else {
            float *pp = part + ((size_t)h * NS + s) * (2 + D);
            pp[2 + d] = v;
            if (d == 0) {
                pp[0] = m_run;
                pp[1] = l_run;
            }
        }
    }
}

// out[h][d] = sum_s o_s[d] e^(m_s - M) / sum_s l_s e^(m_s - M) (splits without
// a position have l_s = 0 and weight 0). One wave reads every split's
// (max, sum) at once and forms the weights; then each dimension's loads are
// independent of one another.
__global__ __launch_bounds__(kMaxHeadDim) void k_attn_combine(const float *__restrict__ part,
                                                              int NS, int D,
                                                              uint16_t *__restrict__ out)
{
    __shared__ float wgt[kMaxSplits];
    __shared__ float inv_l;
    const int h = blockIdx.x, tid = threadIdx.x;
    const float *ph = part + (size_t)h * NS * (2 + D);
    if (tid < 64) {
        const bool has = tid < NS;
        const float m = has ? ph[tid * (2 + D)] : -INFINITY;
        const float l = has ? ph[tid * (2 + D) + 1] : 0.f;
        const bool valid = l > 0.f;
        float M = valid ? m : -INFINITY;
        M = segment_max(M, 64);
        const float w = valid ? expf(m - M) : 0.f;
        const float sum = segment_sum(l * w, 64);
        if (has)
            wgt[tid] = w;
        if (tid == 0)
            inv_l = sum > 0.f ? 1.f / sum : 0.f;
    }
    __syncthreads();
    if (tid >= D)
        return;
    float v = 0.f;
#pragma unroll 8
    for (int s = 0; s < NS; ++s)
        v = fmaf(ph[s * (2 + D) + 2 + tid], wgt[s], v);
    out[(size_t)h * D + tid] = f2h(v * inv_l);
}

}  // namespace

q4_status launch_rope_append(const uint16_t *qkv, const RopeArgs &r, hipStream_t stream)
{
    const int pairs = (r.n_heads + 2 * r.n_kv) * r.head_dim / 2;
    hipLaunchKernelGGL(k_rope_append, dim3((pairs + 255) / 256), dim3(256), 0, stream, qkv, r,
                       pairs);
    return check_launch("k_rope_append");
}

size_t attention_part_bytes(const RopeArgs &r)
{
    return (size_t)r.n_heads * kMaxSplits * (2 + r.head_dim) * sizeof(float);
}

namespace {
// Splits of the positions per head for a call bounded by max_len positions.
int attention_splits(const RopeArgs &r, int64_t max_len)
{
    const int64_t cap = (int64_t)r.max_pages * r.page_size;
    const int64_t len = std::max<int64_t>(1, std::min(max_len, cap));
    // one workgroup per head up to one block of positions (no combine step);
    // beyond, about two workgroups per CU over the heads, in splits of whole
    // kSplitGrain pieces, and no fewer splits than blocks of 256 positions
    const int cu = cu_count();
    const int64_t fill = (2 * (int64_t)cu + r.n_heads - 1) / r.n_heads;
    const int64_t by_grain = std::min<int64_t>((len + kSplitGrain - 1) / kSplitGrain, fill);
    const int64_t by_block = (len + kAttnThreads - 1) / kAttnThreads;
    return len <= kAttnThreads ? 1
                               : (int)std::min<int64_t>(kMaxSplits, std::max(by_grain, by_block));
}
}  // namespace

size_t ws_attention(const RopeArgs &r, int64_t max_len)
{
    return attention_splits(r, max_len) > 1 ? kWsHeader + attention_part_bytes(r) : 0;
}

q4_status launch_attention(const uint16_t *q, const uint16_t *kv, const RopeArgs &r,
                           int64_t max_len, uint16_t *out, hipStream_t stream, float *part)
{
    const int NS = attention_splits(r, max_len);
    const float scale = (float)(1.0 / std::sqrt((double)r.head_dim));
    if (NS > 1 && !part) {
        char *ws = static_cast<char *>(workspace(stream, ws_attention(r, max_len)));
        if (!ws)
            return workspace_status();
        part = reinterpret_cast<float *>(ws + kWsHeader);
    }
    const dim3 grid(r.n_heads, NS);
    // blocks of 64 or 128 positions where no split can be longer (the bound on
    // the position count gives the longest split; the kernel loops over blocks
    // either way)
    const int64_t len = std::max<int64_t>(1, std::min<int64_t>(max_len, (int64_t)r.max_pages * r.page_size));
    const int64_t pieces = (len + kSplitGrain - 1) / kSplitGrain;
    const int64_t longest = kSplitGrain * ((pieces + NS - 1) / NS);
    switch (r.head_dim / 8) {
#define Q4_ATTN_CASE(nc)                                                                          \
    case nc:                                                                                      \
        if (longest <= 64)                                                                        \
            hipLaunchKernelGGL((k_attn<nc, 64>), grid, dim3(kAttnThreads), 0, stream, q, kv, r,   \
                               scale, part, out);                                                 \
        else if (longest <= 128)                                                                  \
            hipLaunchKernelGGL((k_attn<nc, 128>), grid, dim3(kAttnThreads), 0, stream, q, kv, r,  \
                               scale, part, out);                                                 \
        else                                                                                      \
            hipLaunchKernelGGL((k_attn<nc, kAttnThreads>), grid, dim3(kAttnThreads), 0, stream, q, \
                               kv, r, scale, part, out);                                          \
        break;
        Q4_ATTN_CASE(1) Q4_ATTN_CASE(2) Q4_ATTN_CASE(4) Q4_ATTN_CASE(6) Q4_ATTN_CASE(8)
        Q4_ATTN_CASE(12) Q4_ATTN_CASE(16) Q4_ATTN_CASE(20) Q4_ATTN_CASE(24) Q4_ATTN_CASE(32)
#undef Q4_ATTN_CASE
    default:
        return fail(Q4_ESHAPE, "no attention kernel for head_dim %d", r.head_dim);
    }
    q4_status st = check_launch("k_attn");
    if (st != Q4_OK || NS == 1)
        return st;
    hipLaunchKernelGGL(k_attn_combine, dim3(r.n_heads), dim3(kMaxHeadDim), 0, stream, part, NS,
                       r.head_dim, out);
    return check_launch("k_attn_combine");
}

}  // namespace q4
