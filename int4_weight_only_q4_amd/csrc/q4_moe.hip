// MoE expert stage for gfx950: every (token, slot) pair runs the matvec of the
// expert it was routed to (BENCH.md, "MoE chunked prefill (2026-08-13)"), and in
// the down stage the slot outputs are combined by routing weight.
//
// The pages ship a per-(token, slot) re-indexing and measure grouping by expert
// ("MoE Phase B") as a loss on Apple, where caches absorb the repeated weight
// reads. On MI355X each distinct expert's weights are streamed from HBM once
// per call instead:
//   1. the pairs are sorted by expert id, stable in pair order, and the
//      distinct experts listed in increasing id order: for a decode-sized
//      routing (at most 256 pairs and 1024 experts) by every expert workgroup
//      itself, otherwise by k_moe_route (one workgroup) into a workspace;
//   2. k_moe_mfma (q4_mfma.hip) runs one grid slice per distinct expert: the
//      expert's pairs are the activation rows of a small matrix-core matvec
//      that reads each weight once;
//   3. k_moe_finish forms the per-pair outputs (or, in the down stage, sums
//      them over the slots in slot order with the routing weights; no
//      floating-point atomics, so results are deterministic).
#include "q4_dequant.h"
#include "q4_moe_route.h"

namespace q4 {
namespace {

enum { MOE_PER_SLOT = 0, MOE_SILU = 1, MOE_COMBINE = 2 };

// The expert matvecs run the dot2 kernel (the single-row arithmetic per pair)
// while the experts get about two pairs each or fewer (P <= 2 E), at most 256
// pairs, and four activation rows fit the staging in LDS; the matrix cores
// take larger batches. (128 experts, top 8: the dot2 kernel up to 32 tokens.)
bool moe_rows_fits(int P, int E, int K) { return P <= 256 && P <= 2 * E && 4 * K <= 24576; }

// Workspace layout (int32): [0] number of distinct experts, [1 .. P] expert of
// each distinct slot (increasing id), [P+1 .. 2P+1] start of each slot's pairs
// in `order`, [2P+2 .. 3P+1] order = pair indices sorted by (expert, pair).
// One workgroup: a bitonic sort of the n (a power of two >= P) keys
// (expert << 32 | pair) in LDS, invalid ids and padding keyed past every
// valid pair, then a block scan over the run starts of the sorted experts.
// P <= Q4_MAX_PAIRS.
__global__ __launch_bounds__(256) void k_moe_route(const int32_t *__restrict__ ids, int P, int E,
                                                   int n, int32_t *__restrict__ meta)
{
    extern __shared__ unsigned long long key[];  // [n]
    __shared__ int red[4];
    int32_t *distinct = meta + 1;
    int32_t *seg = meta + 1 + P;
    int32_t *order = meta + 2 + 2 * P;
    const int t = threadIdx.x;
    constexpr unsigned long long kNone = ~0ull;
    for (int i = t; i < n; i += 256) {
        unsigned long long k = kNone;
        if (i < P) {
            const int e = ids[i];
            if (e >= 0 && e < E)
                k = (unsigned long long)e << 32 | (unsigned)i;
        }
        key[i] = k;
    }
    __syncthreads();
    // ascending bitonic sort: stage (size, stride) compares element lo with
    // lo + stride, ascending where lo & size == 0
    for (int size = 2; size <= n; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = t; i < (n >> 1); i += 256) {
                const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
                const unsigned long long x = key[lo], y = key[hi];
                if ((x > y) == ((lo & size) == 0)) {
                    key[lo] = y;
                    key[hi] = x;
                }
            }
            __syncthreads();
        }
    // thread t owns sorted positions [c t, c t + c): its run starts and valid pairs
    const int c = (n + 255) / 256, i0 = min(n, c * t), i1 = min(n, i0 + c);
    int starts = 0, valid = 0;
    for (int i = i0; i < i1; ++i) {
        const unsigned long long k = key[i];
        if (k == kNone)
            break;
        ++valid;
        starts += (i == 0 || (key[i - 1] >> 32) != (k >> 32)) ? 1 : 0;
    }
    int nd, nvalid;
    int slot = block_exclusive_scan(starts, red, &nd);
    block_exclusive_scan(valid, red, &nvalid);
    for (int i = i0; i < i1; ++i) {
        const unsigned long long k = key[i];
        if (k == kNone)
            break;
        order[i] = (int32_t)(k & 0xFFFFFFFFu);
        if (i == 0 || (key[i - 1] >> 32) != (k >> 32)) {
            distinct[slot] = (int32_t)(k >> 32);
            seg[slot] = i;
            ++slot;
        }
    }
    if (t == 0) {
        meta[0] = nd;
        seg[nd] = nvalid;
    }
}

}  // namespace

namespace {
size_t moe_meta_bytes(int E, int P)
{
    return moe_routes_in_kernel(P, E) ? 0 : ((size_t)(3 * P + 2) * 4 + 255) / 256 * 256;
}
}  // namespace

size_t ws_moe(int E, int N, int K, int P)
{
    return kWsHeader + moe_meta_bytes(E, P) + moe_part_bytes(N, K, P);
}

q4_status launch_moe(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                     const uint16_t *route_w, const uint16_t *x, int64_t ldx,
                     int64_t x_slot_stride, uint16_t *y, int E, int N, int K, int T, int TOPK,
                     int epi_silu, hipStream_t stream)
{
    const int P = T * TOPK;
    const int mode = epi_silu ? MOE_SILU : (route_w ? MOE_COMBINE : MOE_PER_SLOT);
    if (mode == MOE_COMBINE && moe_tokens_fits(T, TOPK, K, x_slot_stride == 0))
        // few pairs: token by token, the combine in the same kernel (no
        // routing step, no finishing kernel)
        return launch_moe_tokens(W, S, ids, route_w, x, ldx, x_slot_stride, y, E, N, K, T, TOPK,
                                 stream);
    const bool in_kernel = moe_routes_in_kernel(P, E);
    const size_t meta_bytes = moe_meta_bytes(E, P);
    char *ws = static_cast<char *>(workspace(stream, ws_moe(E, N, K, P)));
    if (!ws)
        return workspace_status();
    int32_t *meta = in_kernel ? nullptr : reinterpret_cast<int32_t *>(ws + kWsHeader);
    float *part = reinterpret_cast<float *>(ws + kWsHeader + meta_bytes);
    if (!in_kernel) {
        int n = 2;
        while (n < P)
            n <<= 1;
        hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(256), (size_t)n * 8, stream, ids, P, E, n,
                           meta);
        q4_status st = check_launch("k_moe_route");
        if (st != Q4_OK)
            return st;
    }
    if (moe_rows_fits(P, E, K)) {
        // few pairs per expert: the single-row arithmetic per pair; per-pair
        // outputs straight from the expert kernel, the routing-weighted sum
        // over a token's slots by the finishing kernel
        const int out = mode == MOE_SILU ? 2 : (mode == MOE_PER_SLOT ? 1 : 0);
        q4_status st = launch_moe_rows(W, S, ids, meta, x, ldx, x_slot_stride, out, part, y, E,
                                       N, K, T, TOPK, stream);
        if (st != Q4_OK || mode != MOE_COMBINE)
            return st;
        return launch_moe_finish(mode, part, 1, P, N, ids, route_w, y, E, T, TOPK, stream);
    }
    return launch_moe_mfma(W, S, ids, meta, route_w, x, ldx, x_slot_stride, y, part, E, N, K, T,
                           TOPK, mode, stream);
}

}  // namespace q4
