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
// O(P^2) comparisons in one workgroup; P <= Q4_MAX_PAIRS.
__global__ __launch_bounds__(256) void k_moe_route(const int32_t *__restrict__ ids, int P, int E,
                                                   int32_t *__restrict__ meta)
{
    extern __shared__ int32_t sid[];  // [P] expert or -1, then [P] first-occurrence flags
    int32_t *firstocc = sid + P;
    int32_t *distinct = meta + 1;
    int32_t *seg = meta + 1 + P;
    int32_t *order = meta + 2 + 2 * P;
    __shared__ int s_nd, s_valid;
    for (int p = threadIdx.x; p < P; p += 256) {
        const int e = ids[p];
        sid[p] = (e >= 0 && e < E) ? e : -1;
    }
    if (threadIdx.x == 0) {
        s_nd = 0;
        s_valid = 0;
    }
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += 256) {
        const int e = sid[p];
        bool first = e >= 0;
        for (int q = 0; q < p && first; ++q)
            first = sid[q] != e;
        firstocc[p] = first;
    }
    __syncthreads();
    int local_nd = 0, local_valid = 0;
    for (int p = threadIdx.x; p < P; p += 256) {
        const int e = sid[p];
        if (e < 0)
            continue;
        int rank = 0, below = 0, slot = 0;
        for (int q = 0; q < P; ++q) {
            const int f = sid[q];
            if (f < 0)
                continue;
            if (f < e) {
                ++below;
                slot += firstocc[q];
            } else if (f == e && q < p) {
                ++rank;
            }
        }
        order[below + rank] = p;
        if (firstocc[p]) {
            distinct[slot] = e;
            seg[slot] = below;
            ++local_nd;
        }
        ++local_valid;
    }
    atomicAdd(&s_nd, local_nd);
    atomicAdd(&s_valid, local_valid);
    __syncthreads();
    if (threadIdx.x == 0) {
        meta[0] = s_nd;
        seg[s_nd] = s_valid;
    }
}

}  // namespace

q4_status launch_moe(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                     const uint16_t *route_w, const uint16_t *x, int64_t ldx,
                     int64_t x_slot_stride, uint16_t *y, int E, int N, int K, int T, int TOPK,
                     int epi_silu, hipStream_t stream)
{
    const int P = T * TOPK;
    const int mode = epi_silu ? MOE_SILU : (route_w ? MOE_COMBINE : MOE_PER_SLOT);
    const bool in_kernel = moe_routes_in_kernel(P, E);
    const size_t meta_bytes = in_kernel ? 0 : ((size_t)(3 * P + 2) * 4 + 255) / 256 * 256;
    char *ws = static_cast<char *>(
        workspace(stream, kWsHeader + meta_bytes + moe_part_bytes(N, K, P)));
    if (!ws)
        return Q4_EHIP;
    int32_t *meta = in_kernel ? nullptr : reinterpret_cast<int32_t *>(ws + kWsHeader);
    float *part = reinterpret_cast<float *>(ws + kWsHeader + meta_bytes);
    if (!in_kernel) {
        hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(256), (size_t)P * 8, stream, ids, P, E,
                           meta);
        q4_status st = check_launch("k_moe_route");
        if (st != Q4_OK)
            return st;
    }
    if (moe_rows_fits(P, E, K)) {
        // few pairs per expert: the single-row arithmetic per pair, then the outputs
        q4_status st = launch_moe_rows(W, S, ids, meta, x, ldx, x_slot_stride, part, E, N, K, T,
                                       TOPK, stream);
        if (st != Q4_OK)
            return st;
        return launch_moe_finish(mode, part, 1, P, N, ids, route_w, y, E, T, TOPK, stream);
    }
    return launch_moe_mfma(W, S, ids, meta, route_w, x, ldx, x_slot_stride, y, part, E, N, K, T,
                           TOPK, mode, stream);
}

}  // namespace q4
