// MoE expert stage for gfx950: every (token, slot) pair runs the matvec of the
// expert it was routed to (BENCH.md, "MoE chunked prefill (2026-08-13)"), and in
// the down stage the slot outputs are combined by routing weight.
//
// The pages ship a per-(token, slot) re-indexing and measure grouping by expert
// ("MoE Phase B") as a loss on Apple, where caches absorb the repeated weight
// reads. On MI355X each distinct expert's weights are streamed from HBM once
// per call instead:
//   1. k_moe_route (one workgroup) sorts the pairs by expert id, stable in pair
//      order, and lists the distinct experts in increasing id order;
//   2. k_moe_gemv runs one grid row per distinct expert: each wave keeps its
//      weight rows in registers and reuses them for every pair of that expert
//      (activations staged in LDS a few pairs at a time);
//   3. in the down stage, k_moe_combine sums the per-pair f32 results over the
//      slots in slot order (no floating-point atomics, so results are
//      deterministic).
#include "q4_dequant.h"

namespace q4 {
namespace {

enum { MOE_PER_SLOT = 0, MOE_SILU = 1, MOE_COMBINE = 2 };

// Workspace layout (int32): [0] number of distinct experts, [1 .. P] expert of
// each distinct slot (increasing id), [P+1 .. 2P+1] start of each slot's pairs
// in `order`, [2P+2 .. 3P+1] order = pair indices sorted by (expert, pair).
// O(P^2) comparisons in one workgroup; P <= Q4_MAX_PAIRS.
__global__ __launch_bounds__(256) void k_moe_route(const int32_t *__restrict__ ids, int P, int E,
                                                   int32_t *__restrict__ meta,
                                                   uint16_t *__restrict__ y, int out_w,
                                                   int zero_invalid)
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
        if (e < 0) {
            if (zero_invalid)
                for (int i = 0; i < out_w; ++i)
                    y[(int64_t)p * out_w + i] = 0;
            continue;
        }
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

template <int LPR, int NGMAX, int MB, int MODE>
__global__ __launch_bounds__(256) void k_moe_gemv(const uint4 *__restrict__ Wall,
                                                  const uint16_t *__restrict__ Sall,
                                                  const int32_t *__restrict__ meta, int P,
                                                  const uint16_t *__restrict__ x, int64_t ldx,
                                                  int64_t slot_stride, int TOPK,
                                                  uint16_t *__restrict__ y,
                                                  float *__restrict__ part, int N, int G)
{
    constexpr int SPW = 64 / LPR;
    constexpr int RB = 4 * SPW;  // rows per workgroup (one row per segment)
    extern __shared__ uint4 smem[];
    __shared__ float vals[MODE == MOE_SILU ? MB * RB : 1];

    const int slot = blockIdx.y;
    const int nd = meta[0];
    if (slot >= nd)
        return;
    const int e = meta[1 + slot];
    const int p0 = meta[1 + P + slot], p1 = meta[1 + P + slot + 1];
    const int32_t *order = meta + 2 + 2 * P;

    const int K = G * 32;
    const int stride = (K >> 3) + ((G + 3) >> 2);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int seg = lane / LPR, j = lane % LPR;
    const int li = wave * SPW + seg;
    const int half = N >> 1;
    int row;
    bool ok;
    if (MODE == MOE_SILU) {
        const int gi = blockIdx.x * (RB / 2) + (li % (RB / 2));
        ok = gi < half;
        row = li < RB / 2 ? gi : half + gi;
    } else {
        row = blockIdx.x * RB + li;
        ok = row < N;
    }
    if (!ok)
        row = 0;
    const int ng = (G + LPR - 1) / LPR;

    const uint4 *W = Wall + (size_t)e * N * G;
    const uint16_t *S = Sall + (size_t)e * N * G;
    uint4 wv[NGMAX];
    uint32_t sv[NGMAX];
#pragma unroll
    for (int i = 0; i < NGMAX; ++i) {
        // branch-free: lanes past the last group re-read group G - 1, which the
        // accumulation skips (a conditional load would make the compiler wait
        // for each scale inside its branch)
        const size_t off = (size_t)row * G + min(j + LPR * i, G - 1);
        wv[i] = load_weights(W + off);
        sv[i] = load_scale(S + off);
    }

    for (int q0 = p0; q0 < p1; q0 += MB) {
        const int mb = min(MB, p1 - q0);
        __syncthreads();
        for (int m = 0; m < mb; ++m) {
            const int p = order[q0 + m];
            const int t = p / TOPK, s = p % TOPK;
            uint4 *xs = smem + m * stride;
            stage_activation(x + (int64_t)t * ldx + (int64_t)s * slot_stride, K, xs,
                             reinterpret_cast<float *>(xs + (K >> 3)));
        }
        __syncthreads();
        float acc[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m)
            acc[m] = 0.f;
#pragma unroll
        for (int i = 0; i < NGMAX; ++i) {
            const int g = j + LPR * i;
            if (i < ng && g < G) {
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    if (m < mb) {
                        const uint4 *xs = smem + m * stride;
                        const float *cs = reinterpret_cast<const float *>(xs + (K >> 3));
                        acc[m] = fmaf(h2f(sv[i]), group_dot(wv[i], xs, g, cs[g]), acc[m]);
                    }
            }
        }
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int off = LPR / 2; off > 0; off >>= 1)
                acc[m] += __shfl_xor(acc[m], off, 64);

        if (MODE == MOE_SILU) {
            if (j == 0)
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    vals[m * RB + li] = h2f(f2h(acc[m]));
            __syncthreads();
            for (int idx = tid; idx < mb * (RB / 2); idx += 256) {
                const int m = idx / (RB / 2), c = idx % (RB / 2);
                const int gi = blockIdx.x * (RB / 2) + c;
                if (gi < half) {
                    const int p = order[q0 + m];
                    y[(int64_t)p * half + gi] =
                        f2h(silu_mul_f(vals[m * RB + c], vals[m * RB + RB / 2 + c]));
                }
            }
        } else if (j == 0 && ok) {
#pragma unroll
            for (int m = 0; m < MB; ++m)
                if (m < mb) {
                    const int p = order[q0 + m];
                    if (MODE == MOE_PER_SLOT)
                        y[(int64_t)p * N + row] = f2h(acc[m]);
                    else
                        part[(int64_t)p * N + row] = acc[m];
                }
        }
    }
}

__global__ __launch_bounds__(256) void k_moe_combine(const float *__restrict__ part,
                                                     const int32_t *__restrict__ ids,
                                                     const uint16_t *__restrict__ route_w,
                                                     uint16_t *__restrict__ y, int N, int E,
                                                     int TOPK)
{
    const int t = blockIdx.y;
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N)
        return;
    float acc = 0.f;
    for (int s = 0; s < TOPK; ++s) {
        const int p = t * TOPK + s;
        const int e = ids[p];
        if (e >= 0 && e < E)
            acc = fmaf(h2f(route_w[p]), part[(int64_t)p * N + n], acc);
    }
    y[(int64_t)t * N + n] = f2h(acc);
}

template <int LPR, int NGMAX, int MODE>
q4_status run_moe(int mb, dim3 grid, size_t lds, hipStream_t st, const uint4 *W,
                  const uint16_t *S, const int32_t *meta, int P, const uint16_t *x, int64_t ldx,
                  int64_t slot_stride, int TOPK, uint16_t *y, float *part, int N, int G)
{
#define Q4_MOE_LAUNCH(MBV)                                                                        \
    Q4_LAUNCH_MATVEC((k_moe_gemv<LPR, NGMAX, MBV, MODE>), grid, dim3(256), lds, st, W, S, meta, \
                     P, x, ldx, slot_stride, TOPK, y, part, N, G)
    switch (mb) {
    case 8: Q4_MOE_LAUNCH(8); break;
    case 4: Q4_MOE_LAUNCH(4); break;
    case 2: Q4_MOE_LAUNCH(2); break;
    default: Q4_MOE_LAUNCH(1); break;
    }
#undef Q4_MOE_LAUNCH
    return check_launch("k_moe_gemv");
}

template <int MODE>
q4_status dispatch_moe(int lpr, int mb, dim3 grid, size_t lds, hipStream_t st, const uint4 *W,
                       const uint16_t *S, const int32_t *meta, int P, const uint16_t *x,
                       int64_t ldx, int64_t slot_stride, int TOPK, uint16_t *y, float *part,
                       int N, int G)
{
    switch (lpr) {
    case 8: return run_moe<8, 4, MODE>(mb, grid, lds, st, W, S, meta, P, x, ldx, slot_stride, TOPK, y, part, N, G);
    case 16: return run_moe<16, 4, MODE>(mb, grid, lds, st, W, S, meta, P, x, ldx, slot_stride, TOPK, y, part, N, G);
    case 32: return run_moe<32, 4, MODE>(mb, grid, lds, st, W, S, meta, P, x, ldx, slot_stride, TOPK, y, part, N, G);
    default: return run_moe<64, 12, MODE>(mb, grid, lds, st, W, S, meta, P, x, ldx, slot_stride, TOPK, y, part, N, G);
    }
}

}  // namespace

q4_status launch_moe(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                     const uint16_t *route_w, const uint16_t *x, int64_t ldx,
                     int64_t x_slot_stride, uint16_t *y, int E, int N, int K, int T, int TOPK,
                     int epi_silu, hipStream_t stream)
{
    const int P = T * TOPK;
    const int G = K / 32;
    const int mode = epi_silu ? MOE_SILU : (route_w ? MOE_COMBINE : MOE_PER_SLOT);

    const size_t meta_bytes = ((size_t)(3 * P + 2) * 4 + 255) / 256 * 256;
    const size_t part_bytes = mode == MOE_COMBINE ? (size_t)P * N * 4 : 0;
    char *ws = static_cast<char *>(workspace(stream, kWsHeader + meta_bytes + part_bytes));
    if (!ws)
        return Q4_EHIP;
    int32_t *meta = reinterpret_cast<int32_t *>(ws + kWsHeader);
    float *part = reinterpret_cast<float *>(ws + kWsHeader + meta_bytes);

    const int out_w = mode == MOE_SILU ? N / 2 : N;
    hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(256), (size_t)P * 8, stream, ids, P, E, meta, y,
                       out_w, mode != MOE_COMBINE ? 1 : 0);
    q4_status st = check_launch("k_moe_route");
    if (st != Q4_OK)
        return st;

    // lanes per row: least padding with at most 4 groups per lane (LPR < 64)
    int lpr = 64, best = 1 << 30;
    for (int c : {64, 32, 16, 8}) {
        const int ng = (G + c - 1) / c;
        if (c < 64 && ng > 4)
            continue;
        if (c == 64 && ng > 12)
            continue;
        const int waste = ng * c - G;
        if (waste < best) {
            best = waste;
            lpr = c;
        }
    }
    const int rb = 4 * (64 / lpr);
    const int rows = mode == MOE_SILU ? N / 2 : N;
    const int rbo = mode == MOE_SILU ? rb / 2 : rb;
    const size_t row_bytes = ((size_t)(K >> 3) + (size_t)((G + 3) >> 2)) * 16;
    int mb = 8;
    while (mb > 1 && (size_t)mb * row_bytes > 56 * 1024)
        mb >>= 1;
    const int slots = P < E ? P : E;
    dim3 grid((rows + rbo - 1) / rbo, slots);
    const size_t lds = (size_t)mb * row_bytes;
    const uint4 *W4 = reinterpret_cast<const uint4 *>(W);
    switch (mode) {
    case MOE_SILU:
        st = dispatch_moe<MOE_SILU>(lpr, mb, grid, lds, stream, W4, S, meta, P, x, ldx,
                                    x_slot_stride, TOPK, y, part, N, G);
        break;
    case MOE_COMBINE:
        st = dispatch_moe<MOE_COMBINE>(lpr, mb, grid, lds, stream, W4, S, meta, P, x, ldx,
                                       x_slot_stride, TOPK, y, part, N, G);
        break;
    default:
        st = dispatch_moe<MOE_PER_SLOT>(lpr, mb, grid, lds, stream, W4, S, meta, P, x, ldx,
                                        x_slot_stride, TOPK, y, part, N, G);
        break;
    }
    if (st != Q4_OK || mode != MOE_COMBINE)
        return st;
    hipLaunchKernelGGL(k_moe_combine, dim3((N + 255) / 256, T), dim3(256), 0, stream, part, ids,
                       route_w, y, N, E, TOPK);
    return check_launch("k_moe_combine");
}

}  // namespace q4
