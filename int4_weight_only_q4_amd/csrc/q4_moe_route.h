// Routing of a MoE expert stage inside one workgroup (shared by the expert
// kernels). Internal to libq4.
#pragma once

#include "q4_common.h"

namespace q4 {

// Block-wide exclusive prefix sum over 256 threads (wave scans, then the wave
// totals); `red` is 4 ints of LDS. Returns the prefix, *total the sum.
__device__ inline int block_exclusive_scan(int v, int *red, int *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off)
            incl += o;
    }
    if (lane == 63)
        red[wave] = incl;
    __syncthreads();
    int before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        before += w < wave ? red[w] : 0;
        sum += red[w];
    }
    __syncthreads();
    *total = sum;
    return before + incl - v;
}

// Routing of one workgroup when the pairs and experts are few (P <= kFusePairs,
// E <= kFuseExperts). The valid ids' distinct experts, in increasing id order,
// each own ceil(count / per_unit) units of at most per_unit of their pairs
// (per_unit = kFusePairs: one unit per expert); the workgroup takes unit d.
// Returns its expert, or -1 when there are d or fewer units; *npairs is the
// expert's pair count, pairs[] its pairs in pair order (as k_moe_route lists
// them), *first the unit's first position in that list.
constexpr int kFusePairs = 256;
constexpr int kFuseExperts = 1024;
__device__ inline int route_in_workgroup(const int32_t *__restrict__ ids, int P, int E, int d,
                                         int per_unit, int *cnt, int *pairs, int *npairs,
                                         int *first)
{
    __shared__ int red[4];
    __shared__ int s_e, s_first;
    const int t = threadIdx.x;
    for (int i = t; i < E; i += 256)
        cnt[i] = 0;
    if (t == 0)
        s_e = -1;
    __syncthreads();
    const int my = t < P ? ids[t] : -1;
    const bool valid = my >= 0 && my < E;
    if (valid)
        atomicAdd(&cnt[my], 1);
    __syncthreads();
    // thread t owns experts [4t, 4t + 4) and their units
    constexpr int kPer = kFuseExperts / 256;
    int units = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (kPer * t + i < E)
            units += (cnt[kPer * t + i] + per_unit - 1) / per_unit;
    int total;
    int rank = block_exclusive_scan(units, red, &total);
    if (d >= rank && d < rank + units) {
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (kPer * t + i < E) {
                const int u = (cnt[kPer * t + i] + per_unit - 1) / per_unit;
                if (d >= rank && d < rank + u) {
                    s_e = kPer * t + i;
                    s_first = (d - rank) * per_unit;
                }
                rank += u;
            }
    }
    __syncthreads();
    const int e = s_e;
    if (e < 0)
        return -1;
    // the expert's pairs in pair order
    int n_e;
    const int pos = block_exclusive_scan(valid && my == e ? 1 : 0, red, &n_e);
    if (valid && my == e)
        pairs[pos] = t;
    if (t == 0)
        *npairs = n_e;
    *first = s_first;
    __syncthreads();
    return e;
}

}  // namespace q4
