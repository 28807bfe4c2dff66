// Internal interface of the persistent decode-stack kernel (q4_stack.hip).
#pragma once

#include "q4_common.h"

namespace q4 {

// Threads per workgroup (one workgroup per CU), of which the first
// kStackCompute hold weights, and weight chunks (16-byte groups) per compute
// lane per phase: a workgroup covers at most 6144 groups of one matrix per
// phase.
constexpr int kStackThreads = 1024;
constexpr int kStackCompute = 768;
constexpr int kStackNch = 8;
// Copies of every published vector and flag array (one per XCD).
constexpr int kStackCopies = 8;

struct StackParams {
    int n_layers, d, f, n_qkv, v_off, dv;
    float eps;
    const uint32_t *const *W;  // device table [L][4]: QKV, O, gate_up, down
    const uint16_t *const *S;
    const uint16_t *gamma_in, *gamma_post, *gamma_final;
    const uint16_t *r_in, *h_in;
    uint16_t *r_out, *h_out, *trace;
    uint16_t *qkv;                           // plain [n_qkv]
    uint32_t *vbuf, *r1buf, *ubuf, *r2buf;   // tagged [copies][dv], [d], [f], [d]
    uint32_t *flags;                         // [4][copies][workgroups] (V, r1, u, r2)
    uint32_t epoch0;                         // tag of the first phase of this call
    unsigned *err;                           // set on a wait timeout
    int lds_xs, lds_cs, lds_xo, lds_co, lds_st, lds_raw, lds_rowv, lds_lres;  // LDS byte offsets
    int lpr_d, ng_d, lpr_v, ng_v, lpr_f, ng_f;  // single-call layouts for K = d, dv, f
};

const void *stack_kernel();

// Lanes per row and groups per lane that the single-call matvec uses for G
// groups per row (q4_gemv.hip); the persistent kernel replays the same order.
void matvec_layout(int G, int *lpr, int *ng);

}  // namespace q4
