// Internal helpers of libq4 (gfx950). Not part of the C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "q4.h"

namespace q4 {

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Records a message for q4_last_error() on this thread and returns st.
q4_status fail(q4_status st, const char *fmt, ...);

// Wraps a HIP call made by an entry point.
#define Q4_HIP(call)                                                                      \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess)                                                             \
            return ::q4::fail(Q4_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));    \
    } while (0)

// Launch check: hipGetLastError after a kernel launch.
q4_status check_launch(const char *what);

// The events armed by q4_timer_arm for this thread's next matvec launch
// (disarms them), or false if none is armed.
bool take_armed_timer(hipEvent_t *start, hipEvent_t *stop);

// Launch of a matvec kernel: with the armed timer's events (the dispatch
// records its own start and end) when q4_timer_arm armed them, plainly
// otherwise. Wrap a templated kernel name in parentheses.
#define Q4_LAUNCH_MATVEC(kernel, grid, block, lds, stream, ...)                               \
    do {                                                                                  \
        hipEvent_t t0_, t1_;                                                              \
        if (::q4::take_armed_timer(&t0_, &t1_))                                           \
            hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, t0_, t1_, 0, __VA_ARGS__); \
        else                                                                              \
            hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);            \
    } while (0)

// Library-owned scratch for one (device, stream): at least `bytes` bytes. Its
// first kWsHeader bytes are reserved (zero-initialised); callers place their
// own data after them. A call that needs more than the stream holds allocates
// a larger buffer, except during graph capture (then it fails with Q4_ERANGE);
// the replaced buffer stays allocated. Returns nullptr (and sets the error) on
// failure.
constexpr size_t kCounterBytes = 256;
constexpr size_t kWsHeader = kCounterBytes;
void *workspace(hipStream_t stream, size_t bytes);
// The status of this thread's last workspace() failure (Q4_ERANGE during graph
// capture, Q4_EHIP for a HIP error).
q4_status workspace_status();

// Workspace bytes (header included, 0 = none) that each launcher asks
// workspace() for; the launchers and q4_workspace_bytes share them.
size_t ws_rows(int N, int K, int M);   // launch_gemv_batched, launch_gemv_f32, affine rows
size_t ws_argmax(int N, int M);
size_t ws_lm_head(int N, int K, int M);
size_t ws_gemm(int N, int K, int M, bool affine, int64_t ldx);
size_t ws_moe(int E, int N, int K, int P);
struct RopeArgs;
size_t ws_attention(const RopeArgs &r, int64_t max_len);
// Compute units of the current device (cached per device; 256 if unknown).
int cu_count();

inline bool overlaps(const void *a, size_t an, const void *b, size_t bn)
{
    if (!a || !b || an == 0 || bn == 0)
        return false;
    auto pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + bn && pb < pa + an;
}

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Kernel launchers shared between entry points (defined in q4_gemv.hip etc.).
struct EpiArgs {
    int kind = Q4_EPI_NONE;
    const uint16_t *res_in = nullptr;
    const uint16_t *gamma = nullptr;
    uint16_t *res_out = nullptr;
    float eps = 0.f;
    const uint16_t *norm_gamma = nullptr;  // prologue: normalise x first
};

q4_status launch_gemv(const uint32_t *W, const uint16_t *S, const uint16_t *x, uint16_t *y,
                      int N, int K, const EpiArgs &epi, hipStream_t stream);

// One matvec with an optional RMSNorm prologue and a per-row epilogue; no
// synchronisation between workgroups is ever needed.
//   prologue: x (16-byte aligned), or, when norm_src is set, the activation
//             f16(RMSNorm(norm_src) * norm_gamma) (both length K, 16-byte
//             aligned), computed by every workgroup with the canonical
//             summation order of q4_add_rmsnorm (bit-identical to it)
//   epilogue: NONE  y[n] = f16(acc)
//             SILU  y[i] = f16(silu(f16(acc_i)) * f16(acc_{N/2+i}))
//             RESID res_out[n] = f16(f16(acc) + res_in[n])
//             LOGITS yf[n] = acc (f32); when cand is set, cand[workgroup] =
//                    the largest argmax_key of the workgroup's rows
//             ROPE   the rows are Q, K, V heads (rope geometry): Q and K
//                    pairs rotated, Q to q_out, K and V into the cache slot
struct RopeArgs {
    int n_heads = 0, n_kv = 0, head_dim = 0, page_size = 0, max_pages = 0, n_pages = 0;
    float base = 10000.f;
    const int32_t *pos = nullptr;
    const int32_t *page_table = nullptr;
    uint16_t *kv = nullptr;
    uint16_t *q_out = nullptr;
};
struct GemvOp {
    enum { NONE = 0, SILU = 1, RESID = 2, LOGITS = 3, ROPE = 4 };
    const uint32_t *W = nullptr;
    const uint16_t *S = nullptr;
    int N = 0, K = 0;
    const uint16_t *x = nullptr;
    const uint16_t *norm_src = nullptr;
    const uint16_t *norm_gamma = nullptr;
    float norm_eps = 0.f;
    int epi = NONE;
    uint16_t *y = nullptr;
    const uint16_t *res_in = nullptr;
    uint16_t *res_out = nullptr;
    float *yf = nullptr;
    unsigned long long *cand = nullptr;
    RopeArgs rope;
    // the MLX affine format (biases [N][K/64], scales [N][K/64]): plain NONE
    // epilogue with x only
    const uint16_t *bias = nullptr;
};
q4_status launch_gemv_op(const GemvOp &op, hipStream_t stream);
// Workgroups of one launch_gemv_op for N rows of K (the candidates LOGITS writes).
int matvec_blocks(int N, int K);
// MoE expert matvecs on the matrix cores (q4_mfma.hip): meta from the routing
// kernel, or nullptr when moe_routes_in_kernel(P, E); part = f32 scratch of
// moe_part_bytes(N, K, T * TOPK); mode 0 per-slot outputs, 1 SiLU-multiply of
// the gate and up halves, 2 routing-weighted combine.
q4_status launch_moe_mfma(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                          const int32_t *meta, const uint16_t *route_w, const uint16_t *x,
                          int64_t ldx, int64_t x_slot_stride, uint16_t *y, float *part, int E,
                          int N, int K, int T, int TOPK, int mode, hipStream_t stream);
size_t moe_part_bytes(int N, int K, int P);
// The outputs of an expert stage from per-pair f32 partials part[ks][pair][n]
// (KS splits), per mode (q4_mfma.hip).
q4_status launch_moe_finish(int mode, const float *part, int KS, int P, int N,
                            const int32_t *ids, const uint16_t *route_w, uint16_t *y, int E,
                            int T, int TOPK, hipStream_t stream);
// Expert matvecs with the single-row arithmetic per (token, slot) pair
// (q4_gemv.hip), P = T * TOPK <= 256 pairs; routing from meta, or in each
// workgroup when meta == nullptr (moe_routes_in_kernel). out: 0 per-pair f32
// results part[pair][n] (for launch_moe_finish), 1 f16 outputs y[pair][n],
// 2 y[pair][i] = f16(silu(f16(gate_i)) * f16(up_i)) over N / 2 (N even); in
// forms 1 and 2 pairs with an id outside [0, E) get zeros.
// The down stage with the routing-weighted combine, token by token (few
// pairs, moe_tokens_fits): one kernel, no routing step, no per-pair results.
// shared_x: every slot reads the token's one activation row (x_slot_stride 0).
bool moe_tokens_fits(int T, int TOPK, int K, bool shared_x);
q4_status launch_moe_tokens(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                            const uint16_t *route_w, const uint16_t *x, int64_t ldx,
                            int64_t x_slot_stride, uint16_t *y, int E, int N, int K, int T,
                            int TOPK, hipStream_t stream);
q4_status launch_moe_rows(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                          const int32_t *meta, const uint16_t *x, int64_t ldx,
                          int64_t x_slot_stride, int out, float *part, uint16_t *y, int E, int N,
                          int K, int T, int TOPK, hipStream_t stream);
// Whether the expert kernel routes by itself (meta == nullptr) for P pairs and E experts.
bool moe_routes_in_kernel(int P, int E);
// M >= 2 rows on the matrix cores (q4_mfma.hip): f16 outputs y, or f32
// outputs yf when yf is set (y is then ignored); bias set: the MLX affine
// format (scales and biases [N][K/64])
q4_status launch_gemv_mfma(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                           uint16_t *y, float *yf, int64_t ldy, int N, int K, int M,
                           hipStream_t stream, const uint16_t *bias = nullptr);
// M >= 2 rows on the matrix cores with the subnormal nibble unpack and the K
// quarters reduced inside the workgroup (no workspace), for K with
// mma_fits(N, K, M, bias != nullptr); y f16 or yf f32 as launch_gemv_mfma.
// cand set: each workgroup also leaves its largest argmax_key of every row's
// results in cand[m * mma_blocks(N) + workgroup] (M * mma_blocks(N) keys).
// bias set: the MLX affine format (scales and biases [N][K/64]).
bool mma_fits(int N, int K, int M, bool aff = false);
int mma_blocks(int N);
q4_status launch_gemv_mma(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                          uint16_t *y, float *yf, int64_t ldy, int N, int K, int M,
                          hipStream_t stream, unsigned long long *cand = nullptr,
                          const uint16_t *bias = nullptr);
// One matrix-core launch for mt <= 16 activation rows. With mfma_splits(K) > 1
// it leaves f32 partials part[ks][m][n] (mfma_part_bytes(N, K) bytes) and
// writes neither y nor yf; otherwise the results go to yf (f32) when set, else
// to y (f16).
int mfma_splits(int K);
size_t mfma_part_bytes(int N, int K);
q4_status launch_mfma_rows(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                           uint16_t *y, float *yf, int64_t ldy, int N, int K, int mt,
                           float *part, hipStream_t stream, const uint16_t *bias = nullptr);
// RoPE + KV append from a stored qkv vector, and decode attention (q4_attn.hip)
q4_status launch_rope_append(const uint16_t *qkv, const RopeArgs &r, hipStream_t stream);
// part: f32 scratch of attention_part_bytes(r), or nullptr for the library
// workspace of the stream
size_t attention_part_bytes(const RopeArgs &r);
q4_status launch_attention(const uint16_t *q, const uint16_t *kv, const RopeArgs &r,
                           int64_t max_len, uint16_t *out, hipStream_t stream,
                           float *part = nullptr);
// LM head and greedy argmax (q4_lmhead.hip)
q4_status launch_gemv_f32(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                          float *y, int64_t ldy, int N, int K, int M, hipStream_t stream);
q4_status launch_argmax(const float *v, int64_t ld, int N, int M, int32_t *index,
                        hipStream_t stream);
q4_status launch_lm_head_argmax(const uint32_t *W, const uint16_t *S, const uint16_t *x,
                                int64_t ldx, float *logits, int64_t ldl, int32_t *tokens, int N,
                                int K, int M, hipStream_t stream);
// Prefill matmul on the matrix cores (q4_gemm.hip): exact weights, or
// weights rounded to f16 when exact is false; bias set: the MLX affine format
// (scales and biases [N][K/64], exact weights only).
q4_status launch_gemm(const uint32_t *W, const uint16_t *S, const uint16_t *X, int64_t ldx,
                      uint16_t *Y, int64_t ldy, int N, int K, int M, bool exact,
                      hipStream_t stream, const uint16_t *bias = nullptr);
// M = 2..4 activation rows with the single-row kernel's arithmetic per row
// (bit-identical to M single-row matvecs) when M * K <= 24576 (staging in LDS);
// given the symmetric format's N, not for M >= 3 on LM-head-sized matrices
// (N K >= 2^26) that the matrix-core kernel takes (its time does not grow with
// M: the Qwen3-4B LM head at M = 4 measured 53 against 72 us).
bool gemv_rows_fits(int M, int K, int64_t N = 0);
// (yf set: f32 outputs there, y ignored)
q4_status launch_gemv_rows(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                           uint16_t *y, int64_t ldy, int N, int K, int M, hipStream_t stream,
                           const uint16_t *bias = nullptr, float *yf = nullptr);
q4_status launch_gemv_batched(const uint32_t *W, const uint16_t *S, const uint16_t *x,
                              int64_t ldx, uint16_t *y, int64_t ldy, int N, int K, int M,
                              hipStream_t stream);
q4_status launch_add_rmsnorm(const uint16_t *a, const uint16_t *res_in, const uint16_t *gamma,
                             uint16_t *out, uint16_t *res_out, int D, int M, float eps,
                             hipStream_t stream);
q4_status launch_silu_mul(const uint16_t *gu, uint16_t *out, int F, int M, hipStream_t stream);
q4_status launch_pack(const uint8_t *codes, uint32_t *packed, int64_t words, hipStream_t stream);
q4_status launch_unpack(const uint32_t *packed, uint8_t *codes, int64_t words, hipStream_t stream);
q4_status launch_moe(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                     const uint16_t *route_w, const uint16_t *x, int64_t ldx,
                     int64_t x_slot_stride, uint16_t *y, int E, int N, int K, int T, int TOPK,
                     int epi_silu, hipStream_t stream);

// ---------------------------------------------------------------------------
// Device side
// ---------------------------------------------------------------------------

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Round an f32 value to binary16, nearest even (the default mode of
// v_cvt_f16_f32). The empty asm makes the f32 value opaque, so the compiler
// cannot fuse a preceding multiply into a single-rounding v_fma_mix*_f16 in
// some kernels and not in others: every path rounds the same f32 value.
__device__ __forceinline__ uint16_t f2h(float f)
{
    asm("" : "+v"(f));  // opaque (no fusion across the rounding), freely scheduled
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// silu(g) * u in f32, g and u already binary16 values. One definition for every
// kernel, so fused and unfused paths give identical bits.
__device__ __forceinline__ float silu_mul_f(float g, float u)
{
    // g * sigma(g) with the hardware reciprocal (v_rcp_f32, within 1 ulp)
    float s = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
    return s * u;
}

// Canonical order of an RMSNorm's sum of squares over a row of D values:
// thread t visits the 8-element chunks c = t, t + 256, ... ([8c, 8c + 8) cut at
// D), elements in order, ss = fmaf(v, v, ss); then block_sum_256. Every kernel
// that normalises (standalone or as a matvec prologue) follows it, so their
// results are bit-identical.

// Cross-lane sums without the LDS crossbar (ds_bpermute, which a shuffle
// becomes): DPP moves inside each 16-lane row, permlane swaps across rows.
// dpp<CTRL>(v): v of another lane of the row (CTRL: 0xB1 lane i ^ 1, 0x4E
// lane i ^ 2, 0x141 lane 7 - i within each 8, 0x128 lane i ^ 8).
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Cross-row exchanges of a wave (rows = lanes 16r .. 16r + 15): swap16
// exchanges row 1 of a with row 0 of b and row 3 of a with row 2 of b; swap32
// exchanges rows 2, 3 of a with rows 0, 1 of b. Written as inline assembly:
// this compiler has generated code that reads one output of the permlane-swap
// builtins twice and the other not at all. The s_nop give the wait states
// between a VALU write and the swap's read, and between the swap and a read of
// its results, which the compiler cannot insert around inline assembly.
__device__ __forceinline__ void swap16(uint32_t &a, uint32_t &b)
{
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 0" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ void swap32(uint32_t &a, uint32_t &b)
{
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 0" : "+v"(a), "+v"(b));
}

// v(lane) + v(lane ^ 16), the same bits in both lanes of a pair
__device__ __forceinline__ float add_xor16(float v)
{
    uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
    swap16(a, b);
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// v(lane) + v(lane ^ 32), the same bits in both lanes of a pair
__device__ __forceinline__ float add_xor32(float v)
{
    uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
    swap32(a, b);
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Sum over each aligned segment of w lanes (w = 8, 16, 32 or 64), in one fixed
// order; every lane of a segment ends with the same bits. The runtime-w form
// performs the same steps.
__device__ __forceinline__ float segment_sum(float v, int w)
{
    if (w >= 64)
        v = add_xor32(v);
    if (w >= 32)
        v = add_xor16(v);
    if (w >= 16)
        v += dpp<0x128>(v);
    v += dpp<0x141>(v);
    v += dpp<0x4E>(v);
    v += dpp<0xB1>(v);
    return v;
}

// Maximum (fmaxf) over each aligned segment of w lanes, as segment_sum;
// every lane of a segment ends with the same value.
__device__ __forceinline__ float segment_max(float v, int w)
{
    if (w >= 64) {
        uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
        swap32(a, b);
        v = fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
    }
    if (w >= 32) {
        uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
        swap16(a, b);
        v = fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
    }
    if (w >= 16)
        v = fmaxf(v, dpp<0x128>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0xB1>(v));
    return v;
}

// Sum over the four lanes of each aligned quad (partners i ^ 1, then i ^ 2).
__device__ __forceinline__ float quad_sum(float v)
{
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    return v;
}

// 1 / sqrt(mean + eps) of an RMSNorm from its sum of squares over D values:
// the hardware reciprocal and reciprocal square root (v_rcp_f32, v_rsq_f32,
// each within 1 ulp) as rsq(ss * rcp(D) + eps), no IEEE division. One
// definition for every kernel that normalises, so their results agree bit
// for bit.
__device__ __forceinline__ float rms_inv(float ss, int D, float eps)
{
    return __builtin_amdgcn_rsqf(fmaf(ss, __builtin_amdgcn_rcpf((float)D), eps));
}

// Block-wide sum over 256 threads in a fixed order: segment_sum over each
// wave, then the four wave totals added in wave order. `red` is 4 floats of LDS.
__device__ __forceinline__ float block_sum_256(float v, float *red)
{
    v = segment_sum(v, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        red[wave] = v;
    __syncthreads();
    float t = ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();
    return t;
}

// Order-preserving 64-bit key of (value, index) for a greedy argmax: a larger
// value gives a larger key and, between equal values, the smaller index does;
// -0 equals +0 and a NaN ranks above every number. Key 0 is below every value.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx)
{
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    if (v != v)
        u = 0xFFFFFFFFu;                       // NaN: above +inf (0xFF800000)
    else if (v == 0.0f)
        u = 0x80000000u;                       // either zero
    else
        u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)u << 32) | (0xFFFFFFFFu - idx);
}

__device__ __forceinline__ int32_t argmax_index(unsigned long long key)
{
    return (int32_t)(0xFFFFFFFFu - (uint32_t)key);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long k)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(k, off, 64);
        k = o > k ? o : k;
    }
    return k;
}

// One RoPE pair of a decode step (the fused QKV epilogue and the unfused
// kernel share it, so their results are identical): pair p of the
// (n_heads + 2 n_kv) * head_dim / 2 pairs, x1 and x2 the stored f16 values of
// rows head * head_dim + i and + head_dim / 2. Query pairs are rotated into
// q_out, key pairs rotated into the cache, value pairs copied into it. The
// angle pos * base^(-2i / head_dim) is taken in binary64 and reduced to
// [-pi, pi] there; its cosine and sine are then taken in f32 (error ~1e-7),
// the rotation in f32.
// The part of a pair's work that needs no matvec result, split off so that a
// fused epilogue can take it (the position, the angle, the cache page) while
// the weights stream: rope_pair_prepare with the step's position, then
// rope_pair_finish with the pair's values.
struct RopePair {
    float c, s;
    uint16_t *dst;  // the pair's first element (q_out or the cache slot); null: nothing stored
    int half;
    bool rotate;    // Q and K pairs; V pairs are copied
};

__device__ __forceinline__ RopePair rope_pair_prepare(const RopeArgs &r, int p, int pos)
{
    RopePair o;
    o.half = r.head_dim >> 1;
    const int head = p / o.half, i = p - head * o.half;
    o.c = 1.f;
    o.s = 0.f;
    o.dst = nullptr;
    o.rotate = head < r.n_heads + r.n_kv;
    if (o.rotate) {
        const double theta =
            (double)pos * exp2(-2.0 * (double)i / (double)r.head_dim * log2((double)r.base));
        const double two_pi = 6.283185307179586;
        const float red = (float)(theta - two_pi * rint(theta / two_pi));
        sincosf(red, &o.s, &o.c);
    }
    if (head < r.n_heads) {
        o.dst = r.q_out + head * r.head_dim + i;
        return o;
    }
    const bool is_v = head >= r.n_heads + r.n_kv;
    const int kvh = head - r.n_heads - (is_v ? r.n_kv : 0);
    if (pos < 0)
        return o;
    const int lp = pos / r.page_size, slot = pos - lp * r.page_size;
    if (lp >= r.max_pages)
        return o;
    const int pp = r.page_table[lp];
    if (pp < 0 || pp >= r.n_pages)
        return o;
    o.dst = r.kv + (((size_t)pp * 2 + (is_v ? 1 : 0)) * r.n_kv + kvh) *
                       (size_t)r.page_size * r.head_dim +
            (size_t)slot * r.head_dim + i;
    return o;
}

__device__ __forceinline__ void rope_pair_finish(const RopePair &o, float x1, float x2)
{
    if (!o.dst)
        return;
    const float y1 = x1 * o.c - x2 * o.s;
    const float y2 = x2 * o.c + x1 * o.s;
    o.dst[0] = f2h(o.rotate ? y1 : x1);
    o.dst[o.half] = f2h(o.rotate ? y2 : x2);
}

__device__ __forceinline__ void rope_pair_store(const RopeArgs &r, int p, float x1, float x2)
{
    rope_pair_finish(rope_pair_prepare(r, p, *r.pos), x1, x2);
}

}  // namespace q4
