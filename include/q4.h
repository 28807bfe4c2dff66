/*
 * q4.h -- C ABI of libq4, an MI355X (gfx950) library for the single-token
 * decode matmul over q4f16_1 group-quantised int4 weights, with the
 * dequantisation fused into the matmul.
 *
 * Weight format (Zero TVM Documentation, "Q4F16 quantization format"):
 *   packed  uint32 [N][K/8]   eight 4-bit codes per word; element k = 8j + i of
 *                             a row lives in word j, bits 4i..4i+3
 *   scales  binary16 [N][K/32] one scale per 32 consecutive K elements
 *   value   w[n][k] = (code - 7) * scale[n][k/32]
 * y = W x: weights are stored by output row (the "NT" matmul of RESEARCH.md,
 * "1. Dispatch profile", and shader 5 of "WGSL Kernel Roles").
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device, owned
 *     by the caller; the library never frees them. binary16 values are passed
 *     as uint16_t bit patterns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without synchronising. Argument errors are detected on
 *     the host before anything is enqueued and returned synchronously; nothing
 *     is launched then. Kernel faults surface at the caller's next
 *     synchronisation.
 *   - Shapes: K must be a multiple of 32 and at most Q4_MAX_K; dimensions are
 *     positive. Alignment: packed weights and the activation input of a matvec
 *     16 bytes (row strides of batched / MoE activations multiples of 8
 *     elements); every other binary16 vector 2 bytes. Tensors from a device
 *     allocator satisfy this.
 *   - Outputs must not overlap any input of the same call (Q4_EALIAS). This
 *     includes the residual rule of the ping-pong buffers (Zero TVM
 *     Documentation, "Ping-pong residual buffers"): res_out != res_in.
 *   - Accumulation is f32; results are rounded to binary16 (nearest even).
 *     Results are bit-identical from run to run for the same arguments on the
 *     same device (fixed reduction order, no floating-point atomics).
 *   - Entry points that need scratch memory (split partials of the batched,
 *     prefill and attention kernels, MoE routing and partials, LM-head argmax
 *     candidates, the stack's intermediate vectors) use a library-owned
 *     workspace per (device, stream); concurrent calls on distinct streams do
 *     not share it. q4_workspace_bytes / q4_attention_workspace_bytes /
 *     q4_stack_workspace_bytes give what a call needs and q4_workspace_reserve
 *     allocates it ahead of time. A call whose need exceeds the stream's
 *     workspace allocates a larger one (hipMalloc; the header is cleared in
 *     stream order, no device synchronisation) and keeps the replaced buffer
 *     until q4_workspace_release, since work already enqueued or a HIP graph
 *     captured earlier may still use it. During HIP graph capture on the
 *     stream nothing is allocated: such a call returns Q4_ERANGE and enqueues
 *     nothing, so reserve before capturing. Calls on one stream are ordered by
 *     the stream and may share the workspace.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum q4_status {
    Q4_OK = 0,
    Q4_EINVAL = 1, /* NULL pointer, non-positive dimension, unknown mode      */
    Q4_ESHAPE = 2, /* K % 32 != 0, odd row count for a SiLU split, ...       */
    Q4_EALIGN = 3, /* pointer not aligned as stated above                    */
    Q4_EALIAS = 4, /* an output overlaps an input                            */
    Q4_ERANGE = 5, /* a size beyond a supported maximum                      */
    Q4_EHIP = 6    /* HIP runtime error (allocation, launch)                 */
} q4_status;

/* Largest supported reduction length (the activation vector is staged in LDS). */
#define Q4_MAX_K 24576

/* A hipStream_t. */
typedef void *q4_stream;

/* Library version string. */
const char *q4_version(void);

/* Message for the last non-OK status returned on the calling thread. */
const char *q4_last_error(void);

/* Number of bytes one int4 weight occupies in this format (0.5625 = 4.5 bits):
 * K/8 * 4 + K/32 * 2 bytes per row of K weights. Host-only helper. */
double q4_bytes_per_weight(void);

/* ---------------------------------------------------------------------------
 * q4_pack -- "Q4F16 quantization format": codes u8[N][K] with values 0..15 ->
 * packed u32[N][K/8], code of element 8j+i into bits 4i..4i+3 of word j.
 * Codes above 15 are not checked on the device; only their low 4 bits are used.
 * Alignment: packed 16 bytes; codes any.
 */
q4_status q4_pack(const uint8_t *codes, uint32_t *packed, int64_t N, int64_t K,
                  q4_stream stream);

/* q4_unpack -- inverse of q4_pack (u32[N][K/8] -> u8[N][K]); a test hook. */
q4_status q4_unpack(const uint32_t *packed, uint8_t *codes, int64_t N, int64_t K,
                    q4_stream stream);

/* ---------------------------------------------------------------------------
 * q4_gemv -- the decode matmul ("WGSL Kernel Roles", shader 5 "int4 Matmul";
 * RESEARCH.md "Matmul Shader Analysis"):
 *   y[n] = f16( sum_k (code[n][k] - 7) * S[n][k/32] * x[k] ),  f32 accumulation
 * W u32[N][K/8], S f16[N][K/32], x f16[K], y f16[N].
 */
q4_status q4_gemv(const uint32_t *W, const uint16_t *S, const uint16_t *x, uint16_t *y,
                  int64_t N, int64_t K, q4_stream stream);

/* ---------------------------------------------------------------------------
 * q4_gemv_batched -- M activation rows sharing one weight read (BENCH.md,
 * "Falsifiability result: batched M-dim matmul"):
 *   y[m*ldy + n] = f16( sum_k w[n][k] * x[m*ldx + k] ),  m = 0..M-1
 * ldx >= K, ldy >= N (elements). 1 <= M <= Q4_MAX_M.
 */
#define Q4_MAX_M 64
q4_status q4_gemv_batched(const uint32_t *W, const uint16_t *S, const uint16_t *x,
                          int64_t ldx, uint16_t *y, int64_t ldy, int64_t N, int64_t K,
                          int64_t M, q4_stream stream);

/* ---------------------------------------------------------------------------
 * q4_moe_gemv -- one expert stage of a MoE layer (BENCH.md, "MoE chunked
 * prefill (2026-08-13)": every (token, slot) runs its own expert's matmul; the
 * slot outputs are combined by routing weight; "MoE Phase B": grouping the
 * (token, slot) rows by expert so each expert's weights are read once).
 *   W u32[E][N][K/8], S f16[E][N][K/32]   expert weights, stacked
 *   ids i32[T][TOPK]                       expert of (token t, slot s), 0 <= id < E
 *   x                                      activation of (t, s) starts at
 *                                          x + t*ldx + s*x_slot_stride (f16[K]);
 *                                          x_slot_stride = 0 shares one row per token
 *   v(t, s) = W[ids[t][s]] . x(t, s)       (f32)
 * Modes:
 *   epi_silu != 0, route_w == NULL : y f16[T][TOPK][N/2] =
 *        f16( silu(f16(v[:N/2])) * f16(v[N/2:]) )   (gate_up stage; N even)
 *   epi_silu == 0, route_w == NULL : y f16[T][TOPK][N] = f16(v)
 *   epi_silu == 0, route_w f16[T][TOPK] : y f16[T][N] =
 *        f16( sum_s route_w[t][s] * v(t, s) )       (down stage + combine)
 * epi_silu together with route_w is Q4_EINVAL. The (t, s) pairs are grouped by
 * expert, so each distinct expert's weights are read once per group of its
 * pairs: groups of up to 4 pairs while experts get about two pairs each or
 * fewer (at most 256 pairs), otherwise groups of up to 16 on the matrix cores;
 * an expert with more pairs than one group re-reads its rows, mostly from
 * cache. Exception: the down stage with the combine at T*TOPK <= 32 runs token
 * by token (each token's experts read for that token, the combine in the same
 * kernel). Ids are validated on the device; an out-of-range id contributes
 * zeros. T*TOPK <= Q4_MAX_PAIRS.
 */
#define Q4_MAX_PAIRS 4096
q4_status q4_moe_gemv(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                      const uint16_t *route_w, const uint16_t *x, int64_t ldx,
                      int64_t x_slot_stride, uint16_t *y, int64_t E, int64_t N, int64_t K,
                      int64_t T, int64_t TOPK, int epi_silu, q4_stream stream);

/* ---------------------------------------------------------------------------
 * q4_add_rmsnorm -- fused residual add + RMSNorm ("WGSL Kernel Roles", shaders 2
 * and 7; "Ping-pong residual buffers"), for M rows of length D:
 *   res_out = f16(a + res_in)          (a == NULL: res_out = res_in)
 *   out     = f16( res_out / sqrt(mean(res_out^2) + eps) * gamma )
 * a, res_in, out, res_out f16[M][D]; gamma f16[D]. res_out must not overlap
 * res_in; out must not overlap a or res_in. D <= Q4_MAX_K.
 */
q4_status q4_add_rmsnorm(const uint16_t *a, const uint16_t *res_in, const uint16_t *gamma,
                         uint16_t *out, uint16_t *res_out, int64_t D, int64_t M, float eps,
                         q4_stream stream);

/* ---------------------------------------------------------------------------
 * q4_silu_mul -- split-SiLU-multiply (RESEARCH.md, "1. Dispatch profile": gate
 * split + SiLU + elementwise multiply; shader 6 "Fused FFN": gate and up share
 * one row-concatenated matrix, gate first):
 *   out[m][i] = f16( silu(gu[m][i]) * gu[m][F + i] ),  silu(z) = z / (1 + e^-z)
 * gu f16[M][2F], out f16[M][F].
 */
q4_status q4_silu_mul(const uint16_t *gu, uint16_t *out, int64_t F, int64_t M,
                      q4_stream stream);

/* ---------------------------------------------------------------------------
 * q4_gemv_ex -- q4_gemv with a fused prologue and/or epilogue. The results are
 * bit-identical to the unfused sequence of calls named below.
 *   prologue (norm_gamma != NULL): x is a residual f16[K]; the matvec input is
 *                        q4_add_rmsnorm(NULL, x, norm_gamma, h, ., K, 1, eps)'s h,
 *                        computed inside the matvec (norm_gamma 16-byte aligned).
 *                        Not combined with Q4_EPI_ADD_RMSNORM.
 *   Q4_EPI_NONE        : as q4_gemv.
 *   Q4_EPI_SILU_MUL    : rows [0, N/2) are gate, [N/2, N) are up; y f16[N/2] =
 *                        q4_silu_mul(q4_gemv(W, S, x)).   N even.
 *   Q4_EPI_ADD_RMSNORM : t = q4_gemv(W, S, x) (f16[N], not stored);
 *                        q4_add_rmsnorm(t, res_in, gamma, y, res_out, N, 1, eps).
 *                        N <= Q4_MAX_K. Runs as the matvec with the residual add
 *                        in its per-row epilogue followed by a one-workgroup
 *                        normalisation (no synchronisation inside a kernel).
 */
typedef enum q4_epi_kind { Q4_EPI_NONE = 0, Q4_EPI_SILU_MUL = 1, Q4_EPI_ADD_RMSNORM = 2 } q4_epi_kind;

typedef struct q4_epilogue {
    int kind;                    /* q4_epi_kind                                  */
    const uint16_t *res_in;      /* ADD_RMSNORM: running residual f16[N]          */
    const uint16_t *gamma;       /* ADD_RMSNORM: norm weights f16[N]              */
    uint16_t *res_out;           /* ADD_RMSNORM: new residual f16[N], != res_in   */
    float eps;                   /* both norms                                    */
    const uint16_t *norm_gamma;  /* prologue norm weights f16[K], or NULL         */
} q4_epilogue;

q4_status q4_gemv_ex(const uint32_t *W, const uint16_t *S, const uint16_t *x, uint16_t *y,
                     int64_t N, int64_t K, const q4_epilogue *epi, q4_stream stream);

/* ---------------------------------------------------------------------------
 * q4_gemv_affine -- the MLX affine 4-bit format (Zero TVM Documentation, the
 * Qwen3.6-35B-A3B entry: affine w = s * q + b, group 64; BENCH.md, "Affine
 * wide loads"): M activation rows, unsigned codes q (0..15) packed as for
 * q4_gemv (the pages give no other order), scales and biases per 64 codes:
 *   y[m*ldy + n] = f16( sum_k (S[n][k/64] * q[n][k] + B[n][k/64]) * x[m*ldx + k] )
 * W u32[N][K/8], S and B f16[N][K/64] (2-byte aligned), K % 64 == 0; x and y
 * as for q4_gemv_batched. f32 accumulation; M = 1 runs the single-row kernel,
 * M = 2..4 with M*K <= 24576 the same arithmetic per row (each row equals its
 * M = 1 result bit for bit), larger M the matrix cores (exact integer
 * operands, scale and bias in f32).
 */
q4_status q4_gemv_affine(const uint32_t *W, const uint16_t *S, const uint16_t *B,
                         const uint16_t *x, int64_t ldx, uint16_t *y, int64_t ldy, int64_t N,
                         int64_t K, int64_t M, q4_stream stream);

/* ---------------------------------------------------------------------------
 * q4_gemm -- the prefill (many-token) int4 matmul (BENCH.md, "Tiled batched
 * GEMM (2026-08-12)" and "Subgroup-matrix GEMM graduated": chunked prefill
 * runs the matmul over M >= 64 activation rows at once, f16 matrix-unit
 * fragments with f32 accumulation):
 *   y[m*ldy + n] = f16( sum_k w[n][k] * x[m*ldx + k] ),  m = 0..M-1
 * with, by `weights`:
 *   Q4_GEMM_EXACT      w = (q - 7) * s exactly, as q4_gemv_batched (the
 *                      codes enter the matrix cores, each 32-value group's
 *                      f32 sum is scaled by s);
 *   Q4_GEMM_F16_WEIGHT w = f16((q - 7) * s): the dequantised weight rounded to
 *                      binary16, as the format's dequantization formula
 *                      computes it (Zero TVM Documentation, "Q4F16
 *                      quantization format"); no per-group scaling of sums.
 * W, S as for q4_gemv; x f16 rows, 16-byte aligned, ldx % 8 == 0, ldx >= K;
 * y f16, 2-byte aligned, ldy >= N, caller-owned, not overlapping the inputs.
 * 1 <= M <= Q4_MAX_GEMM_M. f32 accumulation over K in an order fixed by
 * (M, N, K). A call whose tile grid would fill under half the GPU splits K:
 * f32 partials in the library workspace of the stream, summed in split order
 * by a second kernel; otherwise one kernel launch. Q4_EINVAL for an unknown
 * `weights`.
 */
#define Q4_MAX_GEMM_M 65536
typedef enum q4_gemm_weights { Q4_GEMM_EXACT = 0, Q4_GEMM_F16_WEIGHT = 1 } q4_gemm_weights;
q4_status q4_gemm(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                  uint16_t *y, int64_t ldy, int64_t N, int64_t K, int64_t M, int weights,
                  q4_stream stream);

/* ---------------------------------------------------------------------------
 * q4_gemm_affine -- the prefill matmul in the MLX affine format (Zero TVM
 * Documentation, the Qwen3.6-35B-A3B entry: w = s * q + b, group 64; BENCH.md,
 * "Subgroup-matrix GEMM graduated" and "GEMM microbench": the _affine prefill
 * GEMMs at the qwen3mlx chunk shapes):
 *   y[m*ldy + n] = f16( sum_k (S[n][k/64] * q[n][k] + B[n][k/64]) * x[m*ldx + k] )
 * W, S, B as for q4_gemv_affine (K % 64 == 0); x, y as for q4_gemm.
 * 1 <= M <= Q4_MAX_GEMM_M. Exact weights: the codes q enter the matrix cores
 * and each 32-value sum is scaled by s; the bias enters as b * (sum of x over
 * the group), the group sums split into binary16 hi and lo. Uses the library workspace of the
 * stream (the group sums, and f32 partials when K is split).
 */
q4_status q4_gemm_affine(const uint32_t *W, const uint16_t *S, const uint16_t *B,
                         const uint16_t *x, int64_t ldx, uint16_t *y, int64_t ldy, int64_t N,
                         int64_t K, int64_t M, q4_stream stream);

/* ---------------------------------------------------------------------------
 * LM head and greedy sampling (Zero TVM Documentation, "Decode loop": the LM
 * head's matmul writes the logits and an argmax picks the next token; shader
 * 10, "Argmax Sampler"; RESEARCH.md, "Why Fewer Dispatches Matter", the
 * per-decode dispatch table and the note below it: the LM head is the int4
 * matmul with f32 outputs, for a stable argmax).
 *
 * q4_gemv_f32 -- the matmul with f32 outputs (no rounding to f16):
 *   y[m*ldy + n] = sum_k w[n][k] * x[m*ldx + k],  f32 accumulation, m < M
 * W, S as for q4_gemv; x f16 rows (16-byte aligned, ldx % 8 == 0, ldx >= K);
 * y f32 (4-byte aligned, ldy >= N), caller-owned, must not overlap the inputs.
 * 1 <= M <= Q4_MAX_M.
 */
q4_status q4_gemv_f32(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                      float *y, int64_t ldy, int64_t N, int64_t K, int64_t M,
                      q4_stream stream);

/* q4_argmax -- greedy token of each of M rows of N f32 values v[m*ld ...]:
 *   index[m] = the smallest n whose v[m*ld + n] is the row's maximum,
 * where -0 equals +0 and a NaN ranks above every number (the first NaN wins);
 * the pages leave ties and NaN open. v 4-byte aligned, ld >= N, 1 <= N <
 * 2^31, 1 <= M <= 65535; index int32[M] (4-byte aligned), caller-owned, must
 * not overlap v. Deterministic (no atomics).
 */
q4_status q4_argmax(const float *v, int64_t ld, int64_t N, int64_t M, int32_t *index,
                    q4_stream stream);

/* q4_lm_head_argmax -- q4_gemv_f32 into logits (f32, rows of ldl >= N) and
 * q4_argmax of each row into tokens int32[M], in one call (for M = 1, and on
 * the matrix cores for M >= 2 where the activation rows fit in LDS, the
 * matmul's workgroups hand their rows' best (value, index) to a one-workgroup
 * reduction; the logits are not read back). Arguments and errors as for the
 * two calls; logits and tokens must not overlap each other or the inputs.
 */
q4_status q4_lm_head_argmax(const uint32_t *W, const uint16_t *S, const uint16_t *x,
                            int64_t ldx, float *logits, int64_t ldl, int32_t *tokens, int64_t N,
                            int64_t K, int64_t M, q4_stream stream);

/* ---------------------------------------------------------------------------
 * RoPE, paged KV cache and decode attention (Zero TVM Documentation, "KV
 * cache"; shader 3 "QKV + RoPE + KV-append (fused, decode)"; shader 4 "Paged
 * Attention"; shaders 8 and 9 "KV Append" and "RoPE"; BENCH.md, split-K
 * attention with a combine step).
 *
 * Geometry: the QKV matvec rows are n_heads query heads, then n_kv key heads,
 * then n_kv value heads, head_dim rows each. RoPE turns the pairs (i, i +
 * head_dim/2) of every query and key head by theta_i = pos * rope_base^(-2i /
 * head_dim) (the pages pair dim and dim + 48 of a 96-dim head; they give no
 * base: Phi-3 uses 10000). Cache: kv_pages f16
 * [n_pages][2 (K, V)][n_kv][page_size][head_dim]; position t lives in physical
 * page page_table[t / page_size], slot t % page_size (the pages use 16-slot
 * pages and an identity table for one sequence). The position is read from
 * device memory (pos: one int32), as the pages bind a position map.
 * Positions, table entries or pages outside the table (max_pages entries) or
 * the cache (n_pages pages) are neither written nor read.
 * Rounding: the Q, K, V rows are rounded to f16 as a separate matvec stores
 * them, rotated in f32 (angles from binary64) and stored as f16.
 */
typedef struct q4_attn_desc {
    int64_t n_heads;    /* query heads */
    int64_t n_kv;       /* key/value heads; divides n_heads */
    int64_t head_dim;   /* multiple of 8, <= 256 */
    int64_t page_size;  /* slots per page */
    int64_t max_pages;  /* entries of page_table */
    int64_t n_pages;    /* physical pages in kv_pages */
    float rope_base;    /* e.g. 10000 */
} q4_attn_desc;

/* Bytes of one cache page: 2 * n_kv * page_size * head_dim * 2. Host-only. */
int64_t q4_kv_page_bytes(const q4_attn_desc *desc);

/* q4_qkv_rope_append -- the fused decode step: qkv = W . x (W u32[N][K/8],
 * S f16[N][K/32], N = (n_heads + 2 n_kv) * head_dim, x f16[K]); q_out f16
 * [n_heads * head_dim] gets the rotated query; the rotated key and the value
 * are written to the cache slot of *pos. */
q4_status q4_qkv_rope_append(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t K,
                             const q4_attn_desc *desc, const int32_t *pos,
                             const int32_t *page_table, uint16_t *kv_pages, uint16_t *q_out,
                             q4_stream stream);

/* q4_rope_append -- the same step from an already stored f16 qkv vector
 * [(n_heads + 2 n_kv) * head_dim] (the unfused path; bit-identical results). */
q4_status q4_rope_append(const uint16_t *qkv, const q4_attn_desc *desc, const int32_t *pos,
                         const int32_t *page_table, uint16_t *kv_pages, uint16_t *q_out,
                         q4_stream stream);

/* q4_attention_decode -- out f16[n_heads * head_dim]: for query head h and
 * key/value head h / (n_heads / n_kv),
 *   out[h] = sum_{t <= *pos} softmax_t(q_h . k_t / sqrt(head_dim)) v_t
 * over the cached positions 0 .. *pos. The positions are split over up to 32
 * workgroups per head (max_len, the caller's bound on *pos + 1, sizes the
 * split; a larger *pos is still attended in full, only more slowly) whose
 * partial softmax states (max, sum, weighted values) a second kernel combines
 * in split order. q f16, 16-byte aligned; out must not overlap
 * q or the cache. */
q4_status q4_attention_decode(const uint16_t *q, const uint16_t *kv_pages,
                              const int32_t *page_table, const int32_t *pos, int64_t max_len,
                              const q4_attn_desc *desc, uint16_t *out, q4_stream stream);

/* ---------------------------------------------------------------------------
 * q4_stack_decode -- one decode token through a stack of decoder layers whose
 * attention is replaced by the single-position identity on the V slice
 * (Zero TVM Documentation, "Decode loop": per layer QKV matmul -> attention ->
 * O matmul -> add+RMSNorm -> gate_up + SiLU*mul -> down -> add+RMSNorm; with one
 * cached position the softmax weight is 1, so attention returns V).
 * Per layer L (r, h: residual and normalised hidden state, f16[d]):
 *   qkv = f16(Wqkv[L] . h)                       Wqkv: n_qkv x d
 *   o   = f16(Wo[L] . qkv[v_off : v_off + dv])   Wo:   d x dv
 *   (r, h) = add_rmsnorm(o, r, gamma_post[L])
 *   u   = silu_mul(f16(Wgu[L] . h))              Wgu:  2f x d
 *   dn  = f16(Wdn[L] . u)                        Wdn:  d x f
 *   (r, h) = add_rmsnorm(dn, r, L+1 < n_layers ? gamma_in[L+1] : gamma_final)
 * The descriptor holds HOST arrays of n_layers DEVICE pointers per matrix, and
 * device pointers to gamma_in f16[n_layers][d], gamma_post f16[n_layers][d],
 * gamma_final f16[d]. r_in/h_in are read, r_out/h_out written (f16[d]); inputs
 * and outputs must not overlap. trace (may be NULL) receives the state after
 * every layer: f16[n_layers][2][d] as (r, h) pairs.
 * mode: Q4_STACK_AUTO and Q4_STACK_MULTI (the same path) run four matvec
 * launches per layer; the dependent steps are ordered by kernel boundaries,
 * which on gfx950 cost less than any grid-wide synchronisation inside a
 * kernel while the weights stream. Any other mode is Q4_EINVAL.
 * Workspace: q4_stack_workspace_bytes(desc, NULL) bytes of the stream's.
 */
typedef struct q4_stack_desc {
    int64_t n_layers, d, f, n_qkv, v_off, dv;
    float eps;
    const uint32_t *const *Wqkv;
    const uint16_t *const *Sqkv;
    const uint32_t *const *Wo;
    const uint16_t *const *So;
    const uint32_t *const *Wgu;
    const uint16_t *const *Sgu;
    const uint32_t *const *Wdn;
    const uint16_t *const *Sdn;
    const uint16_t *gamma_in;
    const uint16_t *gamma_post;
    const uint16_t *gamma_final;
    int mode; /* q4_stack_mode */
} q4_stack_desc;

typedef enum q4_stack_mode { Q4_STACK_AUTO = 0, Q4_STACK_MULTI = 1 } q4_stack_mode;

q4_status q4_stack_decode(const q4_stack_desc *desc, const uint16_t *r_in,
                          const uint16_t *h_in, uint16_t *r_out, uint16_t *h_out,
                          uint16_t *trace, q4_stream stream);

/* q4_stack_decode_noalloc -- q4_stack_decode (same arguments, same kernels, the
 * same bits) for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. It allocates nothing
 * and uses no stream workspace: its intermediate vectors live in a fixed
 * scratch array of Q4_NOALLOC_SCRATCH_BYTES in the library's device image,
 * one per GPU, held until the process ends. A stack whose
 * q4_stack_workspace_bytes(desc, NULL) exceeds that is Q4_ERANGE (nothing
 * enqueued). Every call on a GPU shares that GPU's scratch: calls that overlap
 * on one GPU (e.g. on two streams at once) race; calls ordered on one stream do
 * not. The scratch keeps the last call's contents; nothing in it needs to
 * start at zero. */
#define Q4_NOALLOC_SCRATCH_BYTES (1 << 20)
q4_status q4_stack_decode_noalloc(const q4_stack_desc *desc, const uint16_t *r_in,
                                  const uint16_t *h_in, uint16_t *r_out, uint16_t *h_out,
                                  uint16_t *trace, q4_stream stream);

/* q4_stack_decode_attn -- the same stack with the real attention step in place
 * of the single-position identity ("Decode loop"): per layer
 *   q = RoPE(f16(Wqkv[L] . h)) queries; the rotated key and the value of the
 *       token written to kv_pages[L] at *pos (as q4_qkv_rope_append)
 *   a = attention of q over positions 0 .. *pos of kv_pages[L]
 *       (as q4_attention_decode)
 *   o = f16(Wo[L] . a), then add+RMSNorm, gate_up + SiLU*mul, down, add+RMSNorm
 *       as in q4_stack_decode.
 * The descriptor's n_qkv must be (n_heads + 2 n_kv) * head_dim and dv must be
 * n_heads * head_dim (v_off is unused). attn->kv_pages is a HOST array of
 * n_layers device caches of attn->geom's geometry; the page table and the
 * position (device) are shared by the layers. Workspace:
 * q4_stack_workspace_bytes(desc, attn) bytes of the stream's. */
typedef struct q4_stack_attn {
    const q4_attn_desc *geom;
    uint16_t *const *kv_pages;
    const int32_t *page_table;
    const int32_t *pos;
    int64_t max_len;
} q4_stack_attn;

q4_status q4_stack_decode_attn(const q4_stack_desc *desc, const q4_stack_attn *attn,
                               const uint16_t *r_in, const uint16_t *h_in, uint16_t *r_out,
                               uint16_t *h_out, uint16_t *trace, q4_stream stream);

/* ---------------------------------------------------------------------------
 * Workspace (the library-owned scratch of a stream; see the conventions at the
 * top). Sizes are in bytes and include a 256-byte header; 0 means the call
 * needs none (or the arguments are invalid). Host-only; no device work.
 *
 * q4_workspace_bytes -- the most any one matmul-family call on an N x K
 * matrix with M activation rows needs: q4_gemv_batched, q4_gemv_f32,
 * q4_gemv_affine (M <= Q4_MAX_M), q4_lm_head_argmax (M <= Q4_MAX_M),
 * q4_argmax over M rows of N (M <= 65535), q4_gemm and q4_gemm_affine (M <=
 * Q4_MAX_GEMM_M, any ldx), q4_moe_gemv with M = T * TOPK pairs (any E).
 * q4_gemv, q4_gemv_ex, q4_qkv_rope_append, q4_rope_append, q4_add_rmsnorm,
 * q4_silu_mul, q4_pack and q4_unpack use no workspace.
 */
size_t q4_workspace_bytes(int64_t N, int64_t K, int64_t M);

/* q4_attention_workspace_bytes -- what q4_attention_decode needs for the
 * geometry and max_len (its split partials; 0 when one split suffices). */
size_t q4_attention_workspace_bytes(const q4_attn_desc *desc, int64_t max_len);

/* q4_stack_workspace_bytes -- what q4_stack_decode (attn NULL) or
 * q4_stack_decode_attn needs: the intermediate vectors of a layer and, with
 * attention, its output and split partials. */
size_t q4_stack_workspace_bytes(const q4_stack_desc *desc, const q4_stack_attn *attn);

/* q4_workspace_reserve -- makes the workspace of `stream` on the current
 * device at least `bytes` large (allocating as a growing call does; Q4_ERANGE
 * during graph capture on the stream if it would have to grow). After it, no
 * call on the stream whose need is at most `bytes` allocates or synchronises,
 * so such calls may be captured into a HIP graph. */
q4_status q4_workspace_reserve(q4_stream stream, size_t bytes);

/* q4_workspace_release -- synchronises `stream` and frees its workspace and
 * every buffer it replaced. The caller guarantees that no HIP graph still to
 * be launched uses them. Q4_OK if the stream has none. */
q4_status q4_workspace_release(q4_stream stream);

/* Measurement hook (not part of the method): q4_timer_arm(slot) makes the next
 * matvec kernel that this thread launches through libq4 record its dispatch
 * start and end (the kernel's own execution, as a profiler's kernel trace
 * sees it) on the slot's library-owned HIP events; q4_timer_read(slot, &us)
 * waits for that launch and returns its duration in microseconds. slot: 0..63,
 * per thread. Q4_EINVAL for a bad slot or a slot never armed and launched. A
 * slot armed while another is armed replaces it. */
q4_status q4_timer_arm(int slot);
q4_status q4_timer_read(int slot, float *us);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
