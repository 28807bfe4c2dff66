/*
 * q4_oracle.c -- plain, slow, single-threaded CPU oracle for the int4
 * (q4f16_1) decode path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library may include, link,
 * load or call this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it. It shares no code, header, table or
 * constant generator with the GPU library.
 *
 * Every floating-point value is computed in IEEE binary64 from the exact
 * binary16 / uint32 input bytes. The only roundings to binary16 happen where
 * the library's call boundary stores binary16 (a residual that is written back,
 * an activation that feeds the next matmul); results that are compared against
 * the GPU are returned in binary64.
 *
 * Sources (the Zero-TVM pages):
 *  - Zero TVM Documentation, "Q4F16 quantization format": eight 4-bit codes per
 *    uint32, element i of a word in bits 4i..4i+3; one binary16 scale per 32
 *    weights; value = (nibble - 7) * scale; q_weight shapes [N, K/8], q_scale
 *    shapes [N, K/32].
 *  - Zero TVM Documentation, "WGSL Kernel Roles", shader 5 (int4 Matmul):
 *    dequantize-on-the-fly matvec y = W x, weights stored by output row.
 *  - Zero TVM Documentation, shaders 2 and 7 (RMSNorm, Fused Add + RMSNorm):
 *    residual_out = A + B; output = x / sqrt(mean(x^2) + eps) * gamma.
 *  - RESEARCH.md, "1. Dispatch profile": the FFN gate split, SiLU and
 *    elementwise multiply; Zero TVM Documentation, shader 6 (Fused FFN): the
 *    gate and up projections share one row-concatenated gate_up matrix.
 *  - BENCH.md, "Falsifiability result: batched M-dim matmul": M activation rows
 *    sharing one weight matrix.
 *  - BENCH.md, "MoE chunked prefill (2026-08-13)": each (token, slot) runs its
 *    own expert's matmul and the slot outputs are combined by routing weight.
 *  - Zero TVM Documentation, "Decode loop" and "Ping-pong residual buffers":
 *    the per-layer chain QKV -> attention -> O -> add+norm -> FFN -> add+norm,
 *    then the LM head and the argmax of its logits (shader 10, "Argmax
 *    Sampler"); RESEARCH.md, "Why Fewer Dispatches Matter": the LM head's
 *    matmul writes f32 logits.
 *
 * Every function here has at least one pin in tests/test_oracle_pins.py
 * (closed forms, special cases, brute force, library routines); none is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary64, written from the format definition.       */
/* ------------------------------------------------------------------------ */

/* Exact decode of a binary16 bit pattern. */
double q4o_h2d(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* zero or subnormal */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);  /* (1.m) * 2^(e-15) */
    return sign ? -v : v;
}

/* binary64 -> binary16, round to nearest, ties to even; overflow to infinity. */
uint16_t q4o_d2h(double v)
{
    if (isnan(v))
        return 0x7E00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a >= 65520.0)                 /* halfway between 65504 and 2^16 rounds up */
        return sign | 0x7C00;
    if (a < ldexp(1.0, -14)) {        /* subnormal range: multiples of 2^-24 */
        double q = rint(ldexp(a, 24)); /* rint rounds half to even */
        return sign | (uint16_t)q;    /* q == 1024 is the smallest normal */
    }
    int ex;
    frexp(a, &ex);                    /* a = f * 2^ex, f in [0.5, 1) */
    int E = ex - 1;                   /* a in [2^E, 2^(E+1)) */
    double m = rint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (m >= 2048.0) {
        m = 1024.0;
        E += 1;
    }
    if (E + 15 >= 31)
        return sign | 0x7C00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)m - 1024));
}

void q4o_h2d_array(const uint16_t *h, double *d, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        d[i] = q4o_h2d(h[i]);
}

void q4o_d2h_array(const double *d, uint16_t *h, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        h[i] = q4o_d2h(d[i]);
}

/* ------------------------------------------------------------------------ */
/* Packing (Q4F16 quantization format).                                      */
/* ------------------------------------------------------------------------ */

/* Element k = 8j + i of a row goes to word j, bits 4i..4i+3. */
void q4o_pack(const uint8_t *codes, uint32_t *words, int64_t n, int64_t k)
{
    int64_t wpr = k / 8;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < wpr; ++j) {
            uint32_t w = 0;
            for (int i = 0; i < 8; ++i)
                w |= (uint32_t)(codes[r * k + 8 * j + i] & 0xF) << (4 * i);
            words[r * wpr + j] = w;
        }
}

/* The code of element k of row r. */
static int q4o_code(const uint32_t *words, int64_t k_total, int64_t r, int64_t k)
{
    uint32_t w = words[r * (k_total / 8) + k / 8];
    return (int)((w >> (4 * (k % 8))) & 0xF);
}

void q4o_unpack(const uint32_t *words, uint8_t *codes, int64_t n, int64_t k)
{
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c)
            codes[r * k + c] = (uint8_t)q4o_code(words, k, r, c);
}

/* Dequantised weight (q - 7) * scale, exact in binary64. */
static double q4o_weight(const uint32_t *W, const uint16_t *S, int64_t k_total,
                         int64_t r, int64_t k)
{
    int q = q4o_code(W, k_total, r, k);
    double s = q4o_h2d(S[r * (k_total / 32) + k / 32]);
    return (double)(q - 7) * s;
}

void q4o_dequant(const uint32_t *W, const uint16_t *S, int64_t n, int64_t k, double *w)
{
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c)
            w[r * k + c] = q4o_weight(W, S, k, r, c);
}

/* ------------------------------------------------------------------------ */
/* Matvec: y[r] = sum_k w[r][k] * x[k]  (int4 Matmul, shader 5).             */
/* ------------------------------------------------------------------------ */

static double q4o_row_dot(const uint32_t *W, const uint16_t *S, const uint16_t *x,
                          int64_t k, int64_t r)
{
    double acc = 0.0;
    for (int64_t c = 0; c < k; ++c)
        acc += q4o_weight(W, S, k, r, c) * q4o_h2d(x[c]);
    return acc;
}

void q4o_gemv(const uint32_t *W, const uint16_t *S, const uint16_t *x,
              int64_t n, int64_t k, double *y)
{
    for (int64_t r = 0; r < n; ++r)
        y[r] = q4o_row_dot(W, S, x, k, r);
}

/* Selected rows only, for spot checks of full-size outputs. */
void q4o_gemv_rows(const uint32_t *W, const uint16_t *S, const uint16_t *x,
                   int64_t n, int64_t k, const int64_t *rows, int64_t nrows, double *y)
{
    (void)n;
    for (int64_t i = 0; i < nrows; ++i)
        y[i] = q4o_row_dot(W, S, x, k, rows[i]);
}

/* M activation rows x[m*ldx ...] sharing W: y[m][r]. */
void q4o_gemv_batched(const uint32_t *W, const uint16_t *S, const uint16_t *x,
                      int64_t ldx, int64_t n, int64_t k, int64_t m, double *y)
{
    for (int64_t b = 0; b < m; ++b)
        for (int64_t r = 0; r < n; ++r)
            y[b * n + r] = q4o_row_dot(W, S, x + b * ldx, k, r);
}

/* ------------------------------------------------------------------------ */
/* Fused add + RMSNorm (shaders 2 and 7).                                    */
/* ------------------------------------------------------------------------ */

/*
 * For each of m rows of length d:
 *   res_out = f16(a + r)            (a == NULL: res_out = r, a plain RMSNorm)
 *   out     = res_out / sqrt(mean(res_out^2) + eps) * gamma    (binary64)
 * The residual is rounded because the ping-pong residual buffers hold binary16.
 */
void q4o_add_rmsnorm(const uint16_t *a, const uint16_t *r, const uint16_t *gamma,
                     int64_t d, int64_t m, double eps, uint16_t *res_out, double *out)
{
    for (int64_t b = 0; b < m; ++b) {
        const uint16_t *rr = r + b * d;
        uint16_t *ro = res_out + b * d;
        for (int64_t i = 0; i < d; ++i)
            ro[i] = a ? q4o_d2h(q4o_h2d(a[b * d + i]) + q4o_h2d(rr[i])) : rr[i];
        double ss = 0.0;
        for (int64_t i = 0; i < d; ++i) {
            double v = q4o_h2d(ro[i]);
            ss += v * v;
        }
        double inv = 1.0 / sqrt(ss / (double)d + eps);
        for (int64_t i = 0; i < d; ++i)
            out[b * d + i] = q4o_h2d(ro[i]) * inv * q4o_h2d(gamma[i]);
    }
}

/* ------------------------------------------------------------------------ */
/* Split-SiLU-multiply: gu = [gate | up] -> silu(gate) * up.                 */
/* ------------------------------------------------------------------------ */

static double q4o_silu(double z)
{
    return z / (1.0 + exp(-z));
}

void q4o_silu_mul(const uint16_t *gu, int64_t f, int64_t m, double *out)
{
    for (int64_t b = 0; b < m; ++b)
        for (int64_t i = 0; i < f; ++i) {
            double g = q4o_h2d(gu[b * 2 * f + i]);
            double u = q4o_h2d(gu[b * 2 * f + f + i]);
            out[b * f + i] = q4o_silu(g) * u;
        }
}

/* ------------------------------------------------------------------------ */
/* MoE expert stage (per (token, slot) expert matmul + routing combine).     */
/* ------------------------------------------------------------------------ */

/*
 * W: uint32[E][n][k/8], S: f16[E][n][k/32], ids: int32[t][topk].
 * The activation of (token i, slot s) starts at x + i*ldx + s*x_slot_stride.
 * mode (matching the library):
 *   epi_silu != 0                : y[i][s][n/2] = silu(f16(v)[:n/2]) * f16(v)[n/2:]
 *   epi_silu == 0, route_w NULL  : y[i][s][n]   = v
 *   epi_silu == 0, route_w given : y[i][n]      = sum_s route_w[i][s] * v
 * where v = W[ids[i][s]] . x(i, s) in binary64.
 */
void q4o_moe_stage(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                   const uint16_t *route_w, const uint16_t *x, int64_t ldx,
                   int64_t x_slot_stride, int64_t e_count, int64_t n, int64_t k,
                   int64_t t, int64_t topk, int epi_silu, double *y)
{
    (void)e_count;
    double *v = (double *)malloc(sizeof(double) * (size_t)n);
    uint16_t *vh = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n);
    int64_t wpm = n * (k / 8), spm = n * (k / 32);
    if (!epi_silu && route_w)
        memset(y, 0, sizeof(double) * (size_t)(t * n));
    for (int64_t i = 0; i < t; ++i)
        for (int64_t s = 0; s < topk; ++s) {
            int64_t e = ids[i * topk + s];
            const uint16_t *xv = x + i * ldx + s * x_slot_stride;
            q4o_gemv(W + e * wpm, S + e * spm, xv, n, k, v);
            if (epi_silu) {
                int64_t f = n / 2;
                for (int64_t r = 0; r < n; ++r)
                    vh[r] = q4o_d2h(v[r]);
                q4o_silu_mul(vh, f, 1, y + (i * topk + s) * f);
            } else if (!route_w) {
                memcpy(y + (i * topk + s) * n, v, sizeof(double) * (size_t)n);
            } else {
                double w = q4o_h2d(route_w[i * topk + s]);
                for (int64_t r = 0; r < n; ++r)
                    y[i * n + r] += w * v[r];
            }
        }
    free(v);
    free(vh);
}

/* ------------------------------------------------------------------------ */
/* One decoder layer of the stack (decode loop, attention := V slice).       */
/* ------------------------------------------------------------------------ */

/*
 *   qkv = f16(Wqkv . h)                     rows n_qkv
 *   v   = qkv[v_off : v_off + dv]           single-position attention output
 *   o   = f16(Wo . v)                       rows d, K = dv
 *   (r1, h1) = add_rmsnorm(o, r, gamma_post)
 *   u   = f16(silu_mul(f16(Wgu . h1)))      Wgu rows 2f
 *   dn  = f16(Wdn . u)                      rows d, K = f
 *   (r2, h2) = add_rmsnorm(dn, r1, gamma_next)
 * r_out = r2, h_out = f16(h2), h_out_f64 = h2 (may be NULL).
 */
void q4o_layer(int64_t d, int64_t f, int64_t n_qkv, int64_t v_off, int64_t dv,
               const uint32_t *Wqkv, const uint16_t *Sqkv,
               const uint32_t *Wo, const uint16_t *So,
               const uint32_t *Wgu, const uint16_t *Sgu,
               const uint32_t *Wdn, const uint16_t *Sdn,
               const uint16_t *gamma_post, const uint16_t *gamma_next, double eps,
               const uint16_t *r_in, const uint16_t *h_in,
               uint16_t *r_out, uint16_t *h_out, double *h_out_f64)
{
    int64_t big = n_qkv > 2 * f ? n_qkv : 2 * f;
    double *tmp = (double *)malloc(sizeof(double) * (size_t)big);
    uint16_t *qkv = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n_qkv);
    uint16_t *o = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);
    uint16_t *r1 = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);
    uint16_t *h1 = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);
    uint16_t *gu = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(2 * f));
    uint16_t *u = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)f);
    uint16_t *dn = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);

    q4o_gemv(Wqkv, Sqkv, h_in, n_qkv, d, tmp);
    q4o_d2h_array(tmp, qkv, n_qkv);
    q4o_gemv(Wo, So, qkv + v_off, d, dv, tmp);
    q4o_d2h_array(tmp, o, d);
    q4o_add_rmsnorm(o, r_in, gamma_post, d, 1, eps, r1, tmp);
    q4o_d2h_array(tmp, h1, d);
    q4o_gemv(Wgu, Sgu, h1, 2 * f, d, tmp);
    q4o_d2h_array(tmp, gu, 2 * f);
    q4o_silu_mul(gu, f, 1, tmp);
    q4o_d2h_array(tmp, u, f);
    q4o_gemv(Wdn, Sdn, u, d, f, tmp);
    q4o_d2h_array(tmp, dn, d);
    q4o_add_rmsnorm(dn, r1, gamma_next, d, 1, eps, r_out, tmp);
    q4o_d2h_array(tmp, h_out, d);
    if (h_out_f64)
        memcpy(h_out_f64, tmp, sizeof(double) * (size_t)d);

    free(tmp); free(qkv); free(o); free(r1); free(h1); free(gu); free(u); free(dn);
}

/*
 * n_layers layers in sequence. Per-layer weights are given as arrays of
 * pointers. gamma_post: f16[n_layers][d]; gamma_in: f16[n_layers][d] (the input
 * norm of each layer; layer L's second add+norm uses gamma_in[L+1]);
 * gamma_final: f16[d] (used after the last layer). r, h hold the state in
 * binary16 and are updated in place. h_f64 (may be NULL) receives the final
 * normalised output in binary64. trace_r / trace_h (may be NULL) receive the
 * state after every layer, f16[n_layers][d].
 */
void q4o_stack(int64_t n_layers, int64_t d, int64_t f, int64_t n_qkv, int64_t v_off,
               int64_t dv,
               const uint32_t *const *Wqkv, const uint16_t *const *Sqkv,
               const uint32_t *const *Wo, const uint16_t *const *So,
               const uint32_t *const *Wgu, const uint16_t *const *Sgu,
               const uint32_t *const *Wdn, const uint16_t *const *Sdn,
               const uint16_t *gamma_in, const uint16_t *gamma_post,
               const uint16_t *gamma_final, double eps,
               uint16_t *r, uint16_t *h, double *h_f64,
               uint16_t *trace_r, uint16_t *trace_h)
{
    uint16_t *r2 = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);
    uint16_t *h2 = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);
    for (int64_t L = 0; L < n_layers; ++L) {
        const uint16_t *g_next = (L + 1 < n_layers) ? gamma_in + (L + 1) * d : gamma_final;
        q4o_layer(d, f, n_qkv, v_off, dv, Wqkv[L], Sqkv[L], Wo[L], So[L], Wgu[L], Sgu[L],
                  Wdn[L], Sdn[L], gamma_post + L * d, g_next, eps, r, h, r2, h2,
                  (L + 1 == n_layers) ? h_f64 : NULL);
        memcpy(r, r2, sizeof(uint16_t) * (size_t)d);
        memcpy(h, h2, sizeof(uint16_t) * (size_t)d);
        if (trace_r)
            memcpy(trace_r + L * d, r, sizeof(uint16_t) * (size_t)d);
        if (trace_h)
            memcpy(trace_h + L * d, h, sizeof(uint16_t) * (size_t)d);
    }
    free(r2);
    free(h2);
}

/* ------------------------------------------------------------------------ */
/* LM head and greedy sampling (Zero TVM Documentation, "Decode loop": the   */
/* LM-head matmul writes the logits and the argmax picks the next token;     */
/* shader 10 "Argmax Sampler"; RESEARCH.md, "Why Fewer Dispatches Matter",   */
/* the per-decode dispatch table and the note below it: the LM head is the   */
/* f32-output variant of the int4 matmul, kept in f32 for a stable argmax).  */
/* ------------------------------------------------------------------------ */

/*
 * Index of the largest of n >= 1 values. The pages take the next token as
 * the argmax of the logits and leave ties and NaN open; read here as: ties go
 * to the smallest index, -0 equals +0 (IEEE comparison), and a NaN counts as
 * larger than every number, so the first NaN wins.
 */
int64_t q4o_argmax(const double *v, int64_t n)
{
    int64_t best = 0;
    for (int64_t i = 1; i < n; ++i) {
        if (isnan(v[best]))
            break;
        if (isnan(v[i]) || v[i] > v[best])
            best = i;
    }
    return best;
}

/*
 * For each of m activation rows x[b*ldx ...]: logits[b][r] = W[r] . x_b in
 * binary64 (no rounding: the f32 logits of the library are compared against
 * them) and token[b] = the argmax of those exact logits.
 */
void q4o_lm_head(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                 int64_t n, int64_t k, int64_t m, double *logits, int64_t *token)
{
    for (int64_t b = 0; b < m; ++b) {
        for (int64_t r = 0; r < n; ++r)
            logits[b * n + r] = q4o_row_dot(W, S, x + b * ldx, k, r);
        token[b] = q4o_argmax(logits + b * n, n);
    }
}

/* ------------------------------------------------------------------------ */
/* RoPE, paged KV cache and decode attention (Zero TVM Documentation,       */
/* "KV cache"; shader 3 "QKV + RoPE + KV-append"; shader 4 "Paged            */
/* Attention"; shaders 8 and 9, "KV Append" and "RoPE"; "Phi-3 model         */
/* constants"; BENCH.md, split-K attention).                                 */
/* ------------------------------------------------------------------------ */

/*
 * Rotary position embedding of n_heads head vectors of head_dim values at
 * position pos: within each head the pairs are (i, i + head_dim/2), as the
 * fused QKV shader pairs dim and dim + 48 of a 96-dim head, and pair i turns
 * by theta_i = pos * base^(-2i/head_dim). The pages give no base; 10000 is the
 * caller's reading.
 */
void q4o_rope(const double *in, double *out, int64_t n_heads, int64_t head_dim, int64_t pos,
              double base)
{
    const int64_t half = head_dim / 2;
    for (int64_t h = 0; h < n_heads; ++h) {
        const double *a = in + h * head_dim;
        double *b = out + h * head_dim;
        for (int64_t i = 0; i < half; ++i) {
            const double theta = (double)pos * pow(base, -2.0 * (double)i / (double)head_dim);
            const double c = cos(theta), s = sin(theta);
            b[i] = a[i] * c - a[i + half] * s;
            b[i + half] = a[i + half] * c + a[i] * s;
        }
    }
}

/*
 * The decode step around the QKV matvec for one token at position pos: qkv =
 * f16(W . x) (rows: n_heads query heads, then n_kv key heads, then n_kv value
 * heads, head_dim each), as the separate matvec stores it; q and k rotated in
 * binary64 and returned unrounded (q_rot [n_heads][head_dim], k_rot
 * [n_kv][head_dim]); v is the stored f16 slice, returned as its values.
 */
void q4o_qkv_rope(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t k,
                  int64_t n_heads, int64_t n_kv, int64_t head_dim, int64_t pos, double base,
                  double *q_rot, double *k_rot, double *v)
{
    const int64_t nq = n_heads * head_dim, nk = n_kv * head_dim;
    const int64_t n = nq + 2 * nk;
    double *y = (double *)malloc(sizeof(double) * (size_t)n);
    for (int64_t r = 0; r < n; ++r)
        y[r] = q4o_h2d(q4o_d2h(q4o_row_dot(W, S, x, k, r)));
    q4o_rope(y, q_rot, n_heads, head_dim, pos, base);
    q4o_rope(y + nq, k_rot, n_kv, head_dim, pos, base);
    for (int64_t r = 0; r < nk; ++r)
        v[r] = y[nq + nk + r];
    free(y);
}

/*
 * Decode attention for one query token over L cached positions: K and V are
 * f16 [L][n_kv][head_dim] in position order (as read back from the pages);
 * query head h uses key/value head h / (n_heads / n_kv). For each head
 *   out[h] = sum_t softmax_t(q_h . k_t * scale) v_t,  scale = 1/sqrt(head_dim)
 * in binary64, the softmax taken with its maximum subtracted.
 */
void q4o_attention(const uint16_t *q, const uint16_t *kc, const uint16_t *vc, int64_t L,
                   int64_t n_heads, int64_t n_kv, int64_t head_dim, double *out)
{
    const int64_t group = n_heads / n_kv;
    const double scale = 1.0 / sqrt((double)head_dim);
    double *s = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    for (int64_t h = 0; h < n_heads; ++h) {
        const int64_t kvh = h / group;
        double m = -INFINITY;
        for (int64_t t = 0; t < L; ++t) {
            double dot = 0.0;
            for (int64_t j = 0; j < head_dim; ++j)
                dot += q4o_h2d(q[h * head_dim + j]) *
                       q4o_h2d(kc[(t * n_kv + kvh) * head_dim + j]);
            s[t] = dot * scale;
            if (s[t] > m)
                m = s[t];
        }
        double l = 0.0;
        for (int64_t t = 0; t < L; ++t) {
            s[t] = exp(s[t] - m);
            l += s[t];
        }
        for (int64_t j = 0; j < head_dim; ++j) {
            double acc = 0.0;
            for (int64_t t = 0; t < L; ++t)
                acc += s[t] * q4o_h2d(vc[(t * n_kv + kvh) * head_dim + j]);
            out[h * head_dim + j] = acc / l;
        }
    }
    free(s);
}

/*
 * One decoder layer with the real attention step in place of the
 * single-position identity (Zero TVM Documentation, "Decode loop": QKV with
 * RoPE and the KV append -> paged attention -> O -> add+norm -> FFN ->
 * add+norm). The token sits at position pos; kc_prev, vc_prev hold the cached
 * f16 rows of positions 0 .. pos-1 ([pos][n_kv][hd]). Rounded to f16 where a
 * call stores f16: the rotated query, the appended key and value (returned in
 * k_new, v_new), the attention output, then as q4o_layer.
 */
void q4o_layer_attn(int64_t d, int64_t f, int64_t n_heads, int64_t n_kv, int64_t hd,
                    int64_t pos, double base,
                    const uint32_t *Wqkv, const uint16_t *Sqkv,
                    const uint32_t *Wo, const uint16_t *So,
                    const uint32_t *Wgu, const uint16_t *Sgu,
                    const uint32_t *Wdn, const uint16_t *Sdn,
                    const uint16_t *gamma_post, const uint16_t *gamma_next, double eps,
                    const uint16_t *r_in, const uint16_t *h_in,
                    const uint16_t *kc_prev, const uint16_t *vc_prev,
                    uint16_t *r_out, uint16_t *h_out, double *h_out_f64,
                    uint16_t *k_new, uint16_t *v_new)
{
    const int64_t nq = n_heads * hd, nk = n_kv * hd, L = pos + 1;
    double *qd = (double *)malloc(sizeof(double) * (size_t)nq);
    double *kd = (double *)malloc(sizeof(double) * (size_t)nk);
    double *vd = (double *)malloc(sizeof(double) * (size_t)nk);
    uint16_t *q = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)nq);
    uint16_t *kc = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(L * nk));
    uint16_t *vc = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(L * nk));
    int64_t big = 2 * f > nq ? 2 * f : nq;
    double *tmp = (double *)malloc(sizeof(double) * (size_t)big);
    uint16_t *att = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)nq);
    uint16_t *o = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);
    uint16_t *ra = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);
    uint16_t *h1 = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);
    uint16_t *gu = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(2 * f));
    uint16_t *u = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)f);
    uint16_t *dn = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)d);

    q4o_qkv_rope(Wqkv, Sqkv, h_in, d, n_heads, n_kv, hd, pos, base, qd, kd, vd);
    q4o_d2h_array(qd, q, nq);
    q4o_d2h_array(kd, k_new, nk);
    q4o_d2h_array(vd, v_new, nk);
    if (pos > 0) {
        memcpy(kc, kc_prev, sizeof(uint16_t) * (size_t)(pos * nk));
        memcpy(vc, vc_prev, sizeof(uint16_t) * (size_t)(pos * nk));
    }
    memcpy(kc + pos * nk, k_new, sizeof(uint16_t) * (size_t)nk);
    memcpy(vc + pos * nk, v_new, sizeof(uint16_t) * (size_t)nk);
    q4o_attention(q, kc, vc, L, n_heads, n_kv, hd, tmp);
    q4o_d2h_array(tmp, att, nq);
    q4o_gemv(Wo, So, att, d, nq, tmp);
    q4o_d2h_array(tmp, o, d);
    q4o_add_rmsnorm(o, r_in, gamma_post, d, 1, eps, ra, tmp);
    q4o_d2h_array(tmp, h1, d);
    q4o_gemv(Wgu, Sgu, h1, 2 * f, d, tmp);
    q4o_d2h_array(tmp, gu, 2 * f);
    q4o_silu_mul(gu, f, 1, tmp);
    q4o_d2h_array(tmp, u, f);
    q4o_gemv(Wdn, Sdn, u, d, f, tmp);
    q4o_d2h_array(tmp, dn, d);
    q4o_add_rmsnorm(dn, ra, gamma_next, d, 1, eps, r_out, tmp);
    q4o_d2h_array(tmp, h_out, d);
    if (h_out_f64)
        memcpy(h_out_f64, tmp, sizeof(double) * (size_t)d);

    free(qd); free(kd); free(vd); free(q); free(kc); free(vc); free(tmp); free(att);
    free(o); free(ra); free(h1); free(gu); free(u); free(dn);
}

/* ------------------------------------------------------------------------ */
/* MLX affine 4-bit format (Zero TVM Documentation, "Qwen3.6-35B-A3B MoE":    */
/* affine w = s*q + b with group 64; BENCH.md, "Affine wide loads": a group  */
/* of 64 codes is eight uint32 words, a vec2<u32> one quarter of it).       */
/* ------------------------------------------------------------------------ */

/*
 * Weight r, k of an affine matrix: codes packed as in the Q4F16 format
 * (element i of a word in bits 4i..4i+3; the pages give no other order), q
 * unsigned in 0..15, and w = S[r][k/64] * q + B[r][k/64] with binary16 scales
 * and biases, exact in binary64.
 */
static double q4o_weight_affine(const uint32_t *W, const uint16_t *S, const uint16_t *B,
                                int64_t k_total, int64_t r, int64_t k)
{
    const int q = q4o_code(W, k_total, r, k);
    const int64_t gi = r * (k_total / 64) + k / 64;
    return q4o_h2d(S[gi]) * (double)q + q4o_h2d(B[gi]);
}

/* y[b][r] = sum_k w[r][k] * x[b*ldx + k] for m activation rows, binary64. */
void q4o_gemv_affine(const uint32_t *W, const uint16_t *S, const uint16_t *B,
                     const uint16_t *x, int64_t ldx, int64_t n, int64_t k, int64_t m, double *y)
{
    for (int64_t b = 0; b < m; ++b)
        for (int64_t r = 0; r < n; ++r) {
            double acc = 0.0;
            for (int64_t c = 0; c < k; ++c)
                acc += q4o_weight_affine(W, S, B, k, r, c) * q4o_h2d(x[b * ldx + c]);
            y[b * n + r] = acc;
        }
}

/* ------------------------------------------------------------------------ */
/* Weights rounded to binary16 first (Zero TVM Documentation, "Q4F16       */
/* quantization format": the dequantization formula multiplies f16(q - 7)   */
/* by the binary16 scale in binary16, so the weight it yields is the exact  */
/* product rounded once to binary16).                                       */
/* ------------------------------------------------------------------------ */

/* y[b][r] = sum_k f16((q - 7) * s) * x[b*ldx + k] for m rows, binary64 sums. */
void q4o_gemv_w16(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                  int64_t n, int64_t k, int64_t m, double *y)
{
    for (int64_t b = 0; b < m; ++b)
        for (int64_t r = 0; r < n; ++r) {
            double acc = 0.0;
            for (int64_t c = 0; c < k; ++c) {
                const double w16 = q4o_h2d(q4o_d2h(q4o_weight(W, S, k, r, c)));
                acc += w16 * q4o_h2d(x[b * ldx + c]);
            }
            y[b * n + r] = acc;
        }
}
