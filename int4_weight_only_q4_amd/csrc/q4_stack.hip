// Persistent decode-stack kernel for gfx950: one cooperative launch runs every
// layer of one token ("Decode loop" of the Zero TVM Documentation with the
// attention replaced by the single-position identity on the V slice).
//
// Layout: one 1024-thread workgroup per CU, all co-resident (cooperative
// launch). Each matvec of a layer is one "phase"; workgroup b owns a contiguous
// slice of the phase's rows, i.e. a contiguous byte range of the packed
// weights, and its compute lanes take consecutive 16-byte groups of that range,
// so every weight load instruction is fully coalesced.
//
// Synchronisation between phases is carried by the data: every element that a
// later phase reads (V slice, residual after O, SiLU output, residual after
// down) is published as a 32-bit word = binary16 value | 16-bit phase tag << 16,
// written with a device-coherent store; a consumer accepts a chunk only when
// every word carries the expected tag (and re-reads it otherwise). No counters,
// fences or grid barriers are needed (each word is written atomically and
// validates itself). So that consumers do not flood the memory system with
// polls, each workgroup also writes one tagged flag word per phase after its
// data, and consumers watch the flags (one 1 KB read per poll) before they read
// the data once. Every wait is bounded: on a timeout the kernel records an
// error and finishes.
//
// Roles inside a workgroup: waves 0..11 stream the weights (non-temporal loads)
// and compute; waves 12..15 (256 lanes) do every cross-workgroup read: they
// poll the flags, read the published vector and stage it into LDS (with the
// RMSNorm where the phase has one, in the 256-lane canonical summation order).
// The vector-memory counter of a wave retires in order, so keeping the polls
// and reads in waves that never have weight loads outstanding keeps them off
// the weights' queue. A phase's weight loads are issued right after the
// previous phase is published, so they stream while the workgroup waits for
// the other workgroups. The Q/K rows of the QKV matrix (not consumed
// downstream) are computed while the staging waves wait for the V slice. The
// residual rows a workgroup adds in the O and down epilogues are exactly the
// rows it wrote itself, so they stay in LDS.
//
// Results are bit-identical to the multi-kernel path (q4_gemv_ex chain): the
// per-row reduction replays the single-call kernel's lane order (LPR lanes,
// groups j, j + LPR, ..., fused multiply-add, then the xor butterfly), and the
// RMSNorm uses the canonical summation order.
#include "q4_dequant.h"
#include "q4_stack.h"

namespace q4 {
namespace {

constexpr int kThreads = kStackThreads;
constexpr int kWavesPB = kThreads / 64;
constexpr int kCompute = kStackCompute;   // waves 0..11: weights and compute
constexpr int kStagers = kThreads - kCompute;  // waves 12..15: cross-workgroup reads
static_assert(kStagers == 256, "the staging lanes replay the 256-lane canonical order");
constexpr unsigned kSpinLimit = 1u << 21;  // polls before giving up

// Every published vector (and its flag array) exists in kCopies copies, one per
// group of workgroups (blockIdx mod kCopies, i.e. per XCD under the round-robin
// dispatch of workgroups to XCDs): a producer writes all copies, a consumer
// reads its own, so each copy is read by nb / kCopies workgroups and no few
// memory channels serve the whole chip's reads.
constexpr int kCopies = kStackCopies;

__device__ __forceinline__ int my_copy() { return (int)(blockIdx.x % kCopies); }

// Element i of a published vector of length len, all copies.
__device__ __forceinline__ void publish(uint32_t *buf, int len, int i, uint16_t v, uint32_t tag)
{
    const uint32_t w = (uint32_t)v | (tag << 16);
#pragma unroll
    for (int c = 0; c < kCopies; ++c)
        __hip_atomic_store(buf + (size_t)c * len + i, w, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// One flag word per workgroup and phase kind (all copies), written after its
// data. flags: [kCopies][nb].
__device__ __forceinline__ void publish_flag(uint32_t *flags, int nb, int b, uint32_t tag)
{
    if ((int)threadIdx.x < kCopies)
        __hip_atomic_store(flags + (size_t)threadIdx.x * nb + b, tag, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// One wave: bounded wait until all nb flags of this workgroup's copy carry `tag`.
__device__ __forceinline__ void poll_flags(const uint32_t *flags, int nb, uint32_t tag,
                                           unsigned *err)
{
    const int lane = threadIdx.x & 63;
    flags += (size_t)my_copy() * nb;
    for (unsigned it = 0;; ++it) {
        bool ok = true;
        for (int i = lane; i < nb; i += 64)
            ok = ok && __hip_atomic_load(const_cast<uint32_t *>(flags + i), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == tag;
        if (__all(ok))
            break;
        if (it >= kSpinLimit ||
            ((it & 255) == 255 &&
             __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
            __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

struct Lds {
    uint4 *xs;      // staged activation, pair-interleaved chunks [K/8]
    float *cs;      // 7 * group sums [K/32]
    uint4 *xo;      // the O phase's activation (staged while Q/K still use xs)
    float *co;
    float2 *st;     // per-chunk (scale, group sum of (c - 7) x) [chunks of the phase]
    uint4 *raw;     // residual chunks of a norm [d/8]
    float *rowv;    // SiLU: rounded gate|up row values
    float *lres;    // this workgroup's rows of the residual (O / down slice)
    float *red;     // 4 floats
};

// Weights of one phase for this workgroup: virtual rows v in [0, nv); for a
// SiLU phase the first nrow are gate rows row0.., the next nrow the up rows
// half + row0... Its groups form one contiguous range of the packed matrix (two
// for a SiLU phase), so chunk cl of the workgroup sits at W0[cl] (or W1[cl - n0])
// and its group index within the row is cl mod G.
struct PhaseMap {
    const uint4 *W0, *W1;
    const uint16_t *S0, *S1;
    int G, row0, nrow, half, silu, lpr, ng;
    __device__ int nv() const { return silu ? 2 * nrow : nrow; }
    __device__ int n0() const { return nrow * G; }
    __device__ int row_of(int v) const { return v < nrow ? row0 + v : half + row0 + (v - nrow); }
};

// Compute lanes: issue the loads of this lane's chunks of the phase.
__device__ __forceinline__ void issue_loads(const PhaseMap &m, uint4 (&wv)[kStackNch],
                                            uint32_t (&sv)[kStackNch])
{
    const uint32_t n0 = (uint32_t)m.n0(), total = (uint32_t)(m.silu ? 2 * n0 : n0);
    const uint32_t t = threadIdx.x;
    if (t >= (uint32_t)kCompute)
        return;
#pragma unroll
    for (int i = 0; i < kStackNch; ++i) {
        const uint32_t cl = t + (uint32_t)kCompute * i;
        if (cl < total) {
            if (cl < n0) {
                wv[i] = load_weights(m.W0 + cl);
                sv[i] = load_scale(m.S0 + cl);
            } else {
                wv[i] = load_weights(m.W1 + (cl - n0));
                sv[i] = load_scale(m.S1 + (cl - n0));
            }
        }
    }
}

__device__ __forceinline__ void compute_chunks(const PhaseMap &m, const uint4 (&wv)[kStackNch],
                                               const uint32_t (&sv)[kStackNch], const uint4 *xs,
                                               const float *cs, float2 *st)
{
    const int total = m.silu ? 2 * m.n0() : m.n0();
    const int t = threadIdx.x;
    if (t >= kCompute)
        return;
    const int step = kCompute % m.G;
    int g = t % m.G;
#pragma unroll
    for (int i = 0; i < kStackNch; ++i) {
        const int cl = t + kCompute * i;
        if (cl < total)
            st[cl] = make_float2(h2f(sv[i]), group_dot(wv[i], xs, g, cs[g]));
        g += step;
        if (g >= m.G)
            g -= m.G;
    }
}

// Row value of virtual row v as the single-call kernel forms it: lanes j of an
// LPR-lane segment accumulate groups j, j + LPR, ... with fmaf, then the xor
// butterfly. Called by whole waves; returns the value in lane j == 0 of each
// segment. `v` may be out of range (then the segment computes garbage).
__device__ __forceinline__ float reduce_row(const PhaseMap &m, int v, int j, const float2 *st)
{
    float acc = 0.f;
    if (v < m.nv())
        for (int i = 0; i < m.ng; ++i) {
            const int g = j + m.lpr * i;
            if (g < m.G) {
                const float2 e = st[v * m.G + g];
                acc = fmaf(e.x, e.y, acc);
            }
        }
    return segment_sum(acc, m.lpr);
}

__device__ __forceinline__ bool chunk_ready(const uint64_t (&q)[4], uint32_t tag)
{
    bool ok = true;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        ok = ok && (uint32_t)(q[k] >> 16 & 0xFFFF) == tag && (uint32_t)(q[k] >> 48) == tag;
    return ok;
}

__device__ __forceinline__ void load_chunk_words(const uint32_t *buf, int c, uint64_t (&q)[4])
{
    uint64_t *p = const_cast<uint64_t *>(reinterpret_cast<const uint64_t *>(buf + 8 * c));
#pragma unroll
    for (int k = 0; k < 4; ++k)
        q[k] = __hip_atomic_load(p + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Staging lanes s = 0..255: read chunks c = s + 256 i of this workgroup's copy
// of a tagged buffer of `chunks` chunks, kReadBatch chunks per lane in flight at a time, re-reading a
// chunk until all its words carry `tag` (bounded: on timeout sets *err and
// goes on). fn(c, valid, value) is called for every i by every lane (so it may
// shuffle within the wave).
constexpr int kReadBatch = 4;

template <typename F>
__device__ __forceinline__ void read_tagged(const uint32_t *buf, int chunks, uint32_t tag,
                                            unsigned *err, F &&fn)
{
    const int s = threadIdx.x - kCompute;
    buf += (size_t)my_copy() * chunks * 8;
    for (int base = 0; base < chunks; base += kStagers * kReadBatch) {
        uint64_t q[kReadBatch][4];
#pragma unroll
        for (int i = 0; i < kReadBatch; ++i) {
            const int c = base + s + kStagers * i;
            if (c < chunks)
                load_chunk_words(buf, c, q[i]);
        }
        for (unsigned it = 0;; ++it) {
            bool ok = true;
#pragma unroll
            for (int i = 0; i < kReadBatch; ++i) {
                const int c = base + s + kStagers * i;
                ok = ok && (c >= chunks || chunk_ready(q[i], tag));
            }
            if (ok)
                break;
            if (it >= kSpinLimit ||
                ((it & 1023) == 1023 &&
                 __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
                __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
#pragma unroll
            for (int i = 0; i < kReadBatch; ++i) {
                const int c = base + s + kStagers * i;
                if (c < chunks && !chunk_ready(q[i], tag))
                    load_chunk_words(buf, c, q[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < kReadBatch; ++i) {
            const int c = base + s + kStagers * i;
            uint4 v;
            v.x = (uint32_t)(q[i][0] & 0xFFFF) | (uint32_t)((q[i][0] >> 32 & 0xFFFF) << 16);
            v.y = (uint32_t)(q[i][1] & 0xFFFF) | (uint32_t)((q[i][1] >> 32 & 0xFFFF) << 16);
            v.z = (uint32_t)(q[i][2] & 0xFFFF) | (uint32_t)((q[i][2] >> 32 & 0xFFFF) << 16);
            v.w = (uint32_t)(q[i][3] & 0xFFFF) | (uint32_t)((q[i][3] >> 32 & 0xFFFF) << 16);
            fn(c, c < chunks, v);
        }
    }
}

// Staging lanes: stage a plain (src) or published (tagged, after the flags of
// phase `tag` are all set) K-vector into xs / cs. No barrier inside.
__device__ __forceinline__ void stage_vector(const uint16_t *plain, const uint32_t *tagged,
                                             uint32_t tag, const uint32_t *flags, int nb, int K,
                                             uint4 *xs, float *cs, unsigned *err)
{
    const int chunks = K >> 3;
    const int s = threadIdx.x - kCompute;
    if (plain) {
        for (int base = 0; base < chunks; base += kStagers) {
            const int c = base + s;
            const uint4 v = c < chunks ? reinterpret_cast<const uint4 *>(plain)[c]
                                       : make_uint4(0, 0, 0, 0);
            put_chunk(v, c, c < chunks, xs, cs);
        }
        return;
    }
    poll_flags(flags, nb, tag, err);
    read_tagged(tagged, chunks, tag, err,
                [&](int c, bool valid, uint4 v) { put_chunk(v, c, valid, xs, cs); });
}

// f16(RMSNorm(residual) * gamma) of a published residual, staged into xs / cs
// by the staging lanes in two halves around a workgroup barrier. They form the
// 256-lane canonical order: lane s sums the squares of chunks s, s + 256, ...
// in element order with fused multiply-add, then each wave's xor butterfly,
// then the four wave sums in order. norm_sum also writes the residual to rout,
// norm_apply the normalised values to hout / hout2 (plain binary16, when
// non-null).
__device__ __forceinline__ void norm_sum(const uint32_t *tagged, uint32_t tag,
                                         const uint32_t *flags, int nb, int K, const Lds &l,
                                         unsigned *err, uint16_t *rout)
{
    const int chunks = K >> 3;
    const int s = threadIdx.x - kCompute;
    poll_flags(flags, nb, tag, err);
    float ss = 0.f;
    read_tagged(tagged, chunks, tag, err, [&](int c, bool valid, uint4 v) {
        if (!valid)
            return;
        l.raw[c] = v;
        if (rout)
            reinterpret_cast<uint4 *>(rout)[c] = v;
        float f[8];
        chunk_to_float(v, f);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            ss = fmaf(f[e], f[e], ss);
    });
    ss = segment_sum(ss, 64);
    if ((threadIdx.x & 63) == 0)
        l.red[s >> 6] = ss;
}

__device__ __forceinline__ void norm_apply(const uint16_t *gamma, float eps, int K, const Lds &l,
                                           uint16_t *hout, uint16_t *hout2)
{
    const int chunks = K >> 3;
    const int s = threadIdx.x - kCompute;
    const float tot = ((l.red[0] + l.red[1]) + l.red[2]) + l.red[3];
    const float inv = rms_inv(tot, K, eps);
    for (int base = 0; base < chunks; base += kStagers) {
        const int c = base + s;
        uint4 hv = make_uint4(0, 0, 0, 0);
        if (c < chunks) {
            float f[8], g8[8];
            chunk_to_float(l.raw[c], f);
            chunk_to_float(reinterpret_cast<const uint4 *>(gamma)[c], g8);
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                h[e] = f2h(f[e] * inv * g8[e]);
            hv = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                            h[6] | (h[7] << 16));
            if (hout)
                reinterpret_cast<uint4 *>(hout)[c] = hv;
            if (hout2)
                reinterpret_cast<uint4 *>(hout2)[c] = hv;
        }
        put_chunk(hv, c, c < chunks, l.xs, l.cs);
    }
}

__device__ __forceinline__ uint32_t phase_tag(uint32_t epoch0, int ph)
{
    return (epoch0 + (uint32_t)ph) % 0xFFFFu;
}

__device__ __forceinline__ int slice_lo(int n, int b, int nb) { return (int)((int64_t)n * b / nb); }

// Weights of phase `which` (0 V rows, 1 Q/K rows, 2 O, 3 gate_up, 4 down) of
// layer L for workgroup b.
__device__ __forceinline__ PhaseMap map_of(const StackParams &p, int which, int L, int b, int nb)
{
    PhaseMap m;
    const int mat = which <= 1 ? 0 : which - 1;  // V, QK -> the QKV matrix
    const uint4 *W = reinterpret_cast<const uint4 *>(p.W[L * 4 + mat]);
    const uint16_t *S = p.S[L * 4 + mat];
    const int d = p.d, f = p.f;
    m.silu = 0;
    m.half = 0;
    switch (which) {
    case 0:  // V rows (the last dv rows of the QKV matrix)
        m.G = d >> 5;
        m.row0 = p.v_off + slice_lo(p.dv, b, nb);
        m.nrow = slice_lo(p.dv, b + 1, nb) - slice_lo(p.dv, b, nb);
        m.lpr = p.lpr_d;
        m.ng = p.ng_d;
        break;
    case 1:  // Q/K rows
        m.G = d >> 5;
        m.row0 = slice_lo(p.v_off, b, nb);
        m.nrow = slice_lo(p.v_off, b + 1, nb) - m.row0;
        m.lpr = p.lpr_d;
        m.ng = p.ng_d;
        break;
    case 2:  // O
        m.G = p.dv >> 5;
        m.row0 = slice_lo(d, b, nb);
        m.nrow = slice_lo(d, b + 1, nb) - m.row0;
        m.lpr = p.lpr_v;
        m.ng = p.ng_v;
        break;
    case 3:  // gate_up (gate rows and matching up rows)
        m.G = d >> 5;
        m.row0 = slice_lo(f, b, nb);
        m.nrow = slice_lo(f, b + 1, nb) - m.row0;
        m.half = f;
        m.silu = 1;
        m.lpr = p.lpr_d;
        m.ng = p.ng_d;
        break;
    default:  // down
        m.G = f >> 5;
        m.row0 = slice_lo(d, b, nb);
        m.nrow = slice_lo(d, b + 1, nb) - m.row0;
        m.lpr = p.lpr_f;
        m.ng = p.ng_f;
        break;
    }
    m.W0 = W + (size_t)m.row0 * m.G;
    m.S0 = S + (size_t)m.row0 * m.G;
    m.W1 = W + (size_t)(m.half + m.row0) * m.G;
    m.S1 = S + (size_t)(m.half + m.row0) * m.G;
    return m;
}

// Reduction of a phase over its virtual rows by all 16 waves; fn(v, value)
// runs in lane j == 0 of each segment for every valid virtual row.
template <typename F>
__device__ __forceinline__ void reduce_rows(const PhaseMap &m, const float2 *st, F &&fn)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int spw = 64 / m.lpr;
    const int seg = lane / m.lpr, j = lane % m.lpr;
    const int nv = m.nv();
    for (int v0 = 0; v0 < nv; v0 += kWavesPB * spw) {
        const int v = v0 + wave * spw + seg;
        const float acc = reduce_row(m, v, j, st);
        if (j == 0 && v < nv)
            fn(v, acc);
    }
}

// The layer loop, instantiated once per role so that neither role carries the
// other's registers (a spill reload would wait behind the weight loads). Both
// instantiations pass the same workgroup barriers in the same order; each
// __syncthreads below is reached by every wave of the workgroup.
template <bool STAGER>
__device__ __forceinline__ void layer_loop(const StackParams &p, const Lds &l)
{
    const int b = blockIdx.x, nb = gridDim.x;
    const int t = threadIdx.x;
    const int d = p.d, f = p.f;
    const int fl = kCopies * nb;  // flags of one phase kind: [kCopies][nb]
    uint32_t *const flag_v = p.flags, *const flag_r1 = p.flags + fl;
    uint32_t *const flag_u = p.flags + 2 * fl, *const flag_r2 = p.flags + 3 * fl;
    uint4 wv[kStackNch];  // compute role: this lane's weight chunks of a phase
    uint32_t sv[kStackNch];

    PhaseMap cur = map_of(p, 0, 0, b, nb);
    if (!STAGER)
        issue_loads(cur, wv, sv);

    for (int L = 0; L < p.n_layers; ++L) {
        const int ph = 4 * L;  // tags: V ph, r1 ph+1, u ph+2, r2 ph+3
        const bool last = L + 1 == p.n_layers;
        const bool tr = p.trace && b == 0 && L > 0;
        // ---- QKV input: h_in, or RMSNorm(r2 of the previous layer) ----------
        if (L == 0) {
            if (STAGER)
                stage_vector(p.h_in, nullptr, 0, nullptr, nb, d, l.xs, l.cs, p.err);
        } else {
            if (STAGER)
                norm_sum(p.r2buf, phase_tag(p.epoch0, ph - 1), flag_r2, nb, d, l, p.err,
                         tr ? p.trace + (size_t)(2 * (L - 1)) * d : nullptr);
            __syncthreads();
            if (STAGER)
                norm_apply(p.gamma_in + L * d, p.eps, d, l,
                           tr ? p.trace + (size_t)(2 * (L - 1) + 1) * d : nullptr, nullptr);
        }
        __syncthreads();
        // ---- V rows: published for the O phase ------------------------------
        if (!STAGER)
            compute_chunks(cur, wv, sv, l.xs, l.cs, l.st);
        __syncthreads();
        {
            const uint32_t tg = phase_tag(p.epoch0, ph);
            reduce_rows(cur, l.st, [&](int v, float acc) {
                const int row = cur.row_of(v);
                const uint16_t y = f2h(acc);
                p.qkv[row] = y;
                publish(p.vbuf, p.dv, row - p.v_off, y, tg);
            });
            __syncthreads();
            publish_flag(flag_v, nb, b, tg);
        }
        // ---- Q/K rows (compute role) while the stagers wait for V -----------
        const PhaseMap qk = map_of(p, 1, L, b, nb);
        if (STAGER) {
            stage_vector(nullptr, p.vbuf, phase_tag(p.epoch0, ph), flag_v, nb, p.dv, l.xo, l.co,
                         p.err);
        } else {
            issue_loads(qk, wv, sv);
            compute_chunks(qk, wv, sv, l.xs, l.cs, l.st);
        }
        __syncthreads();
        const PhaseMap o = map_of(p, 2, L, b, nb);
        if (!STAGER)
            issue_loads(o, wv, sv);
        reduce_rows(qk, l.st, [&](int v, float acc) { p.qkv[qk.row_of(v)] = f2h(acc); });
        __syncthreads();
        // ---- O: residual add in the epilogue --------------------------------
        if (!STAGER)
            compute_chunks(o, wv, sv, l.xo, l.co, l.st);
        __syncthreads();
        {
            const uint32_t tg = phase_tag(p.epoch0, ph + 1);
            reduce_rows(o, l.st, [&](int v, float acc) {
                const uint16_t r1 = f2h(h2f(f2h(acc)) + l.lres[v]);
                l.lres[v] = h2f(r1);
                publish(p.r1buf, d, o.row_of(v), r1, tg);
            });
            __syncthreads();
            publish_flag(flag_r1, nb, b, tg);
        }
        // ---- gate_up: RMSNorm prologue, SiLU-multiply epilogue --------------
        const PhaseMap gu = map_of(p, 3, L, b, nb);
        if (STAGER)
            norm_sum(p.r1buf, phase_tag(p.epoch0, ph + 1), flag_r1, nb, d, l, p.err, nullptr);
        else
            issue_loads(gu, wv, sv);
        __syncthreads();
        if (STAGER)
            norm_apply(p.gamma_post + L * d, p.eps, d, l, nullptr, nullptr);
        __syncthreads();
        if (!STAGER)
            compute_chunks(gu, wv, sv, l.xs, l.cs, l.st);
        __syncthreads();
        reduce_rows(gu, l.st, [&](int v, float acc) { l.rowv[v] = h2f(f2h(acc)); });
        __syncthreads();
        {
            const uint32_t tg = phase_tag(p.epoch0, ph + 2);
            for (int i = t; i < gu.nrow; i += kThreads)
                publish(p.ubuf, f, gu.row0 + i, f2h(silu_mul_f(l.rowv[i], l.rowv[gu.nrow + i])),
                        tg);
            __syncthreads();
            publish_flag(flag_u, nb, b, tg);
        }
        // ---- down: residual add in the epilogue -----------------------------
        const PhaseMap dn = map_of(p, 4, L, b, nb);
        if (STAGER)
            stage_vector(nullptr, p.ubuf, phase_tag(p.epoch0, ph + 2), flag_u, nb, f, l.xs, l.cs,
                         p.err);
        else
            issue_loads(dn, wv, sv);
        __syncthreads();
        if (!STAGER)
            compute_chunks(dn, wv, sv, l.xs, l.cs, l.st);
        __syncthreads();
        {
            const uint32_t tg = phase_tag(p.epoch0, ph + 3);
            reduce_rows(dn, l.st, [&](int v, float acc) {
                const uint16_t r2 = f2h(h2f(f2h(acc)) + l.lres[v]);
                l.lres[v] = h2f(r2);
                publish(p.r2buf, d, dn.row_of(v), r2, tg);
                if (last)
                    p.r_out[dn.row_of(v)] = r2;
            });
            __syncthreads();
            publish_flag(flag_r2, nb, b, tg);
        }
        if (!STAGER && !last) {
            cur = map_of(p, 0, L + 1, b, nb);
            issue_loads(cur, wv, sv);
        }
    }

    // final RMSNorm of the last residual (workgroup 0)
    if (b == 0) {
        const int Lz = p.n_layers - 1;
        if (STAGER)
            norm_sum(p.r2buf, phase_tag(p.epoch0, 4 * Lz + 3), flag_r2, nb, d, l, p.err,
                     p.trace ? p.trace + (size_t)(2 * Lz) * d : nullptr);
        __syncthreads();
        if (STAGER)
            norm_apply(p.gamma_final, p.eps, d, l, p.h_out,
                       p.trace ? p.trace + (size_t)(2 * Lz + 1) * d : nullptr);
    }
}

__global__ __launch_bounds__(kThreads) void k_stack(StackParams p)
{
    extern __shared__ uint4 smem[];
    __shared__ float red[4];
    const int b = blockIdx.x, nb = gridDim.x;
    const int t = threadIdx.x;

    // LDS carve-up (byte offsets computed by the host)
    char *const lds = reinterpret_cast<char *>(smem);
    Lds l;
    l.xs = reinterpret_cast<uint4 *>(lds + p.lds_xs);
    l.cs = reinterpret_cast<float *>(lds + p.lds_cs);
    l.xo = reinterpret_cast<uint4 *>(lds + p.lds_xo);
    l.co = reinterpret_cast<float *>(lds + p.lds_co);
    l.st = reinterpret_cast<float2 *>(lds + p.lds_st);
    l.raw = reinterpret_cast<uint4 *>(lds + p.lds_raw);
    l.rowv = reinterpret_cast<float *>(lds + p.lds_rowv);
    l.lres = reinterpret_cast<float *>(lds + p.lds_lres);
    l.red = red;

    // this workgroup's residual rows (the O / down slice), kept in LDS; the
    // first barrier of the layer loop orders these writes before their use
    const int rrow0 = slice_lo(p.d, b, nb), rnrow = slice_lo(p.d, b + 1, nb) - rrow0;
    for (int i = t; i < rnrow; i += kThreads)
        l.lres[i] = h2f(p.r_in[rrow0 + i]);

    if (t >= kCompute)
        layer_loop<true>(p, l);
    else
        layer_loop<false>(p, l);
}

}  // namespace

const void *stack_kernel() { return reinterpret_cast<const void *>(&k_stack); }

}  // namespace q4
