// C ABI of libq4: argument validation on the host, workspace management and
// dispatch to the gfx950 kernels. Every check happens before anything is
// enqueued, so an error return means nothing was launched.
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <utility>

#include "q4_common.h"
#include <algorithm>
#include <cstring>
#include <vector>

namespace q4 {

namespace {
thread_local char g_err[512] = "";
thread_local q4_status g_ws_status = Q4_OK;  // last workspace() failure

// q4_timer_arm / q4_timer_read state, per thread
constexpr int kTimerSlots = 64;
struct TimerSlot {
    hipEvent_t start = nullptr, stop = nullptr;
    bool launched = false;
};
thread_local TimerSlot g_timers[kTimerSlots];
thread_local int g_armed = -1;
// Library workspace per (device, stream): the current buffer and the buffers it
// replaced (kept until q4_workspace_release or the end of the process; no HIP
// call is made at static teardown).
struct Workspace {
    void *buf = nullptr;
    size_t bytes = 0;
    std::vector<void *> retired;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
}  // namespace

q4_status fail(q4_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

bool take_armed_timer(hipEvent_t *start, hipEvent_t *stop)
{
    if (g_armed < 0)
        return false;
    TimerSlot &t = g_timers[g_armed];
    g_armed = -1;
    *start = t.start;
    *stop = t.stop;
    t.launched = true;
    return true;
}

q4_status check_launch(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(Q4_EHIP, "launch of %s failed: %s", what, hipGetErrorString(e));
    return Q4_OK;
}

// Compute units of the current device (cached per device; 256 if unknown).
int cu_count()
{
    static int n[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (!n[dev]) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            c = 256;
        n[dev] = c;
    }
    return n[dev];
}

namespace {
// Grows the (device, stream) workspace to at least `bytes` (caller holds
// g_ws_mu). The replaced buffer is not freed: work already enqueued, or a HIP
// graph captured earlier, may still use it; q4_workspace_release frees it.
void *grow_locked(int dev, hipStream_t stream, size_t bytes)
{
    Workspace &e = g_ws[{dev, stream}];
    if (e.buf && e.bytes >= bytes)
        return e.buf;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) {
        g_ws_status = fail(Q4_EHIP, "hipStreamIsCapturing failed");
        return nullptr;
    }
    if (cap != hipStreamCaptureStatusNone) {
        g_ws_status = fail(Q4_ERANGE,
             "the stream's workspace (%zu bytes) is smaller than the %zu bytes this call needs "
             "and cannot grow during graph capture; call q4_workspace_reserve before capturing",
             e.bytes, bytes);
        return nullptr;
    }
    const size_t nb = bytes < (size_t)(1 << 20) ? (size_t)(1 << 20) : bytes;
    void *p = nullptr;
    if (hipMalloc(&p, nb) != hipSuccess) {
        g_ws_status = fail(Q4_EHIP, "hipMalloc of a %zu-byte workspace failed", nb);
        return nullptr;
    }
    // the header is cleared in stream order, ahead of every use on this stream
    if (hipMemsetAsync(p, 0, kCounterBytes, stream) != hipSuccess) {
        (void)hipFree(p);  // nothing was enqueued on it; the error reported is the one below
        g_ws_status = fail(Q4_EHIP, "clearing the workspace header failed");
        return nullptr;
    }
    if (e.buf)
        e.retired.push_back(e.buf);
    e.buf = p;
    e.bytes = nb;
    return p;
}
}  // namespace

void *workspace(hipStream_t stream, size_t bytes)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        g_ws_status = fail(Q4_EHIP, "hipGetDevice failed");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_ws_mu);
    return grow_locked(dev, stream, bytes);
}

q4_status workspace_status() { return g_ws_status == Q4_OK ? Q4_EHIP : g_ws_status; }

}  // namespace q4

using namespace q4;

namespace {

inline hipStream_t as_stream(q4_stream s) { return reinterpret_cast<hipStream_t>(s); }

// Scratch of q4_stack_decode_noalloc: a fixed array in the library's device
// image (each GPU holds its own copy until the process ends), so the call
// allocates nothing. Host code must not pass `scratch` itself to a kernel (in
// host code it names a host-side stand-in): the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocScratchBytes = Q4_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char *g_scratch_dev[kMaxDevices] = {};  // device address of `scratch`, per device

// The device address of `scratch` on the current device.
q4_status scratch_address(char **out)
{
    int dev = 0;
    Q4_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(Q4_ERANGE, "device %d beyond the %d the fixed scratch serves", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(Q4_EHIP, "hipGetSymbolAddress of the fixed scratch failed: %s",
                        hipGetErrorString(e));
        g_scratch_dev[dev] = static_cast<char *>(p);
    }
    *out = g_scratch_dev[dev];
    return Q4_OK;
}

q4_status check_matrix(const uint32_t *W, const uint16_t *S, int64_t N, int64_t K)
{
    if (!W || !S)
        return fail(Q4_EINVAL, "NULL weight or scale pointer");
    if (N <= 0 || K <= 0)
        return fail(Q4_EINVAL, "non-positive shape N=%lld K=%lld", (long long)N, (long long)K);
    if (K % 32)
        return fail(Q4_ESHAPE, "K=%lld is not a multiple of 32", (long long)K);
    if (K > Q4_MAX_K)
        return fail(Q4_ERANGE, "K=%lld exceeds Q4_MAX_K=%d", (long long)K, Q4_MAX_K);
    if (N > (1ll << 30))
        return fail(Q4_ERANGE, "N=%lld is too large", (long long)N);
    if (!aligned(W, 16))
        return fail(Q4_EALIGN, "packed weights must be 16-byte aligned");
    if (!aligned(S, 2))
        return fail(Q4_EALIGN, "scales must be 2-byte aligned");
    return Q4_OK;
}

inline size_t wbytes(int64_t N, int64_t K) { return (size_t)N * (size_t)K / 2; }
inline size_t sbytes(int64_t N, int64_t K) { return (size_t)N * (size_t)K / 16; }

q4_status check_gemv_args(const uint32_t *W, const uint16_t *S, const uint16_t *x, uint16_t *y,
                          int64_t N, int64_t K, int64_t ny)
{
    q4_status st = check_matrix(W, S, N, K);
    if (st != Q4_OK)
        return st;
    if (!x || !y)
        return fail(Q4_EINVAL, "NULL activation or output pointer");
    if (!aligned(x, 16))
        return fail(Q4_EALIGN, "the activation vector must be 16-byte aligned");
    if (!aligned(y, 2))
        return fail(Q4_EALIGN, "the output must be 2-byte aligned");
    const size_t yb = (size_t)ny * 2;
    if (overlaps(y, yb, W, wbytes(N, K)) || overlaps(y, yb, S, sbytes(N, K)) ||
        overlaps(y, yb, x, (size_t)K * 2))
        return fail(Q4_EALIAS, "the output overlaps an input");
    return Q4_OK;
}


// ---------------------------------------------------------------------------
// Decode stack: multi-kernel path (four matvec launches per layer)
// ---------------------------------------------------------------------------
// The attention step of a stack layer (q4_stack_decode_attn): geometry, the
// layers' caches, and the bound on the position.
struct StackAttn {
    RopeArgs geom;  // pos and page_table set; kv and q_out per layer
    uint16_t *const *kv_pages = nullptr;
    int64_t max_len = 0;
};

// Workspace of a stack call: header | qkv | r1 | u | rA | rB [| attention
// output | attention partials] (256-byte aligned pieces); geom: the attention
// geometry, or nullptr for the single-position stack.
struct StackWs {
    size_t q_b, v_b, u_b, a_b, part_b, total;
    StackWs(const q4_stack_desc *d, const RopeArgs *geom)
    {
        auto al = [](size_t b) { return (b + 255) / 256 * 256; };
        q_b = al((size_t)d->n_qkv * 2);
        v_b = al((size_t)d->d * 2);
        u_b = al((size_t)d->f * 2);
        a_b = geom ? al((size_t)d->dv * 2) : 0;
        part_b = geom ? al(attention_part_bytes(*geom)) : 0;
        total = kWsHeader + q_b + 3 * v_b + u_b + a_b + part_b;
    }
};

// buffers: device memory for the call's intermediate vectors (StackWs(d,
// ...).total bytes), or nullptr for the stream's library workspace.
q4_status stack_multi(const q4_stack_desc *d, const StackAttn *attn, const uint16_t *r_in,
                      const uint16_t *h_in, uint16_t *r_out, uint16_t *h_out, uint16_t *trace,
                      hipStream_t st, char *buffers = nullptr)
{
    const int64_t D = d->d, F = d->f;
    const size_t vb = (size_t)D * 2;
    // Per layer four matvecs and no synchronisation between workgroups: the
    // residual add happens row by row in the O / down epilogues, and the
    // RMSNorm that follows it is recomputed by every workgroup of the next
    // matvec while it stages its activation (bit-identical to q4_add_rmsnorm).
    const StackWs w(d, attn ? &attn->geom : nullptr);
    const size_t q_b = w.q_b, v_b = w.v_b, u_b = w.u_b, a_b = w.a_b;
    char *ws = buffers ? buffers : static_cast<char *>(workspace(st, w.total));
    if (!ws)
        return workspace_status();
    uint16_t *qkv = reinterpret_cast<uint16_t *>(ws + kWsHeader);
    uint16_t *att = reinterpret_cast<uint16_t *>(ws + kWsHeader + q_b + 3 * v_b + u_b);
    float *part = reinterpret_cast<float *>(ws + kWsHeader + q_b + 3 * v_b + u_b + a_b);
    char *p = ws + kWsHeader + q_b;
    uint16_t *r1 = reinterpret_cast<uint16_t *>(p);
    uint16_t *u = reinterpret_cast<uint16_t *>(p + v_b);
    uint16_t *rp[2] = {reinterpret_cast<uint16_t *>(p + v_b + u_b),
                       reinterpret_cast<uint16_t *>(p + 2 * v_b + u_b)};

    const uint16_t *rc = r_in;
    for (int64_t L = 0; L < d->n_layers; ++L) {
        const bool last = L + 1 == d->n_layers;
        uint16_t *r2 = last ? r_out : rp[L & 1];
        const uint16_t *g_next = last ? d->gamma_final : d->gamma_in + (L + 1) * D;
        q4_status s;
        GemvOp qk;
        qk.W = d->Wqkv[L];
        qk.S = d->Sqkv[L];
        qk.N = (int)d->n_qkv;
        qk.K = (int)D;
        if (L == 0) {
            qk.x = h_in;
        } else {  // h = RMSNorm(r) * gamma_in[L], recomputed in the prologue
            qk.norm_src = rc;
            qk.norm_gamma = d->gamma_in + L * D;
            qk.norm_eps = d->eps;
        }
        const uint16_t *o_in = qkv + d->v_off;  // single position: attention returns V
        if (attn) {
            // RoPE and the cache write in the QKV epilogue, then attention
            qk.epi = GemvOp::ROPE;
            qk.rope = attn->geom;
            qk.rope.kv = attn->kv_pages[L];
            qk.rope.q_out = qkv;
            if ((s = launch_gemv_op(qk, st)) != Q4_OK)
                return s;
            if ((s = launch_attention(qkv, attn->kv_pages[L], attn->geom, attn->max_len, att, st,
                                      part)) != Q4_OK)
                return s;
            o_in = att;
        } else {
            qk.epi = GemvOp::NONE;
            qk.y = qkv;
            if ((s = launch_gemv_op(qk, st)) != Q4_OK)
                return s;
        }
        GemvOp o;
        o.W = d->Wo[L];
        o.S = d->So[L];
        o.N = (int)D;
        o.K = (int)d->dv;
        o.x = o_in;
        o.epi = GemvOp::RESID;
        o.res_in = rc;
        o.res_out = r1;
        if ((s = launch_gemv_op(o, st)) != Q4_OK)
            return s;
        GemvOp gu;
        gu.W = d->Wgu[L];
        gu.S = d->Sgu[L];
        gu.N = (int)(2 * F);
        gu.K = (int)D;
        gu.norm_src = r1;
        gu.norm_gamma = d->gamma_post + L * D;
        gu.norm_eps = d->eps;
        gu.epi = GemvOp::SILU;
        gu.y = u;
        if ((s = launch_gemv_op(gu, st)) != Q4_OK)
            return s;
        GemvOp dn;
        dn.W = d->Wdn[L];
        dn.S = d->Sdn[L];
        dn.N = (int)D;
        dn.K = (int)F;
        dn.x = u;
        dn.epi = GemvOp::RESID;
        dn.res_in = r1;
        dn.res_out = r2;
        if ((s = launch_gemv_op(dn, st)) != Q4_OK)
            return s;
        if (trace) {
            uint16_t *tr = trace + (2 * L) * D;
            Q4_HIP(hipMemcpyAsync(tr, r2, vb, hipMemcpyDeviceToDevice, st));
            if ((s = launch_add_rmsnorm(nullptr, r2, g_next, tr + D, nullptr, (int)D, 1, d->eps,
                                        st)) != Q4_OK)
                return s;
        }
        rc = r2;
    }
    return launch_add_rmsnorm(nullptr, r_out, d->gamma_final, h_out, nullptr, (int)D, 1, d->eps,
                              st);
}


q4_status check_f32_matvec(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                           const float *y, int64_t ldy, int64_t N, int64_t K, int64_t M)
{
    q4_status st = check_matrix(W, S, N, K);
    if (st != Q4_OK)
        return st;
    if (!x || !y)
        return fail(Q4_EINVAL, "NULL activation or output pointer");
    if (M < 1 || M > Q4_MAX_M)
        return fail(Q4_ERANGE, "M=%lld outside [1, %d]", (long long)M, Q4_MAX_M);
    if (ldx < K || ldy < N)
        return fail(Q4_EINVAL, "leading dimensions too small (ldx=%lld, ldy=%lld)",
                    (long long)ldx, (long long)ldy);
    if (!aligned(x, 16) || ldx % 8)
        return fail(Q4_EALIGN, "activation rows must be 16-byte aligned (ldx %% 8 == 0)");
    if (!aligned(y, 4))
        return fail(Q4_EALIGN, "the f32 output must be 4-byte aligned");
    const size_t yb = ((size_t)(M - 1) * ldy + N) * 4, xb = ((size_t)(M - 1) * ldx + K) * 2;
    if (overlaps(y, yb, W, wbytes(N, K)) || overlaps(y, yb, S, sbytes(N, K)) ||
        overlaps(y, yb, x, xb))
        return fail(Q4_EALIAS, "the output overlaps an input");
    return Q4_OK;
}

q4_status check_argmax(const float *v, int64_t ld, int64_t N, int64_t M, const int32_t *index)
{
    if (!v || !index)
        return fail(Q4_EINVAL, "NULL logits or index pointer");
    if (N < 1 || M < 1)
        return fail(Q4_EINVAL, "non-positive shape N=%lld M=%lld", (long long)N, (long long)M);
    if (N > 0x7FFFFFFFll || M > 65535)
        return fail(Q4_ERANGE, "N=%lld or M=%lld too large", (long long)N, (long long)M);
    if (ld < N)
        return fail(Q4_EINVAL, "leading dimension ld=%lld < N", (long long)ld);
    if (!aligned(v, 4) || !aligned(index, 4))
        return fail(Q4_EALIGN, "logits and index must be 4-byte aligned");
    if (overlaps(index, (size_t)M * 4, v, ((size_t)(M - 1) * ld + N) * 4))
        return fail(Q4_EALIAS, "the index output overlaps the logits");
    return Q4_OK;
}

q4_status check_attn_desc(const q4_attn_desc *d, RopeArgs *r)
{
    if (!d)
        return fail(Q4_EINVAL, "NULL attention descriptor");
    if (d->n_heads < 1 || d->n_kv < 1 || d->n_heads % d->n_kv)
        return fail(Q4_EINVAL, "n_kv must divide n_heads (n_heads=%lld, n_kv=%lld)",
                    (long long)d->n_heads, (long long)d->n_kv);
    if (d->head_dim < 8 || d->head_dim % 8 || d->head_dim > 256)
        return fail(Q4_ESHAPE, "head_dim=%lld must be a multiple of 8 in [8, 256]",
                    (long long)d->head_dim);
    if (d->page_size < 1 || d->max_pages < 1 || d->n_pages < 1)
        return fail(Q4_EINVAL, "page_size, max_pages and n_pages must be positive");
    if (d->max_pages * d->page_size > (1ll << 30) || d->n_pages > (1ll << 30) ||
        (d->n_heads + 2 * d->n_kv) * d->head_dim > (1ll << 30))
        return fail(Q4_ERANGE, "attention geometry too large");
    if (!(d->rope_base > 0.f))
        return fail(Q4_EINVAL, "rope_base must be positive");
    r->n_heads = (int)d->n_heads;
    r->n_kv = (int)d->n_kv;
    r->head_dim = (int)d->head_dim;
    r->page_size = (int)d->page_size;
    r->max_pages = (int)d->max_pages;
    r->n_pages = (int)d->n_pages;
    r->base = d->rope_base;
    return Q4_OK;
}

inline size_t kv_bytes(const RopeArgs &r)
{
    return (size_t)r.n_pages * 2 * r.n_kv * r.page_size * r.head_dim * 2;
}

q4_status check_rope_io(const RopeArgs &r, const int32_t *pos, const int32_t *page_table,
                        uint16_t *kv, uint16_t *q_out)
{
    if (!pos || !page_table || !kv || !q_out)
        return fail(Q4_EINVAL, "NULL position, page table, cache or q_out pointer");
    if (!aligned(pos, 4) || !aligned(page_table, 4) || !aligned(kv, 16) || !aligned(q_out, 2))
        return fail(Q4_EALIGN, "misaligned position, page table (4), cache (16) or q_out (2)");
    const size_t qb = (size_t)r.n_heads * r.head_dim * 2;
    if (overlaps(q_out, qb, kv, kv_bytes(r)) || overlaps(q_out, qb, page_table, (size_t)r.max_pages * 4) ||
        overlaps(kv, kv_bytes(r), page_table, (size_t)r.max_pages * 4) ||
        overlaps(q_out, qb, pos, 4) || overlaps(kv, kv_bytes(r), pos, 4))
        return fail(Q4_EALIAS, "q_out, the cache, the page table and the position overlap");
    return Q4_OK;
}
// Validation shared by the two stack entry points; vslice: the V rows of the
// QKV output feed O directly.
q4_status check_stack(const q4_stack_desc *d, const uint16_t *r_in, const uint16_t *h_in,
                      uint16_t *r_out, uint16_t *h_out, uint16_t *trace, bool vslice)
{
    if (!d)
        return fail(Q4_EINVAL, "NULL descriptor");
    if (d->n_layers <= 0 || d->d <= 0 || d->f <= 0 || d->n_qkv <= 0 || d->dv <= 0 || d->v_off < 0)
        return fail(Q4_EINVAL, "non-positive stack dimension");
    if (vslice && d->v_off + d->dv > d->n_qkv)
        return fail(Q4_ESHAPE, "V slice [%lld, %lld) outside the QKV rows", (long long)d->v_off,
                    (long long)(d->v_off + d->dv));
    if (vslice && d->v_off % 8)
        return fail(Q4_EALIGN, "v_off must be a multiple of 8 (16-byte aligned slice)");
    if (!d->Wqkv || !d->Sqkv || !d->Wo || !d->So || !d->Wgu || !d->Sgu || !d->Wdn || !d->Sdn ||
        !d->gamma_in || !d->gamma_post || !d->gamma_final)
        return fail(Q4_EINVAL, "NULL pointer in the stack descriptor");
    if (!r_in || !h_in || !r_out || !h_out)
        return fail(Q4_EINVAL, "NULL state pointer");
    if (!(d->eps >= 0.f))
        return fail(Q4_EINVAL, "eps must be non-negative");
    const int64_t D = d->d, F = d->f;
    if (!aligned(h_in, 16) || !aligned(r_in, 2) || !aligned(r_out, 2) || !aligned(h_out, 2) ||
        (trace && !aligned(trace, 2)))
        return fail(Q4_EALIGN, "h_in must be 16-byte aligned, other state vectors 2-byte");
    if (!aligned(d->gamma_in, 16) || !aligned(d->gamma_post, 16) || !aligned(d->gamma_final, 2))
        return fail(Q4_EALIGN, "gamma_in / gamma_post must be 16-byte aligned");
    const size_t vb = (size_t)D * 2;
    const void *ins[2] = {r_in, h_in};
    const void *outs[2] = {r_out, h_out};
    for (const void *o : outs) {
        for (const void *i : ins)
            if (overlaps(o, vb, i, vb))
                return fail(Q4_EALIAS, "stack outputs overlap its inputs");
        if (trace && overlaps(o, vb, trace, (size_t)d->n_layers * 2 * vb))
            return fail(Q4_EALIAS, "stack outputs overlap the trace");
    }
    if (overlaps(r_out, vb, h_out, vb))
        return fail(Q4_EALIAS, "r_out overlaps h_out");
    for (int64_t L = 0; L < d->n_layers; ++L) {
        q4_status st;
        if ((st = check_matrix(d->Wqkv[L], d->Sqkv[L], d->n_qkv, D)) != Q4_OK ||
            (st = check_matrix(d->Wo[L], d->So[L], D, d->dv)) != Q4_OK ||
            (st = check_matrix(d->Wgu[L], d->Sgu[L], 2 * F, D)) != Q4_OK ||
            (st = check_matrix(d->Wdn[L], d->Sdn[L], D, F)) != Q4_OK)
            return st;
    }
    const int mode = d->mode;
    if (mode != Q4_STACK_AUTO && mode != Q4_STACK_MULTI)
        return fail(Q4_EINVAL, "unknown stack mode %d (Q4_STACK_AUTO or Q4_STACK_MULTI)", mode);
    return Q4_OK;
}
}  // namespace

extern "C" {

const char *q4_version(void) { return "libq4 0.1 (gfx950)"; }

const char *q4_last_error(void) { return g_err; }

q4_status q4_timer_arm(int slot)
{
    if (slot < 0 || slot >= q4::kTimerSlots)
        return fail(Q4_EINVAL, "timer slot %d outside 0..%d", slot, q4::kTimerSlots - 1);
    q4::TimerSlot &t = q4::g_timers[slot];
    if (!t.start) {
        Q4_HIP(hipEventCreate(&t.start));
        Q4_HIP(hipEventCreate(&t.stop));
    }
    t.launched = false;
    q4::g_armed = slot;
    return Q4_OK;
}

q4_status q4_timer_read(int slot, float *us)
{
    if (slot < 0 || slot >= q4::kTimerSlots || !us)
        return fail(Q4_EINVAL, "timer slot %d outside 0..%d or NULL output", slot,
                    q4::kTimerSlots - 1);
    q4::TimerSlot &t = q4::g_timers[slot];
    if (!t.launched)
        return fail(Q4_EINVAL, "timer slot %d was not armed for a launch", slot);
    Q4_HIP(hipEventSynchronize(t.stop));
    float ms = 0.f;
    Q4_HIP(hipEventElapsedTime(&ms, t.start, t.stop));
    *us = ms * 1e3f;
    return Q4_OK;
}

double q4_bytes_per_weight(void) { return 4.0 / 8.0 + 2.0 / 32.0; }

q4_status q4_pack(const uint8_t *codes, uint32_t *packed, int64_t N, int64_t K, q4_stream stream)
{
    if (!codes || !packed)
        return fail(Q4_EINVAL, "NULL pointer");
    if (N <= 0 || K <= 0)
        return fail(Q4_EINVAL, "non-positive shape");
    if (K % 32)
        return fail(Q4_ESHAPE, "K=%lld is not a multiple of 32", (long long)K);
    if (!aligned(packed, 16))
        return fail(Q4_EALIGN, "packed weights must be 16-byte aligned");
    if (overlaps(codes, (size_t)N * K, packed, wbytes(N, K)))
        return fail(Q4_EALIAS, "codes and packed words overlap");
    return launch_pack(codes, packed, N * K / 8, as_stream(stream));
}

q4_status q4_unpack(const uint32_t *packed, uint8_t *codes, int64_t N, int64_t K, q4_stream stream)
{
    if (!codes || !packed)
        return fail(Q4_EINVAL, "NULL pointer");
    if (N <= 0 || K <= 0)
        return fail(Q4_EINVAL, "non-positive shape");
    if (K % 32)
        return fail(Q4_ESHAPE, "K=%lld is not a multiple of 32", (long long)K);
    if (!aligned(packed, 4))
        return fail(Q4_EALIGN, "packed weights must be 4-byte aligned");
    if (overlaps(codes, (size_t)N * K, packed, wbytes(N, K)))
        return fail(Q4_EALIAS, "codes and packed words overlap");
    return launch_unpack(packed, codes, N * K / 8, as_stream(stream));
}

q4_status q4_gemv(const uint32_t *W, const uint16_t *S, const uint16_t *x, uint16_t *y, int64_t N,
                  int64_t K, q4_stream stream)
{
    q4_status st = check_gemv_args(W, S, x, y, N, K, N);
    if (st != Q4_OK)
        return st;
    return launch_gemv(W, S, x, y, (int)N, (int)K, EpiArgs{}, as_stream(stream));
}

q4_status q4_gemv_ex(const uint32_t *W, const uint16_t *S, const uint16_t *x, uint16_t *y,
                     int64_t N, int64_t K, const q4_epilogue *epi, q4_stream stream)
{
    EpiArgs e;
    if (epi) {
        e.kind = epi->kind;
        e.norm_gamma = epi->norm_gamma;
        e.eps = epi->eps;
    }
    if (e.norm_gamma) {
        if (e.kind == Q4_EPI_ADD_RMSNORM)
            return fail(Q4_EINVAL, "a normalising prologue is not combined with add+RMSNorm");
        if (!aligned(e.norm_gamma, 16))
            return fail(Q4_EALIGN, "norm_gamma must be 16-byte aligned");
        if (!(e.eps >= 0.f))
            return fail(Q4_EINVAL, "eps must be non-negative");
    }
    if (e.kind != Q4_EPI_NONE && e.kind != Q4_EPI_SILU_MUL && e.kind != Q4_EPI_ADD_RMSNORM)
        return fail(Q4_EINVAL, "unknown epilogue kind %d", e.kind);
    if (e.kind == Q4_EPI_SILU_MUL && (N % 2))
        return fail(Q4_ESHAPE, "SiLU-multiply needs an even row count, N=%lld", (long long)N);
    const int64_t ny = e.kind == Q4_EPI_SILU_MUL ? N / 2 : N;
    q4_status st = check_gemv_args(W, S, x, y, N, K, ny);
    if (st != Q4_OK)
        return st;
    if (e.kind == Q4_EPI_ADD_RMSNORM) {
        e.res_in = epi->res_in;
        e.gamma = epi->gamma;
        e.res_out = epi->res_out;
        e.eps = epi->eps;
        if (!e.res_in || !e.gamma || !e.res_out)
            return fail(Q4_EINVAL, "add+RMSNorm epilogue needs res_in, gamma and res_out");
        if (N > Q4_MAX_K)
            return fail(Q4_ERANGE, "add+RMSNorm epilogue over N=%lld > Q4_MAX_K rows",
                        (long long)N);
        if (!aligned(e.res_in, 2) || !aligned(e.gamma, 2) || !aligned(e.res_out, 2))
            return fail(Q4_EALIGN, "epilogue vectors must be 2-byte aligned");
        const size_t vb = (size_t)N * 2;
        if (overlaps(e.res_out, vb, e.res_in, vb))
            return fail(Q4_EALIAS, "res_out overlaps res_in (use two residual buffers)");
        if (overlaps(e.res_out, vb, y, vb) || overlaps(y, vb, e.res_in, vb) ||
            overlaps(y, vb, e.gamma, vb) || overlaps(e.res_out, vb, e.gamma, vb) ||
            overlaps(e.res_out, vb, x, (size_t)K * 2) || overlaps(e.res_out, vb, W, wbytes(N, K)) ||
            overlaps(e.res_out, vb, S, sbytes(N, K)))
            return fail(Q4_EALIAS, "an epilogue output overlaps an input or another output");
        if (!(e.eps >= 0.f))
            return fail(Q4_EINVAL, "eps must be non-negative");
    }
    return launch_gemv(W, S, x, y, (int)N, (int)K, e, as_stream(stream));
}

q4_status q4_gemv_batched(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                          uint16_t *y, int64_t ldy, int64_t N, int64_t K, int64_t M,
                          q4_stream stream)
{
    q4_status st = check_matrix(W, S, N, K);
    if (st != Q4_OK)
        return st;
    if (!x || !y)
        return fail(Q4_EINVAL, "NULL activation or output pointer");
    if (M < 1 || M > Q4_MAX_M)
        return fail(Q4_ERANGE, "M=%lld outside [1, %d]", (long long)M, Q4_MAX_M);
    if (ldx < K || ldy < N)
        return fail(Q4_EINVAL, "leading dimensions too small (ldx=%lld, ldy=%lld)",
                    (long long)ldx, (long long)ldy);
    if (!aligned(x, 16) || ldx % 8)
        return fail(Q4_EALIGN, "activation rows must be 16-byte aligned (ldx %% 8 == 0)");
    if (!aligned(y, 2))
        return fail(Q4_EALIGN, "the output must be 2-byte aligned");
    const size_t yb = ((size_t)(M - 1) * ldy + N) * 2, xb = ((size_t)(M - 1) * ldx + K) * 2;
    if (overlaps(y, yb, W, wbytes(N, K)) || overlaps(y, yb, S, sbytes(N, K)) ||
        overlaps(y, yb, x, xb))
        return fail(Q4_EALIAS, "the output overlaps an input");
    return launch_gemv_batched(W, S, x, ldx, y, ldy, (int)N, (int)K, (int)M, as_stream(stream));
}

namespace {
// Shared checks of the prefill matmuls: x, y, M and the sizes of the scales
// (sb bytes) and biases (bb bytes, 0 without).
q4_status check_gemm_io(const uint32_t *W, const uint16_t *S, const uint16_t *B, size_t sb,
                        size_t bb, const uint16_t *x, int64_t ldx, const uint16_t *y, int64_t ldy,
                        int64_t N, int64_t K, int64_t M)
{
    if (!x || !y)
        return fail(Q4_EINVAL, "NULL activation or output pointer");
    if (M < 1 || M > Q4_MAX_GEMM_M)
        return fail(Q4_ERANGE, "M=%lld outside [1, %d]", (long long)M, Q4_MAX_GEMM_M);
    if ((M + 63) / 64 * ((N + 127) / 128) > 0x7FFFFFFFll)
        return fail(Q4_ERANGE, "M=%lld x N=%lld needs too many tiles", (long long)M, (long long)N);
    if (ldx < K || ldy < N)
        return fail(Q4_EINVAL, "leading dimensions too small (ldx=%lld, ldy=%lld)",
                    (long long)ldx, (long long)ldy);
    if (!aligned(x, 16) || ldx % 8)
        return fail(Q4_EALIGN, "activation rows must be 16-byte aligned (ldx %% 8 == 0)");
    if (!aligned(y, 2))
        return fail(Q4_EALIGN, "the output must be 2-byte aligned");
    const size_t yb = ((size_t)(M - 1) * ldy + N) * 2, xb = ((size_t)(M - 1) * ldx + K) * 2;
    if (overlaps(y, yb, W, wbytes(N, K)) || overlaps(y, yb, S, sb) || overlaps(y, yb, B, bb) ||
        overlaps(y, yb, x, xb))
        return fail(Q4_EALIAS, "the output overlaps an input");
    return Q4_OK;
}
}  // namespace

q4_status q4_gemm_affine(const uint32_t *W, const uint16_t *S, const uint16_t *B,
                         const uint16_t *x, int64_t ldx, uint16_t *y, int64_t ldy, int64_t N,
                         int64_t K, int64_t M, q4_stream stream)
{
    q4_status st = check_matrix(W, S, N, K);
    if (st != Q4_OK)
        return st;
    if (K % 64)
        return fail(Q4_ESHAPE, "K=%lld is not a multiple of 64 (affine groups)", (long long)K);
    if (!B)
        return fail(Q4_EINVAL, "NULL bias pointer");
    if (!aligned(B, 2))
        return fail(Q4_EALIGN, "the biases must be 2-byte aligned");
    const size_t sb = (size_t)N * (K / 64) * 2;
    if ((st = check_gemm_io(W, S, B, sb, sb, x, ldx, y, ldy, N, K, M)) != Q4_OK)
        return st;
    return launch_gemm(W, S, x, ldx, y, ldy, (int)N, (int)K, (int)M, true, as_stream(stream), B);
}

q4_status q4_gemm(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                  uint16_t *y, int64_t ldy, int64_t N, int64_t K, int64_t M, int weights,
                  q4_stream stream)
{
    q4_status st = check_matrix(W, S, N, K);
    if (st != Q4_OK)
        return st;
    if (weights != Q4_GEMM_EXACT && weights != Q4_GEMM_F16_WEIGHT)
        return fail(Q4_EINVAL, "unknown weights mode %d", weights);
    if ((st = check_gemm_io(W, S, nullptr, sbytes(N, K), 0, x, ldx, y, ldy, N, K, M)) != Q4_OK)
        return st;
    return launch_gemm(W, S, x, ldx, y, ldy, (int)N, (int)K, (int)M,
                       weights == Q4_GEMM_EXACT, as_stream(stream));
}

q4_status q4_gemv_f32(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t ldx,
                      float *y, int64_t ldy, int64_t N, int64_t K, int64_t M, q4_stream stream)
{
    q4_status st = check_f32_matvec(W, S, x, ldx, y, ldy, N, K, M);
    if (st != Q4_OK)
        return st;
    return launch_gemv_f32(W, S, x, ldx, y, ldy, (int)N, (int)K, (int)M, as_stream(stream));
}

q4_status q4_argmax(const float *v, int64_t ld, int64_t N, int64_t M, int32_t *index,
                    q4_stream stream)
{
    q4_status st = check_argmax(v, ld, N, M, index);
    if (st != Q4_OK)
        return st;
    return launch_argmax(v, ld, (int)N, (int)M, index, as_stream(stream));
}

q4_status q4_lm_head_argmax(const uint32_t *W, const uint16_t *S, const uint16_t *x,
                            int64_t ldx, float *logits, int64_t ldl, int32_t *tokens, int64_t N,
                            int64_t K, int64_t M, q4_stream stream)
{
    q4_status st = check_f32_matvec(W, S, x, ldx, logits, ldl, N, K, M);
    if (st != Q4_OK)
        return st;
    if (!tokens)
        return fail(Q4_EINVAL, "NULL token pointer");
    if (!aligned(tokens, 4))
        return fail(Q4_EALIGN, "tokens must be 4-byte aligned");
    const size_t lb = ((size_t)(M - 1) * ldl + N) * 4, tb = (size_t)M * 4;
    if (overlaps(tokens, tb, logits, lb) || overlaps(tokens, tb, W, wbytes(N, K)) ||
        overlaps(tokens, tb, S, sbytes(N, K)) ||
        overlaps(tokens, tb, x, ((size_t)(M - 1) * ldx + K) * 2))
        return fail(Q4_EALIAS, "tokens overlap another argument");
    return launch_lm_head_argmax(W, S, x, ldx, logits, ldl, tokens, (int)N, (int)K, (int)M,
                                 as_stream(stream));
}

int64_t q4_kv_page_bytes(const q4_attn_desc *desc)
{
    if (!desc)
        return 0;
    return 2 * desc->n_kv * desc->page_size * desc->head_dim * 2;
}

q4_status q4_qkv_rope_append(const uint32_t *W, const uint16_t *S, const uint16_t *x, int64_t K,
                             const q4_attn_desc *desc, const int32_t *pos,
                             const int32_t *page_table, uint16_t *kv_pages, uint16_t *q_out,
                             q4_stream stream)
{
    RopeArgs r;
    q4_status st = check_attn_desc(desc, &r);
    if (st != Q4_OK)
        return st;
    const int64_t N = (int64_t)(r.n_heads + 2 * r.n_kv) * r.head_dim;
    if ((st = check_matrix(W, S, N, K)) != Q4_OK)
        return st;
    if (!x)
        return fail(Q4_EINVAL, "NULL activation");
    if (!aligned(x, 16))
        return fail(Q4_EALIGN, "the activation vector must be 16-byte aligned");
    if ((st = check_rope_io(r, pos, page_table, kv_pages, q_out)) != Q4_OK)
        return st;
    const size_t qb = (size_t)r.n_heads * r.head_dim * 2, xb = (size_t)K * 2;
    if (overlaps(q_out, qb, x, xb) || overlaps(q_out, qb, W, wbytes(N, K)) ||
        overlaps(q_out, qb, S, sbytes(N, K)) || overlaps(kv_pages, kv_bytes(r), x, xb) ||
        overlaps(kv_pages, kv_bytes(r), W, wbytes(N, K)) ||
        overlaps(kv_pages, kv_bytes(r), S, sbytes(N, K)))
        return fail(Q4_EALIAS, "q_out or the cache overlaps an input");
    r.pos = pos;
    r.page_table = page_table;
    r.kv = kv_pages;
    r.q_out = q_out;
    GemvOp op;
    op.W = W;
    op.S = S;
    op.N = (int)N;
    op.K = (int)K;
    op.x = x;
    op.epi = GemvOp::ROPE;
    op.rope = r;
    return launch_gemv_op(op, as_stream(stream));
}

q4_status q4_rope_append(const uint16_t *qkv, const q4_attn_desc *desc, const int32_t *pos,
                         const int32_t *page_table, uint16_t *kv_pages, uint16_t *q_out,
                         q4_stream stream)
{
    RopeArgs r;
    q4_status st = check_attn_desc(desc, &r);
    if (st != Q4_OK)
        return st;
    if (!qkv)
        return fail(Q4_EINVAL, "NULL qkv");
    if (!aligned(qkv, 2))
        return fail(Q4_EALIGN, "qkv must be 2-byte aligned");
    if ((st = check_rope_io(r, pos, page_table, kv_pages, q_out)) != Q4_OK)
        return st;
    const size_t nb = (size_t)(r.n_heads + 2 * r.n_kv) * r.head_dim * 2;
    if (overlaps(q_out, (size_t)r.n_heads * r.head_dim * 2, qkv, nb) ||
        overlaps(kv_pages, kv_bytes(r), qkv, nb))
        return fail(Q4_EALIAS, "q_out or the cache overlaps qkv");
    r.pos = pos;
    r.page_table = page_table;
    r.kv = kv_pages;
    r.q_out = q_out;
    return launch_rope_append(qkv, r, as_stream(stream));
}

q4_status q4_attention_decode(const uint16_t *q, const uint16_t *kv_pages,
                              const int32_t *page_table, const int32_t *pos, int64_t max_len,
                              const q4_attn_desc *desc, uint16_t *out, q4_stream stream)
{
    RopeArgs r;
    q4_status st = check_attn_desc(desc, &r);
    if (st != Q4_OK)
        return st;
    if (!q || !kv_pages || !page_table || !pos || !out)
        return fail(Q4_EINVAL, "NULL query, cache, page table, position or output pointer");
    if (max_len < 1)
        return fail(Q4_EINVAL, "max_len must be positive");
    const int nc = r.head_dim / 8;
    if (nc != 1 && nc != 2 && nc != 4 && nc != 6 && nc != 8 && nc != 12 && nc != 16 && nc != 20 &&
        nc != 24 && nc != 32)
        return fail(Q4_ESHAPE, "no attention kernel for head_dim %d", r.head_dim);
    if (!aligned(q, 2) || !aligned(kv_pages, 16) || !aligned(page_table, 4) || !aligned(pos, 4) ||
        !aligned(out, 2))
        return fail(Q4_EALIGN, "misaligned query, cache (16), page table, position or output");
    const size_t ob = (size_t)r.n_heads * r.head_dim * 2;
    if (overlaps(out, ob, q, ob) || overlaps(out, ob, kv_pages, kv_bytes(r)) ||
        overlaps(out, ob, page_table, (size_t)r.max_pages * 4) || overlaps(out, ob, pos, 4))
        return fail(Q4_EALIAS, "the output overlaps an input");
    r.pos = pos;
    r.page_table = page_table;
    return launch_attention(q, kv_pages, r, max_len, out, as_stream(stream));
}

q4_status q4_gemv_affine(const uint32_t *W, const uint16_t *S, const uint16_t *B,
                         const uint16_t *x, int64_t ldx, uint16_t *y, int64_t ldy, int64_t N,
                         int64_t K, int64_t M, q4_stream stream)
{
    q4_status st = check_matrix(W, S, N, K);
    if (st != Q4_OK)
        return st;
    if (K % 64)
        return fail(Q4_ESHAPE, "K=%lld is not a multiple of 64 (affine groups)", (long long)K);
    if (!B || !x || !y)
        return fail(Q4_EINVAL, "NULL bias, activation or output pointer");
    if (M < 1 || M > Q4_MAX_M)
        return fail(Q4_ERANGE, "M=%lld outside [1, %d]", (long long)M, Q4_MAX_M);
    if (ldx < K || ldy < N)
        return fail(Q4_EINVAL, "leading dimensions too small (ldx=%lld, ldy=%lld)",
                    (long long)ldx, (long long)ldy);
    if (!aligned(x, 16) || ldx % 8)
        return fail(Q4_EALIGN, "activation rows must be 16-byte aligned (ldx %% 8 == 0)");
    if (!aligned(y, 2) || !aligned(B, 2))
        return fail(Q4_EALIGN, "the output and the biases must be 2-byte aligned");
    const size_t yb = ((size_t)(M - 1) * ldy + N) * 2, xb = ((size_t)(M - 1) * ldx + K) * 2;
    const size_t sb = (size_t)N * (K / 64) * 2;
    if (overlaps(y, yb, W, wbytes(N, K)) || overlaps(y, yb, S, sb) || overlaps(y, yb, B, sb) ||
        overlaps(y, yb, x, xb))
        return fail(Q4_EALIAS, "the output overlaps an input");
    hipStream_t s = as_stream(stream);
    if (M == 1) {
        GemvOp op;
        op.W = W;
        op.S = S;
        op.bias = B;
        op.N = (int)N;
        op.K = (int)K;
        op.x = x;
        op.y = y;
        return launch_gemv_op(op, s);
    }
    if (gemv_rows_fits((int)M, (int)K))  // a few rows: the single-row arithmetic per row
        return launch_gemv_rows(W, S, x, ldx, y, ldy, (int)N, (int)K, (int)M, s, B);
    return launch_gemv_mfma(W, S, x, ldx, y, nullptr, ldy, (int)N, (int)K, (int)M, s, B);
}

q4_status q4_moe_gemv(const uint32_t *W, const uint16_t *S, const int32_t *ids,
                      const uint16_t *route_w, const uint16_t *x, int64_t ldx,
                      int64_t x_slot_stride, uint16_t *y, int64_t E, int64_t N, int64_t K,
                      int64_t T, int64_t TOPK, int epi_silu, q4_stream stream)
{
    if (E <= 0 || T <= 0 || TOPK <= 0)
        return fail(Q4_EINVAL, "non-positive E, T or TOPK");
    q4_status st = check_matrix(W, S, N, K);
    if (st != Q4_OK)
        return st;
    if (!ids || !x || !y)
        return fail(Q4_EINVAL, "NULL ids, activation or output pointer");
    if (epi_silu && route_w)
        return fail(Q4_EINVAL, "the SiLU epilogue and the routing combine are separate stages");
    if (epi_silu && (N % 2))
        return fail(Q4_ESHAPE, "SiLU-multiply needs an even row count, N=%lld", (long long)N);
    if (T * TOPK > Q4_MAX_PAIRS)
        return fail(Q4_ERANGE, "T*TOPK=%lld exceeds Q4_MAX_PAIRS=%d", (long long)(T * TOPK),
                    Q4_MAX_PAIRS);
    if ((int64_t)E * N > (1ll << 31))
        return fail(Q4_ERANGE, "E*N is too large");
    if (x_slot_stride < 0 || ldx < 0)
        return fail(Q4_EINVAL, "negative stride");
    if (!aligned(x, 16) || ldx % 8 || x_slot_stride % 8)
        return fail(Q4_EALIGN, "activation rows must be 16-byte aligned (strides %% 8 == 0)");
    if (!aligned(ids, 4) || (route_w && !aligned(route_w, 2)) || !aligned(y, 2))
        return fail(Q4_EALIGN, "misaligned ids, routing weights or output");
    const int64_t P = T * TOPK;
    const size_t yb = (route_w ? (size_t)T * N : (size_t)P * (epi_silu ? N / 2 : N)) * 2;
    const size_t xb = ((size_t)(T - 1) * ldx + (size_t)(TOPK - 1) * x_slot_stride + K) * 2;
    if (overlaps(y, yb, W, wbytes(E * N, K)) || overlaps(y, yb, S, sbytes(E * N, K)) ||
        overlaps(y, yb, x, xb) || overlaps(y, yb, ids, (size_t)P * 4) ||
        (route_w && overlaps(y, yb, route_w, (size_t)P * 2)))
        return fail(Q4_EALIAS, "the output overlaps an input");
    return launch_moe(W, S, ids, route_w, x, ldx, x_slot_stride, y, (int)E, (int)N, (int)K, (int)T,
                      (int)TOPK, epi_silu, as_stream(stream));
}

q4_status q4_add_rmsnorm(const uint16_t *a, const uint16_t *res_in, const uint16_t *gamma,
                         uint16_t *out, uint16_t *res_out, int64_t D, int64_t M, float eps,
                         q4_stream stream)
{
    if (!res_in || !gamma || !out || !res_out)
        return fail(Q4_EINVAL, "NULL pointer");
    if (D <= 0 || M <= 0)
        return fail(Q4_EINVAL, "non-positive shape");
    if (D > Q4_MAX_K || M > (1 << 20))
        return fail(Q4_ERANGE, "D=%lld or M=%lld too large", (long long)D, (long long)M);
    if (!(eps >= 0.f))
        return fail(Q4_EINVAL, "eps must be non-negative");
    if ((a && !aligned(a, 2)) || !aligned(res_in, 2) || !aligned(gamma, 2) || !aligned(out, 2) ||
        !aligned(res_out, 2))
        return fail(Q4_EALIGN, "binary16 vectors must be 2-byte aligned");
    const size_t b = (size_t)D * M * 2;
    if (overlaps(res_out, b, res_in, b))
        return fail(Q4_EALIAS, "res_out overlaps res_in (use two residual buffers)");
    if (overlaps(out, b, res_in, b) || overlaps(out, b, res_out, b) || overlaps(out, b, a, b) ||
        overlaps(res_out, b, a, b) || overlaps(out, b, gamma, (size_t)D * 2) ||
        overlaps(res_out, b, gamma, (size_t)D * 2))
        return fail(Q4_EALIAS, "an output overlaps an input or the other output");
    return launch_add_rmsnorm(a, res_in, gamma, out, res_out, (int)D, (int)M, eps,
                              as_stream(stream));
}

q4_status q4_silu_mul(const uint16_t *gu, uint16_t *out, int64_t F, int64_t M, q4_stream stream)
{
    if (!gu || !out)
        return fail(Q4_EINVAL, "NULL pointer");
    if (F <= 0 || M <= 0)
        return fail(Q4_EINVAL, "non-positive shape");
    if (F * M > (1ll << 31))
        return fail(Q4_ERANGE, "F*M too large");
    if (!aligned(gu, 2) || !aligned(out, 2))
        return fail(Q4_EALIGN, "binary16 vectors must be 2-byte aligned");
    if (overlaps(out, (size_t)F * M * 2, gu, (size_t)F * M * 4))
        return fail(Q4_EALIAS, "the output overlaps the input");
    return launch_silu_mul(gu, out, (int)F, (int)M, as_stream(stream));
}


size_t q4_workspace_bytes(int64_t N, int64_t K, int64_t M)
{
    if (N < 1 || N > (1ll << 30) || K < 32 || K % 32 || K > Q4_MAX_K || M < 1)
        return 0;
    const int n = (int)N, k = (int)K;
    size_t need = 0;
    if (M <= Q4_MAX_M) {  // batched, f32 and affine matvecs; LM head + argmax
        need = std::max(need, ws_rows(n, k, (int)M));
        need = std::max(need, ws_lm_head(n, k, (int)M));
    }
    if (M <= 65535)  // argmax over M rows of N logits
        need = std::max(need, ws_argmax(n, (int)M));
    if (M <= Q4_MAX_GEMM_M) {  // prefill, both formats (ldx = K needs the most)
        need = std::max(need, ws_gemm(n, k, (int)M, false, K));
        if (K % 64 == 0)
            need = std::max(need, ws_gemm(n, k, (int)M, true, K));
    }
    if (M <= Q4_MAX_PAIRS)  // one MoE expert stage over M (token, slot) pairs, any E
        need = std::max(need, ws_moe(1 << 30, n, k, (int)M));
    return need;
}

size_t q4_attention_workspace_bytes(const q4_attn_desc *desc, int64_t max_len)
{
    RopeArgs r;
    if (max_len < 1 || check_attn_desc(desc, &r) != Q4_OK)
        return 0;
    return ws_attention(r, max_len);
}

size_t q4_stack_workspace_bytes(const q4_stack_desc *desc, const q4_stack_attn *attn)
{
    if (!desc || desc->d <= 0 || desc->f <= 0 || desc->n_qkv <= 0 || desc->dv <= 0)
        return 0;
    RopeArgs r;
    if (attn && check_attn_desc(attn->geom, &r) != Q4_OK)
        return 0;
    return StackWs(desc, attn ? &r : nullptr).total;
}

q4_status q4_workspace_reserve(q4_stream stream, size_t bytes)
{
    if (bytes == 0)
        return Q4_OK;
    return workspace(as_stream(stream), bytes) ? Q4_OK : workspace_status();
}

q4_status q4_workspace_release(q4_stream stream)
{
    hipStream_t st = as_stream(stream);
    int dev = 0;
    Q4_HIP(hipGetDevice(&dev));
    Q4_HIP(hipStreamSynchronize(st));
    Workspace w;
    {
        std::lock_guard<std::mutex> lock(g_ws_mu);
        auto it = g_ws.find({dev, st});
        if (it == g_ws.end())
            return Q4_OK;
        w = std::move(it->second);
        g_ws.erase(it);
    }
    w.retired.push_back(w.buf);
    for (void *p : w.retired)
        Q4_HIP(hipFree(p));
    return Q4_OK;
}

q4_status q4_stack_decode(const q4_stack_desc *d, const uint16_t *r_in, const uint16_t *h_in,
                          uint16_t *r_out, uint16_t *h_out, uint16_t *trace, q4_stream stream)
{
    q4_status s = check_stack(d, r_in, h_in, r_out, h_out, trace, true);
    if (s != Q4_OK)
        return s;
    hipStream_t st = as_stream(stream);
    return stack_multi(d, nullptr, r_in, h_in, r_out, h_out, trace, st);
}

q4_status q4_stack_decode_noalloc(const q4_stack_desc *d, const uint16_t *r_in,
                                  const uint16_t *h_in, uint16_t *r_out, uint16_t *h_out,
                                  uint16_t *trace, q4_stream stream)
{
    q4_status s = check_stack(d, r_in, h_in, r_out, h_out, trace, true);
    if (s != Q4_OK)
        return s;
    const size_t need = StackWs(d, nullptr).total;
    if (need > kNoAllocScratchBytes)
        return fail(Q4_ERANGE,
                    "this stack needs %zu bytes of scratch; the fixed scratch of "
                    "q4_stack_decode_noalloc holds %zu (use q4_stack_decode)",
                    need, kNoAllocScratchBytes);
    char *base = nullptr;
    if ((s = scratch_address(&base)) != Q4_OK)
        return s;
    return stack_multi(d, nullptr, r_in, h_in, r_out, h_out, trace, as_stream(stream), base);
}

q4_status q4_stack_decode_attn(const q4_stack_desc *d, const q4_stack_attn *attn,
                               const uint16_t *r_in, const uint16_t *h_in, uint16_t *r_out,
                               uint16_t *h_out, uint16_t *trace, q4_stream stream)
{
    q4_status s = check_stack(d, r_in, h_in, r_out, h_out, trace, false);
    if (s != Q4_OK)
        return s;
    if (!attn || !attn->kv_pages)
        return fail(Q4_EINVAL, "NULL attention description or cache array");
    StackAttn a;
    if ((s = check_attn_desc(attn->geom, &a.geom)) != Q4_OK)
        return s;
    const RopeArgs &g = a.geom;
    if (d->n_qkv != (int64_t)(g.n_heads + 2 * g.n_kv) * g.head_dim ||
        d->dv != (int64_t)g.n_heads * g.head_dim)
        return fail(Q4_ESHAPE, "n_qkv must be (n_heads + 2 n_kv) * head_dim and dv n_heads * head_dim");
    const int nc = g.head_dim / 8;
    if (nc != 1 && nc != 2 && nc != 4 && nc != 6 && nc != 8 && nc != 12 && nc != 16 && nc != 20 &&
        nc != 24 && nc != 32)
        return fail(Q4_ESHAPE, "no attention kernel for head_dim %d", g.head_dim);
    if (attn->max_len < 1)
        return fail(Q4_EINVAL, "max_len must be positive");
    if (!attn->pos || !attn->page_table || !aligned(attn->pos, 4) || !aligned(attn->page_table, 4))
        return fail(Q4_EINVAL, "NULL or misaligned position or page table");
    const size_t cb = kv_bytes(g), vb = (size_t)d->d * 2;
    for (int64_t L = 0; L < d->n_layers; ++L) {
        uint16_t *kv = attn->kv_pages[L];
        if (!kv || !aligned(kv, 16))
            return fail(Q4_EALIGN, "NULL or misaligned cache of layer %lld", (long long)L);
        if (overlaps(kv, cb, r_out, vb) || overlaps(kv, cb, h_out, vb) ||
            overlaps(kv, cb, r_in, vb) || overlaps(kv, cb, h_in, vb) ||
            overlaps(kv, cb, attn->page_table, (size_t)g.max_pages * 4) ||
            overlaps(kv, cb, attn->pos, 4) ||
            (trace && overlaps(kv, cb, trace, (size_t)d->n_layers * 2 * vb)))
            return fail(Q4_EALIAS, "the cache of layer %lld overlaps another argument", (long long)L);
    }
    a.geom.pos = attn->pos;
    a.geom.page_table = attn->page_table;
    a.kv_pages = attn->kv_pages;
    a.max_len = attn->max_len;
    return stack_multi(d, &a, r_in, h_in, r_out, h_out, trace, as_stream(stream));
}

}  // extern "C"
