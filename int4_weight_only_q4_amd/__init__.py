"""Python binding of libq4, the gfx950 int4 (q4f16_1) decode-matmul library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/q4.h``. PyTorch provides device
memory and streams. There is no CPU fallback: if ``libq4.so`` has not been
built, ``lib()`` raises.

Tensor conventions (all on the current CUDA/HIP device):
  packed weights  int32  [N, K/8]   (the uint32 words, viewed as int32)
  scales          float16 [N, K/32]
  activations     float16
Calls enqueue on ``stream`` (default: torch's current stream) and return
without synchronising.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libq4.so")

Q4_OK, Q4_EINVAL, Q4_ESHAPE, Q4_EALIGN, Q4_EALIAS, Q4_ERANGE, Q4_EHIP = range(7)
EPI_NONE, EPI_SILU_MUL, EPI_ADD_RMSNORM = 0, 1, 2
STACK_AUTO, STACK_MULTI = 0, 1
MAX_K = 24576
MAX_M = 64
MAX_GEMM_M = 65536
MAX_PAIRS = 4096
NOALLOC_SCRATCH_BYTES = 1 << 20

#: Bytes per int4 weight in this format: 4 bits + one f16 scale per 32 weights.
BYTES_PER_WEIGHT = 0.5 + 2.0 / 32.0

ABI_SYMBOLS = (
    "q4_version", "q4_last_error", "q4_bytes_per_weight", "q4_pack", "q4_unpack", "q4_gemv",
    "q4_gemv_batched", "q4_moe_gemv", "q4_add_rmsnorm", "q4_silu_mul", "q4_gemv_ex",
    "q4_stack_decode", "q4_timer_arm", "q4_timer_read", "q4_gemv_f32",
    "q4_argmax", "q4_lm_head_argmax", "q4_kv_page_bytes", "q4_qkv_rope_append",
    "q4_rope_append", "q4_attention_decode", "q4_stack_decode_attn", "q4_gemv_affine",
    "q4_gemm", "q4_gemm_affine", "q4_workspace_bytes", "q4_attention_workspace_bytes",
    "q4_stack_workspace_bytes", "q4_workspace_reserve", "q4_workspace_release",
    "q4_stack_decode_noalloc",
)


class Q4Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__("libq4 status %d: %s" % (status, message))
        self.status = status


class Epilogue(C.Structure):
    _fields_ = [("kind", C.c_int), ("res_in", C.c_void_p), ("gamma", C.c_void_p),
                ("res_out", C.c_void_p), ("eps", C.c_float), ("norm_gamma", C.c_void_p)]


class StackDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int64), ("d", C.c_int64), ("f", C.c_int64),
                ("n_qkv", C.c_int64), ("v_off", C.c_int64), ("dv", C.c_int64),
                ("eps", C.c_float),
                ("Wqkv", C.c_void_p), ("Sqkv", C.c_void_p), ("Wo", C.c_void_p),
                ("So", C.c_void_p), ("Wgu", C.c_void_p), ("Sgu", C.c_void_p),
                ("Wdn", C.c_void_p), ("Sdn", C.c_void_p),
                ("gamma_in", C.c_void_p), ("gamma_post", C.c_void_p),
                ("gamma_final", C.c_void_p), ("mode", C.c_int)]


class AttnDesc(C.Structure):
    _fields_ = [("n_heads", C.c_int64), ("n_kv", C.c_int64), ("head_dim", C.c_int64),
                ("page_size", C.c_int64), ("max_pages", C.c_int64), ("n_pages", C.c_int64),
                ("rope_base", C.c_float)]


class StackAttn(C.Structure):
    _fields_ = [("geom", C.POINTER(AttnDesc)), ("kv_pages", C.c_void_p), ("page_table", C.c_void_p),
                ("pos", C.c_void_p), ("max_len", C.c_int64)]


_P, _I = C.c_void_p, C.c_int64
_SIGS = {
    "q4_version": (C.c_char_p, []),
    "q4_last_error": (C.c_char_p, []),
    "q4_bytes_per_weight": (C.c_double, []),
    "q4_pack": (C.c_int, [_P, _P, _I, _I, _P]),
    "q4_unpack": (C.c_int, [_P, _P, _I, _I, _P]),
    "q4_gemv": (C.c_int, [_P, _P, _P, _P, _I, _I, _P]),
    "q4_gemv_batched": (C.c_int, [_P, _P, _P, _I, _P, _I, _I, _I, _I, _P]),
    "q4_gemm": (C.c_int, [_P, _P, _P, _I, _P, _I, _I, _I, _I, C.c_int, _P]),
    "q4_gemm_affine": (C.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _P]),
    "q4_moe_gemv": (C.c_int, [_P, _P, _P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _I, C.c_int, _P]),
    "q4_add_rmsnorm": (C.c_int, [_P, _P, _P, _P, _P, _I, _I, C.c_float, _P]),
    "q4_silu_mul": (C.c_int, [_P, _P, _I, _I, _P]),
    "q4_gemv_ex": (C.c_int, [_P, _P, _P, _P, _I, _I, C.POINTER(Epilogue), _P]),
    "q4_stack_decode": (C.c_int, [C.POINTER(StackDesc), _P, _P, _P, _P, _P, _P]),
    "q4_timer_arm": (C.c_int, [C.c_int]),
    "q4_timer_read": (C.c_int, [C.c_int, C.POINTER(C.c_float)]),
    "q4_gemv_f32": (C.c_int, [_P, _P, _P, _I, _P, _I, _I, _I, _I, _P]),
    "q4_argmax": (C.c_int, [_P, _I, _I, _I, _P, _P]),
    "q4_lm_head_argmax": (C.c_int, [_P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _P]),
    "q4_kv_page_bytes": (C.c_int64, [C.POINTER(AttnDesc)]),
    "q4_gemv_affine": (C.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _P]),
    "q4_qkv_rope_append": (C.c_int, [_P, _P, _P, _I, C.POINTER(AttnDesc), _P, _P, _P, _P, _P]),
    "q4_rope_append": (C.c_int, [_P, C.POINTER(AttnDesc), _P, _P, _P, _P, _P]),
    "q4_attention_decode": (C.c_int, [_P, _P, _P, _P, _I, C.POINTER(AttnDesc), _P, _P]),
    "q4_stack_decode_attn": (C.c_int, [C.POINTER(StackDesc), C.POINTER(StackAttn), _P, _P, _P, _P,
                                       _P, _P]),
    "q4_workspace_bytes": (C.c_size_t, [_I, _I, _I]),
    "q4_attention_workspace_bytes": (C.c_size_t, [C.POINTER(AttnDesc), _I]),
    "q4_stack_workspace_bytes": (C.c_size_t, [C.POINTER(StackDesc), C.POINTER(StackAttn)]),
    "q4_workspace_reserve": (C.c_int, [_P, C.c_size_t]),
    "q4_workspace_release": (C.c_int, [_P]),
    "q4_stack_decode_noalloc": (C.c_int, [C.POINTER(StackDesc), _P, _P, _P, _P, _P, _P]),
}

_lib = None


def lib():
    """The loaded libq4 (raises if it has not been built).

    torch is imported first so that libq4 binds to the HIP runtime torch has
    loaded (both carry the soname libamdhip64.so.7); loading libq4 first would
    bring a second HIP runtime into the process.
    """
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (loads the process's HIP runtime)
        if not os.path.exists(LIB_PATH):
            raise ImportError("libq4.so is not built (run __graft_entry__.build() or "
                              "python -m int4_weight_only_q4_amd._build)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def version() -> str:
    return lib().q4_version().decode()


def _check(status):
    if status != Q4_OK:
        raise Q4Error(status, lib().q4_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t, dtype, name):
    import torch
    if t is None:
        raise ValueError("%s is required" % name)
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s CUDA tensor" % (name, dtype))
    return t


def pack(codes, out=None, stream=None):
    """codes uint8 [N, K] (values 0..15) -> packed int32 [N, K/8]."""
    import torch
    _need(codes, torch.uint8, "codes")
    n, k = codes.shape
    if out is None:
        out = torch.empty((n, k // 8), dtype=torch.int32, device=codes.device)
    _check(lib().q4_pack(_ptr(codes), _ptr(out), n, k, _stream(stream)))
    return out


def unpack(packed, k=None, out=None, stream=None):
    import torch
    _need(packed, torch.int32, "packed")
    n = packed.shape[0]
    k = packed.shape[1] * 8 if k is None else k
    if out is None:
        out = torch.empty((n, k), dtype=torch.uint8, device=packed.device)
    _check(lib().q4_unpack(_ptr(packed), _ptr(out), n, k, _stream(stream)))
    return out


def gemv(W, S, x, y=None, stream=None):
    """y[N] = f16(W . x) with W packed int32 [N, K/8], S f16 [N, K/32], x f16 [K]."""
    import torch
    n, k = W.shape[0], W.shape[1] * 8
    if y is None:
        y = torch.empty(n, dtype=torch.float16, device=W.device)
    _check(lib().q4_gemv(_ptr(W), _ptr(S), _ptr(x), _ptr(y), n, k, _stream(stream)))
    return y


def gemv_ex(W, S, x, y=None, kind=EPI_NONE, res_in=None, gamma=None, res_out=None, eps=1e-5,
            norm_gamma=None, stream=None):
    """q4_gemv with a fused prologue / epilogue (see include/q4.h)."""
    import torch
    n, k = W.shape[0], W.shape[1] * 8
    if y is None:
        y = torch.empty(n // 2 if kind == EPI_SILU_MUL else n, dtype=torch.float16,
                        device=W.device)
    epi = Epilogue(kind, _ptr(res_in), _ptr(gamma), _ptr(res_out), eps, _ptr(norm_gamma))
    _check(lib().q4_gemv_ex(_ptr(W), _ptr(S), _ptr(x), _ptr(y), n, k, C.byref(epi),
                            _stream(stream)))
    return y


def gemv_batched(W, S, x, y=None, stream=None):
    """x f16 [M, ldx >= K] -> y f16 [M, N]; rows share one weight read."""
    import torch
    n, k = W.shape[0], W.shape[1] * 8
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float16, device=W.device)
    _check(lib().q4_gemv_batched(_ptr(W), _ptr(S), _ptr(x), x.stride(0), _ptr(y), y.stride(0),
                                 n, k, m, _stream(stream)))
    return y


def gemv_affine(W, S, B, x, y=None, stream=None):
    """MLX affine 4-bit matvec: x f16 [K] or [M, K] -> y f16 [N] or [M, N];
    S, B f16 [N, K/64] (w = S*q + B)."""
    import torch
    n, k = W.shape[0], W.shape[1] * 8
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    m = x2.shape[0]
    if y is None:
        y = torch.empty((m, n) if x.dim() > 1 else (n,), dtype=torch.float16, device=W.device)
    y2 = y.unsqueeze(0) if y.dim() == 1 else y
    _check(lib().q4_gemv_affine(_ptr(W), _ptr(S), _ptr(B), _ptr(x2), x2.stride(0), _ptr(y2),
                                y2.stride(0), n, k, m, _stream(stream)))
    return y


GEMM_EXACT = 0
GEMM_F16_WEIGHT = 1


def gemm(W, S, x, y=None, weights=GEMM_EXACT, stream=None):
    """Prefill matmul: x f16 [M, ldx >= K] -> y f16 [M, N] (any M >= 1);
    weights GEMM_EXACT (w = (q - 7) * s) or GEMM_F16_WEIGHT (w rounded to f16)."""
    import torch
    n, k = W.shape[0], W.shape[1] * 8
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float16, device=W.device)
    _check(lib().q4_gemm(_ptr(W), _ptr(S), _ptr(x), x.stride(0), _ptr(y), y.stride(0), n, k, m,
                         int(weights), _stream(stream)))
    return y


def gemm_affine(W, S, B, x, y=None, stream=None):
    """Prefill matmul in the MLX affine format: x f16 [M, ldx >= K] -> y f16 [M, N];
    S, B f16 [N, K/64] (w = S*q + B), exact weights."""
    import torch
    n, k = W.shape[0], W.shape[1] * 8
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float16, device=W.device)
    _check(lib().q4_gemm_affine(_ptr(W), _ptr(S), _ptr(B), _ptr(x), x.stride(0), _ptr(y),
                                y.stride(0), n, k, m, _stream(stream)))
    return y


def _rows(x):
    """A 1-D activation as one row; returns (2-D view, M, leading dimension)."""
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    return x2, x2.shape[0], x2.stride(0)


def gemv_f32(W, S, x, y=None, stream=None):
    """f32 logits: x f16 [K] or [M, K] -> y f32 [N] or [M, N] (no f16 rounding)."""
    import torch
    n, k = W.shape[0], W.shape[1] * 8
    x2, m, ldx = _rows(x)
    if y is None:
        y = torch.empty((m, n) if x.dim() > 1 else (n,), dtype=torch.float32, device=W.device)
    y2 = y.unsqueeze(0) if y.dim() == 1 else y
    _check(lib().q4_gemv_f32(_ptr(W), _ptr(S), _ptr(x2), ldx, _ptr(y2), y2.stride(0), n, k, m,
                             _stream(stream)))
    return y


def argmax(v, index=None, stream=None):
    """Greedy token of each row of f32 logits v [N] or [M, N] -> int32 [1] or [M]
    (ties: smallest index; NaN ranks highest)."""
    import torch
    v2 = v.unsqueeze(0) if v.dim() == 1 else v
    m, n = v2.shape
    if index is None:
        index = torch.empty(m, dtype=torch.int32, device=v.device)
    _check(lib().q4_argmax(_ptr(v2), v2.stride(0), n, m, _ptr(index), _stream(stream)))
    return index


def lm_head_argmax(W, S, x, logits=None, tokens=None, stream=None):
    """LM head with f32 logits and the greedy token of each row:
    x f16 [K] or [M, K] -> (logits f32 [N] or [M, N], tokens int32 [M])."""
    import torch
    n, k = W.shape[0], W.shape[1] * 8
    x2, m, ldx = _rows(x)
    if logits is None:
        logits = torch.empty((m, n) if x.dim() > 1 else (n,), dtype=torch.float32,
                             device=W.device)
    if tokens is None:
        tokens = torch.empty(m, dtype=torch.int32, device=W.device)
    l2 = logits.unsqueeze(0) if logits.dim() == 1 else logits
    _check(lib().q4_lm_head_argmax(_ptr(W), _ptr(S), _ptr(x2), ldx, _ptr(l2), l2.stride(0),
                                   _ptr(tokens), n, k, m, _stream(stream)))
    return logits, tokens


def attn_desc(n_heads, n_kv, head_dim, page_size=16, max_pages=257, n_pages=None,
              rope_base=10000.0):
    """Geometry of the RoPE / paged-KV / attention calls (see include/q4.h)."""
    return AttnDesc(n_heads, n_kv, head_dim, page_size, max_pages,
                    max_pages if n_pages is None else n_pages, rope_base)


def kv_page_bytes(desc):
    return int(lib().q4_kv_page_bytes(C.byref(desc)))


def kv_cache(desc, device="cuda"):
    """A zeroed cache f16 [n_pages][2][n_kv][page_size][head_dim]."""
    import torch
    return torch.zeros((desc.n_pages, 2, desc.n_kv, desc.page_size, desc.head_dim),
                       dtype=torch.float16, device=device)


def qkv_rope_append(W, S, x, desc, pos, page_table, kv, q_out=None, stream=None):
    """Fused decode step: q_out f16 [n_heads * head_dim]; K, V into kv at *pos."""
    import torch
    k = W.shape[1] * 8
    if q_out is None:
        q_out = torch.empty(desc.n_heads * desc.head_dim, dtype=torch.float16, device=W.device)
    _check(lib().q4_qkv_rope_append(_ptr(W), _ptr(S), _ptr(x), k, C.byref(desc), _ptr(pos),
                                    _ptr(page_table), _ptr(kv), _ptr(q_out), _stream(stream)))
    return q_out


def rope_append(qkv, desc, pos, page_table, kv, q_out=None, stream=None):
    """The same step from a stored f16 qkv vector."""
    import torch
    if q_out is None:
        q_out = torch.empty(desc.n_heads * desc.head_dim, dtype=torch.float16, device=qkv.device)
    _check(lib().q4_rope_append(_ptr(qkv), C.byref(desc), _ptr(pos), _ptr(page_table), _ptr(kv),
                                _ptr(q_out), _stream(stream)))
    return q_out


def attention_decode(q, kv, page_table, pos, max_len, desc, out=None, stream=None):
    """out f16 [n_heads * head_dim] = attention of q over cached positions 0..*pos."""
    import torch
    if out is None:
        out = torch.empty(desc.n_heads * desc.head_dim, dtype=torch.float16, device=q.device)
    _check(lib().q4_attention_decode(_ptr(q), _ptr(kv), _ptr(page_table), _ptr(pos), int(max_len),
                                     C.byref(desc), _ptr(out), _stream(stream)))
    return out


def moe_gemv(W, S, ids, x, ldx, x_slot_stride, route_w=None, epi_silu=False, y=None,
             stream=None):
    """One MoE expert stage. W int32 [E, N, K/8], S f16 [E, N, K/32], ids int32 [T, TOPK]."""
    import torch
    e, n, k = W.shape[0], W.shape[1], W.shape[2] * 8
    t, topk = ids.shape
    if y is None:
        if route_w is not None:
            shape = (t, n)
        else:
            shape = (t, topk, n // 2 if epi_silu else n)
        y = torch.empty(shape, dtype=torch.float16, device=W.device)
    _check(lib().q4_moe_gemv(_ptr(W), _ptr(S), _ptr(ids), _ptr(route_w), _ptr(x), ldx,
                             x_slot_stride, _ptr(y), e, n, k, t, topk, int(bool(epi_silu)),
                             _stream(stream)))
    return y


def add_rmsnorm(a, res_in, gamma, out=None, res_out=None, eps=1e-5, stream=None):
    """res_out = f16(a + res_in); out = f16(RMSNorm(res_out) * gamma). Rows of length D."""
    import torch
    d = res_in.shape[-1]
    m = res_in.numel() // d
    if out is None:
        out = torch.empty_like(res_in)
    if res_out is None:
        res_out = torch.empty_like(res_in)
    _check(lib().q4_add_rmsnorm(_ptr(a), _ptr(res_in), _ptr(gamma), _ptr(out), _ptr(res_out),
                                d, m, eps, _stream(stream)))
    return out, res_out


def silu_mul(gu, out=None, stream=None):
    """gu f16 [M, 2F] = [gate | up] -> f16 [M, F]."""
    import torch
    f2 = gu.shape[-1]
    m = gu.numel() // f2
    if out is None:
        out = torch.empty(gu.shape[:-1] + (f2 // 2,), dtype=torch.float16, device=gu.device)
    _check(lib().q4_silu_mul(_ptr(gu), _ptr(out), f2 // 2, m, _stream(stream)))
    return out


class Stack:
    """Holds a q4_stack_desc for a list of layers.

    layers: list of (Wqkv, Sqkv, Wo, So, Wgu, Sgu, Wdn, Sdn) device tensors;
    gamma_in, gamma_post: f16 [L, d]; gamma_final: f16 [d].
    """

    def __init__(self, layers, gamma_in, gamma_post, gamma_final, d, f, n_qkv, v_off, dv,
                 eps=1e-5, mode=STACK_AUTO):
        self.layers = layers
        self.gammas = (gamma_in, gamma_post, gamma_final)
        n = len(layers)
        self._arrays = []
        cols = []
        for j in range(8):
            arr = (C.c_void_p * n)(*[lay[j].data_ptr() for lay in layers])
            self._arrays.append(arr)
            cols.append(C.cast(arr, C.c_void_p))
        self.desc = StackDesc(n, d, f, n_qkv, v_off, dv, eps, *cols, gamma_in.data_ptr(),
                              gamma_post.data_ptr(), gamma_final.data_ptr(), mode)
        self.d = d
        self.n_layers = n

    def decode(self, r_in, h_in, r_out, h_out, trace=None, stream=None):
        _check(lib().q4_stack_decode(C.byref(self.desc), _ptr(r_in), _ptr(h_in), _ptr(r_out),
                                     _ptr(h_out), _ptr(trace), _stream(stream)))

    def decode_noalloc(self, r_in, h_in, r_out, h_out, trace=None, stream=None):
        """decode() through q4_stack_decode_noalloc (no allocation: the
        library's fixed per-GPU scratch)."""
        _check(lib().q4_stack_decode_noalloc(C.byref(self.desc), _ptr(r_in), _ptr(h_in),
                                             _ptr(r_out), _ptr(h_out), _ptr(trace),
                                             _stream(stream)))

    def set_mode(self, mode):
        self.desc.mode = mode

    def decode_attn(self, geom, caches, page_table, pos, max_len, r_in, h_in, r_out, h_out,
                    trace=None, stream=None):
        """One token with the real attention step: caches is a list of one
        device cache per layer (see kv_cache), pos an int32 device tensor."""
        arr = (C.c_void_p * len(caches))(*[c.data_ptr() for c in caches])
        self._attn_keep = (arr, geom)
        a = StackAttn(C.pointer(geom), C.cast(arr, C.c_void_p), page_table.data_ptr(),
                      pos.data_ptr(), int(max_len))
        _check(lib().q4_stack_decode_attn(C.byref(self.desc), C.byref(a), _ptr(r_in), _ptr(h_in),
                                          _ptr(r_out), _ptr(h_out), _ptr(trace),
                                          _stream(stream)))


def workspace_bytes(n, k, m):
    """Workspace bytes the largest matmul-family call on an n x k matrix with m
    activation rows (or MoE pairs) needs (q4_workspace_bytes)."""
    return int(lib().q4_workspace_bytes(int(n), int(k), int(m)))


def attention_workspace_bytes(desc, max_len):
    return int(lib().q4_attention_workspace_bytes(C.byref(desc), int(max_len)))


def stack_workspace_bytes(stack, geom=None):
    """Workspace bytes of stack.decode (geom None) or stack.decode_attn."""
    if geom is None:
        return int(lib().q4_stack_workspace_bytes(C.byref(stack.desc), None))
    a = StackAttn(C.pointer(geom), None, None, None, 1)
    return int(lib().q4_stack_workspace_bytes(C.byref(stack.desc), C.byref(a)))


def workspace_reserve(nbytes, stream=None):
    """Allocate the stream's workspace ahead of time (q4_workspace_reserve)."""
    _check(lib().q4_workspace_reserve(_stream(stream), int(nbytes)))


def workspace_release(stream=None):
    """Synchronise the stream and free its workspace (q4_workspace_release)."""
    _check(lib().q4_workspace_release(_stream(stream)))


def timer_arm(slot):
    """Measurement hook: the next matvec kernel this thread launches records
    its dispatch start and end on timer `slot` (0..63)."""
    _check(lib().q4_timer_arm(int(slot)))


def timer_read(slot):
    """Duration in microseconds of the launch timed on `slot` (waits for it)."""
    us = C.c_float()
    _check(lib().q4_timer_read(int(slot), C.byref(us)))
    return float(us.value)


def stack_decode(stack: Stack, r_in, h_in, r_out, h_out, trace=None, stream=None):
    stack.decode(r_in, h_in, r_out, h_out, trace, stream)
