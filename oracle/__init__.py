"""ctypes wrapper over the plain C oracle (``oracle/q4_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may use this package; the product library never does.

The shared object is built with gcc (``-O2``, no fast-math, no OpenMP), so it is
single-threaded and keeps IEEE semantics. ``load()`` builds it on first use when
it is missing or older than its source; ``build()`` always rebuilds.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_P = C.c_void_p
_I = C.c_int64


def compile_oracle(src: str, out: str) -> None:
    """Compile an oracle source file into a shared object with gcc."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build() -> str:
    compile_oracle(SRC, LIB)
    return LIB


_SIGS = {
    "q4o_h2d": (C.c_double, [C.c_uint16]),
    "q4o_d2h": (C.c_uint16, [C.c_double]),
    "q4o_h2d_array": (None, [_P, _P, _I]),
    "q4o_d2h_array": (None, [_P, _P, _I]),
    "q4o_pack": (None, [_P, _P, _I, _I]),
    "q4o_unpack": (None, [_P, _P, _I, _I]),
    "q4o_dequant": (None, [_P, _P, _I, _I, _P]),
    "q4o_gemv": (None, [_P, _P, _P, _I, _I, _P]),
    "q4o_gemv_rows": (None, [_P, _P, _P, _I, _I, _P, _I, _P]),
    "q4o_gemv_batched": (None, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "q4o_add_rmsnorm": (None, [_P, _P, _P, _I, _I, C.c_double, _P, _P]),
    "q4o_silu_mul": (None, [_P, _I, _I, _P]),
    "q4o_moe_stage": (None, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, C.c_int, _P]),
    "q4o_layer": (None, [_I] * 5 + [_P] * 8 + [_P, _P, C.c_double] + [_P] * 5),
    "q4o_stack": (None, [_I] * 6 + [_P] * 8 + [_P, _P, _P, C.c_double] + [_P] * 5),
    "q4o_argmax": (C.c_int64, [_P, _I]),
    "q4o_lm_head": (None, [_P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "q4o_rope": (None, [_P, _P, _I, _I, _I, C.c_double]),
    "q4o_qkv_rope": (None, [_P, _P, _P, _I, _I, _I, _I, _I, C.c_double, _P, _P, _P]),
    "q4o_attention": (None, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "q4o_gemv_affine": (None, [_P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "q4o_gemv_w16": (None, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "q4o_layer_attn": (None, [_I] * 6 + [C.c_double] + [_P] * 8 + [_P, _P, C.c_double] +
                       [_P] * 9),
}


class Oracle:
    """Typed numpy-facing calls into one oracle shared object."""

    def __init__(self, path: str):
        self.path = path
        self.lib = C.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(self.lib, name)
            fn.restype = res
            fn.argtypes = args

    # -- helpers -------------------------------------------------------------
    @staticmethod
    def _ptr(a):
        return None if a is None else a.ctypes.data

    @staticmethod
    def _u16(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.float16:
            a = a.view(np.uint16)
        assert a.dtype == np.uint16, a.dtype
        return a

    # -- binary16 ------------------------------------------------------------
    def h2d(self, h):
        h = self._u16(h)
        out = np.empty(h.shape, np.float64)
        self.lib.q4o_h2d_array(self._ptr(h), self._ptr(out), h.size)
        return out

    def d2h(self, d):
        d = np.ascontiguousarray(d, dtype=np.float64)
        out = np.empty(d.shape, np.uint16)
        self.lib.q4o_d2h_array(self._ptr(d), self._ptr(out), d.size)
        return out.view(np.float16)

    # -- format --------------------------------------------------------------
    def pack(self, codes):
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        n, k = codes.shape
        out = np.empty((n, k // 8), np.uint32)
        self.lib.q4o_pack(self._ptr(codes), self._ptr(out), n, k)
        return out

    def unpack(self, words, k=None):
        words = np.ascontiguousarray(words, dtype=np.uint32)
        n = words.shape[0]
        k = words.shape[1] * 8 if k is None else k
        out = np.empty((n, k), np.uint8)
        self.lib.q4o_unpack(self._ptr(words), self._ptr(out), n, k)
        return out

    def dequant(self, W, S):
        W = np.ascontiguousarray(W, dtype=np.uint32)
        S = self._u16(S)
        n, k = W.shape[0], W.shape[1] * 8
        out = np.empty((n, k), np.float64)
        self.lib.q4o_dequant(self._ptr(W), self._ptr(S), n, k, self._ptr(out))
        return out

    # -- matvec --------------------------------------------------------------
    def gemv(self, W, S, x):
        W = np.ascontiguousarray(W, dtype=np.uint32)
        S, x = self._u16(S), self._u16(x)
        n, k = W.shape[0], W.shape[1] * 8
        assert x.size == k
        y = np.empty(n, np.float64)
        self.lib.q4o_gemv(self._ptr(W), self._ptr(S), self._ptr(x), n, k, self._ptr(y))
        return y

    def gemv_rows(self, W, S, x, rows):
        W = np.ascontiguousarray(W, dtype=np.uint32)
        S, x = self._u16(S), self._u16(x)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n, k = W.shape[0], W.shape[1] * 8
        y = np.empty(rows.size, np.float64)
        self.lib.q4o_gemv_rows(self._ptr(W), self._ptr(S), self._ptr(x), n, k,
                               self._ptr(rows), rows.size, self._ptr(y))
        return y

    def gemv_batched(self, W, S, X):
        W = np.ascontiguousarray(W, dtype=np.uint32)
        S, X = self._u16(S), self._u16(X)
        n, k = W.shape[0], W.shape[1] * 8
        m = X.shape[0]
        assert X.shape[1] == k
        y = np.empty((m, n), np.float64)
        self.lib.q4o_gemv_batched(self._ptr(W), self._ptr(S), self._ptr(X), k, n, k, m,
                                  self._ptr(y))
        return y

    def gemv_w16(self, W, S, X):
        """Like gemv_batched, with every weight rounded to f16 before the sum."""
        W = np.ascontiguousarray(W, dtype=np.uint32)
        S = self._u16(S)
        one = np.asarray(X).ndim == 1
        X = self._u16(np.atleast_2d(X))
        n, k = W.shape[0], W.shape[1] * 8
        m = X.shape[0]
        assert X.shape[1] == k
        y = np.empty((m, n), np.float64)
        self.lib.q4o_gemv_w16(self._ptr(W), self._ptr(S), self._ptr(X), k, n, k, m, self._ptr(y))
        return y[0] if one else y

    # -- epilogues -----------------------------------------------------------
    # -- MLX affine format ------------------------------------------------------
    def gemv_affine(self, W, S, B, X):
        """X f16 [M, K] (or [K]) -> y f64 [M, N] (or [N]); w = S*q + B, group 64."""
        W = np.ascontiguousarray(W, dtype=np.uint32)
        S, B = self._u16(S), self._u16(B)
        one = np.asarray(X).ndim == 1
        X = self._u16(np.atleast_2d(X))
        n, k = W.shape[0], W.shape[1] * 8
        m = X.shape[0]
        assert X.shape[1] == k and S.shape == (n, k // 64) and B.shape == (n, k // 64)
        y = np.empty((m, n), np.float64)
        self.lib.q4o_gemv_affine(self._ptr(W), self._ptr(S), self._ptr(B), self._ptr(X), k, n, k,
                                 m, self._ptr(y))
        return y[0] if one else y

    # -- LM head and greedy sampling ------------------------------------------
    def argmax(self, v):
        """Index of the largest value (ties: smallest index; NaN ranks highest)."""
        v = np.ascontiguousarray(v, dtype=np.float64).ravel()
        assert v.size >= 1
        return int(self.lib.q4o_argmax(self._ptr(v), v.size))

    def lm_head(self, W, S, X):
        """X f16 [M, K] -> (exact logits f64 [M, N], greedy tokens int64 [M])."""
        W = np.ascontiguousarray(W, dtype=np.uint32)
        S, X = self._u16(S), self._u16(np.atleast_2d(X))
        n, k = W.shape[0], W.shape[1] * 8
        m = X.shape[0]
        assert X.shape[1] == k
        logits = np.empty((m, n), np.float64)
        tokens = np.empty(m, np.int64)
        self.lib.q4o_lm_head(self._ptr(W), self._ptr(S), self._ptr(X), k, n, k, m,
                             self._ptr(logits), self._ptr(tokens))
        return logits, tokens

    # -- RoPE, KV cache, decode attention --------------------------------------
    def rope(self, v, head_dim, pos, base=10000.0):
        """v f64/f16 [n_heads * head_dim] -> rotated f64 (pairs i, i + head_dim/2)."""
        v = np.ascontiguousarray(np.asarray(v, dtype=np.float64).ravel())
        out = np.empty_like(v)
        self.lib.q4o_rope(self._ptr(v), self._ptr(out), v.size // head_dim, head_dim, pos, base)
        return out

    def qkv_rope(self, W, S, x, n_heads, n_kv, head_dim, pos, base=10000.0):
        """-> (q_rot f64 [n_heads*hd], k_rot f64 [n_kv*hd], v f64 [n_kv*hd])."""
        W = np.ascontiguousarray(W, dtype=np.uint32)
        S, x = self._u16(S), self._u16(x)
        k = W.shape[1] * 8
        q = np.empty(n_heads * head_dim, np.float64)
        kr = np.empty(n_kv * head_dim, np.float64)
        v = np.empty(n_kv * head_dim, np.float64)
        self.lib.q4o_qkv_rope(self._ptr(W), self._ptr(S), self._ptr(x), k, n_heads, n_kv,
                              head_dim, pos, base, self._ptr(q), self._ptr(kr), self._ptr(v))
        return q, kr, v

    def attention(self, q, kc, vc, n_heads, n_kv, head_dim):
        """q f16 [n_heads*hd]; kc, vc f16 [L][n_kv][hd] -> f64 [n_heads*hd]."""
        q, kc, vc = self._u16(q), self._u16(kc), self._u16(vc)
        L = kc.size // (n_kv * head_dim)
        out = np.empty(n_heads * head_dim, np.float64)
        self.lib.q4o_attention(self._ptr(q), self._ptr(kc), self._ptr(vc), L, n_heads, n_kv,
                               head_dim, self._ptr(out))
        return out

    def add_rmsnorm(self, a, r, gamma, eps=1e-5):
        r = self._u16(np.atleast_2d(r))
        m, d = r.shape
        a_ = None if a is None else self._u16(np.atleast_2d(a))
        g = self._u16(gamma)
        res_out = np.empty((m, d), np.uint16)
        out = np.empty((m, d), np.float64)
        self.lib.q4o_add_rmsnorm(self._ptr(a_), self._ptr(r), self._ptr(g), d, m, eps,
                                 self._ptr(res_out), self._ptr(out))
        return res_out.view(np.float16), out

    def silu_mul(self, gu):
        gu = self._u16(np.atleast_2d(gu))
        m, f2 = gu.shape
        f = f2 // 2
        out = np.empty((m, f), np.float64)
        self.lib.q4o_silu_mul(self._ptr(gu), f, m, self._ptr(out))
        return out

    # -- MoE -----------------------------------------------------------------
    def moe_stage(self, W, S, ids, route_w, x, ldx, x_slot_stride, n, k, epi_silu):
        """See q4o_moe_stage. W: uint32[E][n][k/8], S: f16[E][n][k/32]."""
        W = np.ascontiguousarray(W, dtype=np.uint32)
        S = self._u16(S)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        t, topk = ids.shape
        rw = None if route_w is None else self._u16(route_w)
        x = self._u16(x)
        e = W.shape[0]
        if epi_silu:
            y = np.empty((t, topk, n // 2), np.float64)
        elif rw is None:
            y = np.empty((t, topk, n), np.float64)
        else:
            y = np.empty((t, n), np.float64)
        self.lib.q4o_moe_stage(self._ptr(W), self._ptr(S), self._ptr(ids), self._ptr(rw),
                               self._ptr(x), ldx, x_slot_stride, e, n, k, t, topk,
                               int(bool(epi_silu)), self._ptr(y))
        return y

    # -- stack ---------------------------------------------------------------
    def layer(self, dims, mats, gamma_post, gamma_next, r, h, eps=1e-5):
        """One decoder layer. dims = (d, f, n_qkv, v_off, dv);
        mats = (Wqkv, Sqkv, Wo, So, Wgu, Sgu, Wdn, Sdn)."""
        d = dims[0]
        mats = [np.ascontiguousarray(m) if m.dtype == np.uint32 else self._u16(m)
                for m in mats]
        r, h = self._u16(r), self._u16(h)
        gp, gn = self._u16(gamma_post), self._u16(gamma_next)
        r_out = np.empty(d, np.uint16)
        h_out = np.empty(d, np.uint16)
        h64 = np.empty(d, np.float64)
        self.lib.q4o_layer(*dims, *[self._ptr(m) for m in mats], self._ptr(gp),
                           self._ptr(gn), eps, self._ptr(r), self._ptr(h), self._ptr(r_out),
                           self._ptr(h_out), self._ptr(h64))
        return r_out.view(np.float16), h_out.view(np.float16), h64

    def layer_attn(self, geom, pos, mats, gamma_post, gamma_next, r, h, kc_prev, vc_prev,
                   eps=1e-5, base=10000.0):
        """One layer with RoPE, the KV append at pos and attention over 0..pos.
        geom = (d, f, n_heads, n_kv, head_dim); kc_prev, vc_prev f16
        [pos][n_kv][head_dim]. Returns (r_out, h_out, h64, k_new, v_new)."""
        d, f, nh, nkv, hd = geom
        mats = [np.ascontiguousarray(m) if m.dtype == np.uint32 else self._u16(m)
                for m in mats]
        r, h = self._u16(r), self._u16(h)
        gp, gn = self._u16(gamma_post), self._u16(gamma_next)
        kp = self._u16(np.ascontiguousarray(kc_prev).reshape(-1)) if pos > 0 else np.zeros(1, np.uint16)
        vp = self._u16(np.ascontiguousarray(vc_prev).reshape(-1)) if pos > 0 else np.zeros(1, np.uint16)
        r_out = np.empty(d, np.uint16)
        h_out = np.empty(d, np.uint16)
        h64 = np.empty(d, np.float64)
        k_new = np.empty(nkv * hd, np.uint16)
        v_new = np.empty(nkv * hd, np.uint16)
        self.lib.q4o_layer_attn(d, f, nh, nkv, hd, pos, base, *[self._ptr(m) for m in mats],
                                self._ptr(gp), self._ptr(gn), eps, self._ptr(r), self._ptr(h),
                                self._ptr(kp), self._ptr(vp), self._ptr(r_out), self._ptr(h_out),
                                self._ptr(h64), self._ptr(k_new), self._ptr(v_new))
        return (r_out.view(np.float16), h_out.view(np.float16), h64, k_new.view(np.float16),
                v_new.view(np.float16))

    def stack(self, dims, layers, gamma_in, gamma_post, gamma_final, r, h, eps=1e-5,
              trace=False):
        """layers: list of (Wqkv, Sqkv, Wo, So, Wgu, Sgu, Wdn, Sdn) per layer."""
        d = dims[0]
        n_layers = len(layers)
        keep = []
        arrs = []
        for j in range(8):
            col = []
            for lay in layers:
                m = lay[j]
                m = np.ascontiguousarray(m) if m.dtype == np.uint32 else self._u16(m)
                keep.append(m)
                col.append(m.ctypes.data)
            arrs.append((C.c_void_p * n_layers)(*col))
        gi, gp, gf = self._u16(gamma_in), self._u16(gamma_post), self._u16(gamma_final)
        r = self._u16(r).copy()
        h = self._u16(h).copy()
        h64 = np.empty(d, np.float64)
        tr = np.empty((n_layers, d), np.uint16) if trace else None
        th = np.empty((n_layers, d), np.uint16) if trace else None
        self.lib.q4o_stack(n_layers, *dims, *[C.cast(a, C.c_void_p) for a in arrs],
                           self._ptr(gi), self._ptr(gp), self._ptr(gf), eps,
                           self._ptr(r), self._ptr(h), self._ptr(h64), self._ptr(tr),
                           self._ptr(th))
        out = (r.view(np.float16), h.view(np.float16), h64)
        if trace:
            out = out + (tr.view(np.float16), th.view(np.float16))
        return out


_default = None


def load() -> Oracle:
    """The oracle built from ``q4_oracle.c`` (compiled on first use if stale)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB)
    return _default


def load_variant(source_text: str, tag: str) -> Oracle:
    """Compile an edited copy of the oracle source (used to plant mistakes in
    tests of the tests) and load it."""
    d = tempfile.mkdtemp(prefix="q4o_%s_" % tag)
    src = os.path.join(d, "q4_oracle_%s.c" % tag)
    with open(src, "w") as fh:
        fh.write(source_text)
    out = os.path.join(d, "liboracle_%s.so" % tag)
    compile_oracle(src, out)
    return Oracle(out)
