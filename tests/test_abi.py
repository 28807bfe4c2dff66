"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* libq4.so loads and exports every function declared in include/q4.h.
* Argument validation returns the documented status before anything is
  enqueued: these calls use fake (never dereferenced) pointer values.
* The byte accounting of the format matches the pages' figures.
"""
import ctypes as C
import json
import os
import re

import pytest

import int4_weight_only_q4_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(q4.ABI_SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = q4.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert "gfx950" in q4.version()


def test_bytes_per_weight():
    assert q4.lib().q4_bytes_per_weight() == 0.5625 == q4.BYTES_PER_WEIGHT


def test_per_token_bytes_match_bandwidth_ceiling_passage():
    """Zero TVM Documentation, 'The memory-bandwidth ceiling': the q4 shape table
    summed over 32 layers plus the LM head (and one embedding row) is ~2.09 GB
    per token, ~5.2 ms at 400 GB/s, ~191 tok/s."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "phi3_q4f16_shapes.json")))
    t = g["tensors"]

    def tensor_bytes(name, rows=None):
        n, words = t[name]["q_weight"]
        k = words * 8
        return (rows if rows is not None else n) * k * q4.BYTES_PER_WEIGHT

    layer = sum(tensor_bytes(x) for x in ("qkv_proj", "o_proj", "gate_up", "down"))
    total = g["layers"] * layer + tensor_bytes("lm_head") + tensor_bytes("embedding", rows=1)
    assert abs(total / 1e9 - g["bytes_per_token_GB_approx"]) < 0.005
    assert abs(total / (g["bus_GB_per_s"] * 1e9) * 1e3 - g["ms_per_token_approx"]) < 0.05
    assert abs(g["bus_GB_per_s"] * 1e9 / total - g["tok_per_s_ceiling_approx"]) < 1.0
    assert g["layers"] * layer == 2_038_431_744      # the 32-layer stack without LM head


def test_density_matches_mlc_build():
    """MLC-COMPILE.md: a q4f16_1 build reports 4.503 bits/param; the quantised
    weights cost exactly 4.5 bits each, the rest being unquantised tensors."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "mlc_density.json")))
    bits = q4.BYTES_PER_WEIGHT * 8
    assert bits == 4.5 and 0 <= g["bits_per_param"] - bits < 0.01


# ---------------------------------------------------------------------------
# validation: fake device pointers, never dereferenced
# ---------------------------------------------------------------------------
A = 0x7F0000000000  # 16-byte aligned fake addresses, far apart
B = A + 0x10000000
X = A + 0x20000000
Y = A + 0x30000000
R = A + 0x40000000


def status(fn, *args):
    return getattr(q4.lib(), fn)(*args)


def test_gemv_validation():
    assert status("q4_gemv", None, B, X, Y, 16, 64, None) == q4.Q4_EINVAL
    assert status("q4_gemv", A, B, X, Y, 0, 64, None) == q4.Q4_EINVAL
    assert status("q4_gemv", A, B, X, Y, 16, 48, None) == q4.Q4_ESHAPE
    assert status("q4_gemv", A, B, X, Y, 16, q4.MAX_K + 32, None) == q4.Q4_ERANGE
    assert status("q4_gemv", A + 4, B, X, Y, 16, 64, None) == q4.Q4_EALIGN
    assert status("q4_gemv", A, B, X + 2, Y, 16, 64, None) == q4.Q4_EALIGN
    # output inside the weights / the activation
    assert status("q4_gemv", A, B, X, A + 64, 16, 64, None) == q4.Q4_EALIAS
    assert status("q4_gemv", A, B, X, X + 8, 16, 64, None) == q4.Q4_EALIAS
    assert "overlaps" in q4.lib().q4_last_error().decode()


def test_gemv_ex_validation():
    ep = q4.Epilogue(7, None, None, None, 1e-5)
    assert status("q4_gemv_ex", A, B, X, Y, 16, 64, C.byref(ep), None) == q4.Q4_EINVAL
    ep = q4.Epilogue(q4.EPI_SILU_MUL, None, None, None, 1e-5)
    assert status("q4_gemv_ex", A, B, X, Y, 15, 64, C.byref(ep), None) == q4.Q4_ESHAPE
    ep = q4.Epilogue(q4.EPI_ADD_RMSNORM, R, None, R + 4096, 1e-5)
    assert status("q4_gemv_ex", A, B, X, Y, 16, 64, C.byref(ep), None) == q4.Q4_EINVAL
    # the ping-pong rule: res_out may not overlap res_in
    ep = q4.Epilogue(q4.EPI_ADD_RMSNORM, R, R + 8192, R + 16, 1e-5)
    assert status("q4_gemv_ex", A, B, X, Y, 16, 64, C.byref(ep), None) == q4.Q4_EALIAS
    ep = q4.Epilogue(q4.EPI_ADD_RMSNORM, R, R + 8192, R + 4096, -1.0)
    assert status("q4_gemv_ex", A, B, X, Y, 16, 64, C.byref(ep), None) == q4.Q4_EINVAL
    # a normalising prologue: aligned gamma, not together with add+RMSNorm
    ep = q4.Epilogue(q4.EPI_ADD_RMSNORM, R, R + 8192, R + 4096, 1e-5, R + 16384)
    assert status("q4_gemv_ex", A, B, X, Y, 16, 64, C.byref(ep), None) == q4.Q4_EINVAL
    ep = q4.Epilogue(q4.EPI_SILU_MUL, None, None, None, 1e-5, R + 2)
    assert status("q4_gemv_ex", A, B, X, Y, 16, 64, C.byref(ep), None) == q4.Q4_EALIGN


def test_batched_validation():
    assert status("q4_gemv_batched", A, B, X, 64, Y, 16, 16, 64, 0, None) == q4.Q4_ERANGE
    assert status("q4_gemv_batched", A, B, X, 64, Y, 16, 16, 64, q4.MAX_M + 1, None) == q4.Q4_ERANGE
    assert status("q4_gemv_batched", A, B, X, 60, Y, 16, 16, 64, 2, None) == q4.Q4_EINVAL
    assert status("q4_gemv_batched", A, B, X, 68, Y, 16, 16, 64, 2, None) == q4.Q4_EALIGN
    assert status("q4_gemv_batched", A, B, X, 64, X + 64, 16, 16, 64, 2, None) == q4.Q4_EALIAS


def test_moe_validation():
    args = [A, B, R, None, X, 64, 0, Y, 8, 16, 64, 2, 4, 1, None]
    bad = list(args); bad[3] = R + 4096   # SiLU epilogue together with a routing combine
    assert status("q4_moe_gemv", *bad) == q4.Q4_EINVAL
    bad = list(args); bad[9] = 15          # odd N with SiLU
    assert status("q4_moe_gemv", *bad) == q4.Q4_ESHAPE
    bad = list(args); bad[12] = 5000; bad[13] = 1   # too many (token, slot) pairs
    assert status("q4_moe_gemv", *bad) == q4.Q4_ERANGE
    bad = list(args); bad[6] = 4          # slot stride breaks 16-byte alignment
    assert status("q4_moe_gemv", *bad) == q4.Q4_EALIGN
    bad = list(args); bad[7] = R          # output over the ids
    assert status("q4_moe_gemv", *bad) == q4.Q4_EALIAS


def test_norm_and_silu_validation():
    assert status("q4_add_rmsnorm", None, R, B, Y, R, 64, 1, 1e-5, None) == q4.Q4_EALIAS
    assert status("q4_add_rmsnorm", None, R, None, Y, X, 64, 1, 1e-5, None) == q4.Q4_EINVAL
    assert status("q4_add_rmsnorm", None, R, B, R + 64, X, 64, 1, 1e-5, None) == q4.Q4_EALIAS
    assert status("q4_silu_mul", X, X + 64, 64, 1, None) == q4.Q4_EALIAS
    assert status("q4_silu_mul", X, Y, 0, 1, None) == q4.Q4_EINVAL


def test_stack_validation():
    arr = (C.c_void_p * 1)(A)
    sarr = (C.c_void_p * 1)(B)
    ptr = C.cast(arr, C.c_void_p)
    sptr = C.cast(sarr, C.c_void_p)
    d = q4.StackDesc(1, 64, 64, 192, 128, 64, 1e-5, ptr, sptr, ptr, sptr, ptr, sptr, ptr, sptr,
                     R, R + 4096, R + 8192)
    st = q4.lib().q4_stack_decode
    assert st(None, X, X + 4096, Y, Y + 4096, None, None) == q4.Q4_EINVAL
    # outputs over inputs
    assert st(C.byref(d), X, X + 4096, X, Y + 4096, None, None) == q4.Q4_EALIAS
    d.v_off = 160
    assert st(C.byref(d), X, X + 4096, Y, Y + 4096, None, None) == q4.Q4_ESHAPE
    d.v_off = 124
    d.dv = 64
    assert st(C.byref(d), X, X + 4096, Y, Y + 4096, None, None) == q4.Q4_EALIGN
    d.v_off = 128
    d.d = 48
    assert st(C.byref(d), X, X + 4096, Y, Y + 4096, None, None) == q4.Q4_ESHAPE


def test_pack_validation():
    assert status("q4_pack", None, A, 4, 64, None) == q4.Q4_EINVAL
    assert status("q4_pack", X, A, 4, 40, None) == q4.Q4_ESHAPE
    assert status("q4_pack", X, A + 4, 4, 64, None) == q4.Q4_EALIGN
    assert status("q4_pack", X, X + 16, 4, 64, None) == q4.Q4_EALIAS


def test_timer_validation():
    L = q4.lib()
    assert L.q4_timer_arm(-1) == q4.Q4_EINVAL
    assert L.q4_timer_arm(64) == q4.Q4_EINVAL
    us = C.c_float()
    assert L.q4_timer_read(64, C.byref(us)) == q4.Q4_EINVAL
    assert L.q4_timer_read(3, None) == q4.Q4_EINVAL
    # slot 7 was never armed for a launch on this thread
    assert L.q4_timer_read(7, C.byref(us)) == q4.Q4_EINVAL


def test_lm_head_validation():
    # q4_gemv_f32: W, S, x, ldx, y, ldy, N, K, M
    assert status("q4_gemv_f32", A, B, X, 64, None, 16, 16, 64, 1, None) == q4.Q4_EINVAL
    assert status("q4_gemv_f32", A, B, X, 64, Y, 16, 16, 64, 0, None) == q4.Q4_ERANGE
    assert status("q4_gemv_f32", A, B, X, 64, Y, 8, 16, 64, 2, None) == q4.Q4_EINVAL
    assert status("q4_gemv_f32", A, B, X, 64, Y + 2, 16, 16, 64, 1, None) == q4.Q4_EALIGN
    assert status("q4_gemv_f32", A, B, X, 64, X + 64, 16, 16, 64, 1, None) == q4.Q4_EALIAS
    # q4_argmax: v, ld, N, M, index
    assert status("q4_argmax", None, 16, 16, 1, Y, None) == q4.Q4_EINVAL
    assert status("q4_argmax", X, 16, 0, 1, Y, None) == q4.Q4_EINVAL
    assert status("q4_argmax", X, 8, 16, 2, Y, None) == q4.Q4_EINVAL
    assert status("q4_argmax", X, 1 << 31, 1 << 31, 1, Y, None) == q4.Q4_ERANGE
    assert status("q4_argmax", X, 16, 16, 65536, Y, None) == q4.Q4_ERANGE
    assert status("q4_argmax", X + 2, 16, 16, 1, Y, None) == q4.Q4_EALIGN
    assert status("q4_argmax", X, 16, 16, 1, X + 60, None) == q4.Q4_EALIAS
    # q4_lm_head_argmax: W, S, x, ldx, logits, ldl, tokens, N, K, M
    assert status("q4_lm_head_argmax", A, B, X, 64, Y, 16, None, 16, 64, 1, None) == q4.Q4_EINVAL
    assert status("q4_lm_head_argmax", A, B, X, 64, Y, 16, R + 2, 16, 64, 1, None) == q4.Q4_EALIGN
    assert status("q4_lm_head_argmax", A, B, X, 64, Y, 16, Y + 32, 16, 64, 1, None) == q4.Q4_EALIAS
    assert status("q4_lm_head_argmax", A, B, X, 64, Y, 16, X, 16, 64, 1, None) == q4.Q4_EALIAS
    assert status("q4_lm_head_argmax", A, B, X, 64, Y, 16, R, 16, 48, 1, None) == q4.Q4_ESHAPE


def test_kv_cache_geometry_matches_page_table():
    """Zero TVM Documentation, 'KV cache': 16-slot pages of 196,608 bytes (32
    heads x 16 slots x 96 dims x K+V x 2 bytes), 257 pages ~ 4096 tokens,
    ~50 MB per layer and ~1.6 GB for 32 layers."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "kv_cache_phi3.json")))
    assert g["heads"] * g["head_dim"] == g["hidden"]
    d = q4.attn_desc(g["heads"], g["heads"], g["head_dim"], g["page_size"], g["max_pages"])
    assert q4.kv_page_bytes(d) == g["bytes_per_page"]
    per_layer = g["max_pages"] * g["bytes_per_page"]
    assert abs(per_layer / 1e6 - g["per_layer_MB_approx"]) < 1.0
    assert abs(g["layers"] * per_layer / 1e9 - g["total_GB_approx"]) < 0.05
    assert abs(g["max_pages"] * g["page_size"] - g["context_tokens_approx"]) <= g["page_size"]


def test_attention_validation():
    L = q4.lib()
    d = q4.attn_desc(32, 32, 96)
    args = lambda **kw: [kw.get(k, v) for k, v in
                         (("W", A), ("S", B), ("x", X), ("K", 3072), ("d", C.byref(d)),
                          ("pos", R), ("pt", R + 64), ("kv", R + 65536), ("q", Y), ("s", None))]
    assert L.q4_qkv_rope_append(*args(d=None)) == q4.Q4_EINVAL
    bad = q4.attn_desc(32, 5, 96)  # n_kv does not divide n_heads
    assert L.q4_qkv_rope_append(*args(d=C.byref(bad))) == q4.Q4_EINVAL
    bad = q4.attn_desc(32, 32, 100)  # head_dim not a multiple of 8
    assert L.q4_qkv_rope_append(*args(d=C.byref(bad))) == q4.Q4_ESHAPE
    assert L.q4_qkv_rope_append(*args(K=48)) == q4.Q4_ESHAPE
    assert L.q4_qkv_rope_append(*args(pos=None)) == q4.Q4_EINVAL
    assert L.q4_qkv_rope_append(*args(kv=R + 65536 + 8)) == q4.Q4_EALIGN
    assert L.q4_qkv_rope_append(*args(q=R + 65536 + 64)) == q4.Q4_EALIAS  # q_out inside the cache
    assert L.q4_rope_append(None, C.byref(d), R, R + 64, R + 65536, Y, None) == q4.Q4_EINVAL
    assert L.q4_rope_append(X, C.byref(d), R, R + 64, X + 64, Y, None) == q4.Q4_EALIAS
    att = L.q4_attention_decode
    assert att(X, R + 65536, R + 64, R, 0, C.byref(d), Y, None) == q4.Q4_EINVAL
    assert att(X, R + 65536 + 2, R + 64, R, 16, C.byref(d), Y, None) == q4.Q4_EALIGN
    assert att(X, R + 65536, R + 64, R, 16, C.byref(d), X + 2, None) == q4.Q4_EALIAS
    odd = q4.attn_desc(4, 4, 80)  # a multiple of 8 without a kernel
    assert att(X, R + 65536, R + 64, R, 16, C.byref(odd), Y, None) == q4.Q4_ESHAPE


def test_stack_attention_validation():
    arr = (C.c_void_p * 1)(A)
    sarr = (C.c_void_p * 1)(B)
    ptr, sptr = C.cast(arr, C.c_void_p), C.cast(sarr, C.c_void_p)
    g = q4.attn_desc(4, 2, 64, 16, 8, 8)
    kv = (C.c_void_p * 1)(R + 0x100000)
    a = q4.StackAttn(C.pointer(g), C.cast(kv, C.c_void_p), R, R + 64, 128)
    # n_qkv = (4 + 4) * 64 = 512, dv = 256
    d = q4.StackDesc(1, 256, 512, 512, 0, 256, 1e-5, ptr, sptr, ptr, sptr, ptr, sptr, ptr, sptr,
                     R + 4096, R + 8192, R + 12288)
    st = q4.lib().q4_stack_decode_attn
    assert st(C.byref(d), None, X, X + 4096, Y, Y + 4096, None, None) == q4.Q4_EINVAL
    d.dv = 192
    assert st(C.byref(d), C.byref(a), X, X + 4096, Y, Y + 4096, None, None) == q4.Q4_ESHAPE
    d.dv = 256
    d.mode = 2  # no such mode (only the multi-kernel path exists)
    assert st(C.byref(d), C.byref(a), X, X + 4096, Y, Y + 4096, None, None) == q4.Q4_EINVAL
    d.mode = q4.STACK_AUTO
    a.max_len = 0
    assert st(C.byref(d), C.byref(a), X, X + 4096, Y, Y + 4096, None, None) == q4.Q4_EINVAL
    a.max_len = 128
    kv[0] = Y  # the cache over the outputs
    assert st(C.byref(d), C.byref(a), X, X + 4096, Y, Y + 4096, None, None) == q4.Q4_EALIAS


def test_affine_validation():
    f = q4.lib().q4_gemv_affine
    assert f(A, B, None, X, 128, Y, 16, 16, 128, 1, None) == q4.Q4_EINVAL
    assert f(A, B, R, X, 96, Y, 16, 16, 96, 1, None) == q4.Q4_ESHAPE      # K % 64
    assert f(A, B, R, X, 128, Y, 16, 16, 128, 0, None) == q4.Q4_ERANGE
    assert f(A, B, R, X, 128, Y, 8, 16, 128, 2, None) == q4.Q4_EINVAL     # ldy < N
    assert f(A, B, R + 1, X, 128, Y, 16, 16, 128, 1, None) == q4.Q4_EALIGN
    assert f(A, B, R, X, 128, R, 16, 16, 128, 1, None) == q4.Q4_EALIAS    # y over the biases


def test_gemm_validation():
    f = q4.lib().q4_gemm
    assert f(A, B, None, 128, Y, 16, 16, 128, 1, 0, None) == q4.Q4_EINVAL
    assert f(A, B, X, 128, Y, 16, 16, 128, 4, 2, None) == q4.Q4_EINVAL     # unknown weights mode
    assert f(A, B, X, 96, Y, 16, 16, 100, 4, 0, None) == q4.Q4_ESHAPE      # K % 32
    assert f(A, B, X, 128, Y, 16, 16, 128, 0, 0, None) == q4.Q4_ERANGE     # M < 1
    assert f(A, B, X, 128, Y, 16, 16, 128, q4.MAX_GEMM_M + 1, 1, None) == q4.Q4_ERANGE
    assert f(A, B, X, 120, Y, 16, 16, 128, 4, 0, None) == q4.Q4_EINVAL     # ldx < K
    assert f(A, B, X, 128, Y, 8, 16, 128, 4, 0, None) == q4.Q4_EINVAL      # ldy < N
    assert f(A, B, X + 8, 128, Y, 16, 16, 128, 4, 0, None) == q4.Q4_EALIGN
    assert f(A, B, X, 132, Y, 16, 16, 128, 4, 0, None) == q4.Q4_EALIGN     # ldx % 8
    assert f(A, B, X, 128, Y + 1, 16, 16, 128, 4, 0, None) == q4.Q4_EALIGN
    assert f(A, B, X, 128, X + 64, 16, 16, 128, 4, 0, None) == q4.Q4_EALIAS  # y over x
    assert f(A, B, X, 128, B, 16, 16, 128, 4, 1, None) == q4.Q4_EALIAS     # y over the scales


def test_gemm_affine_validation():
    f = q4.lib().q4_gemm_affine
    assert f(A, B, None, X, 128, Y, 16, 16, 128, 4, None) == q4.Q4_EINVAL     # no biases
    assert f(A, B, R, X, 96, Y, 16, 16, 96, 4, None) == q4.Q4_ESHAPE        # K % 64
    assert f(A, B, R, X, 128, Y, 16, 16, 128, 0, None) == q4.Q4_ERANGE      # M < 1
    assert f(A, B, R, X, 128, Y, 8, 16, 128, 4, None) == q4.Q4_EINVAL       # ldy < N
    assert f(A, B, R + 1, X, 128, Y, 16, 16, 128, 4, None) == q4.Q4_EALIGN
    assert f(A, B, R, X + 8, 128, Y, 16, 16, 128, 4, None) == q4.Q4_EALIGN
    assert f(A, B, R, X, 128, R, 16, 16, 128, 4, None) == q4.Q4_EALIAS      # y over the biases


# ---------------------------------------------------------------------------
# workspace sizes (host-only queries; no device work)
# ---------------------------------------------------------------------------

def _al(b):
    return (b + 255) // 256 * 256


def test_workspace_bytes_invalid_shapes_are_zero():
    f = q4.lib().q4_workspace_bytes
    assert f(0, 256, 1) == 0
    assert f(16, 100, 1) == 0                 # K % 32
    assert f(16, q4.MAX_K + 32, 1) == 0       # K > Q4_MAX_K
    assert f(16, 256, 0) == 0


def test_workspace_bytes_at_each_entry_points_maximum_shapes():
    """Every matmul-family entry point at its largest shape gets a finite size
    that covers the 256-byte header, and the size never shrinks as M grows
    (prefill partials, MoE pairs, argmax rows)."""
    f = q4.lib().q4_workspace_bytes
    cases = [
        (151936, 2560, q4.MAX_M),          # LM head / batched matvec, largest M
        (151936, 2560, 1),                 # LM head + argmax at one row
        (65536, q4.MAX_K, q4.MAX_M),       # batched matvec at the largest K
        (16384, q4.MAX_K, q4.MAX_GEMM_M),  # prefill, largest M and K
        (1536, 2048, q4.MAX_PAIRS),        # one MoE stage, largest pair count
        (2048, 768, q4.MAX_PAIRS),
    ]
    for n, k, m in cases:
        b = f(n, k, m)
        assert 256 < b < (1 << 36), (n, k, m, b)
    for n, k in ((3072, 8192), (19456, 2560), (512, 256)):
        prev = 0
        for m in (1, 2, 5, 16, 64, 256, 1024, 4096):
            b = f(n, k, m)
            assert b >= prev, (n, k, m)
            prev = b


def test_attention_workspace_bytes():
    """One split (at most 256 positions) needs nothing; more positions need the
    split partials: (max, sum, weighted values) per head and split, 32 splits."""
    g = q4.attn_desc(32, 32, 96)
    f = q4.lib().q4_attention_workspace_bytes
    assert f(C.byref(g), 1) == 0
    assert f(C.byref(g), 256) == 0
    assert f(C.byref(g), 4096) == 256 + 32 * 32 * (2 + 96) * 4
    assert f(C.byref(g), 0) == 0
    assert f(None, 4096) == 0


def test_stack_workspace_bytes():
    """header | qkv | r1 | u | two residual buffers [| attention output |
    attention partials], each 256-byte aligned (Phi-3-mini shapes)."""
    arr = (C.c_void_p * 1)(A)
    ptr = C.cast(arr, C.c_void_p)
    d = q4.StackDesc(32, 3072, 8192, 9216, 6144, 3072, 1e-5, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                     ptr, R, R + 4096, R + 8192)
    f = q4.lib().q4_stack_workspace_bytes
    base = 256 + _al(9216 * 2) + 3 * _al(3072 * 2) + _al(8192 * 2)
    assert f(C.byref(d), None) == base
    g = q4.attn_desc(32, 32, 96)
    a = q4.StackAttn(C.pointer(g), None, None, None, 1024)
    assert f(C.byref(d), C.byref(a)) == base + _al(3072 * 2) + _al(32 * 32 * (2 + 96) * 4)
    assert f(None, None) == 0


def test_noalloc_stack_refuses_vectors_beyond_the_fixed_scratch():
    """q4_stack_decode_noalloc checks on the host that the stack's intermediate
    vectors fit its fixed scratch; a larger stack is Q4_ERANGE with nothing
    enqueued (fake device addresses are never touched)."""
    arr = (C.c_void_p * 1)(A)
    ptr = C.cast(arr, C.c_void_p)
    f = q4.lib().q4_stack_decode_noalloc
    # 600000 QKV rows: 1.2 MB of qkv alone
    d = q4.StackDesc(1, 256, 512, 600000, 512, 256, 1e-5, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                     ptr, R, R + 4096, R + 8192)
    assert q4.lib().q4_stack_workspace_bytes(C.byref(d), None) > q4.NOALLOC_SCRATCH_BYTES
    assert f(C.byref(d), X, X + 4096, Y, Y + 4096, None, None) == q4.Q4_ERANGE
    assert "fixed scratch" in q4.lib().q4_last_error().decode()
    assert f(None, X, X + 4096, Y, Y + 4096, None, None) == q4.Q4_EINVAL
