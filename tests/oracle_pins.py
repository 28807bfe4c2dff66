"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError if
the oracle disagrees with a closed form, a special case, a brute-force count,
a library routine or a value printed on the pages. The same functions run
against deliberately broken copies of the oracle in ``test_oracle_pins.py`` to
show that a plausible mistake anywhere in it fails at least one pin.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import datagen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _mat(o, seed, n, k, codes=None):
    c = datagen.codes(seed, n, k) if codes is None else np.asarray(codes, np.uint8)
    s = datagen.scales(seed + 1, n, k)
    return c, o.pack(c), s


def _f16(v):
    return np.asarray(v, dtype=np.float64).astype(np.float16)


# --------------------------------------------------------------------------
# binary16 conversion: reduces to numpy's IEEE conversions (library routine)
# --------------------------------------------------------------------------

def pin_h2d_every_pattern(o):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = o.h2d(h)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_d2h_round_to_nearest_even(o):
    # every midpoint between consecutive finite binary16 values (ties), their
    # binary64 neighbours, plus random values over the whole range
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2
    cand = np.concatenate([mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), lo,
                           [65504.0, 65519.99, 65520.0, 1e6, 0.0, 2.0 ** -25, 2.0 ** -26,
                            3 * 2.0 ** -26]])
    rng = np.random.default_rng(11)
    cand = np.concatenate([cand, rng.normal(0, 1, 20000), rng.uniform(-7e4, 7e4, 20000),
                           rng.uniform(-1e-4, 1e-4, 20000)])
    cand = np.concatenate([cand, -cand])
    got = o.d2h(cand).view(np.uint16)
    with np.errstate(over="ignore"):
        ref = cand.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]
    # ties go to the even mantissa: 1 + 2^-11 -> 1, 1 + 3*2^-11 -> 1 + 2^-9
    assert o.d2h(np.array([1 + 2.0 ** -11]))[0] == 1.0
    assert o.d2h(np.array([1 + 3 * 2.0 ** -11]))[0] == 1 + 2.0 ** -9


# --------------------------------------------------------------------------
# packing: closed forms of "element i of a word lives in bits 4i..4i+3"
# (Zero TVM Documentation, "Q4F16 quantization format")
# --------------------------------------------------------------------------

def pin_pack_closed_form(o):
    assert o.pack(np.array([[0, 1, 2, 3, 4, 5, 6, 7]], np.uint8))[0, 0] == 0x76543210
    assert o.pack(np.array([[15, 0, 0, 0, 0, 0, 0, 0]], np.uint8))[0, 0] == 0x0000000F
    assert o.pack(np.array([[0, 0, 0, 0, 0, 0, 0, 15]], np.uint8))[0, 0] == 0xF0000000
    w = o.pack(np.array([[1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 0]], np.uint8))
    assert list(w[0]) == [0x87654321, 0x0FEDCBA9]


def pin_unpack_inverts_pack(o):
    c = datagen.codes(5, 7, 96)
    assert np.array_equal(o.unpack(o.pack(c)), c)
    w = np.array([[0x76543210, 0xFEDCBA98]], np.uint32)
    assert list(o.unpack(w)[0]) == list(range(16))


def pin_shapes_match_page_table(o):
    g = _golden("phi3_q4f16_shapes.json")
    for name, t in g["tensors"].items():
        words, groups = t["q_weight"][1], t["q_scale"][1]
        k = words * 8
        assert groups * 32 == k, name
        c = datagen.codes(3, 2, k)
        assert o.pack(c).shape == (2, words), name
    u = _golden("int4_matmul_uniforms.json")
    assert u["input_dim"] // 8 == u["K_groups"]
    assert u["input_dim"] // u["group_size"] == u["scale_stride"]
    c = datagen.codes(4, 1, u["input_dim"])
    assert o.pack(c).shape[1] == u["K_groups"]
    t = _golden("tvm_matmul_structure.json")
    assert t["threads"] * t["iterations"] * t["codes_per_word"] == t["dot_length"]
    assert o.pack(datagen.codes(6, 1, t["dot_length"])).shape[1] == t["threads"] * t["iterations"]


# --------------------------------------------------------------------------
# matvec pins
# --------------------------------------------------------------------------

def pin_one_hot_reproduces_column(o):
    """x = e_k gives y[n] = (q[n][k] - 7) * S[n][k // 32] exactly, for every k
    (every nibble position of every word and every group)."""
    n, k = 6, 96
    codes, W, S = _mat(o, 21, n, k)
    Sd = S.astype(np.float64)
    for kk in range(k):
        x = np.zeros(k, np.float16)
        x[kk] = 1.0
        y = o.gemv(W, S, x)
        expect = (codes[:, kk].astype(np.float64) - 7.0) * Sd[:, kk // 32]
        assert np.array_equal(y, expect), kk


def pin_all_sevens_zero(o):
    n, k = 9, 128
    _, W, S = _mat(o, 22, n, k, codes=np.full((n, k), 7, np.uint8))
    x = datagen.activations(23, 1, k)[0]
    assert np.array_equal(o.gemv(W, S, x), np.zeros(n))


def pin_scale_linearity(o):
    n, k = 11, 160
    _, W, S = _mat(o, 24, n, k)
    x = datagen.activations(25, 1, k)[0]
    y1 = o.gemv(W, S, x)
    y2 = o.gemv(W, (S.astype(np.float64) * 2).astype(np.float16), x)
    assert np.array_equal(y2, 2 * y1)


def pin_x_linearity(o):
    n, k = 8, 64
    _, W, S = _mat(o, 26, n, k)
    r = np.random.default_rng(27)
    x1 = (r.integers(-64, 64, k) / 64.0).astype(np.float16)
    x2 = (r.integers(-64, 64, k) / 64.0).astype(np.float16)
    x3 = (x1.astype(np.float64) + x2.astype(np.float64)).astype(np.float16)
    assert np.array_equal(x3.astype(np.float64), x1.astype(np.float64) + x2.astype(np.float64))
    y = o.gemv(W, S, x1) + o.gemv(W, S, x2)
    assert np.allclose(o.gemv(W, S, x3), y, rtol=0, atol=1e-12)


def pin_all_fifteen_closed_form(o):
    """codes all 15 -> y[n] = 8 * sum_g S[n][g] * sum_{k in g} x[k]."""
    n, k = 5, 256
    _, W, S = _mat(o, 28, n, k, codes=np.full((n, k), 15, np.uint8))
    x = datagen.activations(29, 1, k)[0]
    gs = x.astype(np.float64).reshape(k // 32, 32).sum(axis=1)
    expect = 8.0 * (S.astype(np.float64) * gs[None, :]).sum(axis=1)
    assert np.allclose(o.gemv(W, S, x), expect, rtol=1e-13, atol=1e-13)


def pin_brute_force_every_code_every_position(o):
    """Row n holds code (n + k) % 16 at column k, so across 16 rows every code
    value sits at every nibble position of every word; exact rational sums."""
    n, k = 16, 64
    codes = (np.arange(n)[:, None] + np.arange(k)[None, :]) % 16
    codes = codes.astype(np.uint8)
    _, W, S = _mat(o, 30, n, k, codes=codes)
    x = datagen.activations(31, 1, k)[0]
    y = o.gemv(W, S, x)
    xf = [Fraction(float(v)) for v in x]
    for r in range(n):
        acc = Fraction(0)
        for c in range(k):
            acc += (int(codes[r, c]) - 7) * Fraction(float(S[r, c // 32])) * xf[c]
        assert abs(Fraction(y[r]) - acc) <= Fraction(1, 2 ** 40) * (1 + abs(acc)), r


def pin_matvec_equals_library_matmul(o):
    """Against numpy's float64 matmul of the matrix dequantised from the codes
    (ragged sizes, several groups)."""
    n, k = 37, 224
    codes, W, S = _mat(o, 32, n, k)
    x = datagen.activations(33, 1, k)[0]
    dense = (codes.astype(np.float64) - 7.0) * np.repeat(S.astype(np.float64), 32, axis=1)
    assert np.allclose(o.dequant(W, S), dense, rtol=0, atol=0)
    assert np.allclose(o.gemv(W, S, x), dense @ x.astype(np.float64), rtol=1e-12, atol=1e-12)
    rows = np.array([36, 0, 17])
    assert np.array_equal(o.gemv_rows(W, S, x, rows), o.gemv(W, S, x)[rows])


def pin_batched(o):
    n, k, m = 13, 96, 5
    codes, W, S = _mat(o, 34, n, k)
    X = datagen.activations(35, m, k)
    dense = (codes.astype(np.float64) - 7.0) * np.repeat(S.astype(np.float64), 32, axis=1)
    Y = o.gemv_batched(W, S, X)
    assert Y.shape == (m, n)
    assert np.allclose(Y, X.astype(np.float64) @ dense.T, rtol=1e-12, atol=1e-12)
    same = np.repeat(X[:1], 4, axis=0)
    Ys = o.gemv_batched(W, S, same)
    assert all(np.array_equal(Ys[0], Ys[i]) for i in range(4))


# --------------------------------------------------------------------------
# add + RMSNorm pins (shaders 2 and 7)
# --------------------------------------------------------------------------

def pin_rmsnorm_constant_input(o):
    d = 64
    for c in (0.5, 3.0, -2.0, 0.0078125):
        r = np.full(d, c, np.float16)
        g = np.ones(d, np.float16)
        res, out = o.add_rmsnorm(None, r, g, eps=1e-5)
        assert np.array_equal(res[0].view(np.uint16), r.view(np.uint16))
        expect = c / math.sqrt(c * c + 1e-5)
        assert np.allclose(out[0], expect, rtol=1e-14, atol=0)


def pin_rmsnorm_one_nonzero(o):
    """r = [c, 0, ..., 0] has mean square c^2 / D, so out[0] = c / sqrt(c^2/D + eps)."""
    for d in (8, 100):
        c = 0.25
        r = np.zeros(d, np.float16)
        r[0] = c
        g = _f16(np.linspace(0.5, 1.5, d))
        _, out = o.add_rmsnorm(None, r, g, eps=1e-5)
        expect = c / math.sqrt(c * c / d + 1e-5) * float(g[0])
        assert np.allclose(out[0, 0], expect, rtol=1e-14)
        assert np.all(out[0, 1:] == 0)


def pin_rmsnorm_unit_rms(o):
    d = 48
    r = np.where(np.arange(d) % 2 == 0, 1.0, -1.0).astype(np.float16)
    g = datagen.gammas(36, 1, d)[0]
    _, out = o.add_rmsnorm(None, r, g, eps=0.0)
    assert np.array_equal(out[0], r.astype(np.float64) * g.astype(np.float64))


def pin_rmsnorm_scale_invariance(o):
    d = 96
    r = datagen.activations(37, 1, d)[0]
    g = datagen.gammas(38, 1, d)[0]
    r2 = (r.astype(np.float64) * 2).astype(np.float16)
    _, a = o.add_rmsnorm(None, r, g, eps=0.0)
    _, b = o.add_rmsnorm(None, r2, g, eps=0.0)
    assert np.allclose(a, b, rtol=1e-14, atol=1e-14)


def pin_add_residual_rounding(o):
    d = 4
    g = np.ones(d, np.float16)
    a = np.array([1.0, 1.0, 0.0, 2.0], np.float16)
    r = np.array([2.0 ** -11, 3 * 2.0 ** -11, 0.75, 2.0 ** -10], np.float16)
    res, _ = o.add_rmsnorm(a, r, g)
    # ties round to even; an exact sum is kept as is
    assert list(res[0].astype(np.float64)) == [1.0, 1 + 2.0 ** -9, 0.75, 2.0]
    # a == 0 leaves the residual bit-identical
    rr = datagen.activations(39, 1, 64)[0]
    res2, _ = o.add_rmsnorm(np.zeros(64, np.float16), rr, np.ones(64, np.float16))
    assert np.array_equal(res2[0].view(np.uint16), rr.view(np.uint16))


def pin_add_then_norm(o):
    """out is RMSNorm of the stored (rounded) residual: with a = r the residual
    doubles exactly and the norm is that of r (eps = 0)."""
    d = 32
    r = datagen.activations(40, 1, d)[0]
    g = datagen.gammas(41, 1, d)[0]
    res, out = o.add_rmsnorm(r, r, g, eps=0.0)
    assert np.array_equal(res[0].astype(np.float64), 2 * r.astype(np.float64))
    _, ref = o.add_rmsnorm(None, r, g, eps=0.0)
    assert np.allclose(out, ref, rtol=1e-14, atol=1e-15)


def pin_eps_inside_sqrt(o):
    c = 2.0 ** -8
    r = np.array([c], np.float16)
    _, out = o.add_rmsnorm(None, r, np.ones(1, np.float16), eps=1e-5)
    assert np.allclose(out[0, 0], c / math.sqrt(c * c + 1e-5), rtol=1e-14)


# --------------------------------------------------------------------------
# split-SiLU-multiply pins (RESEARCH.md, "1. Dispatch profile")
# --------------------------------------------------------------------------

def _gu(gate, up):
    return np.concatenate([np.asarray(gate, np.float16), np.asarray(up, np.float16)])


def pin_silu_special_values(o):
    out = o.silu_mul(_gu([0.0, 20.0, -30.0, 0.0], [5.0, 1.0, 1.0, 0.0]))[0]
    assert out[0] == 0.0 and out[3] == 0.0
    assert abs(out[1] - 20.0) < 20.0 * 3e-9          # 20 * sigmoid(20)
    assert -3e-12 < out[2] < -2.7e-12                 # -30 * sigmoid(-30)
    # tiny gate: silu(z) = z/2 + z^2/4 + O(z^4)
    z = 2.0 ** -12
    t = o.silu_mul(_gu([z], [1.0]))[0, 0]
    assert abs(t - (z / 2 + z * z / 4)) < 1e-15


def pin_silu_odd_identity(o):
    """silu(z) - silu(-z) = z for every z."""
    g = datagen.normal_f16(42, 256, 0.0, 4.0)
    pos = o.silu_mul(_gu(g, np.ones_like(g)))[0]
    neg = o.silu_mul(_gu(-g, np.ones_like(g)))[0]
    assert np.allclose(pos - neg, g.astype(np.float64), rtol=0, atol=1e-14)


def pin_silu_gate_first(o):
    """The first half of [gate | up] is the gate: gate 20, up 1 gives ~20 (the
    other order would give silu(1) * 20 ~ 14.6); up scales linearly."""
    out = o.silu_mul(_gu([20.0, 1.0], [1.0, 20.0]))[0]
    assert abs(out[0] - 20.0) < 1e-6
    assert abs(out[1] - 20.0 / (1 + math.exp(-1.0))) < 1e-12
    g = datagen.normal_f16(43, 64)
    u = datagen.normal_f16(44, 64)
    a = o.silu_mul(_gu(g, u))[0]
    b = o.silu_mul(_gu(g, (u.astype(np.float64) * 2).astype(np.float16)))[0]
    assert np.array_equal(b, 2 * a)


# --------------------------------------------------------------------------
# MoE pins (BENCH.md, "MoE chunked prefill"; "MoE Phase B")
# --------------------------------------------------------------------------

def _experts(o, seed, e, n, k, codes_fn=None):
    W = np.empty((e, n, k // 8), np.uint32)
    S = np.empty((e, n, k // 32), np.float16)
    for i in range(e):
        c = datagen.codes(seed + 2 * i, n, k) if codes_fn is None else codes_fn(i)
        W[i] = o.pack(c)
        S[i] = datagen.scales(seed + 2 * i + 1, n, k)
    return W, S


def pin_moe_one_hot_routing_is_dense_chain(o):
    e, d, f, t, topk = 6, 64, 32, 3, 3
    Wg, Sg = _experts(o, 50, e, 2 * f, d)
    Wd, Sd = _experts(o, 80, e, d, f)
    ids = np.array([[4, 1, 2], [0, 5, 3], [2, 3, 4]], np.int32)
    x = datagen.activations(51, t, d)
    u = o.moe_stage(Wg, Sg, ids, None, x, d, 0, 2 * f, d, epi_silu=True)
    u16 = u.astype(np.float16)
    for slot in range(topk):
        w = np.zeros((t, topk), np.float16)
        w[:, slot] = 1.0
        y = o.moe_stage(Wd, Sd, ids, w, u16, topk * f, f, d, f, epi_silu=False)
        for i in range(t):
            ex = ids[i, slot]
            gu = o.gemv(Wg[ex], Sg[ex], x[i]).astype(np.float16)
            uu = o.silu_mul(gu)[0].astype(np.float16)
            dn = o.gemv(Wd[ex], Sd[ex], uu)
            assert np.array_equal(y[i], dn), (slot, i)


def pin_moe_slot_permutation(o):
    e, d, f, t, topk = 5, 32, 32, 2, 4
    Wd, Sd = _experts(o, 90, e, d, f)
    ids, w = datagen.routing(91, t, e, topk)
    u = datagen.activations(92, t * topk, f).reshape(t, topk, f)
    y = o.moe_stage(Wd, Sd, ids, w, u, topk * f, f, d, f, epi_silu=False)
    p = np.array([2, 0, 3, 1])
    y2 = o.moe_stage(Wd, Sd, ids[:, p], w[:, p], np.ascontiguousarray(u[:, p]), topk * f, f,
                     d, f, epi_silu=False)
    assert np.allclose(y, y2, rtol=1e-13, atol=1e-13)


def pin_moe_identical_experts(o):
    e, d, f, t, topk = 4, 32, 32, 3, 3
    c = datagen.codes(93, d, f)
    Wd, Sd = _experts(o, 94, e, d, f, codes_fn=lambda i: c)
    Sd[:] = Sd[0]
    ids, w = datagen.routing(95, t, e, topk)
    xa = datagen.activations(96, t, f)
    u = np.repeat(xa[:, None, :], topk, axis=1)      # same activation in every slot
    y = o.moe_stage(Wd, Sd, ids, w, u, topk * f, f, d, f, epi_silu=False)
    for i in range(t):
        dense = o.gemv(Wd[0], Sd[0], xa[i])
        assert np.allclose(y[i], w[i].astype(np.float64).sum() * dense, rtol=1e-13, atol=1e-13)


def pin_moe_per_slot_outputs(o):
    e, d, n, t, topk = 5, 64, 48, 2, 3
    W, S = _experts(o, 97, e, n, d)
    ids, _ = datagen.routing(98, t, e, topk)
    x = datagen.activations(99, t * topk, d)
    y = o.moe_stage(W, S, ids, None, x, topk * d, d, n, d, epi_silu=False)
    for i in range(t):
        for s in range(topk):
            ex = ids[i, s]
            assert np.array_equal(y[i, s], o.gemv(W[ex], S[ex], x[i * topk + s]))


# --------------------------------------------------------------------------
# stack pins (decode loop with attention := V slice)
# --------------------------------------------------------------------------

DIMS = (64, 96, 192, 128, 64)          # d, f, n_qkv, v_off, dv


def _layer_mats(o, seed, zero_o_down=False):
    d, f, nq, _, dv = DIMS
    seven = lambda n, k: np.full((n, k), 7, np.uint8)
    mats = []
    for j, (n, k) in enumerate([(nq, d), (d, dv), (2 * f, d), (d, f)]):
        codes = seven(n, k) if (zero_o_down and j in (1, 3)) else datagen.codes(seed + j, n, k)
        mats += [o.pack(codes), datagen.scales(seed + 10 + j, n, k)]
    return mats


def pin_stack_identity_layers(o):
    """O and down codes all 7: both residual adds add zero, so r is unchanged
    and h is RMSNorm(r) with the next layer's gamma."""
    d = DIMS[0]
    L = 3
    layers = [_layer_mats(o, 100 + 20 * i, zero_o_down=True) for i in range(L)]
    gi = datagen.gammas(160, L, d)
    gp = datagen.gammas(161, L, d)
    gf = datagen.gammas(162, 1, d)[0]
    r0 = datagen.activations(163, 1, d)[0]
    h0 = datagen.activations(164, 1, d)[0]
    r, h, h64, tr, th = o.stack(DIMS, layers, gi, gp, gf, r0, h0, trace=True)
    assert np.array_equal(r.view(np.uint16), r0.view(np.uint16))
    for li in range(L):
        g_next = gi[li + 1] if li + 1 < L else gf
        _, ref = o.add_rmsnorm(None, r0, g_next)
        assert np.array_equal(th[li].view(np.uint16), ref[0].astype(np.float16).view(np.uint16))
    _, ref = o.add_rmsnorm(None, r0, gf)
    assert np.array_equal(h64, ref[0])


def pin_stack_only_v_slice_matters(o):
    """Rows of the QKV matrix outside the V slice do not change the result."""
    d, f, nq, v_off, dv = DIMS
    lay = _layer_mats(o, 200)
    lay2 = list(lay)
    codes = o.unpack(lay[0])
    codes[:v_off] = (codes[:v_off] + 5) % 16
    lay2[0] = o.pack(codes)
    gp, gn = datagen.gammas(201, 2, d)
    r0 = datagen.activations(202, 1, d)[0]
    h0 = datagen.activations(203, 1, d)[0]
    a = o.layer(DIMS, lay, gp, gn, r0, h0)
    b = o.layer(DIMS, lay2, gp, gn, r0, h0)
    assert np.array_equal(a[2], b[2])
    codes[v_off] = (codes[v_off] + 3) % 16          # a V row does change it
    lay2[0] = o.pack(codes)
    c = o.layer(DIMS, lay2, gp, gn, r0, h0)
    assert not np.array_equal(a[2], c[2])


def pin_layer_is_composition(o):
    """One layer equals the chain of single ops with f16 stores between them."""
    d, f, nq, v_off, dv = DIMS
    Wq, Sq, Wo, So, Wg, Sg, Wd, Sd = _layer_mats(o, 300)
    gp, gn = datagen.gammas(301, 2, d)
    r0 = datagen.activations(302, 1, d)[0]
    h0 = datagen.activations(303, 1, d)[0]
    r2, h2, h64 = o.layer(DIMS, [Wq, Sq, Wo, So, Wg, Sg, Wd, Sd], gp, gn, r0, h0)
    qkv = o.gemv(Wq, Sq, h0).astype(np.float16)
    oo = o.gemv(Wo, So, qkv[v_off:v_off + dv]).astype(np.float16)
    r1, h1 = o.add_rmsnorm(oo, r0, gp)
    gu = o.gemv(Wg, Sg, h1[0].astype(np.float16)).astype(np.float16)
    u = o.silu_mul(gu)[0].astype(np.float16)
    dn = o.gemv(Wd, Sd, u).astype(np.float16)
    rr, hh = o.add_rmsnorm(dn, r1[0], gn)
    assert np.array_equal(rr[0].view(np.uint16), r2.view(np.uint16))
    assert np.array_equal(hh[0], h64)


def pin_stack_is_layer_sequence(o):
    d = DIMS[0]
    L = 2
    layers = [_layer_mats(o, 400 + 20 * i) for i in range(L)]
    gi = datagen.gammas(460, L, d)
    gp = datagen.gammas(461, L, d)
    gf = datagen.gammas(462, 1, d)[0]
    r0 = datagen.activations(463, 1, d)[0]
    h0 = datagen.activations(464, 1, d)[0]
    r, h, h64 = o.stack(DIMS, layers, gi, gp, gf, r0, h0)
    ra, ha, _ = o.layer(DIMS, layers[0], gp[0], gi[1], r0, h0)
    rb, hb, hb64 = o.layer(DIMS, layers[1], gp[1], gf, ra, ha)
    assert np.array_equal(r.view(np.uint16), rb.view(np.uint16))
    assert np.array_equal(h64, hb64)


# -- LM head and greedy argmax ------------------------------------------------
# The pages pick the next token as the argmax of the LM head's logits (Zero TVM
# Documentation, shader 10 "Argmax Sampler") and leave ties and NaN open; the
# reading pinned here: ties go to the smallest index, -0 equals +0, a NaN ranks
# above every number (the first NaN wins).

def pin_argmax_special_cases(o):
    inf, nan = np.inf, np.nan
    cases = [
        ([3.0], 0), ([1.0, 2.0, 3.0], 2), ([3.0, 2.0, 1.0], 0),
        ([2.0, 5.0, 5.0, 1.0], 1),            # tie: the smaller index
        ([-0.0, 0.0], 0), ([0.0, -0.0], 0),   # -0 == +0
        ([-inf, -inf, -inf], 0), ([-1.0, -inf], 0), ([1e308, inf], 1),
        ([-2.0, -1.0, -3.0], 1),
        ([1.0, nan, 5.0, nan], 1), ([inf, nan], 1), ([nan, inf], 0), ([nan], 0),
    ]
    for v, want in cases:
        assert o.argmax(v) == want, (v, want)


def pin_argmax_brute_force(o):
    """Every sequence of length 1..4 over seven special values against the
    maximum of the key (rank, -index), rank putting NaN above every number."""
    import itertools
    import math
    vals = [-np.inf, -1.0, -0.0, 0.0, 1.0, np.inf, np.nan]

    def key(v, i):
        return ((1, 0.0) if math.isnan(v[i]) else (0, v[i]), -i)

    for n in range(1, 5):
        for v in itertools.product(vals, repeat=n):
            want = max(range(n), key=lambda i: key(v, i))
            assert o.argmax(list(v)) == want, (v, want)


def pin_argmax_matches_numpy(o):
    """numpy.argmax is the same definition: the first occurrence of the
    maximum, a NaN counting as the maximum."""
    rng = np.random.default_rng(7)
    for trial in range(40):
        n = int(rng.integers(1, 3000))
        v = rng.integers(-4, 5, n).astype(np.float64)  # few levels: many ties
        if trial % 3 == 0:
            v[rng.integers(0, n, 2)] = np.nan
        assert o.argmax(v) == int(np.argmax(v)), trial
    for seed in range(3):  # f32 logits of the Phi-3 vocabulary size
        v = np.random.default_rng(seed).standard_normal(32064).astype(np.float32)
        assert o.argmax(v) == int(np.argmax(v))


def pin_lm_head_planted_maximum(o):
    """All codes 7 (weight 0) except row r0 (codes 15, weight 8 s) and x > 0:
    every logit is 0 but logit r0 = 8 sum_k s x_k > 0, so the token is r0; a
    copy of row r0 at a larger index does not change it."""
    n, k = 96, 256
    codes = np.full((n, k), 7, np.uint8)
    r0, r1 = 37, 80
    codes[r0] = 15
    codes[r1] = 15
    W = o.pack(codes)
    S = datagen.scales(501, n, k)
    S[r1] = S[r0]
    x = np.abs(datagen.activations(502, 1, k)).astype(np.float16)
    logits, tok = o.lm_head(W, S, x)
    assert tok[0] == r0
    s = o.h2d(S[r0])
    xs = o.h2d(x[0])
    want = sum(8.0 * s[c // 32] * xs[c] for c in range(k))
    assert logits[0, r0] == logits[0, r1]
    assert abs(logits[0, r0] - want) <= 1e-12 * abs(want)
    others = np.delete(logits[0], [r0, r1])
    assert np.all(others == 0.0)


def pin_lm_head_rows_are_matvec_then_argmax(o):
    """Each row's logits are the matvec of that activation row (one-hot rows
    give a weight column exactly) and its token is their argmax."""
    n, k, m = 200, 512, 3
    _, W, S = _mat(o, 510, n, k)
    X = datagen.activations(511, m, k)
    X[1] = 0
    X[1, 77] = 1.0  # one-hot: logits = column 77 exactly
    logits, tok = o.lm_head(W, S, X)
    col = o.dequant(W, S)[:, 77]
    assert np.array_equal(logits[1], col)
    for b in range(m):
        y = o.gemv(W, S, X[b])
        assert np.array_equal(logits[b], y)
        assert tok[b] == int(np.argmax(y))


# -- RoPE, KV cache, decode attention ------------------------------------------
# RoPE pairs (i, i + head_dim/2) of a head and turns pair i by pos * base^(-2i/d)
# (Zero TVM Documentation, shader 3: a RoPE pair is dim and dim + 48 of a 96-dim
# head); attention is softmax(q . K^T / sqrt(d)) V per head (shader 4).

def pin_rope_closed_form(o):
    """Unit vectors turn by the closed-form angle: theta_0 = pos, theta_1 = pos *
    10000^(-2/96); the partner of dim i is dim i + 48."""
    d = 96
    cases = [(0, 1), (48, 1), (1, 3), (49, 3), (47, 2)]
    for dim, pos in cases:
        v = np.zeros(2 * d)
        v[d + dim] = 1.0  # second head
        r = o.rope(v, d, pos)
        i = dim % 48
        theta = pos * 10000.0 ** (-2.0 * i / d)
        c, s_ = math.cos(theta), math.sin(theta)
        want = np.zeros(2 * d)
        if dim < 48:
            want[d + i], want[d + i + 48] = c, s_
        else:
            want[d + i], want[d + i + 48] = -s_, c
        assert np.allclose(r, want, rtol=0, atol=1e-15), (dim, pos)


def pin_rope_position_zero_is_identity(o):
    v = datagen.activations(601, 1, 3 * 96)[0].astype(np.float64)
    assert np.array_equal(o.rope(v, 96, 0), v)


def pin_rope_preserves_pair_norms_and_relative_positions(o):
    """Each pair keeps its length, and the rotated dot product of a query at m
    and a key at n depends only on m - n."""
    d = 96
    q = datagen.activations(602, 1, 4 * d)[0].astype(np.float64)
    k = datagen.activations(603, 1, 4 * d)[0].astype(np.float64)
    for pos in (1, 17, 4095):
        r = o.rope(q, d, pos).reshape(4, 2, 48)
        a = q.reshape(4, 2, 48)
        assert np.allclose((r ** 2).sum(1), (a ** 2).sum(1), rtol=1e-12, atol=1e-12)
    for m, n, c in ((5, 2, 7), (100, 40, 900), (3, 3, 50)):
        qa, ka = o.rope(q, d, m).reshape(4, d), o.rope(k, d, n).reshape(4, d)
        qb, kb = o.rope(q, d, m + c).reshape(4, d), o.rope(k, d, n + c).reshape(4, d)
        assert np.allclose((qa * ka).sum(1), (qb * kb).sum(1), rtol=1e-9, atol=1e-9)


def _attn_numpy(q, kc, vc, n_heads, n_kv, d):
    """Independent formulation: numpy matmuls and scipy's softmax."""
    from scipy.special import softmax
    q = q.astype(np.float64).reshape(n_heads, d)
    L = kc.size // (n_kv * d)
    K = kc.astype(np.float64).reshape(L, n_kv, d)
    V = vc.astype(np.float64).reshape(L, n_kv, d)
    out = np.empty((n_heads, d))
    for h in range(n_heads):
        kv = h // (n_heads // n_kv)
        p = softmax(K[:, kv, :] @ q[h] / math.sqrt(d))
        out[h] = p @ V[:, kv, :]
    return out.ravel()


def pin_attention_matches_library_softmax(o):
    for (nh, nkv, d, L, seed) in ((4, 4, 96, 37, 610), (8, 2, 64, 100, 611), (2, 1, 32, 1, 612)):
        q = datagen.activations(seed, 1, nh * d)[0]
        kc = datagen.activations(seed + 1, L, nkv * d)
        vc = datagen.activations(seed + 2, L, nkv * d)
        got = o.attention(q, kc, vc, nh, nkv, d)
        assert np.allclose(got, _attn_numpy(q, kc, vc, nh, nkv, d), rtol=1e-12, atol=1e-12)


def pin_attention_special_cases(o):
    """One position returns its value exactly; equal keys average the values;
    a dominant key returns its value; GQA equals MHA with repeated kv heads."""
    d, nh = 96, 4
    q = datagen.activations(620, 1, nh * d)[0]
    kc = datagen.activations(621, 1, nh * d)
    vc = datagen.activations(622, 1, nh * d)
    assert np.array_equal(o.attention(q, kc, vc, nh, nh, d), o.h2d(vc[0]))
    L = 10
    k1 = np.tile(datagen.activations(623, 1, nh * d), (L, 1))
    vL = datagen.activations(624, L, nh * d)
    mean = o.h2d(vL).reshape(L, nh * d).mean(0)
    assert np.allclose(o.attention(q, k1, vL, nh, nh, d), mean, rtol=1e-13, atol=1e-13)
    kd = np.zeros((L, nh * d), np.float16)
    kd[4] = (q.astype(np.float64) * 8).astype(np.float16)  # score ~ 8 |q|^2 / sqrt(d)
    got = o.attention(q, kd, vL, nh, nh, d)
    assert np.allclose(got, o.h2d(vL[4]), rtol=0, atol=1e-6)
    nkv = 2
    kg = datagen.activations(625, L, nkv * d)
    vg = datagen.activations(626, L, nkv * d)
    rep = lambda a: np.repeat(a.reshape(L, nkv, d), nh // nkv, axis=1).reshape(L, nh * d)
    assert np.allclose(o.attention(q, kg, vg, nh, nkv, d),
                       o.attention(q, rep(kg), rep(vg), nh, nh, d), rtol=0, atol=1e-15)


def pin_qkv_rope_is_stored_matvec_then_rope(o):
    """q and k are the RoPE of the f16-stored matvec rows; v is the stored V rows."""
    nh, nkv, d, k = 4, 2, 32, 256
    n = (nh + 2 * nkv) * d
    _, W, S = _mat(o, 630, n, k)
    x = datagen.activations(631, 1, k)[0]
    q, kr, v = o.qkv_rope(W, S, x, nh, nkv, d, 21)
    y = o.h2d(o.d2h(o.gemv(W, S, x)))
    assert np.array_equal(q, o.rope(y[:nh * d], d, 21))
    assert np.array_equal(kr, o.rope(y[nh * d:(nh + nkv) * d], d, 21))
    assert np.array_equal(v, y[(nh + nkv) * d:])


def _attn_layer_mats(o, seed, d, f, nq_rows):
    return [m for pair in (_mat(o, seed, nq_rows, d)[1:], _mat(o, seed + 2, d, nq_rows // 3)[1:],
                           _mat(o, seed + 4, 2 * f, d)[1:], _mat(o, seed + 6, d, f)[1:])
            for m in pair]


def pin_layer_attn_at_position_zero_is_the_v_slice_layer(o):
    """With one cached position attention returns that position's value, so
    the layer at pos 0 is the single-position layer that feeds O the V slice of
    the QKV rows (and its key and value rows are the RoPE'd, stored rows)."""
    d, f, nh, hd = 128, 256, 4, 32
    mats = _attn_layer_mats(o, 700, d, f, 3 * nh * hd)
    gp, gn = datagen.gammas(710, 1, d)[0], datagen.gammas(711, 1, d)[0]
    r = datagen.activations(712, 1, d)[0]
    h = datagen.activations(713, 1, d)[0]
    ra, ha, h64a, k_new, v_new = o.layer_attn((d, f, nh, nh, hd), 0, mats, gp, gn, r, h, None, None)
    dims = (d, f, 3 * nh * hd, 2 * nh * hd, nh * hd)  # d, f, n_qkv, v_off, dv
    rb, hb, h64b = o.layer(dims, mats, gp, gn, r, h)
    assert np.array_equal(ra.view(np.uint16), rb.view(np.uint16))
    assert np.array_equal(h64a, h64b)
    q, kr, v = o.qkv_rope(mats[0], mats[1], h, nh, nh, hd, 0)
    assert np.array_equal(k_new.view(np.uint16), o.d2h(kr).view(np.uint16))
    assert np.array_equal(v_new.view(np.uint16), o.d2h(v).view(np.uint16))


def pin_layer_attn_is_rope_attention_then_layer(o):
    """At pos > 0 the O input is the stored attention output over the cached
    rows and the new ones."""
    d, f, nh, nkv, hd, pos = 128, 256, 4, 2, 32, 9
    nrows = (nh + 2 * nkv) * hd
    mats = [m for pair in (_mat(o, 720, nrows, d)[1:], _mat(o, 722, d, nh * hd)[1:],
                           _mat(o, 724, 2 * f, d)[1:], _mat(o, 726, d, f)[1:]) for m in pair]
    gp, gn = datagen.gammas(730, 1, d)[0], datagen.gammas(731, 1, d)[0]
    r = datagen.activations(732, 1, d)[0]
    h = datagen.activations(733, 1, d)[0]
    kc = datagen.activations(734, pos, nkv * hd)
    vc = datagen.activations(735, pos, nkv * hd)
    ra, ha, h64a, k_new, v_new = o.layer_attn((d, f, nh, nkv, hd), pos, mats, gp, gn, r, h, kc, vc)
    q, kr, v = o.qkv_rope(mats[0], mats[1], h, nh, nkv, hd, pos)
    att = o.attention(o.d2h(q), np.vstack([kc, o.d2h(kr)]), np.vstack([vc, o.d2h(v)]), nh, nkv, hd)
    # the rest of the layer from the stored attention output: O, add+norm, FFN, add+norm
    ao = o.d2h(o.gemv(mats[2], mats[3], o.d2h(att)))
    r1, h1 = o.add_rmsnorm(ao, r, gp)
    u = o.d2h(o.silu_mul(o.d2h(o.gemv(mats[4], mats[5], o.d2h(h1)))))
    dn = o.d2h(o.gemv(mats[6], mats[7], u))
    r2, h2 = o.add_rmsnorm(dn, r1, gn)
    assert np.array_equal(ra.view(np.uint16), np.asarray(r2).view(np.uint16).ravel())
    assert np.array_equal(h64a, np.asarray(h2).ravel())


# -- MLX affine format ------------------------------------------------------------
# w = s * q + b with q unsigned, s and b per 64-code group (Zero TVM
# Documentation, the Qwen3.6 MoE model entry; BENCH.md, "Affine wide loads").

def _affine(o, seed, n, k):
    codes = datagen.codes(seed, n, k)
    S = datagen.scales(seed + 1, n, k // 2)  # one per 64 codes
    B = datagen.normal_f16(seed + 2, (n, k // 64), 0.0, 0.05)
    return codes, o.pack(codes), S, B


def pin_affine_one_hot_is_weight(o):
    n, k = 40, 256
    codes, W, S, B = _affine(o, 800, n, k)
    for c in (0, 1, 7, 31, 32, 63, 64, 130, 255):
        x = np.zeros(k, np.float16)
        x[c] = 1.0
        want = o.h2d(S[:, c // 64]) * codes[:, c] + o.h2d(B[:, c // 64])
        assert np.array_equal(o.gemv_affine(W, S, B, x), want), c


def pin_affine_zero_codes_sum_biases(o):
    """All codes 0: y = sum_g b_g * (sum of x over group g)."""
    n, k = 24, 512
    _, _, S, B = _affine(o, 801, n, k)
    W = o.pack(np.zeros((n, k), np.uint8))
    x = datagen.activations(802, 1, k)[0]
    xs = o.h2d(x).reshape(k // 64, 64).sum(1)
    want = (o.h2d(B) * xs).sum(1)
    assert np.allclose(o.gemv_affine(W, S, B, x), want, rtol=1e-13, atol=1e-13)


def pin_affine_matches_symmetric_format(o):
    """With b = -7 s (exact here: s has at most 8 significant bits) and both
    32-halves of a group sharing s, the affine weight equals the q4f16_1 one."""
    n, k = 32, 256
    codes = datagen.codes(803, n, k)
    rng = np.random.default_rng(803)
    S = (rng.integers(20, 200, size=(n, k // 64)) * 2.0 ** -12).astype(np.float16)
    B = (-7.0 * S.astype(np.float64)).astype(np.float16)
    assert np.array_equal(B.astype(np.float64), -7.0 * S.astype(np.float64))
    W = o.pack(codes)
    S32 = np.repeat(S, 2, axis=1)
    x = datagen.activations(804, 2, k)
    assert np.array_equal(o.gemv_affine(W, S, B, x), np.stack([o.gemv(W, S32, x[i]) for i in range(2)]))


def pin_affine_brute_force(o):
    n, k = 3, 128
    codes, W, S, B = _affine(o, 805, n, k)
    x = datagen.activations(806, 1, k)[0]
    xd = [float(v) for v in x.astype(np.float64)]
    for r in range(n):
        acc = Fraction(0)
        for c in range(k):
            w = Fraction(float(S[r, c // 64])) * int(codes[r, c]) + Fraction(float(B[r, c // 64]))
            acc += w * Fraction(xd[c])
        assert abs(o.gemv_affine(W, S, B, x)[r] - float(acc)) <= 1e-12 * (1 + abs(float(acc)))


# -- weights rounded to f16 (the format's dequantization formula multiplies in
# binary16: Zero TVM Documentation, "Q4F16 quantization format") -------------------

def _dense_f16(codes, S):
    """numpy's binary16 product f16(q - 7) * s (exact in float32, rounded once)."""
    q = (codes.astype(np.int32) - 7).astype(np.float16)
    return (q * np.repeat(S, 32, axis=1)).astype(np.float64)


def pin_w16_one_hot_is_numpy_f16_product(o):
    n, k = 24, 128
    codes, W, S = _mat(o, 820, n, k)
    exact = (codes.astype(np.float64) - 7.0) * np.repeat(S.astype(np.float64), 32, axis=1)
    want = _dense_f16(codes, S)
    assert np.any(want != exact), "the sample must hold weights that round"
    for c in (0, 1, 5, 7, 31, 32, 77, 127):
        x = np.zeros(k, np.float16)
        x[c] = 1.0
        assert np.array_equal(o.gemv_w16(W, S, x), want[:, c]), c


def pin_w16_equals_exact_for_power_of_two_scales(o):
    """Scales 2^-e make (q - 7) * s exact in binary16: no rounding happens."""
    n, k, m = 16, 96, 3
    codes = datagen.codes(821, n, k)
    e = np.random.default_rng(821).integers(4, 12, size=(n, k // 32))
    S = (2.0 ** -e).astype(np.float16)
    W = o.pack(codes)
    X = datagen.activations(822, m, k)
    assert np.array_equal(o.gemv_w16(W, S, X), o.gemv_batched(W, S, X))


def pin_w16_matches_library_matmul(o):
    n, k, m = 29, 160, 4
    codes, W, S = _mat(o, 823, n, k)
    X = datagen.activations(824, m, k)
    want = X.astype(np.float64) @ _dense_f16(codes, S).T
    assert np.allclose(o.gemv_w16(W, S, X), want, rtol=1e-12, atol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


# (name, text in q4_oracle.c, replacement)
MUTANTS = [
    ("zero_point_8", "(double)(q - 7) * s", "(double)(q - 8) * s"),
    ("nibble_order_reversed", "(w >> (4 * (k % 8)))", "(w >> (4 * (7 - k % 8)))"),
    ("pack_order_reversed", "<< (4 * i)", "<< (4 * (7 - i))"),
    ("group_index_off_by_one", "S[r * (k_total / 32) + k / 32]",
     "S[r * (k_total / 32) + (k / 32 + 1) % (k_total / 32)]"),
    ("group_of_16", "S[r * (k_total / 32) + k / 32]", "S[r * (k_total / 32) + (k / 16) % (k_total / 32)]"),
    ("scale_dropped", "return (double)(q - 7) * s;", "return (double)(q - 7);"),
    ("h2d_subnormal_scale", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("d2h_truncates", "double m = rint(ldexp(a, 10 - E));", "double m = floor(ldexp(a, 10 - E));"),
    ("gate_up_swapped", "double g = q4o_h2d(gu[b * 2 * f + i]);", "double g = q4o_h2d(gu[b * 2 * f + f + i]);"),
    ("silu_sign", "exp(-z)", "exp(z)"),
    ("eps_outside_sqrt", "sqrt(ss / (double)d + eps)", "(sqrt(ss / (double)d) + eps)"),
    ("mean_over_d_minus_1", "ss / (double)d + eps", "ss / (double)(d - 1) + eps"),
    ("residual_add_dropped", "q4o_h2d(a[b * d + i]) + q4o_h2d(rr[i])", "q4o_h2d(rr[i])"),
    ("gamma_dropped", "* inv * q4o_h2d(gamma[i])", "* inv"),
    ("moe_weight_ignored", "y[i * n + r] += w * v[r];", "y[i * n + r] += v[r];"),
    ("moe_slot_activation_ignored", "x + i * ldx + s * x_slot_stride", "x + i * ldx"),
    ("moe_gu_not_rounded", "vh[r] = q4o_d2h(v[r]);", "vh[r] = q4o_d2h(v[r] * 1.0009765625);"),
    ("stack_wrong_v_slice", "qkv + v_off, d, dv", "qkv, d, dv"),
    ("stack_gamma_next_is_current", "gamma_in + (L + 1) * d", "gamma_in + L * d"),
    ("layer_second_norm_uses_first_residual", "q4o_add_rmsnorm(dn, r1, gamma_next", "q4o_add_rmsnorm(dn, r_in, gamma_next"),
    ("argmax_ties_to_last", "|| v[i] > v[best])", "|| v[i] >= v[best])"),
    ("argmax_nan_ignored", "if (isnan(v[i]) || v[i] > v[best])", "if (v[i] > v[best])"),
    ("argmax_is_argmin", "|| v[i] > v[best])", "|| v[i] < v[best])"),
    ("argmax_skips_first", "int64_t best = 0;\n    for (int64_t i = 1;", "int64_t best = n > 1 ? 1 : 0;\n    for (int64_t i = 2;"),
    ("lm_head_row_stride_ignored", "q4o_row_dot(W, S, x + b * ldx, k, r);\n        token", "q4o_row_dot(W, S, x, k, r);\n        token"),
    ("lm_head_token_of_first_row", "token[b] = q4o_argmax(logits + b * n, n);", "token[b] = q4o_argmax(logits, n);"),
    ("rope_sign", "b[i] = a[i] * c - a[i + half] * s;", "b[i] = a[i] * c + a[i + half] * s;"),
    ("rope_frequency_exponent", "-2.0 * (double)i / (double)head_dim", "-1.0 * (double)i / (double)head_dim"),
    ("rope_position_ignored", "(double)pos * pow(", "1.0 * pow("),
    ("rope_adjacent_pairs", "const int64_t half = head_dim / 2;\n    for (int64_t h = 0; h < n_heads; ++h) {\n        const double *a", "const int64_t half = 1;\n    for (int64_t h = 0; h < n_heads; ++h) {\n        const double *a"),
    ("attention_unscaled", "s[t] = dot * scale;", "s[t] = dot;"),
    ("attention_kv_head_mapping", "const int64_t kvh = h / group;", "const int64_t kvh = h % n_kv;"),
    ("attention_values_from_keys", "acc += s[t] * q4o_h2d(vc[", "acc += s[t] * q4o_h2d(kc["),
    ("qkv_rope_unrounded", "y[r] = q4o_h2d(q4o_d2h(q4o_row_dot(W, S, x, k, r)));", "y[r] = q4o_row_dot(W, S, x, k, r);"),
    ("qkv_rope_v_slice", "v[r] = y[nq + nk + r];", "v[r] = y[nq + r];"),
    ("layer_attn_second_norm_uses_first_residual", "q4o_add_rmsnorm(dn, ra, gamma_next", "q4o_add_rmsnorm(dn, r_in, gamma_next"),
    ("affine_bias_dropped", "return q4o_h2d(S[gi]) * (double)q + q4o_h2d(B[gi]);", "return q4o_h2d(S[gi]) * (double)q;"),
    ("affine_group_of_32", "const int64_t gi = r * (k_total / 64) + k / 64;", "const int64_t gi = r * (k_total / 64) + (k / 32) % (k_total / 64);"),
    ("affine_zero_point_7", "return q4o_h2d(S[gi]) * (double)q + q4o_h2d(B[gi]);", "return q4o_h2d(S[gi]) * (double)(q - 7) + q4o_h2d(B[gi]);"),
    ("layer_attn_o_reads_values", "q4o_gemv(Wo, So, att, d, nq, tmp);", "q4o_gemv(Wo, So, v_new, d, nq, tmp);"),
    ("w16_not_rounded", "const double w16 = q4o_h2d(q4o_d2h(q4o_weight(W, S, k, r, c)));", "const double w16 = q4o_weight(W, S, k, r, c);"),
    ("w16_row_stride_ignored", "acc += w16 * q4o_h2d(x[b * ldx + c]);", "acc += w16 * q4o_h2d(x[c]);"),
    ("layer_attn_new_key_not_cached", "memcpy(kc + pos * nk, k_new, sizeof(uint16_t) * (size_t)nk);", "memcpy(kc + pos * nk, kc, sizeof(uint16_t) * (size_t)nk);"),
]


def mutant(name):
    """The oracle with one planted mistake (compiled on the CPU)."""
    import oracle
    src = open(oracle.SRC).read()
    for n, old, new in MUTANTS:
        if n == name:
            assert src.count(old) == 1, old
            return oracle.load_variant(src.replace(old, new), name)
    raise KeyError(name)

