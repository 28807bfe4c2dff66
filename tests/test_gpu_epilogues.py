"""GPU parity of q4_add_rmsnorm, q4_silu_mul and the fused q4_gemv_ex epilogues.

* standalone ops vs the oracle (residual bit-exact, normalised output and
  SiLU-multiply within tolerance);
* fused epilogues bit-identical to the unfused call sequence they replace, and
  within tolerance of the oracle chain.
"""
import numpy as np
import pytest

import datagen
import oracle
from gpu_common import assert_within, bits, dev_tensor, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.fixture(scope="module")
def q4():
    import int4_weight_only_q4_amd as m
    m.lib()
    return m


def sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("d,m,with_a", [(3072, 1, True), (2560, 4, True), (3072, 2, False),
                                        (37, 3, True), (24576, 1, True)])
def test_add_rmsnorm_vs_oracle(o, q4, d, m, with_a):
    a = datagen.activations(200 + d, m, d) if with_a else None
    r = datagen.activations(201 + d, m, d)
    g = datagen.gammas(202 + d, 1, d)[0]
    out, res_out = q4.add_rmsnorm(None if a is None else dev_tensor(a), dev_tensor(r),
                                  dev_tensor(g), eps=1e-5)
    sync()
    ref_res, ref_out = o.add_rmsnorm(a, r, g, eps=1e-5)
    assert np.array_equal(bits(res_out), ref_res.view(np.uint16))
    assert_within(host(out), ref_out, "add_rmsnorm")


def _offset_copy(t, off):
    """t's values in a fresh buffer starting `off` elements in (off = 1 gives a
    2-byte-aligned, not 16-byte-aligned, view)."""
    import torch
    buf = torch.zeros(t.numel() + 16, dtype=t.dtype, device=t.device)
    v = buf[off:off + t.numel()].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("d,m,with_a", [(2048, 1, True), (4096, 2, False), (5120, 1, True),
                                        (5120, 3, False), (6144, 1, True), (6144, 2, True),
                                        (8192, 1, False)])
def test_add_rmsnorm_row_in_registers_equals_scalar_path(o, q4, d, m, with_a):
    """The add+RMSNorm with the row held in registers (16-byte aligned vectors,
    D % 8 == 0, up to 8192 values: 1 to 4 chunks of 8 values per thread) and the
    general kernel, which the same call takes when a pointer is only 2-byte
    aligned, give the same bits, and both match the oracle."""
    import torch
    a = datagen.activations(210 + d + m, m, d) if with_a else None
    r = datagen.activations(211 + d + m, m, d)
    g = datagen.gammas(212 + d, 1, d)[0]
    ad = None if a is None else dev_tensor(a)
    rd, gd = dev_tensor(r), dev_tensor(g)
    out_v, res_v = q4.add_rmsnorm(ad, rd, gd, eps=1e-5)
    # the same values one element into fresh buffers: every vector misaligned
    ad1 = None if ad is None else _offset_copy(ad, 1)
    rd1, gd1 = _offset_copy(rd, 1), _offset_copy(gd, 1)
    out_s = _offset_copy(torch.empty_like(rd), 1)
    res_s = _offset_copy(torch.empty_like(rd), 1)
    q4.add_rmsnorm(ad1, rd1, gd1, out=out_s, res_out=res_s, eps=1e-5)
    sync()
    assert np.array_equal(bits(out_v), bits(out_s)), "normalised output: vector != scalar path"
    assert np.array_equal(bits(res_v), bits(res_s)), "residual: vector != scalar path"
    ref_res, ref_out = o.add_rmsnorm(a, r, g, eps=1e-5)
    assert np.array_equal(bits(res_v), ref_res.view(np.uint16))
    assert_within(host(out_v), ref_out, "add_rmsnorm d=%d" % d)


@pytest.mark.parametrize("f,m", [(8192, 1), (9728, 2), (768, 16), (37, 3)])
def test_silu_mul_vs_oracle(o, q4, f, m):
    gu = datagen.normal_f16(300 + f, (m, 2 * f), 0.0, 3.0)
    out = q4.silu_mul(dev_tensor(gu))
    sync()
    assert_within(host(out), o.silu_mul(gu), "silu_mul")


def test_silu_mul_special_values(o, q4):
    gate = np.array([0.0, 20.0, -30.0, 65504.0, -65504.0, 1.0], np.float16)
    up = np.array([5.0, 1.0, 1.0, 1.0, 1.0, 20.0], np.float16)
    gu = np.concatenate([gate, up])[None, :]
    out = host(q4.silu_mul(dev_tensor(gu)))
    sync()
    assert_within(out, o.silu_mul(gu), "silu special")
    assert out[0, 0] == 0.0


def _mat(o, seed, n, k):
    codes = datagen.codes(seed, n, k)
    return o.pack(codes), datagen.scales(seed + 1, n, k)


@pytest.mark.parametrize("n,k", [(16384, 3072), (19456, 2560), (74, 96), (3072, 2048)])
def test_silu_epilogue_equals_unfused(o, q4, n, k):
    W, S = _mat(o, 400 + n, n, k)
    x = datagen.activations(402 + n, 1, k)[0]
    Wd, Sd, xd = dev_tensor(W), dev_tensor(S), dev_tensor(x)
    fused = q4.gemv_ex(Wd, Sd, xd, kind=q4.EPI_SILU_MUL)
    unfused = q4.silu_mul(q4.gemv(Wd, Sd, xd)[None, :])[0]
    sync()
    assert np.array_equal(bits(fused), bits(unfused))
    gu = o.d2h(o.gemv(W, S, x))
    assert_within(host(fused), o.silu_mul(gu)[0], "fused silu vs oracle")


@pytest.mark.parametrize("n,k", [(3072, 3072), (3072, 8192), (2560, 9728), (291, 64)])
def test_add_rmsnorm_epilogue_equals_unfused(o, q4, n, k):
    import torch
    W, S = _mat(o, 500 + n, n, k)
    x = datagen.activations(502 + n, 1, k)[0]
    r = datagen.activations(503 + n, 1, n)[0]
    g = datagen.gammas(504 + n, 1, n)[0]
    Wd, Sd, xd, rd, gd = (dev_tensor(v) for v in (W, S, x, r, g))
    for rep in range(2):   # twice: the completion counter must be back at zero
        res_f = torch.empty(n, dtype=torch.float16, device="cuda")
        h_f = q4.gemv_ex(Wd, Sd, xd, kind=q4.EPI_ADD_RMSNORM, res_in=rd, gamma=gd,
                         res_out=res_f, eps=1e-5)
        t = q4.gemv(Wd, Sd, xd)
        h_u, res_u = q4.add_rmsnorm(t, rd, gd, eps=1e-5)
        sync()
        assert np.array_equal(bits(res_f), bits(res_u)), rep
        assert np.array_equal(bits(h_f), bits(h_u)), rep
    res_ref, h_ref = o.add_rmsnorm(o.d2h(o.gemv(W, S, x)), r, g, eps=1e-5)
    assert_within(host(res_f), res_ref[0].astype(np.float64), "residual")
    assert_within(host(h_f), h_ref[0], "fused add+rmsnorm vs oracle")


def test_epilogue_rejects_aliased_residual(q4):
    import torch
    n, k = 64, 64
    Wd = torch.zeros((n, k // 8), dtype=torch.int32, device="cuda")
    Sd = torch.zeros((n, k // 32), dtype=torch.float16, device="cuda")
    xd = torch.zeros(k, dtype=torch.float16, device="cuda")
    r = torch.zeros(n, dtype=torch.float16, device="cuda")
    g = torch.ones(n, dtype=torch.float16, device="cuda")
    with pytest.raises(q4.Q4Error) as ei:
        q4.gemv_ex(Wd, Sd, xd, kind=q4.EPI_ADD_RMSNORM, res_in=r, gamma=g, res_out=r)
    assert ei.value.status == q4.Q4_EALIAS


@pytest.mark.parametrize("n,k,kind", [(16384, 3072, 1), (9216, 3072, 0), (74, 96, 1), (33, 8192, 0)])
def test_norm_prologue_equals_unfused(o, q4, n, k, kind):
    """x := RMSNorm(x) * gamma inside the matvec equals q4_add_rmsnorm then the matvec."""
    W, S = _mat(o, 600 + n, n, k)
    r = datagen.activations(602 + n, 1, k)[0]
    g = datagen.gammas(603 + n, 1, k)[0]
    Wd, Sd, rd, gd = (dev_tensor(v) for v in (W, S, r, g))
    fused = q4.gemv_ex(Wd, Sd, rd, kind=kind, norm_gamma=gd, eps=1e-5)
    h, _ = q4.add_rmsnorm(None, rd, gd, eps=1e-5)
    unfused = q4.gemv_ex(Wd, Sd, h, kind=kind)
    sync()
    assert np.array_equal(bits(fused), bits(unfused))
    _, h_ref = o.add_rmsnorm(None, r, g, eps=1e-5)
    y_ref = o.gemv(W, S, o.d2h(h_ref[0]))
    if kind == 1:
        y_ref = o.silu_mul(o.d2h(y_ref))[0]
    assert_within(host(fused), y_ref, "prologue vs oracle")
