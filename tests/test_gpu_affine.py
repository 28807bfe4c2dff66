"""GPU parity of q4_gemv_affine (the MLX affine 4-bit format) against the oracle.

Bar: per element |y - y_ref| <= 1e-2 + 5e-3 |y_ref| against the binary64
oracle (w = s * q + b, group 64); a one-hot activation gives f16(s * q + b)
bit for bit at M = 1 and on the matrix cores (M >= 2); a reference with the
bias dropped must fail the gate. Shapes: Qwen3-4B's layer matrices (the pages
run Qwen3 as an MLX-affine build), ragged N, and M = 1, 2, 3, 4, 8, 17; at
M = 2..4 every row equals the single-row matvec of that row bit for bit.
"""
import zlib

import numpy as np
import pytest

import datagen
import oracle
import oracle_pins
from gpu_common import assert_within, bits, dev_tensor, host, within

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.fixture(scope="module")
def q4():
    import torch
    import int4_weight_only_q4_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


def make(name, n, k, m):
    seed = datagen.seed_for(8, zlib.crc32(name.encode()) % 1000)
    W = datagen.words(seed, n, k)
    S = datagen.scales(seed + 1, n, k // 2)
    B = datagen.normal_f16(seed + 2, (n, k // 64), 0.0, 0.05)
    X = datagen.activations(seed + 3, m, k)
    return W, S, B, X


def run(q4, W, S, B, X):
    import torch
    x = dev_tensor(X if X.shape[0] > 1 else X[0])
    y = q4.gemv_affine(dev_tensor(W), dev_tensor(S), dev_tensor(B), x)
    torch.cuda.synchronize()
    return host(y).reshape(X.shape[0], -1)


SHAPES = [("qwen3_qkv", 6144, 2560, 1), ("qwen3_gate_up", 19456, 2560, 1),
          ("qwen3_down", 2560, 9728, 1), ("ragged", 333, 640, 1), ("one_group", 5, 64, 1),
          ("qwen3_qkv", 6144, 2560, 8), ("qwen3_down", 2560, 9728, 2), ("ragged", 333, 640, 2),
          ("ragged", 333, 640, 17), ("one_group", 5, 64, 8), ("qwen3_qkv", 6144, 2560, 4),
          ("qwen3_gate_up", 19456, 2560, 3), ("qwen3_gate_up", 19456, 2560, 8),
          ("qwen3_o", 2560, 4096, 8), ("qwen3_down", 2560, 9728, 4)]


@pytest.mark.parametrize("name,n,k,m", SHAPES, ids=["%s-M%d" % (s[0], s[3]) for s in SHAPES])
def test_affine_vs_oracle(o, q4, name, n, k, m):
    W, S, B, X = make(name, n, k, m)
    y = run(q4, W, S, B, X)
    assert_within(y, o.gemv_affine(W, S, B, X), "%s M=%d" % (name, m))


@pytest.mark.parametrize("m", [1, 3, 16])
def test_affine_one_hot_is_exact(o, q4, m):
    n, k = 96, 1024
    codes = datagen.codes(811, n, k)
    W = o.pack(codes)
    S = datagen.scales(812, n, k // 2)
    B = datagen.normal_f16(813, (n, k // 64), 0.0, 0.05)
    ks = np.random.default_rng(m).integers(0, k, m)
    X = np.zeros((m, k), np.float16)
    X[np.arange(m), ks] = 1.0
    y = run(q4, W, S, B, X)
    for i in range(m):
        c = ks[i]
        want = o.d2h(o.h2d(S[:, c // 64]) * codes[:, c] + o.h2d(B[:, c // 64]))
        assert np.array_equal(y[i].view(np.uint16), want.view(np.uint16)), (m, i)


def test_affine_gate_rejects_a_dropped_bias(o, q4):
    W, S, B, X = make("gate", 512, 2048, 1)
    y = run(q4, W, S, B, X)
    assert within(y, o.gemv_affine(W, S, B, X))
    bad = oracle_pins.mutant("affine_bias_dropped")
    assert not within(y, bad.gemv_affine(W, S, B, X))


@pytest.mark.parametrize("n,k,m", [(6144, 2560, 2), (19456, 2560, 4), (2560, 4096, 3), (333, 640, 4),
                                   (2560, 9728, 2)])
def test_affine_few_rows_equal_single_row_matvecs(q4, n, k, m):
    """M = 2..4 (M K <= 24576) runs the single-row affine arithmetic per row."""
    W, S, B, X = make("rows_%d_%d_%d" % (n, k, m), n, k, m)
    Wd, Sd, Bd = dev_tensor(W), dev_tensor(S), dev_tensor(B)
    Y = q4.gemv_affine(Wd, Sd, Bd, dev_tensor(X))
    singles = [q4.gemv_affine(Wd, Sd, Bd, dev_tensor(X[i])) for i in range(m)]
    import torch
    torch.cuda.synchronize()
    b = bits(Y)
    for i in range(m):
        assert np.array_equal(b[i], bits(singles[i])), i
