"""GPU parity of q4_gemm (the prefill matmul on the matrix cores) against the oracle.

Bar: per element |y - y_ref| <= 1e-2 + 5e-3 |y_ref| against the binary64
oracle: gemv_batched (w = (q - 7) s exact) for Q4_GEMM_EXACT, gemv_w16 (w
rounded to f16 first) for Q4_GEMM_F16_WEIGHT, which must also stay within the
bar of the exact result. Bit-exact cases:
* a one-hot activation row gives f16(w) (exact mode) or the f16 weight itself
  (f16 mode) for every weight row, with scales small enough that many of them
  are binary16 subnormals;
* every output row is independent of M and of the row's position in the batch
  (the same bits computed alone and inside a batch of 300) while the launch
  splits K the same way (here: two splits at every M).
Shapes: ragged small cases that the oracle computes whole (tiles of 64 or 128
x 128, steps of 128 values of K, a last step of one group, K split in 2 and 7
parts with a partial last step), and the prefill shapes of Phi-3-mini
(M = 1024) and Qwen3-4B (M = 256, K split) checked on sampled outputs.
"""
import zlib

import numpy as np
import pytest

import datagen
import oracle
from gpu_common import assert_within, dev_tensor, host

pytestmark = pytest.mark.gpu

EXACT, F16W = 0, 1


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
    seed = datagen.seed_for(9, zlib.crc32(name.encode()) % 1000)
    W = datagen.words(seed, n, k)
    S = datagen.scales(seed + 1, n, k)
    X = datagen.activations(seed + 2, m, k)
    return W, S, X


def run(q4, W, S, X, mode, ldx=None, ldy=None):
    import torch
    m, k = X.shape
    n = W.shape[0]
    ldx = ldx or k
    ldy = ldy or n
    xb = np.zeros((m, ldx), np.float16)
    xb[:, :k] = X
    xd = dev_tensor(xb)
    yd = torch.full((m, ldy), 3.0, dtype=torch.float16, device="cuda")
    q4.gemm(dev_tensor(W), dev_tensor(S), xd[:, :k], yd[:, :n], weights=mode)
    torch.cuda.synchronize()
    y = host(yd)
    assert np.all(y[:, n:] == np.float16(3.0)), "wrote past N in the padded rows"
    return y[:, :n]


SMALL = [("tiny", 1, 1, 32), ("one_step_short", 17, 200, 96), ("one_tile", 64, 128, 256),
         ("ragged", 65, 129, 160), ("ragged_tail_group", 130, 300, 544),
         ("square", 256, 256, 1024), ("tall", 1000, 40, 128),
         ("split_tail", 100, 200, 1184), ("many_splits", 64, 128, 4160)]


@pytest.mark.parametrize("mode", [EXACT, F16W], ids=["exact", "f16w"])
@pytest.mark.parametrize("name,m,n,k", SMALL, ids=[s[0] for s in SMALL])
def test_gemm_vs_oracle(o, q4, name, m, n, k, mode):
    W, S, X = make(name, n, k, m)
    y = run(q4, W, S, X, mode)
    exact = o.gemv_batched(W, S, X)
    assert_within(y, exact, "%s vs exact weights" % name)
    if mode == F16W:
        assert_within(y, o.gemv_w16(W, S, X), "%s vs f16 weights" % name)


def test_gemm_strided_rows(o, q4):
    W, S, X = make("strided", 200, 384, 70)
    y = run(q4, W, S, X, EXACT, ldx=392, ldy=216)
    assert_within(y, o.gemv_batched(W, S, X), "strided")


@pytest.mark.parametrize("mode", [EXACT, F16W], ids=["exact", "f16w"])
def test_gemm_one_hot_is_the_weight(o, q4, mode):
    """Row i of X is e_{k_i}: y[i][n] is f16 of the weight at (n, k_i). Scales in
    [2^-12, 2^-8] put many weights below the binary16 normal range."""
    n, k, m = 160, 512, 96
    codes = datagen.codes(901, n, k)
    W = o.pack(codes)
    rng = np.random.default_rng(902)
    S = rng.uniform(2.0 ** -12, 2.0 ** -8, size=(n, k // 32)).astype(np.float16)
    ks = np.concatenate([np.arange(8), rng.integers(0, k, m - 8)])
    X = np.zeros((m, k), np.float16)
    X[np.arange(m), ks] = 1.0
    y = run(q4, W, S, X, mode)
    w = (codes.astype(np.float64) - 7.0) * np.repeat(S.astype(np.float64), 32, axis=1)
    if mode == F16W:
        w = o.h2d(o.d2h(w))
    for i in range(m):
        want = o.d2h(w[:, ks[i]])
        assert np.array_equal(y[i].view(np.uint16), want.view(np.uint16)), (i, ks[i])


@pytest.mark.parametrize("mode", [EXACT, F16W], ids=["exact", "f16w"])
def test_gemm_rows_independent_of_m(q4, mode):
    W, S, X = make("m_invariance", 384, 1024, 300)
    full = run(q4, W, S, X, mode)
    for lo, hi in ((0, 1), (77, 78), (250, 300), (64, 129)):
        part = run(q4, W, S, X[lo:hi], mode)
        assert np.array_equal(part.view(np.uint16), full[lo:hi].view(np.uint16)), (lo, hi)


PREFILL = [("phi3_qkv", 9216, 3072, 1024), ("phi3_o", 3072, 3072, 1024),
           ("phi3_gate_up", 16384, 3072, 1024), ("phi3_down", 3072, 8192, 1024),
           ("qwen3_gate_up", 19456, 2560, 256), ("qwen3_down", 2560, 9728, 256),
           ("qwen3_o", 2560, 4096, 256)]


@pytest.mark.parametrize("mode", [EXACT, F16W], ids=["exact", "f16w"])
@pytest.mark.parametrize("name,n,k,m", PREFILL, ids=[s[0] for s in PREFILL])
def test_gemm_prefill_sampled(o, q4, name, n, k, m, mode):
    """Full-size launch; 12 activation rows x 96 weight rows (first and last of
    each, and random ones) against the oracle, one small oracle call."""
    W, S, X = make(name, n, k, m)
    y = run(q4, W, S, X, mode)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    rows = np.unique(np.r_[0, m - 1, rng.integers(0, m, 10)])
    cols = np.unique(np.r_[0, 127, 128, n - 1, rng.integers(0, n, 92)])
    ref_fn = o.gemv_batched if mode == EXACT else o.gemv_w16
    ref = ref_fn(W[cols], S[cols], X[rows])
    assert_within(y[np.ix_(rows, cols)], ref, "%s sampled" % name)
    assert np.all(np.isfinite(y)), "non-finite outputs"


# -- MLX affine format (w = s * q + b, group 64) ----------------------------------

def make_affine(name, n, k, m):
    seed = datagen.seed_for(9, 500 + zlib.crc32(name.encode()) % 400)
    W = datagen.words(seed, n, k)
    S = datagen.scales(seed + 1, n, k // 2)
    B = datagen.normal_f16(seed + 2, (n, k // 64), 0.0, 0.05)
    X = datagen.activations(seed + 3, m, k)
    return W, S, B, X


def run_affine(q4, W, S, B, X, ldx=None, ldy=None):
    import torch
    m, k = X.shape
    n = W.shape[0]
    ldx = ldx or k
    ldy = ldy or n
    xb = np.zeros((m, ldx), np.float16)
    xb[:, :k] = X
    xd = dev_tensor(xb)
    yd = torch.full((m, ldy), 3.0, dtype=torch.float16, device="cuda")
    q4.gemm_affine(dev_tensor(W), dev_tensor(S), dev_tensor(B), xd[:, :k], yd[:, :n])
    torch.cuda.synchronize()
    y = host(yd)
    assert np.all(y[:, n:] == np.float16(3.0)), "wrote past N in the padded rows"
    return y[:, :n]


AFFINE_SMALL = [("a_tiny", 1, 5, 64), ("a_short", 17, 200, 192), ("a_tile", 64, 128, 256),
                ("a_ragged", 65, 129, 640), ("a_tail", 130, 300, 1088),
                ("a_two_bias_steps_split", 256, 256, 4160)]


@pytest.mark.parametrize("name,m,n,k", AFFINE_SMALL, ids=[s[0] for s in AFFINE_SMALL])
def test_gemm_affine_vs_oracle(o, q4, name, m, n, k):
    W, S, B, X = make_affine(name, n, k, m)
    y = run_affine(q4, W, S, B, X)
    assert_within(y, o.gemv_affine(W, S, B, X), name)


def test_gemm_affine_strided_rows(o, q4):
    W, S, B, X = make_affine("a_strided", 200, 384, 70)
    y = run_affine(q4, W, S, B, X, ldx=392, ldy=216)
    assert_within(y, o.gemv_affine(W, S, B, X), "affine strided")


def test_gemm_affine_one_hot_is_the_weight(o, q4):
    """Row i of X is e_{k_i}: y[i][n] = f16(s q + b) of weight (n, k_i), bit for bit."""
    n, k, m = 160, 1024, 96
    codes = datagen.codes(911, n, k)
    W = o.pack(codes)
    S = datagen.scales(912, n, k // 2)
    B = datagen.normal_f16(913, (n, k // 64), 0.0, 0.05)
    rng = np.random.default_rng(914)
    ks = np.concatenate([np.arange(8), rng.integers(0, k, m - 8)])
    X = np.zeros((m, k), np.float16)
    X[np.arange(m), ks] = 1.0
    y = run_affine(q4, W, S, B, X)
    for i in range(m):
        c = ks[i]
        want = o.d2h(o.h2d(S[:, c // 64]) * codes[:, c] + o.h2d(B[:, c // 64]))
        assert np.array_equal(y[i].view(np.uint16), want.view(np.uint16)), (i, c)


def test_gemm_affine_rows_independent_of_m(q4):
    W, S, B, X = make_affine("a_m_invariance", 384, 1024, 300)
    full = run_affine(q4, W, S, B, X)
    for lo, hi in ((0, 1), (77, 78), (250, 300), (64, 129)):
        part = run_affine(q4, W, S, B, X[lo:hi])
        assert np.array_equal(part.view(np.uint16), full[lo:hi].view(np.uint16)), (lo, hi)


AFFINE_PREFILL = [("qwen3_gate_up", 19456, 2560, 256), ("qwen3_down", 2560, 9728, 256),
                  ("qwen3_o", 2560, 4096, 256), ("qwen3_qkv_1024", 6144, 2560, 1024)]


@pytest.mark.parametrize("name,n,k,m", AFFINE_PREFILL, ids=[s[0] for s in AFFINE_PREFILL])
def test_gemm_affine_prefill_sampled(o, q4, name, n, k, m):
    W, S, B, X = make_affine(name, n, k, m)
    y = run_affine(q4, W, S, B, X)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    rows = np.unique(np.r_[0, m - 1, rng.integers(0, m, 10)])
    cols = np.unique(np.r_[0, 127, 128, n - 1, rng.integers(0, n, 92)])
    ref = o.gemv_affine(W[cols], S[cols], B[cols], X[rows])
    assert_within(y[np.ix_(rows, cols)], ref, "%s sampled" % name)
    assert np.all(np.isfinite(y)), "non-finite outputs"


@pytest.mark.parametrize("mode", [EXACT, F16W], ids=["exact", "f16w"])
def test_gemm_k_max(o, q4, mode):
    """K = Q4_MAX_K (24576, 768 groups): one tile of rows, K split."""
    W, S, X = make("k_max", 40, 24576, 70)
    y = run(q4, W, S, X, mode)
    ref = o.gemv_batched(W, S, X) if mode == EXACT else o.gemv_w16(W, S, X)
    assert_within(y, ref, "K max")


def test_gemm_m_max(o, q4):
    """M = Q4_MAX_GEMM_M (65536 activation rows) on a small matrix: sampled rows
    (the first and last tiles and random ones) against the oracle."""
    m = q4.MAX_GEMM_M
    W, S, X = make("m_max", 24, 64, m)
    y = run(q4, W, S, X, EXACT)
    rng = np.random.default_rng(65536)
    rows = np.unique(np.r_[0, 1, 127, 128, m - 129, m - 1, rng.integers(0, m, 200)])
    assert_within(y[rows], o.gemv_batched(W, S, X[rows]), "M max sampled")
    assert np.all(np.isfinite(y.astype(np.float64)))
