"""GPU parity of the LM head (f32 logits) and the greedy argmax against the oracle.

Bar:
* q4_gemv_f32 logits within |y - y_ref| <= 1e-2 + 5e-3 |y_ref| of the binary64
  oracle; a one-hot activation reproduces the exact weight (q - 7) s bit for
  bit in f32 (most of these values are not binary16 numbers, so an output
  rounded to f16 fails).
* q4_argmax on f32 inputs: the index is bit-exact against the oracle's argmax
  of the same f32 values (ties, -0/+0, infinities and NaN included).
* q4_lm_head_argmax: the logits as above; the token decides on the GPU's f32
  logits while the oracle's logits are exact, so the token must equal the
  oracle's whenever the oracle's top-2 gap exceeds the two tolerances, and in
  every case must be a maximum of the returned logits (first index) whose exact
  logit is within the tolerances of the exact maximum.
Shapes: the Phi-3-mini LM head 32064 x 3072 and the tied Qwen3-4B LM head
151936 x 2560 at full size (M = 1 and M = 8), ragged and small shapes.
"""
import zlib

import numpy as np
import pytest

import datagen
import oracle
from gpu_common import ATOL, RTOL, assert_within, dev_tensor, host

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


def make(o, name, n, k, m):
    seed = datagen.seed_for(6, zlib.crc32(name.encode()) % 1000)
    W = datagen.words(seed, n, k)
    S = datagen.scales(seed + 1, n, k)
    X = datagen.activations(seed + 2, m, k)
    return W, S, X


def sync():
    import torch
    torch.cuda.synchronize()


def tol(ref):
    return ATOL + RTOL * np.abs(ref)


def check_token(tok, logits_gpu, ref, what):
    """tok: GPU token of one row; logits_gpu: the row's returned f32 logits;
    ref: the row's exact logits."""
    assert 0 <= tok < ref.size, what
    assert tok == int(np.argmax(logits_gpu)), "%s: token is not the first maximum of its logits" % what
    best = int(np.argmax(ref))
    if ref.size == 1:
        assert tok == 0, what
        return
    order = np.argsort(ref)[::-1]
    gap = ref[order[0]] - ref[order[1]]
    if gap > tol(ref[order[0]]) + tol(ref[order[1]]):
        assert tok == best, "%s: token %d, oracle %d (gap %.4g)" % (what, tok, best, gap)
    else:
        assert ref[tok] >= ref[best] - tol(ref[tok]) - tol(ref[best]), what


F32_SHAPES = [
    # name, N, K, M
    ("single_512x256", 512, 256, 1),
    ("ragged_37x96", 37, 96, 1),
    ("one_row", 1, 32, 1),
    ("k_max", 67, 24576, 1),
    ("odd_groups", 300, 2080, 1),
    ("phi3_lm_head", 32064, 3072, 1),
    ("batched_3", 1000, 3072, 3),
    ("batched_17_ragged", 333, 2080, 17),
    ("phi3_lm_head_m4", 32064, 3072, 4),
]


@pytest.mark.parametrize("name,n,k,m", F32_SHAPES, ids=[s[0] for s in F32_SHAPES])
def test_gemv_f32_vs_oracle(o, q4, name, n, k, m):
    W, S, X = make(o, name, n, k, m)
    x = X[0] if m == 1 else X
    y = q4.gemv_f32(dev_tensor(W), dev_tensor(S), dev_tensor(x))
    sync()
    ref, _ = o.lm_head(W, S, X)
    assert_within(host(y).reshape(m, n), ref, name)


@pytest.mark.parametrize("m", [1, 2, 9])
def test_gemv_f32_one_hot_is_exact(o, q4, m):
    """x = e_k (rows of M) -> y = (q - 7) s exactly, in f32."""
    n, k = 200, 2080
    W, S, _ = make(o, "one_hot", n, k, 1)
    cols = [0, 1, 7, 8, 31, 32, 1000, 1024, 2079]
    Wd, Sd = dev_tensor(W), dev_tensor(S)
    dq = o.dequant(W, S)
    for c in cols:
        X = np.zeros((m, k), np.float16)
        X[:, c] = 1.0
        y = q4.gemv_f32(Wd, Sd, dev_tensor(X if m > 1 else X[0]))
        sync()
        y = host(y).reshape(m, n).astype(np.float64)
        assert np.array_equal(y, np.broadcast_to(dq[:, c], (m, n))), (m, c)
    # most of these weights are not binary16 values: an f16 output would differ
    assert np.mean(o.h2d(o.d2h(dq[:, cols])) != dq[:, cols]) > 0.25


ARGMAX_CASES = [
    # name, M, N, ties, special
    ("one", 1, 1, False, False),
    ("two", 1, 2, True, True),
    ("tail_255", 2, 255, True, True),
    ("tail_257", 3, 257, True, True),
    ("chunk_4095", 1, 4095, True, False),
    ("chunk_4097", 3, 4097, True, True),
    ("phi3_vocab", 4, 32064, True, True),
    ("qwen3_vocab", 8, 151936, False, True),
    ("qwen3_vocab_ties", 6, 151936, True, False),
    ("over_partial_cap", 1, 5_000_003, True, True),
]


@pytest.mark.parametrize("name,m,n,ties,special", ARGMAX_CASES, ids=[c[0] for c in ARGMAX_CASES])
def test_argmax_bit_exact(o, q4, name, m, n, ties, special):
    import torch
    v = datagen.logits(datagen.seed_for(6, 500 + zlib.crc32(name.encode()) % 400), m, n,
                       ties=ties, special=special)
    ld = n + 5  # rows with a leading dimension larger than N
    buf = np.full((m, ld), 1e30, np.float32)  # padding larger than any row value
    buf[:, :n] = v
    d = torch.from_numpy(buf).cuda()
    idx = q4.argmax(d[:, :n])
    sync()
    got = host(idx).astype(np.int64)
    want = [o.argmax(v[i]) for i in range(m)]
    assert list(got) == want, name


def test_argmax_planted_positions(o, q4):
    """The maximum at the first index, the last index, and shared by all."""
    import torch
    n = 40000
    rows = np.zeros((4, n), np.float32)
    rows[0, 0] = 5.0
    rows[1, n - 1] = 5.0
    rows[2, 1234] = 5.0
    rows[2, 30000] = 5.0
    idx = q4.argmax(torch.from_numpy(rows).cuda())
    sync()
    assert list(host(idx)) == [0, n - 1, 1234, 0]
    assert [o.argmax(r) for r in rows] == [0, n - 1, 1234, 0]


@pytest.mark.parametrize("name,n,k", [("phi3_lm_head", 32064, 3072), ("ragged_1001x96", 1001, 96),
                                      ("single_512x256", 512, 256), ("one_row", 1, 32)])
def test_lm_head_argmax_full(o, q4, name, n, k):
    W, S, X = make(o, name, n, k, 1)
    logits, tok = q4.lm_head_argmax(dev_tensor(W), dev_tensor(S), dev_tensor(X[0]))
    sync()
    ref, ref_tok = o.lm_head(W, S, X)
    lg = host(logits)
    assert_within(lg, ref[0], name)
    check_token(int(host(tok)[0]), lg, ref[0], name)


def test_lm_head_argmax_qwen3_tied_m1(o, q4):
    """Tied Qwen3-4B LM head 151936 x 2560, one token: every logit against the
    oracle, and the token."""
    n, k = 151936, 2560
    W, S, X = make(o, "qwen3_lm_head", n, k, 1)
    logits, tok = q4.lm_head_argmax(dev_tensor(W), dev_tensor(S), dev_tensor(X[0]))
    sync()
    ref, ref_tok = o.lm_head(W, S, X)
    lg = host(logits)
    assert_within(lg, ref[0], "qwen3 lm head")
    check_token(int(host(tok)[0]), lg, ref[0], "qwen3 lm head")


def test_lm_head_argmax_qwen3_tied_m8_sampled(o, q4):
    """The same LM head for 8 tokens on the matrix cores: 1024 sampled logits per
    row against the oracle, and each token against the oracle's on 2 rows whose
    full exact logits are computed; all 8 tokens are the first maximum of their
    returned logits."""
    n, k, m = 151936, 2560, 8
    W, S, X = make(o, "qwen3_lm_head", n, k, m)
    logits, tok = q4.lm_head_argmax(dev_tensor(W), dev_tensor(S), dev_tensor(X))
    sync()
    lg, tk = host(logits), host(tok).astype(np.int64)
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(9).integers(0, n, 1022)]))
    for b in range(m):
        assert tk[b] == int(np.argmax(lg[b])), b
        assert_within(lg[b, rows], o.gemv_rows(W, S, X[b], rows), "row %d" % b)
    for b in (0, 5):
        ref = o.gemv(W, S, X[b])
        check_token(int(tk[b]), lg[b], ref, "row %d" % b)


@pytest.mark.parametrize("n,k,m", [(20000, 3072, 3), (151936, 2560, 2), (1001, 96, 4)])
def test_lm_head_few_rows_equal_single_rows(o, q4, n, k, m):
    """M = 2..4 runs the single-row arithmetic per row (up to N K < 2^26 at M = 3
    and 4): each row's f32 logits and token equal those of the M = 1 LM head on
    that row, bit for bit."""
    W, S, X = make(o, "few_rows_%d" % n, n, k, m)
    Wd, Sd = dev_tensor(W), dev_tensor(S)
    logits, tok = q4.lm_head_argmax(Wd, Sd, dev_tensor(X))
    singles = [q4.lm_head_argmax(Wd, Sd, dev_tensor(X[i])) for i in range(m)]
    sync()
    lg, tk = host(logits), host(tok)
    for i in range(m):
        assert np.array_equal(lg[i].view(np.uint32), host(singles[i][0]).view(np.uint32)), i
        assert int(tk[i]) == int(host(singles[i][1])[0]), i


@pytest.mark.parametrize("m", [3, 4])
def test_lm_head_phi3_few_rows_matrix_cores(o, q4, m):
    """The Phi-3 LM head (N K >= 2^26) at M = 3 and 4 runs on the matrix cores:
    every logit of each row against the oracle, and each token."""
    n, k = 32064, 3072
    W, S, X = make(o, "phi3_lm_head_m%d" % m, n, k, m)
    logits, tok = q4.lm_head_argmax(dev_tensor(W), dev_tensor(S), dev_tensor(X))
    sync()
    lg, tk = host(logits), host(tok).astype(np.int64)
    ref, _ = o.lm_head(W, S, X)
    for b in range(m):
        assert_within(lg[b], ref[b], "row %d" % b)
        check_token(int(tk[b]), lg[b], ref[b], "row %d" % b)


def test_lm_head_more_than_16_rows(o, q4):
    """20 rows on the matrix cores run as two launches of 16 and 4 rows, each
    leaving its workgroups' row candidates for one finish: every logit against
    the oracle, each token, and tokens equal to those of the first maximum of
    the returned logits."""
    n, k, m = 5003, 256, 20
    W, S, X = make(o, "rows20", n, k, m)
    logits, tok = q4.lm_head_argmax(dev_tensor(W), dev_tensor(S), dev_tensor(X))
    sync()
    lg, tk = host(logits), host(tok).astype(np.int64)
    ref, _ = o.lm_head(W, S, X)
    for b in range(m):
        assert_within(lg[b], ref[b], "row %d" % b)
        check_token(int(tk[b]), lg[b], ref[b], "row %d" % b)


def test_lm_head_planted_maximum(o, q4):
    """All weights zero except two identical rows of codes 15 and x > 0: the
    token is the first of them, wherever it falls among the workgroups."""
    k = 256
    for n, r0, r1 in [(5000, 4999, 4999), (5000, 0, 4000), (12345, 777, 12000)]:
        codes = np.full((n, k), 7, np.uint8)
        codes[r0] = 15
        codes[r1] = 15
        W = o.pack(codes)
        S = datagen.scales(601, n, k)
        S[r1] = S[r0]
        x = np.abs(datagen.activations(602, 1, k)[0]).astype(np.float16)
        for m in (1, 2, 4, 8, 18):
            X = np.stack([x] * m)
            logits, tok = q4.lm_head_argmax(dev_tensor(W), dev_tensor(S),
                                            dev_tensor(X if m > 1 else x))
            sync()
            assert list(host(tok)) == [min(r0, r1)] * m, (n, r0, r1, m)


def test_lm_head_consistent_and_repeatable(o, q4):
    """M = 1: the fused LM head's logits equal q4_gemv_f32's bit for bit and its
    token equals q4_argmax of those logits; repeated calls give the same bits."""
    n, k = 32064, 3072
    W, S, X = make(o, "phi3_lm_head_rep", n, k, 1)
    Wd, Sd, xd = dev_tensor(W), dev_tensor(S), dev_tensor(X[0])
    l1, t1 = q4.lm_head_argmax(Wd, Sd, xd)
    l2, t2 = q4.lm_head_argmax(Wd, Sd, xd)
    y = q4.gemv_f32(Wd, Sd, xd)
    t3 = q4.argmax(y)
    sync()
    assert np.array_equal(host(l1).view(np.uint32), host(l2).view(np.uint32))
    assert np.array_equal(host(l1).view(np.uint32), host(y).view(np.uint32))
    assert int(host(t1)[0]) == int(host(t2)[0]) == int(host(t3)[0])


def test_lm_head_writes_only_its_outputs(o, q4):
    import torch
    n, k, m = 777, 512, 2
    W, S, X = make(o, "canary", n, k, m)
    lbuf = torch.full((m, n + 64), 7.0, dtype=torch.float32, device="cuda")
    tbuf = torch.full((m + 8,), -5, dtype=torch.int32, device="cuda")
    q4.lm_head_argmax(dev_tensor(W), dev_tensor(S), dev_tensor(X), logits=lbuf[:, 32:32 + n],
                      tokens=tbuf[4:4 + m])
    sync()
    lb, tb = host(lbuf), host(tbuf).view(np.int32)
    assert np.all(lb[:, :32] == 7.0) and np.all(lb[:, 32 + n:] == 7.0)
    assert np.all(tb[:4] == -5) and np.all(tb[4 + m:] == -5)
    ref, ref_tok = o.lm_head(W, S, X)
    assert_within(lb[:, 32:32 + n], ref, "canary logits")
    for b in range(m):
        check_token(int(tb[4 + b]), lb[b, 32:32 + n], ref[b], "canary row %d" % b)
