"""GPU parity of q4_gemv_batched and q4_moe_gemv against the oracle.

Batched: the Qwen3-4B matrices at batch 8 (8 independent activation rows),
ragged and larger M, identical rows giving identical outputs; at M = 2..4
(the dot2 kernel) every row equals the single-row matvec of that row bit for
bit.
MoE: 128 experts with gate_up 1536 x 2048 and down 2048 x 768, top-8 routing at
token batches 1, 4 and 16 (both stages, combined by routing weight), plus
small cases with repeated experts and an out-of-range id.
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


BATCHED = [
    ("qwen3_qkv", 6144, 2560, 8),
    ("qwen3_o", 2560, 4096, 8),
    ("qwen3_gate_up", 19456, 2560, 8),
    ("qwen3_down", 2560, 9728, 8),
    ("phi3_o_m1", 3072, 3072, 1),
    ("ragged_m13", 37, 96, 13),
    ("m64", 300, 512, 64),
    ("m3_kmax", 33, 24576, 3),
    ("phi3_qkv_m2", 9216, 3072, 2),
    ("phi3_gate_up_m4", 16384, 3072, 4),
    ("phi3_down_m2", 3072, 8192, 2),
    ("qwen3_qkv_m3", 6144, 2560, 3),
    ("ragged_m4", 37, 96, 4),
    # the workgroup-reduced matrix-core kernel: a group count that leaves the
    # last wave's quarter part empty, four 16-row tiles per workgroup with a
    # half-empty last workgroup, 16 rows, and 17 rows (two launches)
    ("mma_ragged_groups_m8", 1000, 2528, 8),
    ("mma_four_tiles_tail_m6", 32800, 256, 6),
    ("mma_m16", 3000, 2048, 16),
    ("mma_m17", 500, 1024, 17),
    # LM-head-sized matrices (N K >= 2^26) at M = 3 and 4 take the matrix
    # cores instead of the few-row kernel
    ("lm_sized_m3", 32768, 2048, 3),
    ("lm_sized_m4", 33000, 2080, 4),
]


@pytest.mark.parametrize("name,n,k,m", BATCHED, ids=[b[0] for b in BATCHED])
def test_batched_vs_oracle(o, q4, name, n, k, m):
    seed = 900 + n + m
    codes = datagen.codes(seed, n, k)
    W, S = o.pack(codes), datagen.scales(seed + 1, n, k)
    X = datagen.activations(seed + 2, m, k)
    Y = q4.gemv_batched(dev_tensor(W), dev_tensor(S), dev_tensor(X))
    sync()
    assert_within(host(Y), o.gemv_batched(W, S, X), name)


def test_batched_lm_head_sampled(o, q4):
    n, k, m = 151936, 2560, 8
    codes = datagen.codes(datagen.seed_for(4, 60), n, k)
    W, S = o.pack(codes), datagen.scales(datagen.seed_for(4, 61), n, k)
    X = datagen.activations(datagen.seed_for(4, 62), m, k)
    Y = host(q4.gemv_batched(dev_tensor(W), dev_tensor(S), dev_tensor(X)))
    sync()
    rows = np.unique(np.random.default_rng(9).integers(0, n, 512))
    for i in range(m):
        assert_within(Y[i, rows], o.gemv_rows(W, S, X[i], rows), "lm head row %d" % i)


def test_batched_identical_rows(o, q4):
    n, k = 2560, 9728
    codes = datagen.codes(71, n, k)
    W, S = o.pack(codes), datagen.scales(72, n, k)
    x = datagen.activations(73, 1, k)
    X = np.repeat(x, 8, axis=0)
    Y = q4.gemv_batched(dev_tensor(W), dev_tensor(S), dev_tensor(X))
    sync()
    b = bits(Y)
    assert all(np.array_equal(b[0], b[i]) for i in range(8))


@pytest.mark.parametrize("n,k,m", [(9216, 3072, 2), (16384, 3072, 3), (3072, 3072, 4),
                                   (3072, 8192, 2), (3072, 8192, 3), (2560, 9728, 2),
                                   (6144, 2560, 4), (37, 96, 3)])
def test_batched_few_rows_equal_single_row_matvecs(q4, n, k, m):
    """M = 2..4 (M K <= 24576) runs the single-row kernel's arithmetic per row:
    every row equals q4_gemv of that row bit for bit."""
    seed = 950 + n + k + m
    W = datagen.words(seed, n, k)
    S = datagen.scales(seed + 1, n, k)
    X = datagen.activations(seed + 2, m, k)
    Wd, Sd = dev_tensor(W), dev_tensor(S)
    Y = q4.gemv_batched(Wd, Sd, dev_tensor(X))
    singles = [q4.gemv(Wd, Sd, dev_tensor(X[i])) for i in range(m)]
    sync()
    b = bits(Y)
    for i in range(m):
        assert np.array_equal(b[i], bits(singles[i])), i


def test_batched_strided_rows(o, q4):
    import torch
    n, k, m = 96, 256, 5
    codes = datagen.codes(81, n, k)
    W, S = o.pack(codes), datagen.scales(82, n, k)
    X = datagen.activations(83, m, k)
    big = torch.zeros((m, k + 64), dtype=torch.float16, device="cuda")
    big[:, :k] = dev_tensor(X)
    out = torch.full((m, n + 8), 7.0, dtype=torch.float16, device="cuda")
    q4.gemv_batched(dev_tensor(W), dev_tensor(S), big[:, :k], y=out[:, :n])
    sync()
    h = host(out)
    assert np.all(h[:, n:] == np.float16(7.0))
    assert_within(h[:, :n], o.gemv_batched(W, S, X), "strided")


# ---------------------------------------------------------------------------
# MoE
# ---------------------------------------------------------------------------

def experts(o, seed, e, n, k):
    W = np.empty((e, n, k // 8), np.uint32)
    S = np.empty((e, n, k // 32), np.float16)
    for i in range(e):
        W[i] = o.pack(datagen.codes(seed + 2 * i, n, k))
        S[i] = datagen.scales(seed + 2 * i + 1, n, k)
    return W, S


@pytest.fixture(scope="module")
def moe128(o):
    """128 experts: gate_up 1536 x 2048, down 2048 x 768 (hidden 2048, ffn 768)."""
    Wg, Sg = experts(o, datagen.seed_for(5, 0), 128, 1536, 2048)
    Wd, Sd = experts(o, datagen.seed_for(5, 1000), 128, 2048, 768)
    return Wg, Sg, Wd, Sd, [dev_tensor(a) for a in (Wg, Sg, Wd, Sd)]


@pytest.mark.parametrize("t", [1, 4, 16])
def test_moe_layer_128_experts(o, q4, moe128, t):
    Wg, Sg, Wd, Sd, (Wgd, Sgd, Wdd, Sdd) = moe128
    topk, hidden, f = 8, 2048, 768
    ids, rw = datagen.routing(datagen.seed_for(5, 2000 + t), t, 128, topk)
    x = datagen.activations(datagen.seed_for(5, 3000 + t), t, hidden)
    idsd, rwd, xd = dev_tensor(ids), dev_tensor(rw), dev_tensor(x)
    u = q4.moe_gemv(Wgd, Sgd, idsd, xd, ldx=hidden, x_slot_stride=0, epi_silu=True)
    y = q4.moe_gemv(Wdd, Sdd, idsd, u, ldx=topk * f, x_slot_stride=f, route_w=rwd)
    sync()
    u_ref = o.moe_stage(Wg, Sg, ids, None, x, hidden, 0, 2 * f, hidden, epi_silu=True)
    assert_within(host(u), u_ref, "gate_up stage")
    # the down stage is checked from the GPU's own stored u (teacher forcing)
    uh = host(u)
    y_ref = o.moe_stage(Wd, Sd, ids, rw, uh, topk * f, f, hidden, f, epi_silu=False)
    assert_within(host(y), y_ref, "down stage + combine")


def test_moe_per_slot_mode_and_repeated_experts(o, q4):
    e, n, k, t, topk = 6, 96, 128, 5, 4
    W, S = experts(o, 1234, e, n, k)
    ids = np.array([[0, 1, 2, 3], [3, 2, 1, 0], [5, 5, 5, 5], [4, 0, 4, 0], [1, 1, 2, 2]],
                   np.int32)
    x = datagen.activations(1240, t * topk, k)
    y = q4.moe_gemv(dev_tensor(W), dev_tensor(S), dev_tensor(ids), dev_tensor(x),
                    ldx=topk * k, x_slot_stride=k)
    sync()
    ref = o.moe_stage(W, S, ids, None, x, topk * k, k, n, k, epi_silu=False)
    assert_within(host(y), ref, "per-slot")


def test_moe_out_of_range_id_contributes_zero(o, q4):
    e, n, k, t, topk = 4, 64, 64, 2, 3
    W, S = experts(o, 1300, e, n, k)
    ids = np.array([[0, 7, 1], [-1, 2, 3]], np.int32)
    rw = np.array([[0.5, 0.25, 0.25], [0.125, 0.5, 0.375]], np.float16)
    x = datagen.activations(1301, t * topk, k)
    y = q4.moe_gemv(dev_tensor(W), dev_tensor(S), dev_tensor(ids), dev_tensor(x),
                    ldx=topk * k, x_slot_stride=k, route_w=dev_tensor(rw))
    yp = q4.moe_gemv(dev_tensor(W), dev_tensor(S), dev_tensor(ids), dev_tensor(x),
                     ldx=topk * k, x_slot_stride=k)
    ys = q4.moe_gemv(dev_tensor(W), dev_tensor(S), dev_tensor(ids), dev_tensor(x),
                     ldx=topk * k, x_slot_stride=k, epi_silu=True)
    sync()
    valid = (ids >= 0) & (ids < e)
    ok = np.where(valid, ids, 0)
    w_eff = np.where(valid, rw, np.float16(0))
    ref = o.moe_stage(W, S, ok.astype(np.int32), w_eff, x, topk * k, k, n, k, epi_silu=False)
    assert_within(host(y), ref, "combine with invalid ids")
    yp = host(yp)
    assert np.all(yp[0, 1] == 0) and np.all(yp[1, 0] == 0)
    # the SiLU-multiply form: zeros for the invalid pairs, the oracle elsewhere
    ref_s = o.moe_stage(W, S, ok.astype(np.int32), None, x, topk * k, k, n, k, epi_silu=True)
    ys = host(ys)
    assert np.all(ys[~valid] == 0)
    assert_within(ys[valid], ref_s[valid], "SiLU form with invalid ids")


def test_moe_deterministic(o, q4, moe128):
    _, _, _, _, (Wgd, Sgd, Wdd, Sdd) = moe128
    ids, rw = datagen.routing(77, 16, 128, 8)
    x = datagen.activations(78, 16, 2048)
    idsd, rwd, xd = dev_tensor(ids), dev_tensor(rw), dev_tensor(x)
    outs = []
    for _ in range(2):
        u = q4.moe_gemv(Wgd, Sgd, idsd, xd, ldx=2048, x_slot_stride=0, epi_silu=True)
        y = q4.moe_gemv(Wdd, Sdd, idsd, u, ldx=8 * 768, x_slot_stride=768, route_w=rwd)
        outs.append(bits(y))
    sync()
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("n,k,m", [(3072, 3072, 8), (2560, 9728, 5), (96, 256, 16),
                                   (19456, 2560, 8), (1000, 2528, 13)])
def test_batched_one_hot_rows_are_exact(o, q4, n, k, m):
    """Row m of X is one-hot at column k_m: y[m][n] = f16((q[n][k_m] - 7) *
    s[n][k_m / 32]) exactly, so the batched path must not round a dequantised
    weight before it is multiplied (only the final f16 rounding remains)."""
    seed = 1700 + n + m
    codes = datagen.codes(seed, n, k)
    W, S = o.pack(codes), datagen.scales(seed + 1, n, k)
    ks = np.random.default_rng(seed).integers(0, k, m)
    X = np.zeros((m, k), np.float16)
    X[np.arange(m), ks] = 1.0
    Y = bits(q4.gemv_batched(dev_tensor(W), dev_tensor(S), dev_tensor(X)))
    sync()
    for i in range(m):
        g = ks[i] // 32  # the oracle dequantises the group holding column k_m
        grp = o.dequant(W[:, 4 * g:4 * g + 4], S[:, g:g + 1])
        assert np.array_equal(Y[i], o.d2h(grp[:, ks[i] % 32]).view(np.uint16)), i


@pytest.mark.parametrize("t,topk,e", [(40, 8, 32), (2, 4, 1100), (32, 8, 64), (32, 8, 1100)])
def test_moe_routing_paths(o, q4, t, topk, e):
    """Routings beyond the in-kernel limit (more than 256 pairs, more than 1024
    experts) take the sorting kernel; 256 pairs exactly stay in the kernel.
    Few pairs per expert (at most two on average) take the dot2 expert kernel:
    with the sorting kernel's list at 8 and 256 pairs (about 230 experts
    listed), the matrix cores otherwise. Per-slot and combine modes against the
    oracle, repeated ids included."""
    n, k = 48, 128
    W, S = experts(o, 1400 + e, e, n, k)
    ids = np.random.default_rng(e + t).integers(0, e, size=(t, topk)).astype(np.int32)
    ids[0, :2] = ids[0, 2]  # the same expert twice within a token
    rw = (np.random.default_rng(t).random((t, topk)) / topk).astype(np.float16)
    x = datagen.activations(1401 + e, t * topk, k)
    Wd, Sd, idsd, xd = dev_tensor(W), dev_tensor(S), dev_tensor(ids), dev_tensor(x)
    yp = q4.moe_gemv(Wd, Sd, idsd, xd, ldx=topk * k, x_slot_stride=k)
    yc = q4.moe_gemv(Wd, Sd, idsd, xd, ldx=topk * k, x_slot_stride=k, route_w=dev_tensor(rw))
    sync()
    assert_within(host(yp), o.moe_stage(W, S, ids, None, x, topk * k, k, n, k, epi_silu=False),
                  "per-slot")
    assert_within(host(yc), o.moe_stage(W, S, ids, rw, x, topk * k, k, n, k, epi_silu=False),
                  "combine")


@pytest.mark.parametrize("e", [12, 1100], ids=["in_kernel_routing", "sorted_routing"])
def test_moe_few_tokens_expert_with_many_pairs(o, q4, e):
    """Few tokens (the dot2 expert path) with one expert repeated into 12 pairs:
    its pairs run in several units of at most 4. Per-slot and combine modes
    against the oracle, an out-of-range id included; every valid per-slot
    output equals the single-row matvec of its expert and activation, bit for
    bit (the same arithmetic per pair). 1100 experts take the sorting kernel."""
    n, k, topk = 80, 256, 6
    W, S = experts(o, 1500 + e, e, n, k)
    ids = np.array([[2, 2, 2, 2, 2, 2], [2, 2, 2, 1, 0, 4], [2, 3, 2, -1, 2, 1]], np.int32)
    t = ids.shape[0]
    rw = (np.random.default_rng(e).random((t, topk)) / topk).astype(np.float16)
    x = datagen.activations(1501 + e, t * topk, k)
    Wd, Sd, idsd, xd = dev_tensor(W), dev_tensor(S), dev_tensor(ids), dev_tensor(x)
    yp = q4.moe_gemv(Wd, Sd, idsd, xd, ldx=topk * k, x_slot_stride=k)
    yc = q4.moe_gemv(Wd, Sd, idsd, xd, ldx=topk * k, x_slot_stride=k, route_w=dev_tensor(rw))
    singles = {}
    for p, ex in enumerate(ids.reshape(-1)):
        if 0 <= ex < e:
            singles[p] = q4.gemv(Wd[ex], Sd[ex], xd[p])
    sync()
    ok = np.where((ids >= 0) & (ids < e), ids, 0).astype(np.int32)
    w_eff = np.where((ids >= 0) & (ids < e), rw, np.float16(0))
    ref_p = o.moe_stage(W, S, ok, None, x, topk * k, k, n, k, epi_silu=False)
    ref_c = o.moe_stage(W, S, ok, w_eff, x, topk * k, k, n, k, epi_silu=False)
    yph = host(yp).reshape(t * topk, n)
    valid = ((ids >= 0) & (ids < e)).reshape(-1)
    assert_within(yph[valid], ref_p.reshape(t * topk, n)[valid], "per-slot")
    assert np.all(yph[~valid] == 0)
    assert_within(host(yc), ref_c, "combine")
    for p, y1 in singles.items():
        assert np.array_equal(yph[p].view(np.uint16), bits(y1)), p


@pytest.mark.parametrize("t,topk,e", [(40, 8, 32), (64, 8, 128), (3, 6, 1100)])
def test_moe_sorted_routing_with_invalid_ids(o, q4, t, topk, e):
    """The sorting kernel's list (more than 256 pairs or more than 1024
    experts) with out-of-range ids and one expert repeated within a token:
    invalid pairs give zero per-slot outputs and no combine term, every other
    output within the bar of the oracle."""
    n, k = 64, 128
    W, S = experts(o, 1600 + e + t, e, n, k)
    rng = np.random.default_rng(1601 + t)
    ids = rng.integers(0, e, size=(t, topk)).astype(np.int32)
    ids[0, :3] = ids[0, 3]
    ids[1, 1] = -1
    ids[t - 1, topk - 1] = e
    ids[t // 2, 0] = e + 5
    rw = (rng.random((t, topk)) / topk).astype(np.float16)
    x = datagen.activations(1602 + t, t * topk, k)
    Wd, Sd, idsd, xd = dev_tensor(W), dev_tensor(S), dev_tensor(ids), dev_tensor(x)
    yp = q4.moe_gemv(Wd, Sd, idsd, xd, ldx=topk * k, x_slot_stride=k)
    yc = q4.moe_gemv(Wd, Sd, idsd, xd, ldx=topk * k, x_slot_stride=k, route_w=dev_tensor(rw))
    sync()
    valid = (ids >= 0) & (ids < e)
    ok = np.where(valid, ids, 0).astype(np.int32)
    w_eff = np.where(valid, rw, np.float16(0))
    ref_p = o.moe_stage(W, S, ok, None, x, topk * k, k, n, k, epi_silu=False)
    ref_c = o.moe_stage(W, S, ok, w_eff, x, topk * k, k, n, k, epi_silu=False)
    yph = host(yp).reshape(t * topk, n)
    v = valid.reshape(-1)
    assert_within(yph[v], ref_p.reshape(t * topk, n)[v], "per-slot")
    assert np.all(yph[~v] == 0)
    assert_within(host(yc), ref_c, "combine")


def test_moe_max_pairs(o, q4):
    """T * TOPK = Q4_MAX_PAIRS (512 tokens x 8 slots over 64 experts): the
    sorting kernel at its largest list and the matrix-core expert kernel,
    per-slot and combine modes against the oracle."""
    e, n, k, t, topk = 64, 32, 64, 512, 8
    W, S = experts(o, 1700, e, n, k)
    rng = np.random.default_rng(1701)
    ids = np.stack([rng.permutation(e)[:topk] for _ in range(t)]).astype(np.int32)
    rw = (rng.random((t, topk)) / topk).astype(np.float16)
    x = datagen.activations(1702, t * topk, k)
    Wd, Sd, idsd, xd = dev_tensor(W), dev_tensor(S), dev_tensor(ids), dev_tensor(x)
    yp = q4.moe_gemv(Wd, Sd, idsd, xd, ldx=topk * k, x_slot_stride=k)
    yc = q4.moe_gemv(Wd, Sd, idsd, xd, ldx=topk * k, x_slot_stride=k, route_w=dev_tensor(rw))
    sync()
    assert_within(host(yp), o.moe_stage(W, S, ids, None, x, topk * k, k, n, k, epi_silu=False),
                  "per-slot")
    assert_within(host(yc), o.moe_stage(W, S, ids, rw, x, topk * k, k, n, k, epi_silu=False),
                  "combine")


@pytest.mark.parametrize("t,topk,n,k", [(2, 4, 83, 1024), (1, 8, 2051, 768), (4, 8, 40, 96),
                                        (3, 5, 17, 32)])
def test_moe_token_wise_combine(o, q4, t, topk, n, k):
    """At most 32 pairs the combine stage runs token by token (the routing-
    weighted sum in the expert kernel): output rows not a multiple of the
    kernel's 8-row blocks, an expert repeated within a token, an out-of-range
    id, against the oracle with the invalid slot's weight set to zero."""
    e = 9
    W, S = experts(o, 1800 + n + k, e, n, k)
    rng = np.random.default_rng(1801 + t * topk)
    ids = rng.integers(0, e, size=(t, topk)).astype(np.int32)
    ids[0, 0] = ids[0, topk - 1]
    ids[t - 1, topk // 2] = -3 if t > 1 else e
    rw = (rng.random((t, topk)) / topk).astype(np.float16)
    x = datagen.activations(1802 + n, t * topk, k)
    yc = q4.moe_gemv(dev_tensor(W), dev_tensor(S), dev_tensor(ids), dev_tensor(x),
                     ldx=topk * k, x_slot_stride=k, route_w=dev_tensor(rw))
    sync()
    valid = (ids >= 0) & (ids < e)
    ok = np.where(valid, ids, 0).astype(np.int32)
    w_eff = np.where(valid, rw, np.float16(0))
    ref = o.moe_stage(W, S, ok, w_eff, x, topk * k, k, n, k, epi_silu=False)
    assert_within(host(yc), ref, "token-wise combine")


@pytest.mark.parametrize("t,topk,n,k", [(2, 4, 84, 1024), (1, 8, 1536, 2048), (4, 8, 40, 96),
                                        (3, 5, 18, 32)])
def test_moe_silu_few_pairs_shared_activation(o, q4, t, topk, n, k):
    """The SiLU-multiply stage at few pairs with every slot reading its token's
    one activation row (slot stride 0): gate rows not a multiple of the row
    block, an expert repeated within a token, an out-of-range id (zeros)
    against the oracle."""
    e = 7
    W, S = experts(o, 1900 + n + k, e, n, k)
    rng = np.random.default_rng(1901 + t * topk)
    ids = rng.integers(0, e, size=(t, topk)).astype(np.int32)
    ids[0, 1] = ids[0, topk - 1]
    ids[t - 1, 0] = e + 1
    x = datagen.activations(1902 + n, t, k)
    ys = q4.moe_gemv(dev_tensor(W), dev_tensor(S), dev_tensor(ids), dev_tensor(x), ldx=k,
                     x_slot_stride=0, epi_silu=True)
    sync()
    valid = (ids >= 0) & (ids < e)
    ok = np.where(valid, ids, 0).astype(np.int32)
    ref = o.moe_stage(W, S, ok, None, x, k, 0, n, k, epi_silu=True)
    ys = host(ys)
    assert np.all(ys[~valid] == 0)
    assert_within(ys[valid], ref[valid], "SiLU-multiply, shared activation")
