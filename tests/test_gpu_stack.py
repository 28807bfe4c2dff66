"""GPU parity of q4_stack_decode (decode layers with attention := V slice).

* a small stack (d=256) against the oracle end to end and layer by layer;
* the full Phi-3-mini-shaped 32-layer stack as benchmarked (same weights and
  launch configuration as bench.py): layers 0, 15 and 31 teacher-forced against
  the oracle from the GPU's traced layer inputs (normalised output within
  tolerance of the oracle's layer; the layer bit-identical to the chain of
  single ABI calls; every op of that chain within tolerance of the oracle fed
  the GPU's own inputs), repeated tokens bit-identical;
* layers whose O and down matrices are all code 7 leave the residual unchanged.
"""
import numpy as np
import pytest

import bench
import datagen
import oracle
from gpu_common import assert_within, assert_within_scaled, bits, dev_tensor, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.fixture(scope="module")
def q4():
    import int4_weight_only_q4_amd as m
    m.lib()
    return m


def check_layer_by_ops(o, q4, p, mats_host, gp, g_next, r_in, h_in, tr_r, tr_h, what):
    """Op-level teacher forcing of one traced stack layer.

    The layer is re-run on the GPU as the chain of single ABI calls it is built
    from; the stack's traced (r, h) must equal that chain bit for bit, and every
    op of the chain is checked against the oracle fed the GPU's own binary16
    inputs (a layer-level tolerance would mix in legitimate one-ulp differences
    of intermediates amplified by the matvecs that follow them)."""
    import torch
    Wq, Sq, Wo, So, Wg, Sg, Wd, Sd = mats_host
    dev = [dev_tensor(m) for m in mats_host]
    v0, dv = p["v_off"], p["dv"]
    rd, hd = dev_tensor(r_in), dev_tensor(h_in)
    gpd, gnd = dev_tensor(gp), dev_tensor(g_next)
    qkv = q4.gemv(dev[0], dev[1], hd)
    r1 = torch.empty_like(rd)
    h1 = q4.gemv_ex(dev[2], dev[3], qkv[v0:v0 + dv], kind=q4.EPI_ADD_RMSNORM, res_in=rd,
                    gamma=gpd, res_out=r1, eps=p["eps"])
    u = q4.gemv_ex(dev[4], dev[5], h1, kind=q4.EPI_SILU_MUL)
    r2 = torch.empty_like(rd)
    h2 = q4.gemv_ex(dev[6], dev[7], u, kind=q4.EPI_ADD_RMSNORM, res_in=r1, gamma=gnd,
                    res_out=r2, eps=p["eps"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(r2), np.asarray(tr_r).view(np.uint16)), what + ": stack r != op chain"
    assert np.array_equal(bits(h2), np.asarray(tr_h).view(np.uint16)), what + ": stack h != op chain"
    qkv_h, r1_h, h1_h, u_h = host(qkv), host(r1), host(h1), host(u)
    f = lambda a: np.abs(np.asarray(a, dtype=np.float64))
    # each op against the oracle, from the GPU's own inputs
    assert_within(qkv_h, o.gemv(Wq, Sq, h_in), what + " qkv")
    o_ref = o.gemv(Wo, So, qkv_h[v0:v0 + dv])
    r1_ref, h1_ref = o.add_rmsnorm(o.d2h(o_ref), r_in, gp, eps=p["eps"])
    assert_within_scaled(r1_h, r1_ref[0], f(o_ref) + f(r_in), what + " r1")
    _, h1_from_r1 = o.add_rmsnorm(None, r1_h, gp, eps=p["eps"])
    assert_within(h1_h, h1_from_r1[0], what + " h1")
    gu_ref = o.d2h(o.gemv(Wg, Sg, h1_h))
    assert_within(u_h, o.silu_mul(gu_ref)[0], what + " u")
    dn_ref = o.gemv(Wd, Sd, u_h)
    r2_ref, _ = o.add_rmsnorm(o.d2h(dn_ref), r1_h, g_next, eps=p["eps"])
    assert_within_scaled(host(r2), r2_ref[0], f(dn_ref) + f(r1_h), what + " r2")
    _, h2_from_r2 = o.add_rmsnorm(None, host(r2), g_next, eps=p["eps"])
    assert_within(host(h2), h2_from_r2[0], what + " h2")


SMALL = dict(d=256, f=512, n_qkv=768, v_off=512, dv=256, layers=4, eps=1e-5)


def _run(q4, stack, st, d, n):
    import torch
    trace = torch.empty((n, 2, d), dtype=torch.float16, device="cuda")
    r_out = torch.empty(d, dtype=torch.float16, device="cuda")
    h_out = torch.empty(d, dtype=torch.float16, device="cuda")
    stack.decode(st["r0"], st["h0"], r_out, h_out, trace=trace)
    torch.cuda.synchronize()
    return host(r_out), host(h_out), host(trace)


def test_small_stack_vs_oracle(o, q4):
    import torch
    p = SMALL
    stack, st = bench.build_stack(q4, torch, p)
    r, h, tr = _run(q4, stack, st, p["d"], p["layers"])
    gi, gp, gf, r0, h0 = st["host"]
    dims = (p["d"], p["f"], p["n_qkv"], p["v_off"], p["dv"])
    layers = [bench.host_layer(p, L) for L in range(p["layers"])]
    # layer by layer from the GPU's own inputs
    for L in range(p["layers"]):
        r_in, h_in = (r0, h0) if L == 0 else (tr[L - 1, 0], tr[L - 1, 1])
        g_next = gi[L + 1] if L + 1 < p["layers"] else gf
        _, _, h64 = o.layer(dims, layers[L], gp[L], g_next, r_in, h_in)
        assert_within(tr[L, 1], h64, "layer %d h" % L)
        check_layer_by_ops(o, q4, p, layers[L], gp[L], g_next, r_in, h_in, tr[L, 0], tr[L, 1],
                           "layer %d" % L)
    assert np.array_equal(tr[-1, 1].view(np.uint16), h.view(np.uint16))
    assert np.array_equal(tr[-1, 0].view(np.uint16), r.view(np.uint16))
    # end to end (4 layers): reported, and within a loose bound
    _, _, h_e2e = o.stack(dims, layers, gi, gp, gf, r0, h0)
    rel = np.linalg.norm(h.astype(np.float64) - h_e2e) / np.linalg.norm(h_e2e)
    assert rel < 2e-2, rel


def test_identity_layers_keep_residual(o, q4):
    import torch
    p = SMALL
    stack, st = bench.build_stack(q4, torch, p, n_layers=2)
    sevens_o = o.pack(np.full((p["d"], p["dv"]), 7, np.uint8))
    sevens_dn = o.pack(np.full((p["d"], p["f"]), 7, np.uint8))
    for L in range(2):
        stack.layers[L][2].copy_(dev_tensor(sevens_o))
        stack.layers[L][6].copy_(dev_tensor(sevens_dn))
    r, h, tr = _run(q4, stack, st, p["d"], 2)
    gi, gp, gf, r0, h0 = st["host"]
    assert_within(r, r0.astype(np.float64), "residual")
    _, ref = o.add_rmsnorm(None, r0, gf)
    assert_within(h, ref[0], "normalised residual")


@pytest.fixture(scope="module")
def phi3(q4):
    import torch
    return bench.build_stack(q4, torch, bench.PHI3)


@pytest.mark.parametrize("layer", [0, 15, 31])
def test_phi3_stack_teacher_forced(o, q4, phi3, layer):
    p = bench.PHI3
    stack, st = phi3
    r, h, tr = _run(q4, stack, st, p["d"], p["layers"])
    gi, gp, gf, r0, h0 = st["host"]
    dims = (p["d"], p["f"], p["n_qkv"], p["v_off"], p["dv"])
    r_in, h_in = (r0, h0) if layer == 0 else (tr[layer - 1, 0], tr[layer - 1, 1])
    g_next = gi[layer + 1] if layer + 1 < p["layers"] else gf
    mats = bench.host_layer(p, layer)
    _, _, h64 = o.layer(dims, mats, gp[layer], g_next, r_in, h_in)
    assert_within(tr[layer, 1], h64, "phi3 layer %d" % layer)
    check_layer_by_ops(o, q4, p, mats, gp[layer], g_next, r_in, h_in, tr[layer, 0],
                       tr[layer, 1], "phi3 layer %d" % layer)


def test_phi3_stack_repeatable(q4, phi3):
    p = bench.PHI3
    stack, st = phi3
    a = _run(q4, stack, st, p["d"], p["layers"])
    b = _run(q4, stack, st, p["d"], p["layers"])
    assert np.array_equal(a[1].view(np.uint16), b[1].view(np.uint16))
    assert np.array_equal(a[0].view(np.uint16), b[0].view(np.uint16))
    assert np.all(np.isfinite(a[1].astype(np.float64))) and np.abs(a[1]).max() > 0


@pytest.mark.parametrize("which", ["small", "phi3"])
def test_stack_graph_replays_equal_eager(q4, phi3, which):
    """The captured token graphs that bench.py replays: every replay (four,
    alternating the two graphs, with eager calls and synchronisations between
    them) gives the bits of the same token computed by eager calls."""
    import torch
    if which == "small":
        p = SMALL
        stack, st = bench.build_stack(q4, torch, p)
    else:
        p = bench.PHI3
        stack, st = phi3
    d = p["d"]
    hs = [st["h0"].clone(), torch.empty_like(st["h0"])]
    r_out = torch.empty(d, dtype=torch.float16, device="cuda")
    _, graphs = bench.token_graphs(torch, stack, hs, r_out)
    for rep in range(4):
        a = rep & 1
        h_ref = torch.empty_like(hs[0])
        r_ref = torch.empty_like(hs[0])
        stack.decode(hs[a], hs[a], r_ref, h_ref)
        torch.cuda.synchronize()
        graphs[a].replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(hs[1 - a]), bits(h_ref)), ("h", rep)
        assert np.array_equal(bits(r_out), bits(r_ref)), ("r", rep)
    assert np.all(np.isfinite(host(hs[0]).astype(np.float64)))


# ---------------------------------------------------------------------------
# the stack with the real attention step (q4_stack_decode_attn)
# ---------------------------------------------------------------------------

def _attn_stack(o, q4, geom, n_layers, seed):
    """Host and device weights of a stack whose QKV rows are n_heads query,
    n_kv key and n_kv value heads, and whose O matrix reads n_heads heads."""
    d, f, nh, nkv, hd = geom
    nrows = (nh + 2 * nkv) * hd
    host_layers, dev_layers = [], []
    for L in range(n_layers):
        mats = []
        for j, (n, k) in enumerate(((nrows, d), (d, nh * hd), (2 * f, d), (d, f))):
            s = seed + 100 * L + 10 * j
            mats += [o.pack(datagen.codes(s, n, k)), datagen.scales(s + 1, n, k)]
        host_layers.append(mats)
        dev_layers.append([dev_tensor(m) for m in mats])
    gi = datagen.gammas(seed + 7, n_layers, d)
    gp = datagen.gammas(seed + 8, n_layers, d)
    gf = datagen.gammas(seed + 9, 1, d)[0]
    return host_layers, dev_layers, gi, gp, gf


@pytest.mark.parametrize("geom,n_layers,pos,max_len,pages", [
    ((256, 512, 4, 2, 64), 3, 37, 128, 8),
    ((256, 512, 4, 4, 64), 2, 0, 128, 8),
    # several splits of the positions (their combine may be the O matvec's
    # prologue): 521 cached positions over 3 splits, and a bound of 1000
    # positions whose later splits are empty
    ((256, 512, 4, 2, 64), 2, 520, 600, 40),
    ((256, 512, 4, 4, 64), 2, 300, 1000, 64)])
def test_stack_with_attention_teacher_forced(o, q4, geom, n_layers, pos, max_len, pages):
    import torch
    d, f, nh, nkv, hd = geom
    eps = 1e-5
    hl, dl, gi, gp, gf = _attn_stack(o, q4, geom, n_layers, 2100 + pos)
    desc = q4.attn_desc(nh, nkv, hd, 16, pages, pages)
    table = (np.array([5, 2, 7, 0, 1, 3, 6, 4], np.int32) if pages == 8
             else np.random.default_rng(pages).permutation(pages).astype(np.int32))
    tab = torch.from_numpy(table).cuda()
    posd = torch.tensor([pos], dtype=torch.int32, device="cuda")
    # caches with random rows for positions < pos (position pos is written by the step)
    caches0 = []
    for L in range(n_layers):
        c = np.zeros((pages, 2, nkv, 16, hd), np.float16)
        if pos:
            t = np.arange(pos)
            c[table[t // 16], 0, :, t % 16, :] = datagen.activations(2200 + L, pos, nkv * hd).reshape(pos, nkv, hd)
            c[table[t // 16], 1, :, t % 16, :] = datagen.activations(2300 + L, pos, nkv * hd).reshape(pos, nkv, hd)
        caches0.append(c)
    caches = [torch.from_numpy(c.copy()).cuda() for c in caches0]
    st = q4.Stack(dl, dev_tensor(gi), dev_tensor(gp), dev_tensor(gf), d, f, (nh + 2 * nkv) * hd, 0,
                  nh * hd, eps=eps)
    r0 = datagen.activations(2400, 1, d)[0]
    h0 = datagen.activations(2401, 1, d)[0]
    r_out = torch.empty(d, dtype=torch.float16, device="cuda")
    h_out = torch.empty(d, dtype=torch.float16, device="cuda")
    trace = torch.empty((n_layers, 2, d), dtype=torch.float16, device="cuda")
    st.decode_attn(desc, caches, tab, posd, max_len, dev_tensor(r0), dev_tensor(h0), r_out, h_out,
                   trace=trace)
    torch.cuda.synchronize()
    tr = host(trace)
    f64 = lambda a: np.abs(np.asarray(a, dtype=np.float64))
    r_in, h_in = r0, h0
    for L in range(n_layers):
        Wq, Sq, Wo, So, Wg, Sg, Wd, Sd = hl[L]
        dev = dl[L]
        g_next = gi[L + 1] if L + 1 < n_layers else gf
        what = "layer %d" % L
        # the chain of single calls from the same inputs and the cache before the step
        kv = torch.from_numpy(caches0[L].copy()).cuda()
        rd, hd_ = dev_tensor(r_in), dev_tensor(h_in)
        q = q4.qkv_rope_append(dev[0], dev[1], hd_, desc, posd, tab, kv)
        a = q4.attention_decode(q, kv, tab, posd, max_len, desc)
        r1 = torch.empty_like(rd)
        h1 = q4.gemv_ex(dev[2], dev[3], a, kind=q4.EPI_ADD_RMSNORM, res_in=rd, gamma=dev_tensor(gp[L]),
                        res_out=r1, eps=eps)
        u = q4.gemv_ex(dev[4], dev[5], h1, kind=q4.EPI_SILU_MUL)
        r2 = torch.empty_like(rd)
        h2 = q4.gemv_ex(dev[6], dev[7], u, kind=q4.EPI_ADD_RMSNORM, res_in=r1,
                        gamma=dev_tensor(g_next), res_out=r2, eps=eps)
        torch.cuda.synchronize()
        assert np.array_equal(bits(r2), tr[L, 0].view(np.uint16)), what + ": stack r != op chain"
        assert np.array_equal(bits(h2), tr[L, 1].view(np.uint16)), what + ": stack h != op chain"
        assert np.array_equal(bits(kv), bits(caches[L])), what + ": stack cache != op chain"
        # every op against the oracle, from the GPU's own inputs
        qr, kr, vr = o.qkv_rope(Wq, Sq, h_in, nh, nkv, hd, pos)
        assert_within(host(q), qr, what + " q")
        c = host(kv)
        t = np.arange(pos + 1)
        kc = c[table[t // 16], 0, :, t % 16, :]
        vc = c[table[t // 16], 1, :, t % 16, :]
        assert_within(kc[pos].ravel(), kr, what + " k")
        assert_within(vc[pos].ravel(), vr, what + " v")
        assert_within(host(a), o.attention(host(q), kc, vc, nh, nkv, hd), what + " attention")
        o_ref = o.gemv(Wo, So, host(a))
        r1_ref, _ = o.add_rmsnorm(o.d2h(o_ref), r_in, gp[L], eps=eps)
        assert_within_scaled(host(r1), r1_ref[0], f64(o_ref) + f64(r_in), what + " r1")
        _, h1_ref = o.add_rmsnorm(None, host(r1), gp[L], eps=eps)
        assert_within(host(h1), h1_ref[0], what + " h1")
        assert_within(host(u), o.silu_mul(o.d2h(o.gemv(Wg, Sg, host(h1))))[0], what + " u")
        dn_ref = o.gemv(Wd, Sd, host(u))
        r2_ref, _ = o.add_rmsnorm(o.d2h(dn_ref), host(r1), g_next, eps=eps)
        assert_within_scaled(host(r2), r2_ref[0], f64(dn_ref) + f64(host(r1)), what + " r2")
        r_in, h_in = tr[L, 0], tr[L, 1]
    assert np.array_equal(bits(r_out), tr[-1, 0].view(np.uint16))


def test_stack_with_attention_graph_replays_equal_eager(o, q4):
    """A captured HIP graph of one decode token with the attention step
    (q4_stack_decode_attn: cache append, split attention and merge kernels,
    matvecs), replayed four times between eager calls: every replay gives the
    eager token's bits and cache. The position grows the cache past one split."""
    import torch
    d, f, nh, nkv, hd = 256, 512, 4, 2, 64
    n_layers, L = 2, 600
    _, dl, gi, gp, gf = _attn_stack(o, q4, (d, f, nh, nkv, hd), n_layers, 2600)
    npages = (L + 15) // 16
    desc = q4.attn_desc(nh, nkv, hd, 16, npages, npages)
    tab = torch.from_numpy(np.random.default_rng(3).permutation(npages).astype(np.int32)).cuda()
    posd = torch.tensor([L - 1], dtype=torch.int32, device="cuda")
    c0 = [torch.from_numpy(datagen.normal_f16(2700 + i, (npages, 2, nkv, 16, hd))).cuda()
          for i in range(n_layers)]
    st = q4.Stack(dl, dev_tensor(gi), dev_tensor(gp), dev_tensor(gf), d, f, (nh + 2 * nkv) * hd, 0,
                  nh * hd, eps=1e-5)
    r0 = dev_tensor(datagen.activations(2800, 1, d)[0])
    h0 = dev_tensor(datagen.activations(2801, 1, d)[0])
    caches = [c.clone() for c in c0]
    r_g = torch.empty(d, dtype=torch.float16, device="cuda")
    h_g = torch.empty(d, dtype=torch.float16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            st.decode_attn(desc, caches, tab, posd, L, r0, h0, r_g, h_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        st.decode_attn(desc, caches, tab, posd, L, r0, h0, r_g, h_g)
    torch.cuda.synchronize()
    for rep in range(4):
        ce = [c.clone() for c in c0]
        r_e = torch.empty_like(r_g)
        h_e = torch.empty_like(h_g)
        st.decode_attn(desc, ce, tab, posd, L, r0, h0, r_e, h_e)
        torch.cuda.synchronize()
        for c, c_0 in zip(caches, c0):
            c.copy_(c_0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(h_g), bits(h_e)), ("h", rep)
        assert np.array_equal(bits(r_g), bits(r_e)), ("r", rep)
        for c, e_ in zip(caches, ce):
            assert torch.equal(c.view(torch.int16), e_.view(torch.int16)), ("cache", rep)
