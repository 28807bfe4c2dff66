"""GPU parity of q4_pack / q4_unpack / q4_gemv against the oracle.

Bar: packed words and unpacked codes bit-exact; matvec outputs within
|y - y_ref| <= 1e-2 + 5e-3 |y_ref| of the binary64 oracle; special cases
(one-hot, scale doubling, repeated runs) bit-exact. Shapes: the 512 x 256
single-GEMV workload, the Phi-3-mini and Qwen3-4B layer matrices at full size,
the MoE expert matrices, and ragged/small/maximal shapes.
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


def make(o, seed, n, k):
    codes = datagen.codes(seed, n, k)
    S = datagen.scales(seed + 1, n, k)
    return codes, o.pack(codes), S


def gpu_gemv(q4, W, S, x):
    import torch
    y = q4.gemv(dev_tensor(W), dev_tensor(S), dev_tensor(x))
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("n,k", [(1, 32), (37, 96), (512, 256), (9216, 3072)])
def test_pack_unpack_bit_exact(o, q4, n, k):
    import torch
    codes = datagen.codes(100 + n, n, k)
    Wd = q4.pack(dev_tensor(codes))
    torch.cuda.synchronize()
    assert np.array_equal(host(Wd), o.pack(codes))
    back = q4.unpack(Wd)
    torch.cuda.synchronize()
    assert np.array_equal(host(back), codes)


def test_pack_uses_low_nibble_only(o, q4):
    import torch
    raw = np.random.default_rng(5).integers(0, 256, size=(8, 64), dtype=np.uint8)
    Wd = q4.pack(dev_tensor(raw))
    torch.cuda.synchronize()
    assert np.array_equal(host(Wd), o.pack(raw & 0xF))


GEMV_SHAPES = [
    ("single_512x256", 512, 256),
    ("phi3_qkv", 9216, 3072),
    ("phi3_o", 3072, 3072),
    ("phi3_gate_up", 16384, 3072),
    ("phi3_down", 3072, 8192),
    ("qwen3_qkv", 6144, 2560),
    ("qwen3_o", 2560, 4096),
    ("qwen3_gate_up", 19456, 2560),
    ("qwen3_down", 2560, 9728),
    ("moe_gate_up", 1536, 2048),
    ("moe_down", 2048, 768),
    ("ragged_37x96", 37, 96),
    ("one_row_one_group", 1, 32),
    ("k64", 5, 64),
    ("k_max", 67, 24576),
    ("odd_groups", 300, 2080),
    ("tp8_shard_qkv", 1152, 3072),
    ("tp8_shard_down", 3072, 1024),
]


@pytest.mark.parametrize("name,n,k", GEMV_SHAPES, ids=[s[0] for s in GEMV_SHAPES])
def test_gemv_vs_oracle(o, q4, name, n, k):
    seed = datagen.seed_for(2, zlib.crc32(name.encode()) % 1000)
    codes, W, S = make(o, seed, n, k)
    x = datagen.activations(seed + 2, 1, k)[0]
    y = gpu_gemv(q4, W, S, x)
    ref = o.gemv(W, S, x)
    assert_within(y, ref, name)


def test_gemv_lm_head_sampled_rows(o, q4):
    """Qwen3-4B LM head 151936 x 2560: every output checked against properties,
    2048 sampled rows (first, last, random) against the oracle row by row."""
    n, k = 151936, 2560
    codes, W, S = make(o, datagen.seed_for(4, 40), n, k)
    x = datagen.activations(datagen.seed_for(4, 42), 1, k)[0]
    y = gpu_gemv(q4, W, S, x)
    rows = np.unique(np.concatenate([[0, 1, n - 2, n - 1],
                                     np.random.default_rng(3).integers(0, n, 2044)]))
    assert_within(y[rows], o.gemv_rows(W, S, x, rows), "lm_head sampled")
    assert np.all(np.isfinite(y.astype(np.float64)))


def test_one_hot_reproduces_column_bit_exact(o, q4):
    n, k = 64, 512
    codes, W, S = make(o, 777, n, k)
    cols = list(range(16)) + [8 * j + (j % 8) for j in range(2, 64, 5)] + [k - 1]
    for kk in cols:
        x = np.zeros(k, np.float16)
        x[kk] = 1.0
        y = gpu_gemv(q4, W, S, x)
        ref = o.d2h(o.gemv(W, S, x))
        assert np.array_equal(y.view(np.uint16), ref.view(np.uint16)), kk


def test_all_sevens_give_zero(o, q4):
    n, k = 96, 3072
    codes = np.full((n, k), 7, np.uint8)
    W = o.pack(codes)
    S = datagen.scales(31, n, k)
    x = datagen.activations(32, 1, k)[0]
    y = gpu_gemv(q4, W, S, x)
    assert np.abs(y.astype(np.float64)).max() < 1e-4


def test_scale_doubling_is_bit_exact(o, q4):
    n, k = 300, 3072
    codes, W, S = make(o, 41, n, k)
    x = datagen.activations(43, 1, k)[0]
    y1 = gpu_gemv(q4, W, S, x)
    y2 = gpu_gemv(q4, W, (S.astype(np.float64) * 2).astype(np.float16), x)
    assert np.array_equal(y2.astype(np.float64), 2 * y1.astype(np.float64))


def test_repeatable_bits(o, q4):
    import torch
    n, k = 9216, 3072
    codes, W, S = make(o, 51, n, k)
    x = datagen.activations(53, 1, k)[0]
    Wd, Sd, xd = dev_tensor(W), dev_tensor(S), dev_tensor(x)
    a = q4.gemv(Wd, Sd, xd)
    b = q4.gemv(Wd, Sd, xd)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(b))


def test_no_write_outside_output_and_inputs_untouched(o, q4):
    import torch
    n, k = 37, 2080
    codes, W, S = make(o, 61, n, k)
    x = datagen.activations(63, 1, k)[0]
    Wd, Sd, xd = dev_tensor(W), dev_tensor(S), dev_tensor(x)
    canary = torch.full((n + 128,), 12345.0, dtype=torch.float16, device="cuda")
    q4.gemv(Wd, Sd, xd, y=canary[64:64 + n])
    torch.cuda.synchronize()
    c = host(canary)
    assert np.all(c[:64] == np.float16(12345.0)) and np.all(c[64 + n:] == np.float16(12345.0))
    assert_within(c[64:64 + n], o.gemv(W, S, x), "canary run")
    assert np.array_equal(host(Wd), W) and np.array_equal(bits(Sd), S.view(np.uint16))
    assert np.array_equal(bits(xd), x.view(np.uint16))


@pytest.mark.parametrize("mutant", ["zero_point_8", "nibble_order_reversed", "group_index_off_by_one",
                                    "scale_dropped", "group_of_16"])
def test_gate_rejects_a_wrong_reference(o, q4, mutant):
    """The tolerance gate is strong enough to see a plausible mistake: the GPU
    output, compared against an oracle with one planted mistake, must fail."""
    n, k = 512, 3072
    codes, W, S = make(o, 71, n, k)
    x = datagen.activations(73, 1, k)[0]
    y = gpu_gemv(q4, W, S, x)
    assert within(y, o.gemv(W, S, x))
    bad = oracle_pins.mutant(mutant)
    assert not within(y, bad.gemv(W, S, x))


def test_dispatch_timer_measures_the_matvec(o, q4):
    """q4_timer_arm makes the next matvec record its own start and end: the
    duration is positive and plausible, the output is unchanged, and a slot is
    consumed by one launch only."""
    import torch
    codes, W, S = make(o, 900, 3072, 3072)
    x = datagen.activations(902, 1, 3072)[0]
    Wd, Sd, xd = dev_tensor(W), dev_tensor(S), dev_tensor(x)
    plain = q4.gemv(Wd, Sd, xd)
    q4.timer_arm(5)
    timed = q4.gemv(Wd, Sd, xd)
    untimed = q4.gemv(Wd, Sd, xd)  # the slot is disarmed after one launch
    us = q4.timer_read(5)
    torch.cuda.synchronize()
    assert 0.1 < us < 10_000
    assert np.array_equal(bits(plain), bits(timed))
    assert np.array_equal(bits(plain), bits(untimed))
