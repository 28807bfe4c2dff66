"""q4_stack_decode_noalloc (the decode token without allocation, on the
library's fixed per-GPU scratch) against q4_stack_decode, called through the C
ABI: two calls in a row, the second on a smaller stack, each bit-identical to
the allocating entry point's result (and so within the tolerance of the
oracle, which the stack tests check for q4_stack_decode); a stack too large for
the fixed scratch is refused before anything is enqueued."""
import ctypes as C

import numpy as np
import pytest

import bench
from gpu_common import bits

pytestmark = pytest.mark.gpu

LARGE = dict(d=1024, f=2048, n_qkv=3072, v_off=2048, dv=1024, layers=3, eps=1e-5)
SMALL = dict(d=256, f=512, n_qkv=768, v_off=512, dv=256, layers=2, eps=1e-5)


@pytest.fixture(scope="module")
def q4():
    import int4_weight_only_q4_amd as m
    m.lib()
    return m


def _both(q4, torch, p):
    stack, st = bench.build_stack(q4, torch, p)
    d, n = p["d"], p["layers"]
    outs = []
    for fn in (q4.lib().q4_stack_decode_noalloc, q4.lib().q4_stack_decode):
        r_out = torch.empty(d, dtype=torch.float16, device="cuda")
        h_out = torch.empty(d, dtype=torch.float16, device="cuda")
        trace = torch.empty((n, 2, d), dtype=torch.float16, device="cuda")
        status = fn(C.byref(stack.desc), C.c_void_p(st["r0"].data_ptr()),
                    C.c_void_p(st["h0"].data_ptr()), C.c_void_p(r_out.data_ptr()),
                    C.c_void_p(h_out.data_ptr()), C.c_void_p(trace.data_ptr()),
                    C.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert status == q4.Q4_OK, q4.lib().q4_last_error().decode()
        outs.append((r_out, h_out, trace))
    torch.cuda.synchronize()
    return outs


def test_noalloc_equals_allocating_entry_point_two_calls(q4):
    import torch
    for p in (LARGE, SMALL):  # the second call on a smaller stack
        (r_a, h_a, t_a), (r_b, h_b, t_b) = _both(q4, torch, p)
        assert np.array_equal(bits(h_a), bits(h_b)), p
        assert np.array_equal(bits(r_a), bits(r_b)), p
        assert np.array_equal(bits(t_a), bits(t_b)), p
        assert np.all(np.isfinite(bits(h_a).view(np.float16).astype(np.float64)))
