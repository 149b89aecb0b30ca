"""dsa_forward_noalloc (the static-scratch variant of dsa_forward, for
callers that cannot allocate) against dsa_forward on the same inputs: two
calls in a row, the second on a smaller problem, results identical bit for
bit (the same kernels over a different workspace)."""
import ctypes

import pytest
import torch

import dsa_top_token_amd as dsa
from dsa_top_token_amd import synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def run_both(w, seed):
    x = {k: v.cuda() for k, v in synth.make_inputs(w, seed=seed).items()}
    idx, O, lse = dsa.forward(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"], w.q_pos0, w.top_k)
    O2 = torch.full_like(O, 7.0)
    idx2 = torch.full_like(idx, -7)
    lse2 = torch.full_like(lse, 7.0)
    dsa.forward_noalloc(x["q_idx"], x["k_idx"], x["Q"], x["K"], x["V"], w.q_pos0, w.top_k, O2,
                        idx2, lse2)
    torch.cuda.synchronize()
    return (idx, O, lse), (idx2, O2, lse2)


def assert_same(a, b, what):
    assert torch.equal(a[0], b[0]), what
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16)), what
    assert torch.equal(a[2], b[2]), what


def test_noalloc_matches_forward_twice(gpu_lib):
    # the full 64 x 128K clustered decode batch (99 MiB of workspace), then a
    # smaller prefill through the same scratch, whose earlier contents must
    # not leak into the result
    big = synth.WORKLOADS["decode_128k_clustered"]
    small = synth.WORKLOADS["prefill_1k"].replace(n_q=700, n_k=700, top_k=48, n_heads=4)
    for w, seed in ((big, 0), (small, 3)):
        say("noalloc %s" % w.name)
        a, b = run_both(w, seed)
        assert_same(a, b, w.name)
    # a third call on the first shape again (scratch left by the prefill)
    w = big.replace(batch=8)
    say("noalloc %s batch 8" % w.name)
    a, b = run_both(w, 1)
    assert_same(a, b, "decode batch 8")


def test_noalloc_refuses_problems_beyond_its_scratch(gpu_lib):
    w = synth.WORKLOADS["prefill_64k"]
    p = dsa.make_problem(w.batch, w.n_q, w.n_k, 0, w.d_idx, w.idx_dtype, w.top_k, w.n_heads)
    assert dsa.workspace_size(p, dsa.OP_FORWARD) > (128 << 20)
    lib = dsa.load()
    dummy = torch.empty(256, dtype=torch.uint8, device="cuda")
    ptr = ctypes.c_void_p(dummy.data_ptr())
    rc = lib.dsa_forward_noalloc(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, None, ptr, None,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == -5  # DSA_E_WORKSPACE, nothing enqueued
    assert b"static scratch" in lib.dsa_last_error()
