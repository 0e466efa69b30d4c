"""Calls in flight on two streams at once. Every entry point enqueues its
work on the caller's stream (torch's current stream here), keeps no state
between calls and touches nothing outside its arguments and workspace, so
two independent problems run concurrently on two streams, each with its own
workspace, must give bitwise the results they give one after the other on
one stream: the loss, row_lse, row_kl, both gradients and a teacher cache."""

import numpy as np
import pytest
import torch

import output_projection_kl_amd as fkl
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _upload(wl, dev):
    def bits(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)

    m = torch.from_numpy(wl.mask).to(dev) if wl.mask is not None else None
    return bits(wl.h_bits), bits(wl.W_bits), torch.from_numpy(wl.t_idx).to(dev), torch.from_numpy(wl.t_logit).to(dev), m


def _run(x, T):
    h, W, ti, tl, m = x
    loss, lse, kl = fkl.forward(h, W, ti, tl, T=T, mask=m, chunk=256, return_row_kl=True)
    gh, gW = fkl.backward(h, W, ti, tl, lse, T=T, mask=m, chunk=256)
    ci, cl = fkl.topk(h, W, 20)
    return [loss, lse, kl, gh, gW, ci, cl]


def test_two_streams_match_one_stream():
    dev = _dev()
    a = _upload(make_workload("tiny", seed_offset=1, N=700, d=136, V=5000, K=7, mask="random25"), dev)
    b = _upload(make_workload("tiny", seed_offset=2, N=520, d=64, V=3000, K=100), dev)
    print("[streams] sequential on one stream", flush=True)
    ref_a, ref_b = _run(a, 0.8), _run(b, 1.5)
    torch.cuda.synchronize()
    ref = [t.cpu() for t in ref_a + ref_b]
    cur = torch.cuda.current_stream()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(cur)
    s2.wait_stream(cur)
    print("[streams] concurrent on two streams", flush=True)
    for _ in range(3):
        with torch.cuda.stream(s1):
            out_a = _run(a, 0.8)
        with torch.cuda.stream(s2):
            out_b = _run(b, 1.5)
        cur.wait_stream(s1)
        cur.wait_stream(s2)
        torch.cuda.synchronize()
        for r, o in zip(ref, out_a + out_b):
            assert torch.equal(r, o.cpu())
