"""The fused loss inside a captured HIP graph (torch.cuda.graph): every launch
of fkl_forward / fkl_backward is a kernel on the caller's stream, with no
allocation, memset or host synchronisation, so a training step can capture
it. Each replay, with eager library work and synchronisations in between,
must reproduce the eager result bit for bit (the path is deterministic)."""

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


def _bits(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def test_forward_backward_replay_in_a_graph():
    dev = _dev()
    wl = make_workload("tiny", N=300, d=136, V=5000, K=7, mask="random25")
    h, W = _bits(wl.h_bits, dev), _bits(wl.W_bits, dev)
    ti, tl = torch.from_numpy(wl.t_idx).to(dev), torch.from_numpy(wl.t_logit).to(dev)
    m = torch.from_numpy(wl.mask).to(dev)
    kw = dict(T=0.8, mask=m, chunk=128, vslab=768)
    fb, bb = fkl.workspace_size(wl.N, wl.d, wl.V, wl.K, 0.8, chunk=128, vslab=768)
    ws = torch.empty(max(fb, bb), dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(wl.N, dtype=torch.float32, device=dev)
    gh = torch.empty((wl.N, wl.d), dtype=torch.float32, device=dev)
    gW = torch.empty((wl.V, wl.d), dtype=torch.float32, device=dev)
    gl = torch.tensor([1.7], device=dev)

    def step():
        fkl.forward(h, W, ti, tl, workspace=ws, loss=loss, row_lse=lse, **kw)
        fkl.backward(h, W, ti, tl, lse, grad_loss=gl, workspace=ws, grad_h=gh, grad_W=gW, **kw)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = (loss.clone(), lse.clone(), gh.clone(), gW.clone())

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    other = make_workload("tiny", 1, N=300, d=136, V=5000, K=7)
    h2, ti2, tl2 = _bits(other.h_bits, dev), torch.from_numpy(other.t_idx).to(dev), torch.from_numpy(other.t_logit).to(dev)
    for rep in range(3):
        for t in (loss, lse, gh, gW):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        for got, want in zip((loss, lse, gh, gW), ref):
            assert torch.equal(got, want)
        # eager library work between replays, on other inputs and its own buffers
        l2, lse2 = fkl.forward(h2, W, ti2, tl2, T=0.8, chunk=128)
        fkl.backward(h2, W, ti2, tl2, lse2, T=0.8, chunk=128)
        torch.cuda.synchronize()


def test_static_forward_and_builder_replay_in_a_graph():
    """fkl_forward_static (no workspace argument, its scratch is the library's
    static array) and the teacher-cache builder (fused route, whose guarded
    redo kernels test a device flag) captured together and replayed: every
    replay reproduces the eager outputs, with eager builder and static-forward
    calls on other inputs in between (they share the static scratch and must
    not leave anything a replay depends on)."""
    dev = _dev()
    wl = make_workload("tiny", N=300, d=136, V=5000, K=7, mask="random25")
    h, W = _bits(wl.h_bits, dev), _bits(wl.W_bits, dev)
    ti, tl = torch.from_numpy(wl.t_idx).to(dev), torch.from_numpy(wl.t_logit).to(dev)
    m = torch.from_numpy(wl.mask).to(dev)
    K = 50
    tb = fkl.topk_workspace_size(wl.N, wl.d, wl.V, K)
    tws = torch.empty(tb, dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(wl.N, dtype=torch.float32, device=dev)
    ci = torch.empty((wl.N, K), dtype=torch.int32, device=dev)
    cl = torch.empty((wl.N, K), dtype=torch.float32, device=dev)

    def step():
        fkl.forward_static(h, W, ti, tl, T=0.8, mask=m, chunk=128, loss=loss, row_lse=lse)
        fkl.topk(h, W, K, workspace=tws, t_idx=ci, t_logit=cl)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = (loss.clone(), lse.clone(), ci.clone(), cl.clone())

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    other = make_workload("tiny", 2, N=280, d=136, V=5000, K=7)
    h2, ti2, tl2 = _bits(other.h_bits, dev), torch.from_numpy(other.t_idx).to(dev), torch.from_numpy(other.t_logit).to(dev)
    for rep in range(3):
        for t in (loss, lse, cl):
            t.fill_(float("nan"))
        ci.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph-static-builder] replay {rep}", flush=True)
        for got, want in zip((loss, lse, ci, cl), ref):
            assert torch.equal(got, want)
        fkl.forward_static(h2, W, ti2, tl2, T=1.1, chunk=64)
        fkl.topk(h2, W, 9)
        torch.cuda.synchronize()
