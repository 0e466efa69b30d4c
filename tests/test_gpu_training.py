"""Training-loop integration of the fused loss (GPU): gradient accumulation
across micro-batches, skipped gradients, bf16 grad_h, and the autograd entry.

Pins: accumulate(a, b) equals a + b against the oracle's two batches; a
skipped gradient leaves its buffer untouched; bf16 grad_h equals the fp32
grad_h of the same call rounded to nearest even (same accumulation order);
autograd's gradients equal the library's for the same upstream gradient and
match the oracle within the parity tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
import output_projection_kl_amd as fkl
from workloads import make_workload

pytestmark = pytest.mark.gpu

GRAD_TOL = 2e-2


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _bits(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _upload(wl, dev):
    m = None if wl.mask is None else torch.from_numpy(wl.mask).to(dev)
    return (_bits(wl.h_bits, dev), _bits(wl.W_bits, dev), torch.from_numpy(wl.t_idx).to(dev),
            torch.from_numpy(wl.t_logit).to(dev), m)


def _rel(got, ref):
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def _ragged(seed, N=300):
    return make_workload("tiny", seed, N=N, d=136, V=5000, K=7, T=0.7, chunk=128, mask="random25")


def test_accumulate_two_micro_batches():
    """Two micro-batches through the same head: the second call accumulates."""
    dev = _dev()
    a, b = _ragged(0), _ragged(1)          # b contributes its rows and teacher; the head is a's
    ha, W, tia, tla, ma = _upload(a, dev)
    hb, _, tib, tlb, mb = _upload(b, dev)
    kw = dict(T=a.T, chunk=a.chunk, vslab=768)
    _, lse_a = fkl.forward(ha, W, tia, tla, mask=ma, **kw)
    _, lse_b = fkl.forward(hb, W, tib, tlb, mask=mb, **kw)
    gh, gW = fkl.backward(ha, W, tia, tla, lse_a, mask=ma, **kw)
    gh, gW = fkl.backward(hb, W, tib, tlb, lse_b, mask=mb, grad_h=gh, grad_W=gW,
                          accumulate_grad_h=True, accumulate_grad_W=True, **kw)
    torch.cuda.synchronize()
    ra_h, ra_W = oracle.backward(a.h(), a.W(), a.t_idx, a.t_logit, a.T, a.mask)
    rb_h, rb_W = oracle.backward(b.h(), a.W(), b.t_idx, b.t_logit, b.T, b.mask)
    e_W = _rel(gW.cpu().numpy(), ra_W + rb_W)
    e_h = _rel(gh.cpu().numpy(), ra_h + rb_h)
    print(f"[train] accumulate: grad_W {e_W:.2e} grad_h {e_h:.2e}", flush=True)
    assert e_W <= GRAD_TOL and e_h <= GRAD_TOL


def test_accumulate_is_a_plus_b():
    """Same inputs twice: accumulating equals adding the two results, up to the
    fp32 summation order (the old value enters before the per-chunk and
    per-slab terms instead of after their sum)."""
    dev = _dev()
    wl = _ragged(2)
    h, W, ti, tl, m = _upload(wl, dev)
    kw = dict(T=wl.T, mask=m, chunk=wl.chunk, vslab=768)
    _, lse = fkl.forward(h, W, ti, tl, **kw)
    gh1, gW1 = fkl.backward(h, W, ti, tl, lse, **kw)
    gh2, gW2 = fkl.backward(h, W, ti, tl, lse, grad_h=gh1.clone(), grad_W=gW1.clone(),
                            accumulate_grad_h=True, accumulate_grad_W=True, **kw)
    torch.cuda.synchronize()
    for got, one in ((gW2, gW1), (gh2, gh1)):
        err = (got - 2 * one).abs().max().item()
        assert err <= 1e-5 * one.abs().max().item(), err


def test_skipped_gradients_are_untouched():
    dev = _dev()
    wl = _ragged(3)
    h, W, ti, tl, m = _upload(wl, dev)
    kw = dict(T=wl.T, mask=m, chunk=wl.chunk, vslab=768)
    _, lse = fkl.forward(h, W, ti, tl, **kw)
    gh_ref, gW_ref = fkl.backward(h, W, ti, tl, lse, **kw)
    gh, gW_none = fkl.backward(h, W, ti, tl, lse, need_grad_W=False, **kw)
    gh_none, gW = fkl.backward(h, W, ti, tl, lse, need_grad_h=False, **kw)
    # a poisoned buffer stays as it was when its gradient is skipped
    poison = torch.full((wl.V, wl.d), float("nan"), device=dev)
    s = fkl.make_shape(wl.N, wl.d, wl.V, wl.K, wl.T, wl.chunk, 768, fkl.SKIP_GRAD_W)
    _, bb = fkl.workspace_size(wl.N, wl.d, wl.V, wl.K, wl.T, wl.chunk, 768, fkl.SKIP_GRAD_W)
    ws = torch.empty(bb, dtype=torch.uint8, device=dev)
    gh3 = torch.empty((wl.N, wl.d), dtype=torch.float32, device=dev)
    import ctypes
    rc = fkl.lib().fkl_backward(ctypes.byref(s), h.data_ptr(), W.data_ptr(), ti.data_ptr(), tl.data_ptr(),
                                m.data_ptr(), None, lse.data_ptr(), None, gh3.data_ptr(), poison.data_ptr(),
                                ws.data_ptr(), ctypes.c_size_t(bb), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    assert gW_none is None and gh_none is None
    assert torch.equal(gh, gh_ref) and torch.equal(gW, gW_ref) and torch.equal(gh3, gh_ref)
    assert torch.isnan(poison).all()


@pytest.mark.parametrize("accumulate", [False, True])
def test_bf16_grad_h_is_the_rounded_fp32_result(accumulate):
    dev = _dev()
    wl = _ragged(4)
    h, W, ti, tl, m = _upload(wl, dev)
    kw = dict(T=wl.T, mask=m, chunk=wl.chunk, vslab=768)
    _, lse = fkl.forward(h, W, ti, tl, **kw)
    gh32, _ = fkl.backward(h, W, ti, tl, lse, need_grad_W=False, **kw)
    old = (torch.randn((wl.N, wl.d), device=dev) * 1e-3).to(torch.bfloat16)
    gh16, _ = fkl.backward(h, W, ti, tl, lse, need_grad_W=False, grad_h=old.clone() if accumulate else None,
                           accumulate_grad_h=accumulate, grad_h_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    want = (old.float() + gh32).to(torch.bfloat16) if accumulate else gh32.to(torch.bfloat16)
    assert gh16.dtype == torch.bfloat16
    assert torch.equal(gh16, want)


def test_autograd_entry_matches_library_and_oracle():
    dev = _dev()
    wl = _ragged(5)
    h, W, ti, tl, m = _upload(wl, dev)
    x = torch.randn((wl.N, 24), device=dev)
    A = (torch.randn((24, wl.d), device=dev) / 5).requires_grad_(True)
    # h = x A (a preceding layer in fp32, rounded to bf16), so the gradient must flow through it
    hh = (x @ A).to(torch.bfloat16)
    hh.retain_grad()
    Wp = W.clone().requires_grad_(True)
    loss = fkl.FusedKLLoss.apply(hh, Wp, ti, tl, wl.T, m, wl.chunk)
    (0.7 * loss).backward()
    torch.cuda.synchronize()
    assert hh.grad.dtype == torch.bfloat16 and Wp.grad.dtype == torch.bfloat16
    _, lse = fkl.forward(hh.detach(), W, ti, tl, T=wl.T, mask=m, chunk=wl.chunk)
    g = torch.tensor([0.7], device=dev)
    gh_lib, gW_lib = fkl.backward(hh.detach(), W, ti, tl, lse, T=wl.T, mask=m, grad_loss=g, chunk=wl.chunk,
                                  grad_h_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(hh.grad, gh_lib)
    assert torch.equal(Wp.grad, gW_lib.to(torch.bfloat16))
    assert torch.allclose(A.grad, x.t() @ gh_lib.float(), rtol=1e-4, atol=1e-6)
    hb = hh.detach().float().cpu().numpy()
    r_gh, r_gW = oracle.backward(hb, wl.W(), wl.t_idx, wl.t_logit, wl.T, wl.mask, grad_loss=0.7)
    assert _rel(hh.grad.float().cpu().numpy(), r_gh) <= GRAD_TOL
    assert _rel(gW_lib.cpu().numpy(), r_gW) <= GRAD_TOL
    # a frozen head: no grad_W requested, none produced
    hh2 = hh.detach().clone().requires_grad_(True)
    fkl.FusedKLLoss.apply(hh2, W, ti, tl, wl.T, m, wl.chunk).backward()
    torch.cuda.synchronize()
    assert hh2.grad is not None and W.grad is None


def test_drop_in_training_steps_track_a_dense_reference():
    """The fused loss as a drop-in KL term: five SGD steps of a small student
    (a linear layer in fp32 feeding h, and an fp32 master copy of the head,
    both cast to bf16 for the loss) follow the same steps taken with a dense
    fp32 torch KL of the same bf16 values. Losses agree to 1e-3 and the
    parameter updates to 3e-2 of their size."""
    dev = _dev()
    wl = make_workload("tiny", 11, N=128, d=64, V=2000, K=8, T=1.5)
    ti = torch.from_numpy(wl.t_idx).to(dev)
    tl = torch.from_numpy(wl.t_logit).to(dev)
    g = torch.Generator(device="cpu").manual_seed(3)
    x = torch.randn((wl.N, 24), generator=g).to(dev)
    A0 = (torch.randn((24, wl.d), generator=g) / 5).to(dev)
    W0 = torch.from_numpy(wl.W()).to(dev)
    p_dense = torch.zeros((wl.N, wl.V), device=dev)
    p_dense.scatter_(1, ti.long(), torch.softmax(tl / wl.T, dim=1))

    def dense_kl(h, Wb):
        logq = torch.log_softmax(h.float() @ Wb.float().t() / wl.T, dim=1)
        logp = torch.where(p_dense > 0, p_dense.clamp_min(1e-30).log(), torch.zeros_like(p_dense))
        return wl.T ** 2 * (p_dense * (logp - logq)).sum(dim=1).mean()

    def run(fused):
        A = A0.clone().requires_grad_(True)
        W = W0.clone().requires_grad_(True)
        losses = []
        for _ in range(5):
            h = (x @ A).to(torch.bfloat16)
            Wb = W.to(torch.bfloat16)
            loss = fkl.FusedKLLoss.apply(h, Wb, ti, tl, wl.T) if fused else dense_kl(h, Wb)
            loss.backward()
            with torch.no_grad():
                A -= 0.5 * A.grad
                W -= 0.5 * W.grad
                A.grad = None
                W.grad = None
            losses.append(float(loss.detach()))
        return losses, A.detach(), W.detach()

    l_f, A_f, W_f = run(True)
    l_r, A_r, W_r = run(False)
    torch.cuda.synchronize()
    print(f"   losses fused {[round(v, 5) for v in l_f]} dense {[round(v, 5) for v in l_r]}", flush=True)
    for a, b in zip(l_f, l_r):
        assert abs(a - b) <= 1e-3 * abs(b)
    assert l_f[-1] < l_f[0]
    for got, ref, start in ((A_f, A_r, A0), (W_f, W_r, W0)):
        step = (ref - start).abs().max().item()
        assert step > 0
        assert (got - ref).abs().max().item() <= 3e-2 * step
