"""The allocation-free forward (fkl_forward_static, through the C ABI)
against the existing entry point fkl_forward with a caller workspace: the
same kernels on the same plan, so the loss, row_lse and row_kl must agree
bit for bit, and both must match the fp64 oracle to the parity bar (loss
1e-3 relative, row_lse 1e-3 absolute, row KL 1e-3 relative). Two static calls
in a row, the second on a smaller input, then the headline shape."""

import numpy as np
import pytest
import torch

import oracle
import output_projection_kl_amd as fkl
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _upload(wl, dev):
    h = torch.from_numpy(np.ascontiguousarray(wl.h_bits).view(np.int16)).to(dev).view(torch.bfloat16)
    W = torch.from_numpy(np.ascontiguousarray(wl.W_bits).view(np.int16)).to(dev).view(torch.bfloat16)
    ti = torch.from_numpy(wl.t_idx).to(dev)
    tl = torch.from_numpy(wl.t_logit).to(dev)
    m = torch.from_numpy(wl.mask).to(dev) if wl.mask is not None else None
    return h, W, ti, tl, m


def _outputs(N, dev):
    return (torch.full((1,), float("nan"), device=dev), torch.full((N,), float("nan"), device=dev),
            torch.full((N,), float("nan"), device=dev))


def test_static_forward_matches_workspace_forward_twice_then_smaller():
    dev = _dev()
    big = make_workload("tiny", 3, N=2000, d=256, V=9000, K=16, mask="random25")
    small = make_workload("tiny", 4, N=300, d=136, V=5000, K=7)
    runs = []
    for wl, T in ((big, 1.0), (small, 0.7)):
        print(f"[no-alloc] static forward N={wl.N} d={wl.d} V={wl.V} K={wl.K} T={T}", flush=True)
        h, W, ti, tl, m = _upload(wl, dev)
        loss_s, lse_s, kl_s = _outputs(wl.N, dev)
        fkl.forward_static(h, W, ti, tl, T=T, mask=m, chunk=256, loss=loss_s, row_lse=lse_s, row_kl=kl_s)
        runs.append((wl, T, h, W, ti, tl, m, loss_s, lse_s, kl_s))
    torch.cuda.synchronize()
    for wl, T, h, W, ti, tl, m, loss_s, lse_s, kl_s in runs:
        loss_w, lse_w, kl_w = fkl.forward(h, W, ti, tl, T=T, mask=m, chunk=256, return_row_kl=True)
        torch.cuda.synchronize()
        assert torch.equal(loss_s, loss_w) and torch.equal(lse_s, lse_w) and torch.equal(kl_s, kl_w)
        r_loss, r_lse, r_kl = oracle.forward(wl.h(), wl.W(), wl.t_idx, wl.t_logit, T, wl.mask)
        e_loss = abs(loss_s.item() - r_loss) / abs(r_loss)
        e_lse = float(np.abs(lse_s.cpu().numpy() - r_lse).max())
        e_kl = float(np.abs(kl_s.cpu().numpy() - r_kl).max() / max(1.0, np.abs(r_kl).max()))
        print(f"   N={wl.N}: loss rel {e_loss:.2e} lse {e_lse:.2e} kl {e_kl:.2e}", flush=True)
        assert e_loss <= 1e-3 and e_lse <= 1e-3 and e_kl <= 1e-3


def test_static_forward_at_the_headline_shape():
    """N=32768, d=2880, V=201088, K=100 in the bench's launch configuration
    (16384-row forward passes, 15.2 MiB of scratch): bit for bit the workspace
    forward."""
    from workloads.device import make_device_workload
    dev = _dev()
    wl = make_device_workload("gptoss20b", dev)
    print(f"[no-alloc] headline {wl.describe()}", flush=True)
    loss_s, lse_s, kl_s = _outputs(wl.N, dev)
    fkl.forward_static(wl.h, wl.W, wl.t_idx, wl.t_logit, T=wl.T, chunk=wl.chunk, loss=loss_s, row_lse=lse_s,
                       row_kl=kl_s)
    loss_w, lse_w, kl_w = fkl.forward(wl.h, wl.W, wl.t_idx, wl.t_logit, T=wl.T, chunk=wl.chunk, return_row_kl=True)
    torch.cuda.synchronize()
    assert torch.equal(loss_s, loss_w) and torch.equal(lse_s, lse_w) and torch.equal(kl_s, kl_w)
    assert torch.isfinite(lse_s).all().item()


def test_static_forward_falls_back_to_shorter_passes():
    """K = 300 over 16384 rows: the default 16384-row forward pass needs more
    than the 32 MiB scratch for its teacher lists, so the static forward takes
    8192-row passes. It must equal fkl_forward run with 8192-row passes (an
    explicit slab keeps the caller's chunk) bit for bit, and the oracle to the
    parity bar."""
    dev = _dev()
    wl = make_workload("tiny", 5, N=16384, d=64, V=5000, K=300, mask="random25")
    fb, _ = fkl.workspace_size(wl.N, wl.d, wl.V, wl.K, 1.0)
    assert fb > fkl.STATIC_SCRATCH_BYTES
    print(f"[no-alloc] fallback N={wl.N} K={wl.K}: default forward workspace {fb} bytes", flush=True)
    h, W, ti, tl, m = _upload(wl, dev)
    loss_s, lse_s, kl_s = _outputs(wl.N, dev)
    fkl.forward_static(h, W, ti, tl, T=1.0, mask=m, loss=loss_s, row_lse=lse_s, row_kl=kl_s)
    loss_w, lse_w, kl_w = fkl.forward(h, W, ti, tl, T=1.0, mask=m, chunk=8192, vslab=1024, return_row_kl=True)
    torch.cuda.synchronize()
    assert torch.equal(loss_s, loss_w) and torch.equal(lse_s, lse_w) and torch.equal(kl_s, kl_w)
    r_loss, r_lse, r_kl = oracle.forward(wl.h(), wl.W(), wl.t_idx, wl.t_logit, 1.0, wl.mask)
    assert abs(loss_s.item() - r_loss) <= 1e-3 * abs(r_loss)
    assert float(np.abs(lse_s.cpu().numpy() - r_lse).max()) <= 1e-3
    assert float(np.abs(kl_s.cpu().numpy() - r_kl).max()) <= 1e-3 * max(1.0, float(np.abs(r_kl).max()))
