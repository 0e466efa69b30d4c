"""GPU parity of the loss variants (per-token weights, hard-label cross-entropy
mixed with the teacher KL) against the oracle's forward_terms / backward_terms.
Tolerances as for the plain loss."""

import numpy as np
import pytest
import torch

import oracle
import output_projection_kl_amd as fkl
from workloads import make_workload

pytestmark = pytest.mark.gpu

LOSS_RTOL = 1e-3
GRAD_TOL = 2e-2


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _bits(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _rel(got, ref):
    s = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (s if s > 0 else 1.0))


def _case(wl, T, weights, labels, a, chunk, vslab, g=1.0):
    dev = _dev()
    h, W = _bits(wl.h_bits, dev), _bits(wl.W_bits, dev)
    ti, tl = torch.from_numpy(wl.t_idx).to(dev), torch.from_numpy(wl.t_logit).to(dev)
    m = None if wl.mask is None else torch.from_numpy(wl.mask).to(dev)
    rw = None if weights is None else torch.from_numpy(weights.astype(np.float32)).to(dev)
    lab = None if labels is None else torch.from_numpy(labels.astype(np.int32)).to(dev)
    kw = dict(T=T, mask=m, chunk=chunk, vslab=vslab, row_weight=rw, label=lab, label_weight=a)
    loss, lse, rl = fkl.forward(h, W, ti, tl, return_row_kl=True, **kw)
    gh, gW = fkl.backward(h, W, ti, tl, lse, grad_loss=torch.tensor([g], device=dev), **kw)
    torch.cuda.synchronize()
    w32 = None if weights is None else weights.astype(np.float32)
    r_loss, r_lse, r_rl = oracle.forward_terms(wl.h(), wl.W(), wl.t_idx, wl.t_logit, T, wl.mask, w32, labels, a)
    r_gh, r_gW = oracle.backward_terms(wl.h(), wl.W(), wl.t_idx, wl.t_logit, T, wl.mask, w32, labels, a,
                                       grad_loss=g)
    e_loss = abs(loss.item() - r_loss) / max(abs(r_loss), 1e-30)
    e_rl = float(np.abs(rl.cpu().numpy() - r_rl).max())
    e_gh, e_gW = _rel(gh.cpu().numpy(), r_gh), _rel(gW.cpu().numpy(), r_gW)
    print(f"[terms] N={wl.N} V={wl.V} T={T} a={a} weights={weights is not None} labels={labels is not None}: "
          f"loss {e_loss:.2e} row {e_rl:.2e} grad_h {e_gh:.2e} grad_W {e_gW:.2e}", flush=True)
    assert e_loss <= LOSS_RTOL
    assert e_rl <= 1e-3 * max(1.0, np.abs(r_rl).max())
    assert e_gh <= GRAD_TOL and e_gW <= GRAD_TOL
    return loss.item(), gh, gW


def _labels(wl, rng):
    """Half the labels are one of the row's teacher indices, half are random."""
    lab = rng.integers(0, wl.V, size=wl.N)
    pick = rng.random(wl.N) < 0.5
    lab[pick] = wl.t_idx[pick, rng.integers(0, wl.K, size=wl.N)[pick]]
    return lab


@pytest.mark.parametrize("T", [1.0, 2.0])
def test_weights_only(T):
    wl = make_workload("tiny", 0, mask="random25")
    w = np.random.default_rng(11).random(wl.N) * 2.0
    _case(wl, T, w, None, 0.0, chunk=64, vslab=1024)


@pytest.mark.parametrize("T,a", [(1.0, 0.3), (2.0, 0.6), (1.0, 1.0)])
def test_labels_mixed_with_teacher(T, a):
    wl = make_workload("tiny", 1)
    _case(wl, T, None, _labels(wl, np.random.default_rng(12)), a, chunk=64, vslab=1024, g=0.7)


def test_weights_and_labels_ragged():
    """Several chunks, slabs and grad_h splits, a mask, weights and labels at once."""
    wl = make_workload("tiny", N=300, d=136, V=5000, K=7, mask="random25")
    rng = np.random.default_rng(13)
    _case(wl, 0.7, rng.random(wl.N) * 3.0, _labels(wl, rng), 0.4, chunk=128, vslab=768, g=2.5)


@pytest.mark.parametrize("K", [129, 700])
def test_labels_with_long_teacher_lists(K):
    """Teacher lists longer than 128 entries take the sorted (bitonic) path of
    the list preparation; hard labels land inside and outside the lists."""
    wl = make_workload("tiny", 3, N=200, d=64, V=3000, K=K, mask="random25")
    rng = np.random.default_rng(14)
    _case(wl, 1.3, rng.random(wl.N) + 0.5, _labels(wl, rng), 0.35, chunk=64, vslab=768, g=0.9)


def test_zero_total_weight():
    wl = make_workload("tiny", 2)
    loss, gh, gW = _case(wl, 1.0, np.zeros(wl.N), None, 0.0, chunk=64, vslab=1024)
    assert loss == 0.0 and gh.abs().max().item() == 0.0 and gW.abs().max().item() == 0.0


def test_autograd_entry_with_terms():
    dev = _dev()
    wl = make_workload("tiny", 3)
    rng = np.random.default_rng(14)
    w = rng.random(wl.N).astype(np.float32)
    lab = _labels(wl, rng).astype(np.int32)
    h = _bits(wl.h_bits, dev).requires_grad_(True)
    W = _bits(wl.W_bits, dev).requires_grad_(True)
    ti, tl = torch.from_numpy(wl.t_idx).to(dev), torch.from_numpy(wl.t_logit).to(dev)
    loss = fkl.FusedKLLoss.apply(h, W, ti, tl, 1.5, None, 64, torch.from_numpy(w).to(dev),
                                 torch.from_numpy(lab).to(dev), 0.25)
    loss.backward()
    torch.cuda.synchronize()
    r_loss, _, _ = oracle.forward_terms(wl.h(), wl.W(), wl.t_idx, wl.t_logit, 1.5, None, w, lab, 0.25)
    r_gh, r_gW = oracle.backward_terms(wl.h(), wl.W(), wl.t_idx, wl.t_logit, 1.5, None, w, lab, 0.25)
    assert abs(loss.item() - r_loss) <= LOSS_RTOL * abs(r_loss)
    assert _rel(h.grad.float().cpu().numpy(), r_gh) <= GRAD_TOL
    assert _rel(W.grad.float().cpu().numpy(), r_gW) <= GRAD_TOL


def test_nonpositive_weights_take_no_part():
    """Rows with a zero, negative or NaN weight count in neither the weighted
    sum nor its normaliser (the rule of the oracle's forward_terms)."""
    wl = make_workload("tiny", 4, mask="random25")
    rng = np.random.default_rng(15)
    w = rng.random(wl.N) + 0.25
    w[[3, 40, 77]] = 0.0
    w[[5, 90, 200]] = -2.0
    w[[11, 150]] = np.nan
    loss, gh, gW = _case(wl, 1.0, w, None, 0.0, chunk=64, vslab=1024)
    dropped = ~(w > 0)
    assert gh[torch.from_numpy(dropped).to(gh.device)].abs().max().item() == 0.0


def test_bad_labels_and_weights_are_refused(monkeypatch):
    """fkl_validate_terms counts rows whose label lies outside [0, V) or whose
    weight is not finite; under FKL_VALIDATE=1 forward and backward refuse
    them with FKL_EINDEX (labels -1 and V, the values an ignore index or an
    off-by-one would leave)."""
    dev = _dev()
    wl = make_workload("tiny", 5, N=64, d=64, V=500, K=9)
    h, W = _bits(wl.h_bits, dev), _bits(wl.W_bits, dev)
    ti, tl = torch.from_numpy(wl.t_idx).to(dev), torch.from_numpy(wl.t_logit).to(dev)
    rng = np.random.default_rng(16)
    good_lab = _labels(wl, rng).astype(np.int32)
    good_w = (rng.random(wl.N) + 0.5).astype(np.float32)
    lab_t = torch.from_numpy(good_lab).to(dev)
    w_t = torch.from_numpy(good_w).to(dev)
    assert fkl.validate_terms(wl.N, wl.V, row_weight=w_t, label=lab_t, label_weight=0.3) == 0
    bad_lab = good_lab.copy()
    bad_lab[4] = -1
    bad_lab[9] = wl.V
    bad_w = good_w.copy()
    bad_w[9] = np.inf                  # same row as a bad label: counted once
    bad_w[20] = np.nan
    bl, bw = torch.from_numpy(bad_lab).to(dev), torch.from_numpy(bad_w).to(dev)
    assert fkl.validate_terms(wl.N, wl.V, label=bl, label_weight=0.3) == 2
    assert fkl.validate_terms(wl.N, wl.V, row_weight=bw) == 2
    assert fkl.validate_terms(wl.N, wl.V, row_weight=bw, label=bl, label_weight=0.3) == 3
    monkeypatch.setenv("FKL_VALIDATE", "1")
    loss, lse = fkl.forward(h, W, ti, tl, row_weight=w_t, label=lab_t, label_weight=0.3)
    torch.cuda.synchronize()
    for kw in (dict(label=bl, label_weight=0.3), dict(row_weight=bw)):
        with pytest.raises(fkl.FklError) as e:
            fkl.forward(h, W, ti, tl, **kw)
        assert e.value.status == 3 and "rows rejected" in str(e.value)
        with pytest.raises(fkl.FklError) as e:
            fkl.backward(h, W, ti, tl, lse, **kw)
        assert e.value.status == 3
