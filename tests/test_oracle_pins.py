"""Pins of the fp64 oracle against things other than itself.

Each test fixes the oracle to an independent fact: a hand-derived closed
form, a library routine that shares no code with the sparse formula (torch's
dense kl_div / cross_entropy / autograd, scipy's rel_entr), finite
differences, or an identity of the mathematics. They are chosen so that a
dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them (see test_pins_catch_planted_mistakes).
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import fkl_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(seed, N=6, d=8, V=32, K=5, scale_h=1.0, mask_frac=0.0):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, d)) * scale_h
    W = rng.standard_normal((V, d)) / np.sqrt(d) * 2.0
    t_idx = np.stack([rng.choice(V, K, replace=False) for _ in range(N)]).astype(np.int32)
    t_logit = np.sort(rng.standard_normal((N, K)) * 3.0, axis=1)[:, ::-1].copy()
    mask = None
    if mask_frac > 0:
        mask = (rng.random(N) >= mask_frac).astype(np.uint8)
        mask[0] = 1
    return h, W, t_idx, t_logit, mask


def _torch_dense_loss(h, W, t_idx, t_logit, T, mask):
    """Dense KL through torch's own kl_div on a rebuilt [N, V] teacher grid."""
    ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    N, V = h.shape[0], W.shape[0]
    a = torch.tensor(np.asarray(t_logit, dtype=np.float64)) / T
    p = torch.softmax(a, dim=1)
    grid = torch.zeros(N, V, dtype=torch.float64)
    grid.scatter_(1, torch.tensor(np.asarray(t_idx, dtype=np.int64)), p)
    logq = torch.log_softmax((ht @ Wt.T) / T, dim=1)
    kl_rows = torch.nn.functional.kl_div(logq, grid, reduction="none").sum(dim=1)
    m = torch.ones(N, dtype=torch.float64) if mask is None else torch.tensor(mask, dtype=torch.float64)
    n = m.sum()
    loss = (T * T) * (kl_rows * m).sum() / n
    loss.backward()
    return loss.item(), kl_rows.detach().numpy(), ht.grad.numpy(), Wt.grad.numpy(), logq


# ---------------------------------------------------------------------------
# Closed-form worked example (tests/golden/worked_example_v3.json)
# ---------------------------------------------------------------------------

def _ev(expr):
    return float(eval(expr, {"__builtins__": {}}, {k: getattr(math, k) for k in ("log", "sqrt", "exp")}))


def test_worked_example_closed_form():
    with open(os.path.join(GOLDEN, "worked_example_v3.json")) as f:
        g = json.load(f)
    inp = g["inputs"]
    h = np.array(inp["h"], dtype=np.float64)
    W = np.array([[_ev(e)] for e in inp["W"]])
    t_idx = np.array(inp["t_idx"], dtype=np.int32)
    t_logit = np.array([[_ev(e) for e in inp["t_logit"]], inp["t_logit_row1"]], dtype=np.float64)
    mask = np.array(inp["mask"], dtype=np.uint8)
    for case in g["cases"]:
        T = case["T"]
        loss, lse, kl = oracle.forward(h, W, t_idx, t_logit, T, mask)
        gh, gW = oracle.backward(h, W, t_idx, t_logit, T, mask)
        assert loss == pytest.approx(_ev(case["loss"]), rel=1e-13, abs=1e-15)
        assert lse[0] == pytest.approx(_ev(case["row_lse0"]), rel=1e-14)
        assert kl[1] == 0.0
        assert gh[0, 0] == pytest.approx(_ev(case["grad_h0"]), rel=1e-12, abs=1e-15)
        assert gh[1, 0] == 0.0
        np.testing.assert_allclose(gW[:, 0], [_ev(e) for e in case["grad_W"]], rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# P1: brute force on a tiny vocabulary vs torch dense kl_div + autograd, scipy
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1.0, 2.0, 0.7])
@pytest.mark.parametrize("mask_frac", [0.0, 0.4])
def test_p1_dense_bruteforce(T, mask_frac):
    h, W, t_idx, t_logit, mask = _rand_problem(11, mask_frac=mask_frac)
    loss_t, kl_t, gh_t, gW_t, logq = _torch_dense_loss(h, W, t_idx, t_logit, T, mask)
    loss, lse, kl = oracle.forward(h, W, t_idx, t_logit, T, mask)
    gh, gW = oracle.backward(h, W, t_idx, t_logit, T, mask)
    valid = np.ones(len(h), bool) if mask is None else mask.astype(bool)
    assert loss == pytest.approx(loss_t, rel=1e-12)
    np.testing.assert_allclose(kl[valid], kl_t[valid], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(gh, gh_t, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(gW, gW_t, rtol=1e-10, atol=1e-14)
    # scipy's rel_entr on the dense grids: sum_v p~ log(p~/q)
    grid = oracle.dense_teacher_grid(t_idx, t_logit, T, W.shape[0])
    q = np.exp(logq.detach().numpy())
    kl_s = scipy.special.rel_entr(grid, q).sum(axis=1)
    np.testing.assert_allclose(kl[valid], kl_s[valid], rtol=1e-11, atol=1e-14)


# ---------------------------------------------------------------------------
# P2: central finite differences of the oracle loss
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1.0, 2.0])
def test_p2_finite_differences(T):
    h, W, t_idx, t_logit, mask = _rand_problem(5, N=8, d=16, V=64, K=8, mask_frac=0.3)
    g = 1.7
    gh, gW = oracle.backward(h, W, t_idx, t_logit, T, mask, grad_loss=g)
    rng = np.random.default_rng(3)
    eps = 1e-5
    for _ in range(12):
        i, j = rng.integers(0, h.shape[0]), rng.integers(0, h.shape[1])
        hp, hm = h.copy(), h.copy()
        hp[i, j] += eps
        hm[i, j] -= eps
        fd = (oracle.forward(hp, W, t_idx, t_logit, T, mask)[0]
              - oracle.forward(hm, W, t_idx, t_logit, T, mask)[0]) / (2 * eps)
        assert g * fd == pytest.approx(gh[i, j], abs=1e-8 * max(1.0, np.abs(gh).max()))
    for _ in range(12):
        i, j = rng.integers(0, W.shape[0]), rng.integers(0, W.shape[1])
        Wp, Wm = W.copy(), W.copy()
        Wp[i, j] += eps
        Wm[i, j] -= eps
        fd = (oracle.forward(h, Wp, t_idx, t_logit, T, mask)[0]
              - oracle.forward(h, Wm, t_idx, t_logit, T, mask)[0]) / (2 * eps)
        assert g * fd == pytest.approx(gW[i, j], abs=1e-8 * max(1.0, np.abs(gW).max()))


# ---------------------------------------------------------------------------
# P3: Gibbs' inequality
# ---------------------------------------------------------------------------

def test_p3_kl_nonnegative():
    for seed in range(5):
        h, W, t_idx, t_logit, mask = _rand_problem(100 + seed, N=16, V=48, K=7, scale_h=3.0)
        loss, _, kl = oracle.forward(h, W, t_idx, t_logit, 1.3)
        assert np.all(kl >= -1e-12)
        assert loss >= -1e-12


# ---------------------------------------------------------------------------
# P4: self-distillation closed form; K = V gives exactly zero
# ---------------------------------------------------------------------------

def test_p4_self_distillation_closed_form():
    h, W, t_idx, _, _ = _rand_problem(21, N=10, d=8, V=40, K=6)
    T = 1.5
    z = h @ W.T
    t_logit = np.take_along_axis(z, t_idx.astype(np.int64), axis=1)  # student's own logits
    _, lse, kl = oracle.forward(h, W, t_idx, t_logit, T)
    s = z / T
    lse_v = scipy.special.logsumexp(s, axis=1)
    lse_k = scipy.special.logsumexp(np.take_along_axis(s, t_idx.astype(np.int64), axis=1), axis=1)
    np.testing.assert_allclose(kl, lse_v - lse_k, rtol=1e-11, atol=1e-13)  # = -log(student mass on idx)
    np.testing.assert_allclose(lse, lse_v, rtol=1e-14)


def test_p4_full_support_is_exactly_zero():
    h, W, _, _, _ = _rand_problem(22, N=5, d=6, V=12, K=1)
    rng = np.random.default_rng(0)
    t_idx = np.stack([rng.permutation(12) for _ in range(5)]).astype(np.int32)
    t_logit = np.take_along_axis(h @ W.T, t_idx.astype(np.int64), axis=1)
    loss, _, kl = oracle.forward(h, W, t_idx, t_logit, 1.0)
    gh, gW = oracle.backward(h, W, t_idx, t_logit, 1.0)
    assert abs(loss) < 1e-14 and np.abs(kl).max() < 1e-14
    assert np.abs(gh).max() < 1e-14 and np.abs(gW).max() < 1e-14


def test_p4_large_margin_student_reproduces_teacher():
    """Student mass concentrated on the teacher's indices: KL ~ 0."""
    rng = np.random.default_rng(7)
    N, d, V, K = 8, 64, 512, 4
    W = rng.standard_normal((V, d)) / np.sqrt(d)
    t_idx = np.stack([rng.choice(V, K, replace=False) for _ in range(N)]).astype(np.int32)
    tgt = rng.standard_normal((N, K)) + 400.0
    h = np.stack([np.linalg.lstsq(W[t_idx[r]], tgt[r], rcond=None)[0] for r in range(N)])
    t_logit = np.take_along_axis(h @ W.T, t_idx.astype(np.int64), axis=1)
    loss, _, _ = oracle.forward(h, W, t_idx, t_logit, 1.0)
    assert 0.0 <= loss < 1e-6


# ---------------------------------------------------------------------------
# P5: K = 1 is cross-entropy; P6: K = V is the textbook full KL
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1.0, 3.0])
def test_p5_single_index_is_cross_entropy(T):
    h, W, t_idx, t_logit, _ = _rand_problem(31, N=12, d=8, V=50, K=1)
    loss, _, _ = oracle.forward(h, W, t_idx, t_logit, T)
    ce = torch.nn.functional.cross_entropy(torch.tensor(h @ W.T / T), torch.tensor(t_idx[:, 0], dtype=torch.int64))
    assert loss == pytest.approx(T * T * ce.item(), rel=1e-12)


def test_p6_full_vocabulary_is_textbook_kl():
    rng = np.random.default_rng(41)
    N, d, V = 7, 5, 9
    h = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d))
    teacher_full = rng.standard_normal((N, V)) * 2
    t_idx = np.stack([rng.permutation(V) for _ in range(N)]).astype(np.int32)
    t_logit = np.take_along_axis(teacher_full, t_idx.astype(np.int64), axis=1)
    T = 1.7
    loss, _, _ = oracle.forward(h, W, t_idx, t_logit, T)
    ref = torch.nn.functional.kl_div(torch.log_softmax(torch.tensor(h @ W.T) / T, 1),
                                     torch.softmax(torch.tensor(teacher_full) / T, 1), reduction="batchmean")
    assert loss == pytest.approx(T * T * ref.item(), rel=1e-12)


# ---------------------------------------------------------------------------
# P7: invariance to the chunk size
# ---------------------------------------------------------------------------

def test_p7_chunk_invariance():
    h, W, t_idx, t_logit, mask = _rand_problem(51, N=64, d=12, V=80, K=9, mask_frac=0.25)
    ref = None
    for chunk in (1, 3, 64, 0):
        loss, lse, kl = oracle.forward(h, W, t_idx, t_logit, 1.2, mask, chunk=chunk)
        gh, gW = oracle.backward(h, W, t_idx, t_logit, 1.2, mask, chunk=chunk)
        if ref is None:
            ref = (loss, lse, gh, gW)
            continue
        assert loss == pytest.approx(ref[0], rel=1e-12)
        np.testing.assert_allclose(lse, ref[1], rtol=1e-13)
        np.testing.assert_allclose(gh, ref[2], rtol=1e-11, atol=1e-15)
        np.testing.assert_allclose(gW, ref[3], rtol=1e-11, atol=1e-15)


# ---------------------------------------------------------------------------
# P8: temperature identity
# ---------------------------------------------------------------------------

def test_p8_temperature_identity():
    h, W, t_idx, t_logit, mask = _rand_problem(61, N=9, d=7, V=30, K=5, mask_frac=0.2)
    T = 2.0
    l_T, lse_T, _ = oracle.forward(h, W, t_idx, t_logit, T, mask)
    l_1, lse_1, _ = oracle.forward(h / T, W, t_idx, t_logit / T, 1.0, mask)
    gh_T, gW_T = oracle.backward(h, W, t_idx, t_logit, T, mask)
    gh_1, gW_1 = oracle.backward(h / T, W, t_idx, t_logit / T, 1.0, mask)
    assert l_T == pytest.approx(T * T * l_1, rel=1e-12)
    np.testing.assert_allclose(lse_T, lse_1, rtol=1e-13)
    np.testing.assert_allclose(gh_T, T * gh_1, rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(gW_T, T * T * gW_1, rtol=1e-11, atol=1e-15)


# ---------------------------------------------------------------------------
# P9: invariances
# ---------------------------------------------------------------------------

def test_p9_invariances():
    h, W, t_idx, t_logit, mask = _rand_problem(71, N=10, d=6, V=25, K=6, mask_frac=0.2)
    T = 1.4
    base_l, _, _ = oracle.forward(h, W, t_idx, t_logit, T, mask)
    base_gh, base_gW = oracle.backward(h, W, t_idx, t_logit, T, mask)
    rng = np.random.default_rng(1)
    # (a) per-row shift of the teacher logits
    shifted = t_logit + rng.standard_normal((len(h), 1)) * 5
    assert oracle.forward(h, W, t_idx, shifted, T, mask)[0] == pytest.approx(base_l, rel=1e-12)
    # (b) permuting the K entries of every row
    perm = np.stack([rng.permutation(t_idx.shape[1]) for _ in range(len(h))])
    pi, pl = np.take_along_axis(t_idx, perm, 1), np.take_along_axis(t_logit, perm, 1)
    assert oracle.forward(h, W, pi, pl, T, mask)[0] == pytest.approx(base_l, rel=1e-12)
    np.testing.assert_allclose(oracle.backward(h, W, pi, pl, T, mask)[1], base_gW, rtol=1e-11, atol=1e-15)
    # (c) relabelling the vocabulary permutes the rows of grad_W
    sigma = rng.permutation(W.shape[0])          # new row j holds old row sigma[j]
    inv = np.argsort(sigma)
    W2, idx2 = W[sigma], inv[t_idx].astype(np.int32)
    l2, _, _ = oracle.forward(h, W2, idx2, t_logit, T, mask)
    gh2, gW2 = oracle.backward(h, W2, idx2, t_logit, T, mask)
    assert l2 == pytest.approx(base_l, rel=1e-12)
    np.testing.assert_allclose(gh2, base_gh, rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(gW2, base_gW[sigma], rtol=1e-11, atol=1e-15)
    # (d) adding one vector to every row of W shifts each row's logits uniformly
    W3 = W + rng.standard_normal((1, W.shape[1]))
    l3, _, _ = oracle.forward(h, W3, t_idx, t_logit, T, mask)
    gh3, gW3 = oracle.backward(h, W3, t_idx, t_logit, T, mask)
    assert l3 == pytest.approx(base_l, rel=1e-11)
    np.testing.assert_allclose(gh3, base_gh, rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(gW3, base_gW, rtol=1e-9, atol=1e-13)


# ---------------------------------------------------------------------------
# P10: zero sums; P11: masking; P12: row_lse
# ---------------------------------------------------------------------------

def test_p10_grad_W_columns_sum_to_zero():
    h, W, t_idx, t_logit, mask = _rand_problem(81, N=12, d=9, V=33, K=4, mask_frac=0.3)
    _, gW = oracle.backward(h, W, t_idx, t_logit, 1.0, mask)
    assert np.abs(gW.sum(axis=0)).max() < 1e-14 * max(1.0, np.abs(gW).max()) * W.shape[0]


def test_p11_mask_equals_sub_batch():
    h, W, t_idx, t_logit, mask = _rand_problem(91, N=14, d=5, V=21, K=3, mask_frac=0.4)
    keep = mask.astype(bool)
    T = 1.1
    l_m, _, kl_m = oracle.forward(h, W, t_idx, t_logit, T, mask)
    l_s, _, _ = oracle.forward(h[keep], W, t_idx[keep], t_logit[keep], T)
    gh_m, gW_m = oracle.backward(h, W, t_idx, t_logit, T, mask)
    gh_s, gW_s = oracle.backward(h[keep], W, t_idx[keep], t_logit[keep], T)
    assert l_m == pytest.approx(l_s, rel=1e-12)
    assert np.all(kl_m[~keep] == 0.0) and np.all(gh_m[~keep] == 0.0)
    np.testing.assert_allclose(gh_m[keep], gh_s, rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(gW_m, gW_s, rtol=1e-12, atol=1e-16)


def test_p11_all_masked_gives_zero():
    h, W, t_idx, t_logit, _ = _rand_problem(92)
    mask = np.zeros(len(h), np.uint8)
    loss, lse, kl = oracle.forward(h, W, t_idx, t_logit, 1.0, mask)
    gh, gW = oracle.backward(h, W, t_idx, t_logit, 1.0, mask)
    assert loss == 0.0 and np.all(kl == 0) and np.all(gh == 0) and np.all(gW == 0)
    assert np.all(np.isfinite(lse))


def test_p12_row_lse_matches_torch():
    h, W, t_idx, t_logit, _ = _rand_problem(101, N=11, V=70)
    _, lse, _ = oracle.forward(h, W, t_idx, t_logit, 0.8)
    ref = torch.logsumexp(torch.tensor(h @ W.T) / 0.8, dim=1).numpy()
    np.testing.assert_allclose(lse, ref, rtol=1e-14)


def test_sampled_row_helpers_match_full():
    h, W, t_idx, t_logit, mask = _rand_problem(111, N=20, d=8, V=40, K=5, mask_frac=0.3)
    T = 1.3
    loss, lse, kl = oracle.forward(h, W, t_idx, t_logit, T, mask)
    gh, _ = oracle.backward(h, W, t_idx, t_logit, T, mask, grad_loss=0.6)
    rows = np.array([0, 3, 7, 19])
    lse_r, kl_r = oracle.forward_rows(h, W, t_idx, t_logit, T, rows)
    np.testing.assert_allclose(lse_r, lse[rows], rtol=1e-14)
    valid = mask.astype(bool)[rows]
    np.testing.assert_allclose(kl_r[valid], kl[rows][valid], rtol=1e-13)
    gh_r = oracle.grad_h_rows(h, W, t_idx, t_logit, T, int(mask.sum()), rows, grad_loss=0.6, mask=mask)
    np.testing.assert_allclose(gh_r, gh[rows], rtol=1e-12, atol=1e-16)


@pytest.mark.parametrize("T,mask_frac", [(1.0, 0.0), (1.7, 0.4)])
def test_sampled_grad_W_rows_match_autograd(T, mask_frac):
    """grad_W_rows (used at full size, where only some vocabulary rows are
    checked) against torch autograd of the dense loss and the full backward."""
    h, W, t_idx, t_logit, mask = _rand_problem(131, N=12, d=8, V=40, K=6, mask_frac=mask_frac)
    _, _, _, gW_t, _ = _torch_dense_loss(h, W, t_idx, t_logit, T, mask)
    _, lse, _ = oracle.forward(h, W, t_idx, t_logit, T, mask)
    rows = np.array([0, 5, int(t_idx[0, 0]), int(t_idx[3, 2]), 39])
    got = oracle.grad_W_rows(h, W, t_idx, t_logit, T, rows, lse, grad_loss=1.0, mask=mask)
    np.testing.assert_allclose(got, gW_t[rows], rtol=1e-10, atol=1e-15)
    _, gW = oracle.backward(h, W, t_idx, t_logit, T, mask, grad_loss=0.3)
    got3 = oracle.grad_W_rows(h, W, t_idx, t_logit, T, rows, lse, grad_loss=0.3, mask=mask)
    np.testing.assert_allclose(got3, gW[rows], rtol=1e-12, atol=1e-16)


# ---------------------------------------------------------------------------
# Teacher-cache builder: top-K of the teacher's logits
# ---------------------------------------------------------------------------

def test_topk_teacher_matches_torch_topk():
    """Continuous random logits (no ties): same index sets, values and order as
    torch.topk in fp64."""
    rng = np.random.default_rng(141)
    h = rng.standard_normal((7, 12))
    W = rng.standard_normal((300, 12))
    idx, val = oracle.topk_teacher(h, W, 17)
    tv, ti = torch.topk(torch.tensor(h @ W.T), 17, dim=1, largest=True, sorted=True)
    np.testing.assert_array_equal(idx, ti.numpy())
    np.testing.assert_allclose(val, tv.numpy(), rtol=1e-15)


def test_topk_teacher_brute_force_with_ties():
    """Integer logits with many ties against a plain sorted() of (-value, index)."""
    rng = np.random.default_rng(142)
    h = rng.integers(-2, 3, size=(5, 4)).astype(np.float64)
    W = rng.integers(-2, 3, size=(40, 4)).astype(np.float64)
    K = 11
    idx, val = oracle.topk_teacher(h, W, K)
    for r in range(5):
        z = [float(sum(h[r, j] * W[v, j] for j in range(4))) for v in range(40)]
        want = sorted(range(40), key=lambda v: (-z[v], v))[:K]
        assert list(idx[r]) == want
        assert list(val[r]) == [z[v] for v in want]
    with pytest.raises(ValueError):
        oracle.topk_teacher(h, W, 41)


# ---------------------------------------------------------------------------
# Loss variants: per-token weights and a hard-label cross-entropy term
# ---------------------------------------------------------------------------

def _torch_terms(h, W, t_idx, t_logit, T, w, label, a):
    """Dense torch reference: kl_div and cross_entropy per row, weighted mean."""
    ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    N, V = h.shape[0], W.shape[0]
    p = torch.softmax(torch.tensor(np.asarray(t_logit, dtype=np.float64)) / T, dim=1)
    grid = torch.zeros(N, V, dtype=torch.float64)
    grid.scatter_(1, torch.tensor(np.asarray(t_idx, dtype=np.int64)), p)
    s = (ht @ Wt.T) / T
    kl = torch.nn.functional.kl_div(torch.log_softmax(s, dim=1), grid, reduction="none").sum(dim=1)
    ce = torch.nn.functional.cross_entropy(s, torch.tensor(label, dtype=torch.int64), reduction="none")
    wt = torch.tensor(w, dtype=torch.float64)
    loss = (T * T) * (wt * ((1 - a) * kl + a * ce)).sum() / wt.sum()
    loss.backward()
    return loss.item(), ht.grad.numpy(), Wt.grad.numpy()


@pytest.mark.parametrize("T,a", [(1.0, 0.3), (2.0, 0.5), (0.8, 1.0)])
def test_loss_terms_match_torch_dense(T, a):
    h, W, t_idx, t_logit, mask = _rand_problem(151, N=9, d=8, V=40, K=6, mask_frac=0.3)
    rng = np.random.default_rng(152)
    w = rng.random(9) * 2.0
    label = rng.integers(0, 40, size=9)
    label[0] = t_idx[0, 2]            # a label that is also a teacher index
    w_eff = w * mask
    loss_t, gh_t, gW_t = _torch_terms(h, W, t_idx, t_logit, T, w_eff, label, a)
    loss, lse, row_l = oracle.forward_terms(h, W, t_idx, t_logit, T, mask, w, label, a)
    gh, gW = oracle.backward_terms(h, W, t_idx, t_logit, T, mask, w, label, a)
    assert loss == pytest.approx(loss_t, rel=1e-12)
    np.testing.assert_allclose(gh, gh_t, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(gW, gW_t, rtol=1e-10, atol=1e-14)


def test_loss_terms_reduce_to_the_plain_loss():
    """No label (or a = 0) with 0/1 weights is the plain masked KL; scaling all
    weights changes nothing."""
    h, W, t_idx, t_logit, mask = _rand_problem(153, N=10, d=8, V=30, K=5, mask_frac=0.4)
    T = 1.4
    loss0, lse0, kl0 = oracle.forward(h, W, t_idx, t_logit, T, mask)
    gh0, gW0 = oracle.backward(h, W, t_idx, t_logit, T, mask, grad_loss=0.6)
    label = np.arange(10) % 30
    for rw, lab, a in ((None, None, 0.0), (np.full(10, 3.5), label, 0.0), (None, None, 0.7)):
        loss, lse, row_l = oracle.forward_terms(h, W, t_idx, t_logit, T, mask, rw, lab, a)
        gh, gW = oracle.backward_terms(h, W, t_idx, t_logit, T, mask, rw, lab, a, grad_loss=0.6)
        assert loss == pytest.approx(loss0, rel=1e-12)
        np.testing.assert_allclose(row_l, kl0, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(gh, gh0, rtol=1e-11, atol=1e-16)
        np.testing.assert_allclose(gW, gW0, rtol=1e-11, atol=1e-16)


def test_loss_terms_label_only_is_cross_entropy():
    h, W, t_idx, t_logit, _ = _rand_problem(154, N=7, d=8, V=25, K=4)
    label = np.array([3, 0, 24, 7, 7, 11, 1])
    T = 1.0
    loss, _, row_l = oracle.forward_terms(h, W, t_idx, t_logit, T, None, None, label, 1.0)
    ce = torch.nn.functional.cross_entropy(torch.tensor(h @ W.T), torch.tensor(label), reduction="none")
    np.testing.assert_allclose(row_l, ce.numpy(), rtol=1e-13)
    assert loss == pytest.approx(ce.mean().item(), rel=1e-13)


def test_oracle_rejects_bad_teacher():
    h, W, t_idx, t_logit, _ = _rand_problem(121)
    bad = t_idx.copy()
    bad[0, 1] = bad[0, 0]
    with pytest.raises(ValueError):
        oracle.forward(h, W, bad, t_logit)
    bad = t_idx.copy()
    bad[1, 0] = W.shape[0]
    with pytest.raises(ValueError):
        oracle.backward(h, W, bad, t_logit)


# ---------------------------------------------------------------------------
# The pins catch plausible mistakes: plant each one in a copy of the oracle's
# arithmetic (on the CPU) and check that some pin fails.
# ---------------------------------------------------------------------------

def _mutant_forward(kind):
    def fwd(h, W, t_idx, t_logit, T=1.0, mask=None, chunk=None):
        h = np.asarray(h, np.float64)
        W = np.asarray(W, np.float64)
        N = h.shape[0]
        valid = np.ones(N, bool) if mask is None else np.asarray(mask) != 0
        s = (h @ W.T) / (1.0 if kind == "no_student_T" else T)
        lse = scipy.special.logsumexp(s, axis=1)
        a = np.asarray(t_logit, np.float64) / (1.0 if kind == "no_teacher_T" else T)
        log_p = a - scipy.special.logsumexp(a, axis=1, keepdims=True)
        p = np.exp(log_p)
        idx = np.asarray(t_idx, np.int64)
        if kind == "shifted_index":
            idx = (idx + 1) % W.shape[0]
        s_t = np.take_along_axis(s, idx, axis=1)
        if kind == "reverse_sign":
            kl = (p * (-log_p + s_t - lse[:, None])).sum(1)
        elif kind == "no_entropy":
            kl = (p * (-s_t + lse[:, None])).sum(1)
        else:
            kl = (p * (log_p - s_t + lse[:, None])).sum(1)
        kl = np.where(valid, kl, 0.0)
        n = valid.sum() if kind != "count_all_rows" else N
        scale = T * T if kind != "no_T2" else 1.0
        return scale * kl.sum() / n, lse, kl
    return fwd


@pytest.mark.parametrize("kind", ["no_student_T", "no_teacher_T", "shifted_index", "reverse_sign",
                                  "no_entropy", "count_all_rows", "no_T2"])
def test_pins_catch_planted_mistakes(kind):
    """Each planted forward mistake breaks the dense brute-force pin (P1)."""
    h, W, t_idx, t_logit, mask = _rand_problem(11, mask_frac=0.4)
    T = 2.0
    loss_t, *_ = _torch_dense_loss(h, W, t_idx, t_logit, T, mask)
    loss_m, _, _ = _mutant_forward(kind)(h, W, t_idx, t_logit, T, mask)
    loss_ok, _, _ = _mutant_forward("none")(h, W, t_idx, t_logit, T, mask)
    assert loss_ok == pytest.approx(loss_t, rel=1e-12)
    assert abs(loss_m - loss_t) > 1e-6 * abs(loss_t)


@pytest.mark.parametrize("kind", ["transposed", "no_scale", "dense_only", "wrong_sign"])
def test_pins_catch_planted_gradient_mistakes(kind):
    """Planted backward mistakes break the autograd pin (P1) or zero sums (P10)."""
    h, W, t_idx, t_logit, mask = _rand_problem(12, N=6, d=6, V=32, K=5, mask_frac=0.3)
    T = 1.5
    _, _, gh_t, gW_t, _ = _torch_dense_loss(h, W, t_idx, t_logit, T, mask)
    valid = mask.astype(bool)
    n = valid.sum()
    s = h @ W.T / T
    q = np.exp(s - scipy.special.logsumexp(s, axis=1, keepdims=True))
    grid = fkl_oracle.dense_teacher_grid(t_idx, t_logit, T, W.shape[0])
    c = (T / n) * valid[:, None]
    G = c * (q - grid)
    if kind == "no_scale":
        G = valid[:, None] * (q - grid)
    elif kind == "dense_only":
        G = c * q
    elif kind == "wrong_sign":
        G = c * (grid - q)
    gh = G @ W
    gW = G.T @ h if kind != "transposed" else (h.T @ G).T[::-1]
    bad = (not np.allclose(gh, gh_t, rtol=1e-8, atol=1e-12)) or (not np.allclose(gW, gW_t, rtol=1e-8, atol=1e-12))
    assert bad


def test_loss_terms_nonpositive_weight_drops_the_row():
    """A zero, negative or NaN weight leaves the row out entirely, exactly as
    the sub-batch without it (the masking pin P11 for weights)."""
    rng = np.random.default_rng(77)
    N, d, V, K, T = 12, 16, 48, 5, 1.3
    h = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d)) / 4
    t_idx = np.stack([rng.choice(V, K, replace=False) for _ in range(N)])
    t_logit = rng.standard_normal((N, K)) * 3
    w = rng.uniform(0.5, 2.0, N)
    w[[2, 7, 9]] = [0.0, -1.5, np.nan]
    keep = np.ones(N, bool)
    keep[[2, 7, 9]] = False
    loss, lse, row_l = oracle.forward_terms(h, W, t_idx, t_logit, T, row_weight=w)
    ref_loss, _, ref_l = oracle.forward_terms(h[keep], W, t_idx[keep], t_logit[keep], T, row_weight=w[keep])
    assert abs(loss - ref_loss) <= 1e-12 * abs(ref_loss)
    assert np.all(row_l[~keep] == 0.0)
    np.testing.assert_allclose(row_l[keep], ref_l, rtol=1e-12, atol=0)
    gh, gW = oracle.backward_terms(h, W, t_idx, t_logit, T, row_weight=w)
    rgh, rgW = oracle.backward_terms(h[keep], W, t_idx[keep], t_logit[keep], T, row_weight=w[keep])
    assert np.all(gh[~keep] == 0.0)
    np.testing.assert_allclose(gh[keep], rgh, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(gW, rgW, rtol=1e-10, atol=1e-14)
