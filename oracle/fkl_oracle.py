"""fp64 reference for the fused chunked KL distillation loss (forward + backward).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

Sources (web pages about the paper "Efficient Knowledge Distillation for LLMs:
Offline Top-K Logits and a Fused Chunked KL Loss"):

* [BLOG] the authors' post, printed on the page "Efficient Offline Top-K
  Logits and Fused Chunked KL Loss Enable Scalable LLM Distillation",
  sections "Two systems changes" and "Scaling to long context lengths".
* [AIX] "Making knowledge distillation cheap enough to run in production",
  the comparison table of Dense / Forward-chunked / Fused chunked KL.

What the pages fix, restated:

* The teacher is kept sparse: per position only its top-K (index, logit)
  pairs are cached; the rest of its distribution is dropped [BLOG "Two
  systems changes"; AIX last paragraph].
* The loss compares the teacher distribution with the student's
  log-probabilities over the whole vocabulary; dense, forward-chunked and
  fused chunked variants compute the same number [BLOG "Two systems
  changes"]. The dense variant is the correctness baseline.
* The fused variant takes the hidden states and the output-projection
  weight, walks the sequence one chunk of positions at a time, forms that
  chunk's logits, adds the chunk's contribution to a running loss and drops
  the chunk; backward recomputes each chunk's logits instead of storing them
  [BLOG "Two systems changes"].

Readings where the pages are silent (no formula is printed anywhere):

* R1 direction: forward KL(teacher || student).
* R2 teacher distribution: softmax over the K cached logits (renormalised),
  zero outside the K indices.
* R3 reduction: mean over valid (unmasked) positions; loss = 0 if none.
* R4 temperature T divides student and teacher logits; the loss is scaled by
  T^2 (Hinton convention). row_lse is logsumexp_v(z/T).
* R5 masked positions contribute to neither the sum nor the count; their
  row_lse is still reported; their gradient rows are exactly zero.
* R6 teacher indices are distinct per row and in [0, V) (precondition).
* R7 upstream gradient: a scalar g multiplying the whole gradient.

Derived gradient (R1-R7; the pages name a closed-form gradient but do not
print it): with s = z/T, q = softmax_v(s), p~ the teacher distribution
scattered onto the vocabulary, c_r = g * (T/n) * mask_r,

    G[r, v] = c_r * (q[r, v] - p~[r, v]),   grad_h = G @ W,   grad_W = G.T @ h

because dKL_r/ds = q - p~ (sum_v p~ = 1) and ds/dz = 1/T, times T^2/n.

Everything is numpy float64. bf16 / fp32 inputs are widened exactly.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "teacher_distribution",
    "forward",
    "backward",
    "forward_rows",
    "grad_h_rows",
    "grad_W_rows",
    "dense_teacher_grid",
    "topk_teacher",
    "forward_terms",
    "backward_terms",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _check_teacher(t_idx: np.ndarray, V: int) -> None:
    """R6: indices in range and distinct within each row."""
    if t_idx.size == 0:
        return
    if t_idx.min() < 0 or t_idx.max() >= V:
        raise ValueError("teacher index out of range")
    srt = np.sort(t_idx, axis=1)
    if np.any(srt[:, 1:] == srt[:, :-1]):
        raise ValueError("duplicate teacher index in a row")


def _valid_rows(mask, N: int) -> np.ndarray:
    if mask is None:
        return np.ones(N, dtype=bool)
    return np.asarray(mask).reshape(N) != 0


def teacher_distribution(t_logit, T: float):
    """R2 + R4: softmax over the K cached teacher logits divided by T.

    Returns (p, log_p), both [N, K] float64.
    [BLOG "Two systems changes": only the cached top-K logits per position
    are kept and the teacher is never expanded beyond them.]
    """
    a = _f64(t_logit) / T
    a_max = a.max(axis=1, keepdims=True)
    log_norm = a_max + np.log(np.exp(a - a_max).sum(axis=1, keepdims=True))
    log_p = a - log_norm
    return np.exp(log_p), log_p


def _chunk_logits(h_c: np.ndarray, W: np.ndarray, T: float) -> np.ndarray:
    """One chunk's temperature-scaled student logits s = (h_c W^T) / T.

    [BLOG "Two systems changes": hidden states of the chunk are projected to
    logits with the output-projection weight.]
    """
    return (h_c @ W.T) / T


def _row_logsumexp(s: np.ndarray) -> np.ndarray:
    m = s.max(axis=1, keepdims=True)
    return m[:, 0] + np.log(np.exp(s - m).sum(axis=1))


def forward(h, W, t_idx, t_logit, T: float = 1.0, mask=None, chunk: int | None = None):
    """Fused chunked KL, forward.

    Walks the positions one chunk at a time: forms that chunk's logits, folds
    its KL terms into a running sum, and drops the chunk before the next one
    [BLOG "Two systems changes"].

    Returns (loss, row_lse [N], row_kl [N]); row_kl is 0 on masked rows.
    """
    h = _f64(h)
    W = _f64(W)
    t_idx = np.asarray(t_idx, dtype=np.int64)
    N, d = h.shape
    V = W.shape[0]
    _check_teacher(t_idx, V)
    valid = _valid_rows(mask, N)
    n = int(valid.sum())
    chunk = N if not chunk else int(chunk)
    row_lse = np.zeros(N)
    row_kl = np.zeros(N)
    running = 0.0
    for c0 in range(0, N, max(chunk, 1)):
        c1 = min(N, c0 + chunk)
        s = _chunk_logits(h[c0:c1], W, T)
        lse = _row_logsumexp(s)
        p, log_p = teacher_distribution(t_logit[c0:c1], T)
        s_at_teacher = np.take_along_axis(s, t_idx[c0:c1], axis=1)
        # R1: KL(p || q) with log q = s - lse, summed over the teacher support.
        kl = (p * (log_p - s_at_teacher + lse[:, None])).sum(axis=1)
        kl = np.where(valid[c0:c1], kl, 0.0)
        row_lse[c0:c1] = lse
        row_kl[c0:c1] = kl
        running += kl.sum()
        del s
    loss = (T * T) * running / n if n > 0 else 0.0
    return float(loss), row_lse, row_kl


def backward(h, W, t_idx, t_logit, T: float = 1.0, mask=None, grad_loss: float = 1.0,
             chunk: int | None = None):
    """Fused chunked KL, backward with recomputation.

    For every chunk the logits are formed again rather than kept from the
    forward pass [BLOG "Two systems changes"]; the chunk's gradient
    G = c (q - p~) then feeds grad_h (rows of the chunk) and grad_W (summed
    over chunks). Rows with c_r = 0 (masked) contribute exactly zero and are
    skipped. Returns (grad_h [N, d], grad_W [V, d]) float64.
    """
    h = _f64(h)
    W = _f64(W)
    t_idx = np.asarray(t_idx, dtype=np.int64)
    N, d = h.shape
    V = W.shape[0]
    _check_teacher(t_idx, V)
    valid = _valid_rows(mask, N)
    n = int(valid.sum())
    grad_h = np.zeros((N, d))
    grad_W = np.zeros((V, d))
    if n == 0:
        return grad_h, grad_W
    scale = float(grad_loss) * T / n
    rows = np.nonzero(valid)[0]
    chunk = len(rows) if not chunk else int(chunk)
    for c0 in range(0, len(rows), max(chunk, 1)):
        rc = rows[c0:c0 + chunk]
        s = _chunk_logits(h[rc], W, T)
        q = np.exp(s - _row_logsumexp(s)[:, None])
        p, _ = teacher_distribution(t_logit[rc], T)
        p_tilde = np.zeros_like(q)
        np.put_along_axis(p_tilde, t_idx[rc], p, axis=1)
        G = scale * (q - p_tilde)
        grad_h[rc] = G @ W
        grad_W += G.T @ h[rc]
        del s, q, p_tilde, G
    return grad_h, grad_W


def forward_rows(h, W, t_idx, t_logit, T: float, rows):
    """Per-row (row_lse, unmasked row KL) for selected rows only.

    Each row's KL needs nothing but that row's logits, so sampled rows of a
    large problem can be checked one by one.
    """
    rows = np.asarray(rows, dtype=np.int64)
    h_r = _f64(np.asarray(h)[rows])
    W = _f64(W)
    idx = np.asarray(t_idx, dtype=np.int64)[rows]
    _check_teacher(idx, W.shape[0])
    s = _chunk_logits(h_r, W, T)
    lse = _row_logsumexp(s)
    p, log_p = teacher_distribution(np.asarray(t_logit)[rows], T)
    kl = (p * (log_p - np.take_along_axis(s, idx, axis=1) + lse[:, None])).sum(axis=1)
    return lse, kl


def grad_h_rows(h, W, t_idx, t_logit, T: float, n_valid: int, rows, grad_loss: float = 1.0,
                mask=None):
    """grad_h for selected rows: G_r @ W with G_r = g (T/n) mask_r (q_r - p~_r)."""
    rows = np.asarray(rows, dtype=np.int64)
    W = _f64(W)
    h_r = _f64(np.asarray(h)[rows])
    idx = np.asarray(t_idx, dtype=np.int64)[rows]
    s = _chunk_logits(h_r, W, T)
    q = np.exp(s - _row_logsumexp(s)[:, None])
    p, _ = teacher_distribution(np.asarray(t_logit)[rows], T)
    p_tilde = np.zeros_like(q)
    np.put_along_axis(p_tilde, idx, p, axis=1)
    m = np.ones(len(rows)) if mask is None else (np.asarray(mask)[rows] != 0).astype(np.float64)
    if n_valid == 0:
        return np.zeros((len(rows), W.shape[1]))
    G = (float(grad_loss) * T / n_valid) * m[:, None] * (q - p_tilde)
    return G @ W


def grad_W_rows(h, W, t_idx, t_logit, T: float, vocab_rows, row_lse, grad_loss: float = 1.0,
                mask=None):
    """grad_W for selected vocabulary rows: sum_r G[r, v] h_r.

    Column v of G needs every row's logit s[r, v] = h_r . W_v / T and every
    row's normaliser; ``row_lse`` must be the oracle's own forward result
    for all rows. Returns [len(vocab_rows), d] float64.
    """
    vocab_rows = np.asarray(vocab_rows, dtype=np.int64)
    h = _f64(h)
    N = h.shape[0]
    valid = _valid_rows(mask, N)
    n = int(valid.sum())
    if n == 0:
        return np.zeros((len(vocab_rows), h.shape[1]))
    Wv = _f64(np.asarray(W)[vocab_rows])
    s = (h @ Wv.T) / T                                   # [N, len(vocab_rows)]
    q = np.exp(s - _f64(row_lse)[:, None])
    p, _ = teacher_distribution(t_logit, T)
    t_idx = np.asarray(t_idx, dtype=np.int64)
    p_tilde = np.zeros_like(q)
    for j, v in enumerate(vocab_rows):
        hit_r, hit_k = np.nonzero(t_idx == v)
        p_tilde[hit_r, j] = p[hit_r, hit_k]
    G = (float(grad_loss) * T / n) * valid[:, None] * (q - p_tilde)
    return G.T @ h


def dense_teacher_grid(t_idx, t_logit, T: float, V: int) -> np.ndarray:
    """The dense teacher grid [N, V]: p~ scattered onto the vocabulary.

    This is what the dense variant rebuilds and the fused variant avoids
    [BLOG "Two systems changes"]; used only by tiny brute-force checks.
    """
    p, _ = teacher_distribution(t_logit, T)
    grid = np.zeros((p.shape[0], V))
    np.put_along_axis(grid, np.asarray(t_idx, dtype=np.int64), p, axis=1)
    return grid


def topk_teacher(h, W, K: int):
    """The offline teacher cache: per row, the K largest logits z = h W^T.

    The cache keeps each position's top-K (index, logit) pairs and nothing
    else of the teacher's distribution [BLOG "Two systems changes"; AIX last
    paragraph]. Logits are exact fp64 dot products of the given values. Order:
    value descending; equal values by the lower vocabulary index first (the
    reading taken for ties, which the pages do not discuss). Returns
    (idx int64 [N, K], val float64 [N, K]).
    """
    h = _f64(h)
    W = _f64(W)
    N, V = h.shape[0], W.shape[0]
    if not 1 <= K <= V:
        raise ValueError("need 1 <= K <= V")
    idx = np.empty((N, K), dtype=np.int64)
    val = np.empty((N, K))
    cols = np.arange(V)
    for r in range(N):
        z = W @ h[r]
        order = np.lexsort((cols, -z))[:K]   # primary key -z, then the index
        idx[r] = order
        val[r] = z[order]
    return idx, val


def _weights(mask, row_weight, N: int) -> np.ndarray:
    """Per-row weight: row_weight (1 if absent) on unmasked rows. A row whose
    weight is not positive (zero, negative or NaN) takes no part in the loss,
    like a masked row (reading R10: weights generalise the 0/1 mask)."""
    w = np.ones(N) if row_weight is None else _f64(row_weight).reshape(N)
    keep = _valid_rows(mask, N) & (w > 0)
    return np.where(keep, w, 0.0)


def forward_terms(h, W, t_idx, t_logit, T: float = 1.0, mask=None, row_weight=None, label=None,
                  label_weight: float = 0.0):
    """Loss variants on the same fused structure (readings; the pages name a
    "choice of loss function" [AIX] but define no variant):

      l_r  = (1 - a) KL(p_r || q_r) + a CE(y_r, q_r)      q_r = softmax(z_r / T)
      loss = T^2 sum_r w_r l_r / sum_r w_r                (0 if sum_r w_r = 0)

    with w_r = row_weight[r] * mask[r] (per-token weights; the mask is the
    0/1 case), y_r = label[r] a hard label, a = label_weight (a = 0 or no
    label: plain KL). Both terms use the loss temperature. Dense per row,
    written directly from the definition. Returns (loss, row_lse, row_l)
    with row_l the unweighted per-row l_r (0 where w_r = 0).
    """
    h = _f64(h)
    W = _f64(W)
    t_idx = np.asarray(t_idx, dtype=np.int64)
    N = h.shape[0]
    _check_teacher(t_idx, W.shape[0])
    w = _weights(mask, row_weight, N)
    a = float(label_weight) if label is not None else 0.0
    s = _chunk_logits(h, W, T)
    lse = _row_logsumexp(s)
    log_q = s - lse[:, None]
    p, log_p = teacher_distribution(t_logit, T)
    kl = (p * (log_p - np.take_along_axis(log_q, t_idx, axis=1))).sum(axis=1)
    ce = np.zeros(N) if label is None else -log_q[np.arange(N), np.asarray(label, dtype=np.int64)]
    row_l = np.where(w > 0, (1.0 - a) * kl + a * ce, 0.0)
    sw = w.sum()
    loss = (T * T) * float((w * row_l).sum()) / sw if sw > 0 else 0.0
    return loss, lse, row_l


def backward_terms(h, W, t_idx, t_logit, T: float = 1.0, mask=None, row_weight=None, label=None,
                   label_weight: float = 0.0, grad_loss: float = 1.0):
    """Gradients of forward_terms: with c_r = g T w_r / sum w,
    G[r, v] = c_r ((1 - a)(q - p~) + a (q - onehot(y_r)))[r, v],
    grad_h = G W, grad_W = G^T h (dl/ds = q - target, ds/dz = 1/T, times T^2)."""
    h = _f64(h)
    W = _f64(W)
    t_idx = np.asarray(t_idx, dtype=np.int64)
    N = h.shape[0]
    w = _weights(mask, row_weight, N)
    sw = w.sum()
    if sw <= 0:
        return np.zeros_like(h), np.zeros_like(W)
    a = float(label_weight) if label is not None else 0.0
    s = _chunk_logits(h, W, T)
    q = np.exp(s - _row_logsumexp(s)[:, None])
    p, _ = teacher_distribution(t_logit, T)
    target = np.zeros_like(q)
    np.put_along_axis(target, t_idx, (1.0 - a) * p, axis=1)
    if label is not None:
        target[np.arange(N), np.asarray(label, dtype=np.int64)] += a
    G = (float(grad_loss) * T * w / sw)[:, None] * (q - target)
    return G @ W, G.T @ h
