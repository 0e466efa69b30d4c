"""Seeded synthetic workloads for the fused chunked KL loss.

No loss arithmetic lives here. The module draws hidden states, a head weight
and a cached top-K teacher with the shapes and value distributions of the
workloads named below, rounds the float draws to bfloat16 (round to nearest
even), and builds the optional row mask.

Every draw comes from numpy's PCG64 with ``SeedSequence(seed).spawn(5)``
sub-streams, one each for [h, W, teacher index, teacher logit, mask].

Teacher cache format (the offline top-K cache of the method): per position,
K distinct vocabulary indices (int32) and their logits (fp32), the logits
sorted in descending order. Two index recipes:

* ``uniform``: K distinct indices uniform in [0, V).
* ``zipf_uniform``: half the indices are pi[rank - 1] with rank ~ Zipf(1.1)
  truncated to [1, V] (pi a per-seed vocabulary permutation), the other half
  uniform; duplicates are rejected. The Zipf half gets the larger logits.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "CONFIGS",
    "Workload",
    "bf16_bits",
    "bf16_to_f32",
    "make_workload",
    "uniform_teacher",
    "zipf_uniform_teacher",
    "packed_document_mask",
]


# name -> shape and recipe. "chunk" is the row chunk the library is called with.
CONFIGS = {
    "tiny": dict(N=256, d=256, V=4096, K=16, T=1.0, chunk=64, seed=1001, teacher="uniform",
                 mask="none"),
    "llama3b": dict(N=8192, d=3072, V=128256, K=100, T=1.0, chunk=1024, seed=1002,
                    teacher="zipf_uniform", mask="none"),
    "gptoss20b": dict(N=32768, d=2880, V=201088, K=100, T=1.0, chunk=4096, seed=1003,
                      teacher="zipf_uniform", mask="none"),
    "long64k": dict(N=65536, d=2880, V=201088, K=100, T=1.0, chunk=4096, seed=1004,
                    teacher="zipf_uniform", mask="packed"),
    "long256k": dict(N=262144, d=2880, V=201088, K=100, T=1.0, chunk=4096, seed=1005,
                     teacher="zipf_uniform", mask="packed"),
    "temp": dict(N=16384, d=4096, V=128256, K=100, T=2.0, chunk=4096, seed=1006,
                 teacher="perturbed_head", mask="none"),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 24
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    for i in range(0, flat_u.size, step):
        b = flat_u[i:i + step].astype(np.uint32)
        b += np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
        flat_o[i:i + step] = (b >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _first_distinct(cand: np.ndarray, valid: np.ndarray, k: int):
    """Per row, the first k distinct valid candidates in position order.

    Returns (rows_ok [N] bool, picked [n_ok, k] int64).
    """
    N, M = cand.shape
    big = np.int64(1) << 62
    key = np.where(valid, cand, big + np.arange(M, dtype=np.int64)[None, :])
    order = np.argsort(key, axis=1, kind="stable")
    sk = np.take_along_axis(key, order, axis=1)
    dup_sorted = np.zeros((N, M), dtype=bool)
    dup_sorted[:, 1:] = sk[:, 1:] == sk[:, :-1]
    first = np.empty((N, M), dtype=bool)
    np.put_along_axis(first, order, ~dup_sorted, axis=1)
    ok = valid & first
    cs = np.cumsum(ok, axis=1)
    rows_ok = cs[:, -1] >= k
    sel = ok & (cs <= k)
    picked = cand[rows_ok][sel[rows_ok]].reshape(-1, k)
    return rows_ok, picked


def uniform_teacher(rng: np.random.Generator, N: int, V: int, K: int) -> np.ndarray:
    """[N, K] int32: K distinct indices per row, uniform over [0, V)."""
    if K > V:
        raise ValueError("K > V")
    out = np.empty((N, K), dtype=np.int64)
    todo = np.arange(N)
    m = max(2 * K, K + 8)
    while todo.size:
        if m >= V:
            # dense fallback: a random permutation prefix per row
            keys = rng.random((todo.size, V))
            out[todo] = np.argsort(keys, axis=1)[:, :K]
            break
        cand = rng.integers(0, V, size=(todo.size, m), dtype=np.int64)
        ok, picked = _first_distinct(cand, np.ones_like(cand, dtype=bool), K)
        out[todo[ok]] = picked
        todo = todo[~ok]
        m *= 2
    return out.astype(np.int32)


def _zipf_cdf(V: int, a: float) -> np.ndarray:
    """CDF of ranks 1..V with P(rank = k) proportional to k^-a (truncated Zipf)."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-a)
    c = np.cumsum(w)
    return c / c[-1]


def zipf_uniform_teacher(rng: np.random.Generator, N: int, V: int, K: int,
                         zipf_a: float = 1.1, block: int = 8192) -> np.ndarray:
    """[N, K] int32: the Zipf half in columns [0, ceil(K/2)), then the uniform half.

    Zipf half: the first ceil(K/2) distinct values pi[rank-1] of a stream of
    ranks drawn from Zipf(zipf_a) truncated to [1, V] (inverse CDF), pi a
    vocabulary permutation drawn once; uniform half: the remaining indices
    uniform in [0, V), distinct from each other and from the Zipf half. Rows
    are generated in blocks of ``block`` rows from the one stream ``rng``.
    """
    if K > V:
        raise ValueError("K > V")
    kz = (K + 1) // 2
    ku = K - kz
    perm = rng.permutation(V).astype(np.int64)
    cdf = _zipf_cdf(V, zipf_a)
    out = np.empty((N, K), dtype=np.int32)
    for b0 in range(0, N, block):
        n = min(N, b0 + block) - b0
        zipf_part = np.empty((n, kz), dtype=np.int64)
        todo = np.arange(n)
        m = 4 * kz
        while todo.size:
            ranks = np.searchsorted(cdf, rng.random((todo.size, m)), side="right")
            cand = perm[np.minimum(ranks, V - 1)]
            ok, picked = _first_distinct(cand, np.ones_like(cand, dtype=bool), kz)
            zipf_part[todo[ok]] = picked
            todo = todo[~ok]
            m *= 2
        blk = np.empty((n, K), dtype=np.int64)
        blk[:, :kz] = zipf_part
        if ku:
            todo = np.arange(n)
            m = 2 * ku + 8
            while todo.size:
                cand = np.concatenate(
                    [zipf_part[todo], rng.integers(0, V, size=(todo.size, m), dtype=np.int64)], axis=1)
                ok, picked = _first_distinct(cand, np.ones_like(cand, dtype=bool), K)
                blk[todo[ok], kz:] = picked[:, kz:]
                todo = todo[~ok]
                m *= 2
        out[b0:b0 + n] = blk
    return out


def sorted_teacher_logits(rng: np.random.Generator, N: int, K: int, std: float = 3.0) -> np.ndarray:
    """[N, K] float32 logits ~ N(0, std^2), sorted descending within each row."""
    x = rng.standard_normal(size=(N, K)) * std
    return (-np.sort(-x, axis=1)).astype(np.float32)


def packed_document_mask(rng: np.random.Generator, N: int, n_docs: int = 8) -> np.ndarray:
    """uint8 [N]: 8 packed documents of random lengths summing to N.

    The last position of each document has no next-token target inside its
    document, so it is masked out (0); every other position is 1.
    """
    mask = np.ones(N, dtype=np.uint8)
    if N == 0:
        return mask
    n_cuts = min(n_docs - 1, max(N - 1, 0))
    cuts = np.sort(rng.choice(np.arange(1, N), size=n_cuts, replace=False)) if n_cuts else []
    for c in cuts:
        mask[c - 1] = 0
    mask[N - 1] = 0
    return mask


@dataclass
class Workload:
    name: str
    N: int
    d: int
    V: int
    K: int
    T: float
    chunk: int
    seed: int
    h_bits: np.ndarray            # uint16 [N, d] bfloat16 bits
    W_bits: np.ndarray            # uint16 [V, d] bfloat16 bits
    t_idx: np.ndarray             # int32 [N, K]
    t_logit: np.ndarray           # float32 [N, K]
    mask: np.ndarray | None = None  # uint8 [N] or None (all valid)
    h_f32: np.ndarray | None = field(default=None, repr=False)  # unrounded draws (fp32 variant)
    W_f32: np.ndarray | None = field(default=None, repr=False)

    def h(self) -> np.ndarray:
        """bf16-exact hidden states as float32."""
        return bf16_to_f32(self.h_bits)

    def W(self) -> np.ndarray:
        """bf16-exact head weight as float32."""
        return bf16_to_f32(self.W_bits)


def make_workload(name: str, seed_offset: int = 0, *, N: int | None = None, mask: str | None = None,
                  keep_f32: bool = False, teacher_builder=None, **overrides) -> Workload:
    """Build the named workload with seed CONFIGS[name]['seed'] + seed_offset.

    ``N`` overrides the row count (same recipe); ``mask`` overrides the mask
    recipe ('none', 'random25', 'packed'); ``overrides`` may change d, V, K,
    T or chunk for reduced-size variants. ``teacher_builder`` is required for
    the 'perturbed_head' recipe (it needs a projection, which lives outside
    this module).
    """
    cfg = dict(CONFIGS[name])
    cfg.update({k: v for k, v in overrides.items() if v is not None})
    if N is not None:
        cfg["N"] = int(N)
    if mask is not None:
        cfg["mask"] = mask
    seed = int(cfg["seed"]) + int(seed_offset)
    s_h, s_w, s_idx, s_logit, s_mask = np.random.SeedSequence(seed).spawn(5)
    Nr, d, V, K = int(cfg["N"]), int(cfg["d"]), int(cfg["V"]), int(cfg["K"])
    h32 = _normal_f32(np.random.default_rng(s_h), (Nr, d), 1.0)
    W32 = _normal_f32(np.random.default_rng(s_w), (V, d), float(1.0 / np.sqrt(d)))
    h_bits = bf16_bits(h32)
    W_bits = bf16_bits(W32)
    rng_idx = np.random.default_rng(s_idx)
    rng_logit = np.random.default_rng(s_logit)
    if cfg["teacher"] == "uniform":
        t_idx = uniform_teacher(rng_idx, Nr, V, K)
        t_logit = sorted_teacher_logits(rng_logit, Nr, K)
    elif cfg["teacher"] == "zipf_uniform":
        t_idx = zipf_uniform_teacher(rng_idx, Nr, V, K)
        t_logit = sorted_teacher_logits(rng_logit, Nr, K)
    elif cfg["teacher"] == "perturbed_head":
        if teacher_builder is None:
            raise ValueError("the perturbed_head teacher needs a teacher_builder")
        t_idx, t_logit = teacher_builder(h_bits, W_bits, rng_idx, K)
    else:
        raise ValueError(f"unknown teacher recipe {cfg['teacher']}")
    rng_mask = np.random.default_rng(s_mask)
    if cfg["mask"] == "none":
        m = None
    elif cfg["mask"] == "random25":
        m = (rng_mask.random(Nr) >= 0.25).astype(np.uint8)
    elif cfg["mask"] == "packed":
        m = packed_document_mask(rng_mask, Nr)
    else:
        raise ValueError(f"unknown mask recipe {cfg['mask']}")
    wl = Workload(name=name, N=Nr, d=d, V=V, K=K, T=float(cfg["T"]), chunk=int(cfg["chunk"]),
                  seed=seed, h_bits=h_bits, W_bits=W_bits, t_idx=np.ascontiguousarray(t_idx),
                  t_logit=np.ascontiguousarray(t_logit), mask=m)
    if keep_f32:
        wl.h_f32, wl.W_f32 = h32, W32
    return wl
