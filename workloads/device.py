"""Full-size workloads with the hidden states and head weight drawn on the GPU.

Same recipe as ``synth.make_workload`` (h ~ N(0, 1), W ~ N(0, 1/d), rounded to
bfloat16; teacher cache and mask from numpy), but h and W come from torch's
seeded device generator, which draws hundreds of millions of normals in
milliseconds instead of minutes. No loss arithmetic lives here.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .synth import (CONFIGS, packed_document_mask, sorted_teacher_logits, uniform_teacher,
                    zipf_uniform_teacher)


@dataclass
class DeviceWorkload:
    name: str
    N: int
    d: int
    V: int
    K: int
    T: float
    chunk: int
    seed: int
    h: "object"        # torch bf16 [N, d] on the device
    W: "object"        # torch bf16 [V, d] on the device
    t_idx: "object"    # torch int32 [N, K] on the device
    t_logit: "object"  # torch fp32 [N, K] on the device
    mask: "object"     # torch uint8 [N] on the device, or None
    t_idx_np: np.ndarray
    t_logit_np: np.ndarray
    mask_np: np.ndarray | None

    def describe(self) -> str:
        return (f"{self.name}: N={self.N} d={self.d} V={self.V} K={self.K} T={self.T:g} "
                f"chunk={self.chunk}")


def _seed_of(ss: np.random.SeedSequence) -> int:
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def perturbed_head(W, seed: int, device):
    """W_t = bf16(float32(W) + 0.1 * N(0, 1/d)), noise from torch's seeded device generator."""
    import torch

    d = W.shape[1]
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    Wt = torch.empty_like(W)
    block = 16384
    for v0 in range(0, W.shape[0], block):
        v1 = min(W.shape[0], v0 + block)
        noise = torch.randn((v1 - v0, d), generator=g, device=device, dtype=torch.float32)
        Wt[v0:v1] = W[v0:v1].float() + noise * float(0.1 / np.sqrt(d))
    return Wt


def perturbed_head_teacher(h, W, K: int, seed: int, device, rows_per_pass: int = 1024):
    """Teacher cache from a perturbed copy of the student head.

    W_t = bf16(float32(W) + 0.1 * N(0, 1/d)); the teacher keeps the exact
    top-K of its fp32 logits h W_t^T per row (values descending), computed in
    float32 on the device without TF32, in passes of rows_per_pass rows.
    Input generation only: the same arrays feed the library and the oracle.
    """
    import torch

    Wt = perturbed_head(W, seed, device)
    Wt32 = Wt.float()
    del Wt
    prev = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    try:
        idx = torch.empty((h.shape[0], K), dtype=torch.int64, device=device)
        val = torch.empty((h.shape[0], K), dtype=torch.float32, device=device)
        for r0 in range(0, h.shape[0], rows_per_pass):
            r1 = min(h.shape[0], r0 + rows_per_pass)
            z = h[r0:r1].float() @ Wt32.t()
            v, i = torch.topk(z, K, dim=1, largest=True, sorted=True)
            idx[r0:r1] = i
            val[r0:r1] = v
            del z
    finally:
        torch.backends.cuda.matmul.allow_tf32 = prev
    del Wt32
    return idx.to(torch.int32).cpu().numpy(), val.cpu().numpy()


def make_device_workload(name: str, device, seed_offset: int = 0, *, N: int | None = None,
                         mask: str | None = None, **overrides) -> DeviceWorkload:
    import torch

    cfg = dict(CONFIGS[name])
    cfg.update({k: v for k, v in overrides.items() if v is not None})
    if N is not None:
        cfg["N"] = int(N)
    if mask is not None:
        cfg["mask"] = mask
    seed = int(cfg["seed"]) + int(seed_offset)
    s_h, s_w, s_idx, s_logit, s_mask = np.random.SeedSequence(seed).spawn(5)
    Nr, d, V, K = int(cfg["N"]), int(cfg["d"]), int(cfg["V"]), int(cfg["K"])

    g = torch.Generator(device=device)
    g.manual_seed(_seed_of(s_h))
    h = torch.empty((Nr, d), dtype=torch.bfloat16, device=device)
    W = torch.empty((V, d), dtype=torch.bfloat16, device=device)
    block = 16384
    for r0 in range(0, Nr, block):
        r1 = min(Nr, r0 + block)
        h[r0:r1] = torch.randn((r1 - r0, d), generator=g, device=device, dtype=torch.float32)
    g.manual_seed(_seed_of(s_w))
    std = float(1.0 / np.sqrt(d))
    for v0 in range(0, V, block):
        v1 = min(V, v0 + block)
        W[v0:v1] = torch.randn((v1 - v0, d), generator=g, device=device, dtype=torch.float32) * std

    rng_idx = np.random.default_rng(s_idx)
    if cfg["teacher"] == "uniform":
        t_idx = uniform_teacher(rng_idx, Nr, V, K)
        t_logit = sorted_teacher_logits(np.random.default_rng(s_logit), Nr, K)
    elif cfg["teacher"] == "zipf_uniform":
        t_idx = zipf_uniform_teacher(rng_idx, Nr, V, K)
        t_logit = sorted_teacher_logits(np.random.default_rng(s_logit), Nr, K)
    elif cfg["teacher"] == "perturbed_head":
        t_idx, t_logit = perturbed_head_teacher(h, W, K, _seed_of(s_idx), device)
    else:
        raise ValueError(f"teacher recipe {cfg['teacher']} is not available for device workloads")
    rng_mask = np.random.default_rng(s_mask)
    if cfg["mask"] == "none":
        m = None
    elif cfg["mask"] == "random25":
        m = (rng_mask.random(Nr) >= 0.25).astype(np.uint8)
    elif cfg["mask"] == "packed":
        m = packed_document_mask(rng_mask, Nr)
    else:
        raise ValueError(f"unknown mask recipe {cfg['mask']}")
    return DeviceWorkload(
        name=name, N=Nr, d=d, V=V, K=K, T=float(cfg["T"]), chunk=int(cfg["chunk"]), seed=seed,
        h=h, W=W, t_idx=torch.from_numpy(t_idx).to(device), t_logit=torch.from_numpy(t_logit).to(device),
        mask=None if m is None else torch.from_numpy(m).to(device),
        t_idx_np=t_idx, t_logit_np=t_logit, mask_np=m)
