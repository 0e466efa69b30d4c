"""Cases run through both builds of the library: the release build in the test
process and the bounds-checking debug build (libfkl_debug.so, FKL_DEBUG) in a
child process started by tests/test_gpu_debug_build.py. Each case returns its
outputs as numpy arrays; the debug build must report no bounds violation and
return the release build's results (up to the rounding order the compiler
picks for each build).

Run as a script: python tests/debug_cases.py OUT.npz [--planted] [--fullsize]
(the library is whatever FKL_LIBRARY names). --planted adds the case whose
gradient-block extent is narrowed (FKL_DEBUG_SHRINK_G=1), which the debug
build must report as an error naming the gradient block. --fullsize adds the
headline shape and the builder's default pass at the large head.
"""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _dev_inputs(wl, torch, dev):
    def bits(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)

    m = torch.from_numpy(wl.mask).to(dev) if wl.mask is not None else None
    return (bits(wl.h_bits), bits(wl.W_bits), torch.from_numpy(wl.t_idx).to(dev),
            torch.from_numpy(wl.t_logit).to(dev), m)


def _np(t):
    return t.float().cpu().numpy() if t.dtype.is_floating_point else t.cpu().numpy()


def case_ragged(fkl, torch, dev):
    """Ragged N/d/V over several chunks and slabs, a random mask, grad_h split
    along the vocabulary, then the same backward accumulated into the result."""
    from workloads import make_workload
    wl = make_workload("tiny", N=300, d=136, V=5000, K=7, mask="random25")
    h, W, ti, tl, m = _dev_inputs(wl, torch, dev)
    loss, lse, kl = fkl.forward(h, W, ti, tl, T=0.7, mask=m, chunk=128, vslab=768, return_row_kl=True)
    gl = torch.tensor([2.5], dtype=torch.float32, device=dev)
    gh, gW = fkl.backward(h, W, ti, tl, lse, T=0.7, mask=m, grad_loss=gl, chunk=128, vslab=768)
    gh2, gW2 = fkl.backward(h, W, ti, tl, lse, T=0.7, mask=m, grad_loss=gl, chunk=128, vslab=768,
                            grad_h=gh.clone(), grad_W=gW.clone(), accumulate_grad_h=True, accumulate_grad_W=True)
    loss_s, lse_s = fkl.forward_static(h, W, ti, tl, T=0.7, mask=m, chunk=128, vslab=768)
    return {"loss": _np(loss), "lse": _np(lse), "kl": _np(kl), "gh": _np(gh), "gW": _np(gW), "gh2": _np(gh2),
            "gW2": _np(gW2), "loss_static": _np(loss_s), "lse_static": _np(lse_s)}


def case_terms_k1024(fkl, torch, dev):
    """K = 1024 (the sorting teacher prep), per-token weights and hard labels,
    a narrow last column block (d = 320), grad_h returned in bf16."""
    from workloads import make_workload
    wl = make_workload("tiny", N=200, d=320, V=3000, K=1024)
    h, W, ti, tl, _ = _dev_inputs(wl, torch, dev)
    rng = np.random.default_rng(11)
    w = torch.from_numpy(rng.uniform(0.0, 2.0, wl.N).astype(np.float32)).to(dev)
    y = torch.from_numpy(rng.integers(0, wl.V, wl.N).astype(np.int32)).to(dev)
    loss, lse, kl = fkl.forward(h, W, ti, tl, T=1.3, chunk=128, return_row_kl=True, row_weight=w, label=y,
                                label_weight=0.3)
    gh, gW = fkl.backward(h, W, ti, tl, lse, T=1.3, chunk=128, grad_h_dtype=torch.bfloat16, row_weight=w, label=y,
                          label_weight=0.3)
    return {"loss": _np(loss), "lse": _np(lse), "kl": _np(kl), "gh": _np(gh), "gW": _np(gW)}


def case_skips(fkl, torch, dev):
    """Each gradient skipped in turn (a frozen head; a frozen body)."""
    from workloads import make_workload
    wl = make_workload("tiny", N=260, d=64, V=1100, K=9)
    h, W, ti, tl, _ = _dev_inputs(wl, torch, dev)
    _, lse = fkl.forward(h, W, ti, tl, chunk=128)
    gh, _ = fkl.backward(h, W, ti, tl, lse, chunk=128, need_grad_W=False)
    _, gW = fkl.backward(h, W, ti, tl, lse, chunk=128, need_grad_h=False)
    return {"gh": _np(gh), "gW": _np(gW)}


def case_topk(fkl, torch, dev):
    """The teacher-cache builder on every route: fused (with a ragged last
    tile and several passes), materialised with a sampled threshold, whole-row,
    and a fused pass that the sample makes fail, so its guarded redo runs."""
    rng = np.random.default_rng(3)
    out = {}
    from workloads import bf16_bits

    def to_dev(x):
        return torch.from_numpy(bf16_bits(np.asarray(x, np.float32)).view(np.int16)).to(dev).view(torch.bfloat16)

    h = to_dev(rng.standard_normal((300, 64)))
    W = to_dev(rng.standard_normal((20000, 64)) / 8.0)
    for name, kw in (("fused", dict(chunk=128)), ("materialized", dict(materialize=True)),
                     ("direct", dict(direct=True))):
        ti, tl = fkl.topk(h, W, 100, **kw)
        out[f"{name}_idx"], out[f"{name}_logit"] = _np(ti), _np(tl)
    # sampled tiles (every 16th full tile of 256) hold the only non-zero
    # logits: fewer than K keys reach the threshold, so the pass is redone
    V = 5000
    cols = np.zeros(V, bool)
    for t in range(0, V // 256, 16):
        cols[t * 256:(t + 1) * 256] = True
    Wf = np.zeros((V, 16), np.float32)
    Wf[cols, 0] = 1.0
    hf = np.zeros((16, 16), np.float32)
    hf[:, 0] = 1.0
    ti, tl = fkl.topk(to_dev(hf), to_dev(Wf), 200)
    out["redo_idx"], out["redo_logit"] = _np(ti), _np(tl)
    return out


def case_fullsize(fkl, torch, dev):
    """The headline shape (two 16384-row forward passes, four 8192-row
    backward passes over 25 slabs of 8192 columns, the full gradient block) and the builder's default 16384-row pass at the
    large head. Summaries of every output (sums and largest magnitudes in
    fp64), and the builder's indices exactly."""
    from workloads.device import make_device_workload, perturbed_head
    wl = make_device_workload("gptoss20b", dev)
    loss, lse = fkl.forward(wl.h, wl.W, wl.t_idx, wl.t_logit, T=wl.T, chunk=wl.chunk)
    gh, gW = fkl.backward(wl.h, wl.W, wl.t_idx, wl.t_logit, lse, T=wl.T, chunk=wl.chunk)
    out = {"loss": _np(loss)}
    for name, t in (("lse", lse), ("gh", gh), ("gW", gW)):
        t64 = t.double()
        out[f"{name}_sum"] = np.array([t64.sum().item(), t64.abs().sum().item(), t64.abs().max().item()])
    del gh, gW, lse, wl
    tw = make_device_workload("temp", dev, N=16384)
    Wt = perturbed_head(tw.W, 4242, dev)
    ti, tl = fkl.topk(tw.h, Wt, 100)
    out["topk_idx"] = _np(ti)
    out["topk_logit_sum"] = np.array([tl.double().sum().item()])
    return out


def case_planted(fkl, torch, dev):
    """Backward whose gradient block is exactly full (512 rows x 2048 columns),
    with its span narrowed by 4 KiB: the debug build must skip the last row's
    stores and report the gradient block."""
    from workloads import make_workload
    wl = make_workload("tiny", N=512, d=64, V=2048, K=5)
    h, W, ti, tl, _ = _dev_inputs(wl, torch, dev)
    _, lse = fkl.forward(h, W, ti, tl, chunk=512, vslab=2048)
    os.environ["FKL_DEBUG_SHRINK_G"] = "1"
    try:
        fkl.backward(h, W, ti, tl, lse, chunk=512, vslab=2048)
        torch.cuda.synchronize()
        msg = ""
    except fkl.FklError as e:
        msg = str(e)
    finally:
        del os.environ["FKL_DEBUG_SHRINK_G"]
    return {"planted_msg": np.array(msg)}


CASES = {"ragged": case_ragged, "terms_k1024": case_terms_k1024, "skips": case_skips, "topk": case_topk}


def run_all(planted: bool = False, fullsize: bool = False) -> dict:
    import torch

    import output_projection_kl_amd as fkl
    dev = torch.device("cuda", 0)
    out = {}
    cases = dict(CASES)
    if fullsize:
        cases["fullsize"] = case_fullsize
    if planted:
        cases["planted"] = case_planted
    for name, fn in cases.items():
        print(f"[debug-cases] {name} with {fkl.library_path()}", flush=True)
        res = fn(fkl, torch, dev)
        torch.cuda.synchronize()
        out.update({f"{name}/{k}": v for k, v in res.items()})
    return out


if __name__ == "__main__":
    res = run_all(planted="--planted" in sys.argv, fullsize="--fullsize" in sys.argv)
    np.savez(sys.argv[1], **res)
    print("[debug-cases] done", flush=True)
