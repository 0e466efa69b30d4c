"""Per-launch event timing (fkl_trace_enable / fkl_trace_read). Every traced
launch is reported exactly once. That holds also when another thread reads the
statistics while launches are still being enqueued: a read takes only the
records whose stop event has been recorded."""

import threading

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


def _add(totals, stats):
    for k in stats:
        assert k["launches"] > 0 and k["total_ms"] >= 0.0 and k["min_ms"] <= k["max_ms"]
        totals[k["name"]] = totals.get(k["name"], 0) + k["launches"]


def test_every_launch_reported_once_with_concurrent_reads():
    dev = _dev()
    wl = make_workload("tiny", N=512, d=64, V=2048, K=8)
    h, W = _bits(wl.h_bits, dev), _bits(wl.W_bits, dev)
    ti, tl = torch.from_numpy(wl.t_idx).to(dev), torch.from_numpy(wl.t_logit).to(dev)
    fkl.trace_read()  # drop anything recorded before
    fkl.trace_enable(True)
    try:
        fkl.forward(h, W, ti, tl, T=1.0)
        torch.cuda.synchronize()
        per_call = {}
        _add(per_call, fkl.trace_read())
        assert per_call.get("fwd_sweep", 0) >= 1, per_call

        calls = 60
        totals, errors = {}, []
        done = threading.Event()

        def reader():
            try:
                while not done.is_set():
                    _add(totals, fkl.trace_read())
            except Exception as e:  # reported below
                errors.append(e)

        t = threading.Thread(target=reader)
        t.start()
        for _ in range(calls):
            fkl.forward(h, W, ti, tl, T=1.0)
        torch.cuda.synchronize()
        done.set()
        t.join()
        _add(totals, fkl.trace_read())
    finally:
        fkl.trace_enable(False)
    assert not errors, errors
    assert totals == {k: v * calls for k, v in per_call.items()}, (totals, per_call)
