"""Seeded generators: determinism, teacher-cache invariants, masks, bf16 rounding."""

import numpy as np
import pytest

from workloads import (bf16_bits, bf16_to_f32, make_workload, packed_document_mask,
                       uniform_teacher, zipf_uniform_teacher)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-9, 1.0 + 3 * 2**-8, -2.5, 3.0e38, 1e-40], np.float32)
    got = bf16_to_f32(bf16_bits(x))
    # bf16 keeps 7 mantissa bits, so the spacing above 1 is 2^-7:
    # 1 + 2^-8 is a tie and goes to the even neighbour 1.0; 1 + 3*2^-9 rounds up to 1 + 2^-7;
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 (odd) and 1 + 2^-6 (even) and goes up
    np.testing.assert_array_equal(got[:5], np.array([1.0, 1.0, 1.0 + 2**-7, 1.0 + 2**-6, -2.5], np.float32))
    assert np.isfinite(got[5])
    # against torch's own conversion
    import torch
    y = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 100
    ref = torch.tensor(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_bits(y), ref)


def test_determinism_and_seed_offsets():
    a = make_workload("tiny")
    b = make_workload("tiny")
    c = make_workload("tiny", seed_offset=1)
    for f in ("h_bits", "W_bits", "t_idx", "t_logit"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.h_bits, c.h_bits)


def _teacher_ok(t_idx, t_logit, V):
    assert t_idx.dtype == np.int32 and t_logit.dtype == np.float32
    assert t_idx.min() >= 0 and t_idx.max() < V
    srt = np.sort(t_idx, axis=1)
    assert not np.any(srt[:, 1:] == srt[:, :-1])
    assert np.all(np.diff(t_logit, axis=1) <= 0)


def test_tiny_workload_shapes_and_distributions():
    w = make_workload("tiny")
    assert w.h_bits.shape == (256, 256) and w.W_bits.shape == (4096, 256)
    _teacher_ok(w.t_idx, w.t_logit, w.V)
    assert abs(w.h().std() - 1.0) < 0.02
    assert abs(w.W().std() * np.sqrt(w.d) - 1.0) < 0.02
    assert abs(w.t_logit.std() - 3.0) < 0.3
    assert w.mask is None


def test_zipf_half_is_heavy_and_distinct():
    rng = np.random.default_rng(5)
    V, K, N = 128256, 100, 2000
    idx = zipf_uniform_teacher(rng, N, V, K)
    assert idx.shape == (N, K)
    srt = np.sort(idx, axis=1)
    assert not np.any(srt[:, 1:] == srt[:, :-1])
    zipf_vals, zipf_counts = np.unique(idx[:, :50], return_counts=True)
    _, uni_counts = np.unique(idx[:, 50:], return_counts=True)
    # the most popular Zipf token appears in nearly every row; uniform tokens rarely repeat
    assert zipf_counts.max() > 0.9 * N
    assert uni_counts.max() < 10


def test_uniform_teacher_small_vocab():
    rng = np.random.default_rng(9)
    idx = uniform_teacher(rng, 300, 20, 20)   # K = V forces full permutations
    assert np.all(np.sort(idx, axis=1) == np.arange(20))


def test_packed_mask_marks_document_ends():
    rng = np.random.default_rng(3)
    m = packed_document_mask(rng, 1000)
    assert m.dtype == np.uint8 and m[-1] == 0
    assert (m == 0).sum() == 8
    w = make_workload("long64k", N=4096, V=1024, d=64)
    assert (w.mask == 0).sum() == 8 and w.mask[-1] == 0


def test_random25_mask_variant():
    w = make_workload("tiny", mask="random25")
    frac = 1.0 - w.mask.mean()
    assert 0.15 < frac < 0.35


@pytest.mark.parametrize("name", ["llama3b", "gptoss20b"])
def test_large_recipes_at_reduced_rows(name):
    w = make_workload(name, N=64, V=2048, d=64)
    _teacher_ok(w.t_idx, w.t_logit, w.V)
    assert w.K == 100
