"""GPU parity of libfkl (through its C ABI) against the fp64 oracle.

Tolerances, for bf16 inputs with fp32 accumulation:
  loss:            |loss - loss_ref| / |loss_ref| <= 1e-3
  grad_h, grad_W:  max |grad - grad_ref| / max |grad_ref| <= 2e-2 (each tensor)
  row_lse:         max |row_lse - ref| <= 1e-3
Both sides read the same bf16-exact h, W and the same teacher cache.
"""

import numpy as np
import pytest
import torch

import oracle
import output_projection_kl_amd as fkl
from workloads import bf16_bits, bf16_to_f32, make_workload

pytestmark = pytest.mark.gpu

LOSS_RTOL = 1e-3
GRAD_TOL = 2e-2
LSE_ATOL = 1e-3


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _bits_to_dev(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _upload(wl, dev):
    h = _bits_to_dev(wl.h_bits, dev)
    W = _bits_to_dev(wl.W_bits, dev)
    ti = torch.from_numpy(wl.t_idx).to(dev)
    tl = torch.from_numpy(wl.t_logit).to(dev)
    m = torch.from_numpy(wl.mask).to(dev) if wl.mask is not None else None
    return h, W, ti, tl, m


def _rel_max(got, ref):
    scale = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (scale if scale > 0 else 1.0))


def _run_gpu(h, W, ti, tl, m, T, chunk=0, vslab=0, grad_loss=None):
    loss, lse, kl = fkl.forward(h, W, ti, tl, T=T, mask=m, chunk=chunk, vslab=vslab, return_row_kl=True)
    gl = None if grad_loss is None else torch.tensor([grad_loss], dtype=torch.float32, device=h.device)
    gh, gW = fkl.backward(h, W, ti, tl, lse, T=T, mask=m, grad_loss=gl, chunk=chunk, vslab=vslab)
    torch.cuda.synchronize()
    return (loss.item(), lse.cpu().numpy(), kl.cpu().numpy(), gh.cpu().numpy(), gW.cpu().numpy())


def _check_full(wl, T=None, chunk=0, vslab=0, grad_loss=1.0, label=""):
    dev = _dev()
    T = wl.T if T is None else T
    print(f"[parity] {label} N={wl.N} d={wl.d} V={wl.V} K={wl.K} T={T} chunk={chunk} vslab={vslab}",
          flush=True)
    h, W, ti, tl, m = _upload(wl, dev)
    loss, lse, kl, gh, gW = _run_gpu(h, W, ti, tl, m, T, chunk, vslab,
                                     None if grad_loss == 1.0 else grad_loss)
    hf, Wf = wl.h(), wl.W()
    r_loss, r_lse, r_kl = oracle.forward(hf, Wf, wl.t_idx, wl.t_logit, T, wl.mask)
    r_gh, r_gW = oracle.backward(hf, Wf, wl.t_idx, wl.t_logit, T, wl.mask, grad_loss=grad_loss)
    e_loss = abs(loss - r_loss) / max(abs(r_loss), 1e-30)
    e_lse = float(np.abs(lse - r_lse).max()) if wl.N else 0.0
    e_gh = _rel_max(gh, r_gh) if wl.N else 0.0
    e_gW = _rel_max(gW, r_gW)
    print(f"   loss {loss:.8g} ref {r_loss:.8g} rel {e_loss:.2e} | lse {e_lse:.2e} | "
          f"grad_h {e_gh:.2e} | grad_W {e_gW:.2e}", flush=True)
    assert e_loss <= LOSS_RTOL
    assert e_lse <= LSE_ATOL
    assert e_gh <= GRAD_TOL
    assert e_gW <= GRAD_TOL
    if wl.N:
        valid = np.ones(wl.N, bool) if wl.mask is None else wl.mask.astype(bool)
        assert np.abs(kl[valid] - r_kl[valid]).max() <= 1e-3 * max(1.0, np.abs(r_kl).max())
        assert np.all(kl[~valid] == 0.0)
        assert np.all(gh[~valid] == 0.0)
    return loss, lse, gh, gW


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("T", [1.0, 2.0])
def test_tiny(seed, T):
    wl = make_workload("tiny", seed_offset=seed)
    _check_full(wl, T=T, chunk=wl.chunk, label="tiny")


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_random_mask_multi_slab(seed):
    wl = make_workload("tiny", seed_offset=seed, mask="random25")
    _check_full(wl, chunk=64, vslab=1024, label="tiny-mask-slabs")


def test_ragged_shapes():
    """N, d and V off every tile size; several chunks and vocabulary slabs, and a ragged tail."""
    wl = make_workload("tiny", N=300, d=136, V=5000, K=7, mask="random25")
    _check_full(wl, T=0.7, chunk=128, vslab=768, grad_loss=2.5, label="ragged")


@pytest.mark.parametrize("d", [320, 264])
def test_hidden_size_with_a_narrow_last_column_block(d):
    """d = 256 + 64 and 256 + 8: the gradient contractions' last column block
    takes the 256 x 64 tile path (grad_h with transposed operands, grad_W with
    a plain one), over several chunks, slabs and vocabulary splits."""
    wl = make_workload("tiny", N=300, d=d, V=3000, K=9, mask="random25")
    _check_full(wl, T=1.3, chunk=128, vslab=768, grad_loss=0.8, label=f"narrow-d{d}")


def test_largest_teacher_list():
    """K = 1024, the largest supported teacher list, over a ragged vocabulary."""
    wl = make_workload("tiny", N=300, d=64, V=3000, K=1024)
    _check_full(wl, T=1.0, chunk=128, vslab=768, label="K=1024")


def test_smallest_hidden_size_and_single_row():
    """d = 8 (one 16-byte chunk per row) and N = 1."""
    _check_full(make_workload("tiny", N=77, d=8, V=1000, K=5), T=1.0, label="d=8")
    _check_full(make_workload("tiny", N=1, d=64, V=700, K=3), T=0.9, label="N=1")


def test_single_teacher_entry():
    wl = make_workload("tiny", N=96, d=64, V=1000, K=1)
    _check_full(wl, T=1.0, chunk=64, label="K=1")


def test_teacher_covers_vocabulary():
    wl = make_workload("tiny", N=40, d=64, V=64, K=64)
    _check_full(wl, T=1.5, label="K=V")


def test_zipf_teacher_reduced_vocab():
    wl = make_workload("llama3b", N=512, d=192, V=9000)
    _check_full(wl, chunk=256, vslab=2048, label="zipf")


def test_largest_hidden_size():
    """d = 65536, the largest supported hidden size (2048 contraction stages per tile)."""
    wl = make_workload("tiny", N=70, d=65536, V=300, K=8)
    _check_full(wl, T=1.0, label="d=65536")


def test_single_word_vocabulary():
    """V = K = 1: student and teacher are both certain of the only token, so the
    loss and both gradients vanish. The gradient block holds bf16(c q) - c p with
    c = T / n, so each of its entries is within c 2^-8 of zero, which bounds the
    gradients: |grad_h| <= c 2^-8 max|W| and |grad_W| <= T 2^-8 max|h|."""
    dev = _dev()
    wl = make_workload("tiny", N=33, d=64, V=1, K=1)
    h, W, ti, tl, m = _upload(wl, dev)
    T = 1.0
    loss, lse, kl, gh, gW = _run_gpu(h, W, ti, tl, m, T)
    r_lse = oracle.forward(wl.h(), wl.W(), wl.t_idx, wl.t_logit, T)[1]
    assert abs(loss) <= 1e-6 and np.abs(kl).max() <= 1e-6
    assert np.abs(lse - r_lse).max() <= LSE_ATOL
    c = T / wl.N
    assert np.abs(gh).max() <= 1.01 * c * 2.0**-8 * np.abs(wl.W()).max()
    assert np.abs(gW).max() <= 1.01 * T * 2.0**-8 * np.abs(wl.h()).max()


def test_confident_student_gradient_precision():
    """A student that puts most of its mass on one token per row and a teacher
    close to it: at that token q and p nearly cancel. G is formed as
    c (q - p) in fp32 and rounded to bf16 once, so each gradient row keeps the
    relative precision of bf16 (rounding c q and c p separately would leave an
    error of about c q 2^-9 at that token, several times the whole row's bf16
    error)."""
    dev = _dev()
    rng = np.random.default_rng(2024)
    N, d, V, K, T = 64, 256, 8192, 16, 1.0
    hf = bf16_to_f32(bf16_bits(rng.standard_normal((N, d)).astype(np.float32)))
    W32 = (rng.standard_normal((V, d)) / np.sqrt(d)).astype(np.float32)
    top = rng.choice(V, N, replace=False)
    W32[top] += (0.75 * hf / np.linalg.norm(hf, axis=1, keepdims=True)).astype(np.float32)
    Wf = bf16_to_f32(bf16_bits(W32))
    z = hf.astype(np.float64) @ Wf.astype(np.float64).T
    zt = z + 0.05 * rng.standard_normal(z.shape)
    t_idx = np.argsort(-zt, axis=1)[:, :K].astype(np.int32)
    t_logit = np.take_along_axis(zt, t_idx, 1).astype(np.float32)
    q_top = np.exp(z[np.arange(N), top] - np.log(np.exp(z - z.max(1, keepdims=True)).sum(1)) - z.max(1))
    assert np.median(q_top) > 0.5      # the student is confident
    h = torch.from_numpy(bf16_bits(hf).view(np.int16)).to(dev).view(torch.bfloat16)
    W = torch.from_numpy(bf16_bits(Wf).view(np.int16)).to(dev).view(torch.bfloat16)
    ti, tl = torch.from_numpy(t_idx).to(dev), torch.from_numpy(t_logit).to(dev)
    _, _, _, gh, gW = _run_gpu(h, W, ti, tl, None, T)
    r_gh, r_gW = oracle.backward(hf, Wf, t_idx, t_logit, T, None)
    row_err = np.linalg.norm(gh - r_gh, axis=1) / np.linalg.norm(r_gh, axis=1)
    print(f"   grad_h row relative error: median {np.median(row_err):.2e} max {row_err.max():.2e}", flush=True)
    assert np.median(row_err) <= 4e-3
    assert _rel_max(gW, r_gW) <= GRAD_TOL


def test_empty_rows():
    dev = _dev()
    d, V, K = 64, 300, 5
    h = torch.empty((0, d), dtype=torch.bfloat16, device=dev)
    W = torch.randn((V, d), device=dev).to(torch.bfloat16)
    ti = torch.empty((0, K), dtype=torch.int32, device=dev)
    tl = torch.empty((0, K), dtype=torch.float32, device=dev)
    loss, lse = fkl.forward(h, W, ti, tl)
    gh, gW = fkl.backward(h, W, ti, tl, lse)
    torch.cuda.synchronize()
    assert loss.item() == 0.0
    assert gW.abs().max().item() == 0.0 and gh.numel() == 0


def test_all_rows_masked():
    wl = make_workload("tiny", N=100, d=64, V=700, K=4)
    wl.mask = np.zeros(wl.N, np.uint8)
    dev = _dev()
    h, W, ti, tl, m = _upload(wl, dev)
    loss, lse, kl, gh, gW = _run_gpu(h, W, ti, tl, m, 1.0)
    assert loss == 0.0 and np.all(kl == 0) and np.all(gh == 0) and np.all(gW == 0)
    r_lse = oracle.forward(wl.h(), wl.W(), wl.t_idx, wl.t_logit, 1.0, wl.mask)[1]
    assert np.abs(lse - r_lse).max() <= LSE_ATOL


def test_self_distillation_is_near_zero():
    """Teacher = the student's own logits at K indices with a wide margin:
    KL = -log Q_r, the student's mass outside those indices, so ~0.

    h is the min-norm solution of W[idx] h = B + noise with B = 100: |h| is
    about B sqrt(K) = 400, so the other logits spread with std B sqrt(K/d) =
    12.5 and their largest stays about 55 below the teacher's, a tail mass
    near V e^-55 ~ 1e-21. The oracle gets the exact fp64 logits as the
    teacher and must give |loss| <= 1e-12 (fp64 rounding at logits ~100).
    The library gets them rounded to fp32 (its input type): the rounding
    changes the exact KL only at second order (~1e-11), and its own fp32
    arithmetic at logits ~100 (ulp ~8e-6, a handful of rounded terms per
    row) bounds |loss| by 1e-4.
    """
    dev = _dev()
    rng = np.random.default_rng(2024)
    N, d, V, K, B = 256, 1024, 4096, 16, 100.0
    W32 = (rng.standard_normal((V, d)) / np.sqrt(d)).astype(np.float32)
    Wb = bf16_bits(W32)
    Wf = bf16_to_f32(Wb).astype(np.float64)
    t_idx = np.stack([rng.choice(V, K, replace=False) for _ in range(N)]).astype(np.int32)
    tgt = rng.standard_normal((N, K)) + B
    h64 = np.stack([np.linalg.lstsq(Wf[t_idx[r]], tgt[r], rcond=None)[0] for r in range(N)])
    hb = bf16_bits(h64.astype(np.float32))
    hf = bf16_to_f32(hb).astype(np.float64)
    s = hf @ Wf.T
    t_exact = np.take_along_axis(s, t_idx.astype(np.int64), axis=1)
    # closed form: KL_r = logsumexp_V(s_r) - logsumexp_K(s_r[idx]) = -log Q_r
    def lse(x):
        m = x.max(axis=1, keepdims=True)
        return (m + np.log(np.exp(x - m).sum(axis=1, keepdims=True)))[:, 0]
    closed = float(np.mean(lse(s) - lse(t_exact)))
    is_teacher = np.zeros((N, V), bool)
    np.put_along_axis(is_teacher, t_idx.astype(np.int64), True, axis=1)
    margin = float(np.min(t_exact.min(axis=1) - np.where(is_teacher, -np.inf, s).max(axis=1)))
    r_loss = oracle.forward(hf, Wf, t_idx, t_exact, 1.0)[0]
    t_logit = t_exact.astype(np.float32)
    h = _bits_to_dev(hb, dev)
    W = _bits_to_dev(Wb, dev)
    loss, lse_g = fkl.forward(h, W, torch.from_numpy(t_idx).to(dev), torch.from_numpy(t_logit).to(dev))
    torch.cuda.synchronize()
    print(f"[self-distill] margin {margin:.1f} closed form {closed:.3e} oracle {r_loss:.3e} "
          f"gpu {loss.item():.3e}", flush=True)
    assert margin > 30.0
    assert 0.0 <= closed <= 1e-12
    assert abs(r_loss) <= 1e-12
    assert abs(loss.item()) <= 1e-4


def test_chunk_invariance():
    dev = _dev()
    wl = make_workload("tiny", seed_offset=5, mask="random25")
    h, W, ti, tl, m = _upload(wl, dev)
    # with vslab = 0 the passes are at least min(N, 16384) rows forward and
    # min(N, 8192) backward; an explicit vslab keeps chunk-row passes
    outs = [_run_gpu(h, W, ti, tl, m, 1.0, chunk=c) for c in (64, 100, 256)]
    outs += [_run_gpu(h, W, ti, tl, m, 1.0, chunk=c, vslab=1024) for c in (64, 100)]
    for o in outs[1:]:
        assert abs(o[0] - outs[0][0]) <= 1e-6 * abs(outs[0][0])
        assert np.abs(o[1] - outs[0][1]).max() <= 1e-5
        assert _rel_max(o[3], outs[0][3]) <= 1e-3
        assert _rel_max(o[4], outs[0][4]) <= 1e-3


def test_chunk_invariance_explicit_slab_8192_rows():
    """8192 rows with an explicit slab, so chunk sets the pass rows in both
    directions: 256, 1024 and 4096 rows per pass (32, 8 and 2 passes) must
    agree with each other (loss within 1e-6, row_lse within 1e-5, gradients
    within 1e-3) and with the oracle."""
    wl = make_workload("tiny", seed_offset=6, N=8192, d=256, V=8192, K=16, mask="random25")
    dev = _dev()
    h, W, ti, tl, m = _upload(wl, dev)
    outs = []
    for c in (256, 1024, 4096):
        p = fkl.plan_info(wl.N, wl.d, wl.V, wl.K, 1.0, chunk=c, vslab=2048)
        assert p["fwd_rows"] == p["bwd_rows"] == c and p["slabs"] == 4
        print(f"[chunk-invariance] chunk {c}: {p['bwd_passes']} passes x {p['slabs']} slabs", flush=True)
        outs.append(_run_gpu(h, W, ti, tl, m, 1.0, chunk=c, vslab=2048))
    for o in outs[1:]:
        assert abs(o[0] - outs[0][0]) <= 1e-6 * abs(outs[0][0])
        assert np.abs(o[1] - outs[0][1]).max() <= 1e-5
        assert _rel_max(o[3], outs[0][3]) <= 1e-3
        assert _rel_max(o[4], outs[0][4]) <= 1e-3
    r_loss, r_lse, _ = oracle.forward(wl.h(), wl.W(), wl.t_idx, wl.t_logit, 1.0, wl.mask)
    r_gh, r_gW = oracle.backward(wl.h(), wl.W(), wl.t_idx, wl.t_logit, 1.0, wl.mask)
    for o in outs:
        assert abs(o[0] - r_loss) <= LOSS_RTOL * abs(r_loss)
        assert np.abs(o[1] - r_lse).max() <= LSE_ATOL
        assert _rel_max(o[3], r_gh) <= GRAD_TOL
        assert _rel_max(o[4], r_gW) <= GRAD_TOL


def test_forward_and_backward_pass_rows_differ():
    """12000 rows with the default slab: the forward runs one pass of 12000
    rows (its floor is 16384), the backward two passes of 8192 and 3808 rows
    (a ragged last row block in both). Against the oracle at the parity bar,
    and against the same call with 1024-row passes in both directions."""
    wl = make_workload("tiny", seed_offset=8, N=12000, d=136, V=3000, K=16, mask="random25")
    dev = _dev()
    p = fkl.plan_info(wl.N, wl.d, wl.V, wl.K, 1.0)
    assert (p["fwd_rows"], p["fwd_passes"], p["bwd_rows"], p["bwd_passes"]) == (12000, 1, 8192, 2)
    print(f"[pass-rows] N={wl.N}: forward {p['fwd_passes']} x {p['fwd_rows']}, "
          f"backward {p['bwd_passes']} x {p['bwd_rows']}", flush=True)
    h, W, ti, tl, m = _upload(wl, dev)
    got = _run_gpu(h, W, ti, tl, m, 1.0)
    alt = _run_gpu(h, W, ti, tl, m, 1.0, chunk=1024, vslab=1024)
    assert abs(got[0] - alt[0]) <= 1e-6 * abs(alt[0])
    assert np.abs(got[1] - alt[1]).max() <= 1e-5
    assert _rel_max(got[3], alt[3]) <= 1e-3
    assert _rel_max(got[4], alt[4]) <= 1e-3
    r_loss, r_lse, _ = oracle.forward(wl.h(), wl.W(), wl.t_idx, wl.t_logit, 1.0, wl.mask)
    r_gh, r_gW = oracle.backward(wl.h(), wl.W(), wl.t_idx, wl.t_logit, 1.0, wl.mask)
    assert abs(got[0] - r_loss) <= LOSS_RTOL * abs(r_loss)
    assert np.abs(got[1] - r_lse).max() <= LSE_ATOL
    assert _rel_max(got[3], r_gh) <= GRAD_TOL
    assert _rel_max(got[4], r_gW) <= GRAD_TOL
    # masked rows: exactly zero gradient rows
    assert np.all(got[3][~wl.mask.astype(bool)] == 0.0)


def test_bitwise_determinism():
    dev = _dev()
    wl = make_workload("tiny", seed_offset=7)
    h, W, ti, tl, m = _upload(wl, dev)
    a = _run_gpu(h, W, ti, tl, m, 1.0, chunk=64, vslab=1024)
    b = _run_gpu(h, W, ti, tl, m, 1.0, chunk=64, vslab=1024)
    assert a[0] == b[0]
    for x, y in zip(a[1:], b[1:]):
        assert np.array_equal(x, y)


def test_validate_teacher():
    dev = _dev()
    wl = make_workload("tiny", N=64, d=64, V=500, K=9)
    ti = torch.from_numpy(wl.t_idx).to(dev)
    tl = torch.from_numpy(wl.t_logit).to(dev)
    assert fkl.validate_teacher(ti, tl, wl.V) == 0
    bad_i = wl.t_idx.copy()
    bad_l = wl.t_logit.copy()
    bad_i[3, 2] = bad_i[3, 5]          # repeated index
    bad_i[10, 0] = wl.V                # out of range
    bad_i[11, 4] = -1                  # negative
    bad_l[20, 1] = np.nan              # non-finite logit
    n_bad = fkl.validate_teacher(torch.from_numpy(bad_i).to(dev), torch.from_numpy(bad_l).to(dev), wl.V)
    assert n_bad == 4


def test_validate_environment_refuses_bad_teacher(monkeypatch):
    """FKL_VALIDATE=1: forward and backward check the teacher lists first and
    refuse a repeated index with FKL_EINDEX; good lists give the usual results."""
    dev = _dev()
    wl = make_workload("tiny", N=64, d=64, V=500, K=9)
    h, W, ti, tl, m = _upload(wl, dev)
    l0, lse0 = fkl.forward(h, W, ti, tl)
    g0 = fkl.backward(h, W, ti, tl, lse0)
    bad_i = wl.t_idx.copy()
    bad_i[3, 2] = bad_i[3, 5]
    bad = torch.from_numpy(bad_i).to(dev)
    monkeypatch.setenv("FKL_VALIDATE", "1")
    l1, lse1 = fkl.forward(h, W, ti, tl)
    g1 = fkl.backward(h, W, ti, tl, lse1)
    torch.cuda.synchronize()
    assert l1.item() == l0.item() and torch.equal(g1[0], g0[0]) and torch.equal(g1[1], g0[1])
    with pytest.raises(fkl.FklError) as e:
        fkl.forward(h, W, bad, tl)
    assert e.value.status == 3 and "1 rows rejected" in str(e.value)
    with pytest.raises(fkl.FklError) as e:
        fkl.backward(h, W, bad, tl, lse1)
    assert e.value.status == 3


def test_caller_workspace_reuse():
    """One workspace buffer serves repeated calls; results match fresh allocations."""
    dev = _dev()
    wl = make_workload("tiny", seed_offset=3)
    h, W, ti, tl, m = _upload(wl, dev)
    fb, bb = fkl.workspace_size(wl.N, wl.d, wl.V, wl.K, 1.0, chunk=64)
    ws = torch.empty(max(fb, bb), dtype=torch.uint8, device=dev)
    l1, lse1 = fkl.forward(h, W, ti, tl, chunk=64, workspace=ws)
    g1 = fkl.backward(h, W, ti, tl, lse1, chunk=64, workspace=ws)
    l2, lse2 = fkl.forward(h, W, ti, tl, chunk=64)
    g2 = fkl.backward(h, W, ti, tl, lse2, chunk=64)
    torch.cuda.synchronize()
    assert l1.item() == l2.item()
    assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1])


def test_workspace_of_any_dtype_is_sized_in_bytes():
    """A caller's workspace is measured in bytes whatever its dtype; one a byte short is refused."""
    dev = _dev()
    wl = make_workload("tiny", seed_offset=4)
    h, W, ti, tl, m = _upload(wl, dev)
    fb, bb = fkl.workspace_size(wl.N, wl.d, wl.V, wl.K, 1.0, chunk=64)
    nb = max(fb, bb)
    ws = torch.empty((nb + 3) // 4, dtype=torch.float32, device=dev)
    l1, lse1 = fkl.forward(h, W, ti, tl, chunk=64, workspace=ws)
    g1 = fkl.backward(h, W, ti, tl, lse1, chunk=64, workspace=ws)
    l2, lse2 = fkl.forward(h, W, ti, tl, chunk=64)
    g2 = fkl.backward(h, W, ti, tl, lse2, chunk=64)
    torch.cuda.synchronize()
    assert l1.item() == l2.item()
    assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1])
    short = torch.empty(fb - 1, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError):
        fkl.forward(h, W, ti, tl, chunk=64, workspace=short)


@pytest.mark.parametrize("T", [0.5, 1.0])
def test_wide_logit_range(T):
    """Logit scale grows ~400x across the vocabulary (row maxima in the last
    tiles far above the first tiles'), exercising the online max offset."""
    from workloads import bf16_bits
    wl = make_workload("tiny", N=256, d=64, V=3000, K=12, seed_offset=11)
    scale = np.linspace(0.1, 40.0, wl.V, dtype=np.float32)[:, None]
    wl.W_bits = bf16_bits(bf16_to_f32(wl.W_bits) * scale)
    _check_full(wl, T=T, chunk=128, vslab=1024, label="wide-range")


def test_large_logits_do_not_overflow():
    """Logits around 10^3 in magnitude: exp must never be taken unshifted."""
    from workloads import bf16_bits
    wl = make_workload("tiny", N=128, d=64, V=1500, K=6, seed_offset=12)
    wl.h_bits = bf16_bits(bf16_to_f32(wl.h_bits) * 64.0)
    wl.W_bits = bf16_bits(bf16_to_f32(wl.W_bits) * 16.0)
    _check_full(wl, T=1.0, label="large-logits")
