"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, plans workspace, and rejects bad arguments before touching a
device (so these run without a GPU)."""

import ctypes
import os
import re
import subprocess

import pytest

import output_projection_kl_amd as fkl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fkl.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fkl_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert _declared_functions() == sorted(fkl.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = fkl.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", fkl.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(L, name)
    assert L.fkl_version() >= 100


def test_status_strings():
    L = fkl.lib()
    for code in range(6):
        assert L.fkl_status_string(code)
    assert L.fkl_status_string(99) == b"unknown status"


def test_workspace_is_independent_of_rows():
    a = fkl.workspace_size(65536, 2880, 201088, 100, 1.0, chunk=4096)
    b = fkl.workspace_size(262144, 2880, 201088, 100, 1.0, chunk=4096)
    assert a == b
    fwd, bwd = a
    # backward holds one bf16 gradient block of chunk x vslab (64 Mi elements by default)
    assert 128 << 20 <= bwd <= (128 << 20) + (16 << 20)
    assert fwd < 16 << 20


def test_workspace_scales_with_chunk_and_slab():
    _, b1 = fkl.workspace_size(32768, 2880, 201088, 100, 1.0, chunk=4096, vslab=4096)
    _, b2 = fkl.workspace_size(32768, 2880, 201088, 100, 1.0, chunk=4096, vslab=8192)
    assert b2 - b1 == 4096 * 4096 * 2


@pytest.mark.parametrize("field,value,status", [
    ("N", -1, 1), ("d", 12, 1), ("d", 0, 1), ("V", 0, 1), ("K", 0, 1), ("K", 2000, 5),
    ("T", 0.0, 1), ("T", -1.0, 1), ("T", float("inf"), 1), ("chunk", -3, 1), ("vslab", -1, 1),
])
def test_shape_errors(field, value, status):
    s = fkl.make_shape(16, 64, 100, 5)
    setattr(s, field, value)
    f = ctypes.c_size_t(0)
    b = ctypes.c_size_t(0)
    assert fkl.lib().fkl_workspace_size(ctypes.byref(s), ctypes.byref(f), ctypes.byref(b)) == status
    assert fkl.lib().fkl_last_error()


def test_k_larger_than_v_rejected():
    s = fkl.make_shape(4, 64, 10, 11)
    assert fkl.lib().fkl_workspace_size(ctypes.byref(s), None, None) == 1


def _fwd(s, h=8192, W=16384, ti=4096, tl=4096, loss=256, lse=256, ws=1 << 20, ws_bytes=1 << 30):
    vp = ctypes.c_void_p
    return fkl.lib().fkl_forward(ctypes.byref(s), vp(h), vp(W), vp(ti), vp(tl), vp(0), vp(0), vp(loss), vp(lse),
                                 vp(0), vp(ws), ctypes.c_size_t(ws_bytes), vp(0))


def test_forward_argument_errors_before_any_device_work():
    s = fkl.make_shape(16, 64, 100, 5)
    assert _fwd(s, h=0) == 1            # NULL h
    assert _fwd(s, W=8) == 1            # misaligned W (needs 16 bytes)
    assert _fwd(s, lse=2) == 1          # misaligned row_lse
    assert _fwd(s, loss=0) == 1         # NULL loss
    assert _fwd(s, ws=0) == 2           # NULL workspace
    assert _fwd(s, ws=1 << 20 | 16) == 2  # misaligned workspace
    assert _fwd(s, ws_bytes=16) == 2    # workspace too small
    assert b"workspace" in fkl.lib().fkl_last_error()


def test_backward_argument_errors_before_any_device_work():
    L = fkl.lib()
    s = fkl.make_shape(16, 64, 100, 5)
    vp = ctypes.c_void_p

    def bwd(grad_h=8192, grad_W=16384, ws_bytes=1 << 30, grad_loss=0):
        return L.fkl_backward(ctypes.byref(s), vp(8192), vp(16384), vp(4096), vp(4096), vp(0), vp(0), vp(256),
                              vp(grad_loss), vp(grad_h), vp(grad_W), vp(1 << 20), ctypes.c_size_t(ws_bytes),
                              vp(0))
    assert bwd(grad_h=0) == 1
    assert bwd(grad_W=0) == 1
    assert bwd(grad_W=2) == 1
    assert bwd(grad_W=16384 + 4) == 1   # grad_W needs 16-byte alignment
    assert bwd(grad_h=8192 + 8) == 1    # so does grad_h
    assert bwd(grad_loss=6) == 1
    assert bwd(ws_bytes=100) == 2


def test_validate_argument_errors():
    L = fkl.lib()
    s = fkl.make_shape(16, 64, 100, 5)
    vp = ctypes.c_void_p
    assert L.fkl_validate_teacher(ctypes.byref(s), vp(4096), vp(4096), vp(0), vp(0)) == 1
    assert L.fkl_validate_teacher(ctypes.byref(s), vp(0), vp(4096), vp(256), vp(0)) == 1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fkl, "_lib", None)
    monkeypatch.setenv("FKL_LIBRARY", str(tmp_path / "missing.so"))
    with pytest.raises(fkl.FklError):
        fkl.lib()


def test_topk_argument_errors_before_any_device_work():
    L = fkl.lib()
    vp = ctypes.c_void_p

    def call(N=16, d=64, V=100, K=5, chunk=0, h=8192, W=16384, ti=4096, tl=4096, ws=1 << 20, ws_bytes=1 << 30,
             flags=0):
        s = fkl.TopkShape(N, d, V, K, chunk, flags)
        return L.fkl_topk(ctypes.byref(s), vp(h), vp(W), vp(ti), vp(tl), vp(ws), ctypes.c_size_t(ws_bytes), vp(0))
    assert call(d=12) == 1
    assert call(K=0) == 1
    assert call(K=101) == 1       # K > V
    assert call(K=2000, V=5000) == 5
    assert call(chunk=-1) == 1
    assert call(flags=0x4) == 1   # unknown flag
    assert call(flags=fkl.TOPK_DIRECT, ws_bytes=16) == 2  # the whole-row route is a known flag
    assert call(h=0) == 1
    assert call(W=8) == 1         # misaligned
    assert call(ti=2) == 1
    assert call(ws=0) == 2
    assert call(ws_bytes=16) == 2
    assert call(N=0, h=0, W=0, ti=0, tl=0, ws=0) == 0   # nothing to do


def test_topk_workspace_sizes():
    """Materialised route: one fp32 logits block of the pass's rows (rounded up
    to 256) x V (rounded up to 256). Fused route (default): the compact copy of
    the sampled tiles of W, then the larger of the pass's fused buffers and the
    logits block of its redo."""
    M = fkl.TOPK_MATERIALIZE
    assert fkl.topk_workspace_size(16384, 4096, 128256, 100, chunk=256, flags=M) == 256 + 256 * 128256 * 4
    assert fkl.topk_workspace_size(1000, 64, 1000, 10, chunk=300, flags=M) == 256 + 512 * 1024 * 4
    b = fkl.topk_workspace_size(16384, 4096, 128256, 100, flags=M)
    assert 256 * 128256 * 4 <= b <= (512 << 20) + 256
    # fused, large head: 16 sampled tiles (every 32nd of 501) of 256 rows x 4096
    # bf16 = 32 MiB, then the one 16384-row pass's buffers, larger than the
    # redo's 1024-row logits block (501 MiB): the sample's fp32 logits, the
    # thresholds, 8 candidate slices per row (4 vocabulary splits x 2 column
    # quarters) of 2 * ceil(1024 / 4) + 16 keys, their counts, and the extra
    # slice of sampled keys (j = ceil(1024 * 4096 / 128256) = 33, 2j + 256 slots)
    R, S = 16384, 16 * 256
    fused = R * S * 4 + R * 8 + R * 8 * 4 + R * 8 * (2 * 256 + 16) * 8 + R * 4 + R * (2 * 33 + 256) * 8
    f = fkl.topk_workspace_size(16384, 4096, 128256, 100)
    assert fused > 1024 * 128256 * 4
    assert f == 256 + S * 4096 * 2 + fused
    assert fkl.topk_workspace_size(16384, 4096, 128256, 100, flags=fkl.TOPK_DIRECT) == b


def test_backward_flags_checked_on_the_host():
    L = fkl.lib()
    vp = ctypes.c_void_p

    def bwd(flags, grad_h=8192, grad_W=16384, ws_bytes=1 << 30):
        s = fkl.make_shape(16, 64, 100, 5, flags=flags)
        return L.fkl_backward(ctypes.byref(s), vp(8192), vp(16384), vp(4096), vp(4096), vp(0), vp(0), vp(256),
                              vp(0), vp(grad_h), vp(grad_W), vp(1 << 20), ctypes.c_size_t(ws_bytes), vp(0))
    assert bwd(0x40) == 1                                   # unknown bit
    assert bwd(0, grad_W=0) == 1                            # grad_W needed
    assert bwd(fkl.SKIP_GRAD_W, grad_W=0, ws_bytes=16) == 2  # NULL grad_W accepted when skipped
    assert bwd(fkl.SKIP_GRAD_H, grad_h=0, ws_bytes=16) == 2  # NULL grad_h accepted when skipped
    assert bwd(fkl.SKIP_GRAD_H | fkl.SKIP_GRAD_W, grad_h=0, grad_W=0) == 0  # nothing to do, no device work


def test_bf16_grad_h_adds_an_fp32_accumulator_to_the_workspace():
    _, b0 = fkl.workspace_size(32768, 2880, 201088, 100, 1.0, chunk=4096)
    _, b1 = fkl.workspace_size(32768, 2880, 201088, 100, 1.0, chunk=4096, flags=fkl.GRAD_H_BF16)
    assert b1 - b0 == 8192 * 2880 * 4      # one backward pass of 8192 rows
    _, b2 = fkl.workspace_size(32768, 2880, 201088, 100, 1.0, chunk=4096,
                               flags=fkl.GRAD_H_BF16 | fkl.SKIP_GRAD_H)
    assert b2 == b0


def test_loss_terms_checked_on_the_host():
    vp = ctypes.c_void_p
    s = fkl.make_shape(16, 64, 100, 5)
    for a in (-0.1, 1.5, float("nan")):
        t = fkl.Terms(None, 4096, a)
        rc = fkl.lib().fkl_forward(ctypes.byref(s), vp(8192), vp(16384), vp(4096), vp(4096), vp(0),
                                   ctypes.byref(t), vp(256), vp(256), vp(0), vp(1 << 20), ctypes.c_size_t(1 << 30),
                                   vp(0))
        assert rc == 1
    t = fkl.Terms(4098, None, 0.0)   # misaligned weights
    rc = fkl.lib().fkl_forward(ctypes.byref(s), vp(8192), vp(16384), vp(4096), vp(4096), vp(0), ctypes.byref(t),
                               vp(256), vp(256), vp(0), vp(1 << 20), ctypes.c_size_t(1 << 30), vp(0))
    assert rc == 1


def test_operand_views_stay_under_2_gib():
    """Each operand view is addressed with a 32-bit byte size: shapes that would
    need a larger h chunk, W slab or gradient block are refused; the default
    slab is capped instead."""
    L = fkl.lib()
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    s = fkl.make_shape(1 << 20, 65536, 50000, 10, chunk=32768)      # h chunk 4 GiB
    assert L.fkl_workspace_size(ctypes.byref(s), ctypes.byref(f), ctypes.byref(b)) == 5
    s = fkl.make_shape(4096, 2880, 1 << 22, 10, chunk=4096, vslab=1 << 20)  # W slab 5.6 GiB
    assert L.fkl_workspace_size(ctypes.byref(s), ctypes.byref(f), ctypes.byref(b)) == 5
    s = fkl.make_shape(4096, 65536, 1 << 22, 10, chunk=256)         # default slab capped
    assert L.fkl_workspace_size(ctypes.byref(s), ctypes.byref(f), ctypes.byref(b)) == 0
    assert b.value < (2 << 30)


def test_backward_pass_rows_follow_gradient_block():
    """With the default slab the forward takes passes of max(chunk, min(N, 16384))
    rows and the backward of max(chunk, min(N, 8192)), so a small chunk does not
    shrink the passes or grow the workspace; an explicit slab keeps chunk-row
    passes."""
    f1024, b1024 = fkl.workspace_size(65536, 3072, 128256, 100, 1.0, chunk=1024)
    f4096, b4096 = fkl.workspace_size(65536, 3072, 128256, 100, 1.0, chunk=4096)
    f8192, b8192 = fkl.workspace_size(65536, 3072, 128256, 100, 1.0, chunk=8192)
    assert b1024 == b4096 == b8192
    assert f1024 == f4096 == f8192
    # gradient block rows x vslab bf16 follows chunk when vslab is given
    # (grad_h skipped so that no vocabulary-split partial sums enter)
    _, b_small = fkl.workspace_size(65536, 3072, 128256, 100, 1.0, chunk=1024, vslab=4096,
                                    flags=fkl.SKIP_GRAD_H)
    _, b_big = fkl.workspace_size(65536, 3072, 128256, 100, 1.0, chunk=4096, vslab=4096,
                                  flags=fkl.SKIP_GRAD_H)
    assert b_big - b_small >= (4096 - 1024) * 4096 * 2
    # N below the pass floor: one pass of N rows
    _, bn = fkl.workspace_size(300, 64, 1000, 5, 1.0, chunk=64)
    _, bn2 = fkl.workspace_size(300, 64, 1000, 5, 1.0, chunk=300)
    assert bn == bn2


def test_plan_info_reports_the_passes_that_run():
    # default slab: forward passes of at least min(N, 16384) rows, backward
    # passes of at least min(N, 8192), slab sized for a 64 Mi-element block
    p = fkl.plan_info(32768, 2880, 201088, 100, 1.0, chunk=4096)
    assert p["fwd_rows"] == 16384 and p["bwd_rows"] == 8192
    assert p["vslab"] == 8192 and p["slabs"] == 25
    assert p["fwd_passes"] == 2 and p["bwd_passes"] == 4
    # N between the two floors: one forward pass, backward passes of 8192
    r = fkl.plan_info(12000, 2880, 201088, 100, 1.0)
    assert (r["fwd_rows"], r["fwd_passes"], r["bwd_rows"], r["bwd_passes"]) == (12000, 1, 8192, 2)
    # at the largest hidden size the floors stay under the 2 GiB operand view
    w = fkl.plan_info(65536, 65536, 1000, 4, 1.0)
    assert w["fwd_rows"] * 65536 * 2 < (1 << 31) and w["bwd_rows"] == 8192
    assert (p["fwd_bytes"], p["bwd_bytes"]) == fkl.workspace_size(32768, 2880, 201088, 100, 1.0, chunk=4096)
    # an explicit slab keeps the caller's chunk in both directions
    q = fkl.plan_info(8192, 3072, 128256, 100, 1.0, chunk=1024, vslab=65536)
    assert q["fwd_rows"] == q["bwd_rows"] == 1024 and q["fwd_passes"] == 8
    assert q["vslab"] == 65536 and q["slabs"] == 2
    z = fkl.plan_info(0, 64, 1000, 4)
    assert z["fwd_passes"] == z["bwd_passes"] == 0
    L = fkl.lib()
    s = fkl.make_shape(16, 64, 1000, 4)
    assert L.fkl_plan_info(ctypes.byref(s), None) == 1


def test_validate_terms_argument_errors_before_any_device_work():
    L = fkl.lib()
    s = fkl.make_shape(16, 64, 1000, 4)
    t = fkl.Terms(None, None, 0.5)
    bad = ctypes.c_void_p(0x1000)
    assert L.fkl_validate_terms(ctypes.byref(s), ctypes.byref(t), None, None) == 1
    assert L.fkl_validate_terms(ctypes.byref(s), ctypes.byref(t), ctypes.c_void_p(0x1002), None) == 1
    assert L.fkl_validate_terms(None, ctypes.byref(t), bad, None) == 1
    t2 = fkl.Terms(None, None, 1.5)
    assert L.fkl_validate_terms(ctypes.byref(s), ctypes.byref(t2), bad, None) == 1
    assert b"label_weight" in L.fkl_last_error()


def test_static_forward_refuses_shapes_beyond_its_scratch():
    """fkl_forward_static checks the shape's forward workspace against the
    static scratch before any device call: even its shorter 8192-row passes of
    K = 1024 teacher entries need about 67 MB, more than the 32 MiB scratch."""
    L = fkl.lib()
    s = fkl.make_shape(32768, 2880, 201088, 1024)
    fb, _ = fkl.workspace_size(32768, 2880, 201088, 1024)
    assert fb > fkl.STATIC_SCRATCH_BYTES
    p = ctypes.c_void_p(0x10000)
    st = L.fkl_forward_static(ctypes.byref(s), p, p, p, p, None, None, p, p, None, None)
    assert st == 2 and b"static scratch" in L.fkl_last_error()
    assert L.fkl_forward_static(ctypes.byref(s), p, p, p, p, None, None, None, p, None, None) == 1
    assert L.fkl_forward_static(None, p, p, p, p, None, None, p, p, None, None) == 1
    # the headline shape fits
    assert fkl.workspace_size(32768, 2880, 201088, 100)[0] <= fkl.STATIC_SCRATCH_BYTES
