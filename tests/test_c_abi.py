"""The C header as a C client sees it (no GPU): tests/c_abi/fkl_layout.c is
compiled as C99 with warnings as errors against include/fkl.h, linked against
libfkl.so and run. Its struct layouts must match the binding's ctypes mirrors,
and its host-only calls must agree with the same calls made through the
binding."""

import ctypes
import os
import shutil
import subprocess

import pytest

import output_projection_kl_amd as fkl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_c_client(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib = fkl.library_path()
    if not os.path.exists(lib):
        pytest.skip("libfkl.so not built")
    exe = tmp_path / "fkl_layout"
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi", "fkl_layout.c"), "-o", str(exe),
           os.path.abspath(lib), f"-Wl,-rpath,{os.path.dirname(os.path.abspath(lib))}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout
    lines = {}
    for line in out.splitlines():
        key, _, rest = line.partition(" ")
        lines[key] = rest.split()
    return lines


def _layout(fields):
    size = int(fields[0])
    offs = {}
    for f in fields[1:]:
        name, _, off = f.partition("=")
        offs[name] = int(off)
    return size, offs


@pytest.mark.parametrize("cname,pytype", [
    ("fkl_shape", fkl.Shape),
    ("fkl_terms", fkl.Terms),
    ("fkl_topk_shape", fkl.TopkShape),
    ("fkl_plan", fkl.PlanInfo),
    ("fkl_kernel_stat", fkl.KernelStat),
])
def test_struct_layouts_match_the_binding(tmp_path, cname, pytype):
    size, offs = _layout(_run_c_client(tmp_path)[cname])
    assert size == ctypes.sizeof(pytype)
    assert set(offs) == {f[0] for f in pytype._fields_}
    for name, off in offs.items():
        assert getattr(pytype, name).offset == off, name


def test_host_calls_from_c_agree_with_the_binding(tmp_path):
    lines = _run_c_client(tmp_path)
    st, fb, bb = (int(x) for x in lines["workspace"])
    assert st == 0
    assert (fb, bb) == fkl.workspace_size(32768, 2880, 201088, 100, 1.0, chunk=4096)
    st, *plan = (int(x) for x in lines["plan"])
    assert st == 0
    assert plan == list(fkl.plan_info(32768, 2880, 201088, 100, 1.0, chunk=4096).values())
    st, tb = (int(x) for x in lines["topk_workspace"])
    assert st == 0 and tb == fkl.topk_workspace_size(16384, 4096, 128256, 100)
    assert lines["null_shape"] == ["1", "message"]
    assert int(lines["version"][0]) == fkl.lib().fkl_version()
