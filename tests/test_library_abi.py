"""The C-ABI library without a GPU: it loads, exports every function that
include/sv.h declares (and the binding exposes each under the same name), its
host-side self-checks pass, and host-detectable argument errors are reported
before any launch."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sv():
    lib_path = os.path.join(ROOT, "draft_verification_sv_amd", "libsv.so")
    if not os.path.exists(lib_path):
        _load_build_script().build()
    import draft_verification_sv_amd as m

    return m


def _load_build_script():
    import importlib.util

    spec = importlib.util.spec_from_file_location("sv_build", os.path.join(ROOT, "draft_verification_sv_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_build_script_loads_without_the_package():
    """The build step must not import the package (which loads the library
    being rebuilt, absent on a fresh checkout)."""
    import subprocess
    import sys

    code = ("import importlib.util, os, sys\n"
            "spec = importlib.util.spec_from_file_location('b', os.path.join('draft_verification_sv_amd', 'build.py'))\n"
            "m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m)\n"
            "cmd = m.command('x.so')\n"
            "assert cmd[0] == 'hipcc' and any(a.startswith('--offload-arch=gfx950') for a in cmd)\n"
            "assert 'draft_verification_sv_amd' not in sys.modules and 'torch' not in sys.modules\n"
            "print('ok')\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stderr
    src = open(os.path.join(ROOT, "__graft_entry__.py")).read()
    body = src[src.index("def build()"):src.index("def smoke()")]
    assert body.index("spec_from_file_location") < body.index("import draft_verification_sv_amd")


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ["sv_softmax_stats", "sv_topp_threshold", "sv_mixture_q", "sv_accept", "sv_residual_sample",
                 "dvl_alloc_pack"]:
        assert must in names


def test_every_declared_symbol_is_exported(sv):
    lib = C.CDLL(sv.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported by libsv.so"
        assert callable(getattr(sv, name)), f"binding lacks {name}"
    assert sorted(sv.EXPORTS) == sorted(declared_functions())


C_CONSUMER = r"""
#include <stdio.h>
#include "sv.h"
int main(void) {
  size_t ws = 0, tws = 0;
  if (sv_workspace_bytes(32, 16, 8, 151936, &ws) != SV_OK || ws == 0) return 1;
  if (sv_tree_workspace_bytes(1024, 4, 151936, &tws) != SV_OK || tws == 0) return 2;
  if (sv_tree_workspace_bytes(1024, 17, 151936, &tws) != SV_ERR_ARG) return 3;
  if (sv_selftest_philox_host() != 0 || sv_selftest_rows_host() != 0) return 4;
  /* every pointer NULL: rejected on the host, nothing launched */
  if (sv_accept(NULL, SV_BF16, 64, 60, NULL, NULL, 1, 1, NULL, NULL, NULL, NULL, NULL, SV_Q_DENSE, NULL, SV_BF16, 64,
                NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) != SV_ERR_ARG) return 5;
  printf("%s\n", sv_status_string(SV_ERR_WORKSPACE));
  return 0;
}
"""


def test_header_compiles_as_c_and_links(sv, tmp_path):
    """A C99 program that includes include/sv.h (strict, -pedantic, warnings as
    errors) links against libsv.so and calls its host-side entry points: the
    boundary needs no C++ and no torch."""
    import shutil
    import subprocess

    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    src = tmp_path / "consumer.c"
    src.write_text(C_CONSUMER)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(sv.LIB_PATH)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                           os.path.join(ROOT, "include"), str(src), "-o", str(exe), "-L", libdir, "-lsv",
                           f"-Wl,-rpath,{libdir}"])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, (out.returncode, out.stderr)
    assert out.stdout.strip() == "workspace too small"


def test_host_selftests(sv):
    assert sv.selftest_host() == {"rows": 0, "philox": 0}


def test_workspace_size_grows_with_problem(sv):
    small = sv.sv_workspace_bytes(4, 16, 0, 1024)
    big = sv.sv_workspace_bytes(32, 16, 8, 151936)
    assert 256 <= small < big
    with pytest.raises(sv.SvError):
        sv.sv_workspace_bytes(0, 16, 0, 1024)
    with pytest.raises(sv.SvError):
        sv.sv_workspace_bytes(4, 65, 0, 1024)


def _buf(n, dt=np.float32):
    a = np.zeros(n + 64, dt)
    off = (-a.ctypes.data) % 16 // a.itemsize
    return a[off:off + n]


def test_argument_errors_are_reported_before_launch(sv):
    z = _buf(4096)
    p = z.ctypes.data
    ws = _buf(1 << 16, np.uint8)
    wp, nb = ws.ctypes.data, ws.nbytes
    L = sv.lib()
    # row pitch not a 16-byte multiple
    assert L.sv_softmax_stats(p, sv.SV_BF16, 63, 60, p, 0, 2, 4, p, p, p, p, wp, nb, None) == sv.SV_ERR_ARG
    # unknown dtype, null pointer, V < 1
    assert L.sv_softmax_stats(p, 5, 64, 60, p, 0, 2, 4, p, p, p, p, wp, nb, None) == sv.SV_ERR_ARG
    assert L.sv_softmax_stats(None, 1, 64, 60, p, 0, 2, 4, p, p, p, p, wp, nb, None) == sv.SV_ERR_ARG
    assert L.sv_softmax_stats(p, 1, 64, 0, p, 0, 2, 4, p, p, p, p, wp, nb, None) == sv.SV_ERR_ARG
    # top-p call needs its outputs
    assert L.sv_topp_threshold(p, 1, 64, 60, p, 0, 2, 4, p, p, p, p, p, None, p, wp, nb, None) == sv.SV_ERR_ARG
    # mixture: K over 64, workspace too small, capacity over R*b
    assert L.sv_mixture_q(p, 1, 64, 64, 65, 16, p, p, 2, 32, p, p, p, p, wp, nb, None) == sv.SV_ERR_ARG
    assert L.sv_mixture_q(p, 1, 64, 64, 8, 16, p, p, 2, 32, p, p, p, p, wp, 256, None) == sv.SV_ERR_WORKSPACE
    assert L.sv_mixture_q(p, 1, 64, 64, 8, 16, p, p, 2, 33, p, p, p, p, wp, nb, None) == sv.SV_ERR_ARG
    # accept: unknown proposal mode, b over 64
    args = [p, 1, 64, 64, p, p, 2, 16, p, p, p, p, p]
    assert L.sv_accept(*args, 9, p, 1, 64, p, p, p, p, p, None, None, None, wp, nb, None) == sv.SV_ERR_ARG
    args65 = [p, 1, 64, 64, p, p, 2, 65, p, p, p, p, p]
    assert L.sv_accept(*args65, 1, None, 1, 0, None, None, p, p, p, None, None, None, wp, nb, None) == sv.SV_ERR_ARG
    # DVL: b over 64, null budget
    assert L.dvl_alloc_pack(p, 4, 65, None, p, p, p, p, p, wp, nb, None) == sv.SV_ERR_ARG
    assert L.dvl_alloc_pack(p, 4, 16, None, None, p, p, p, p, wp, nb, None) == sv.SV_ERR_ARG
    assert sv.sv_status_string(sv.SV_ERR_WORKSPACE) == "workspace too small"


def test_one_hip_runtime_when_the_package_is_imported_first():
    """Importing the package before torch must not load a second HIP runtime
    beside the one torch ships (libsv's launches would then go to streams of
    the other runtime and fail)."""
    import ast
    import subprocess
    import sys

    code = ("import draft_verification_sv_amd, torch\n"
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.returncode == 0, out.stderr
    paths = ast.literal_eval(out.stdout.strip().splitlines()[-1])
    assert len(paths) == 1, paths


def _prototype_params(text: str, name: str) -> list:
    """The parameter declarations of `name`'s prototype in the (comment-free) header."""
    m = re.search(r"\b" + name + r"\s*\(", text)
    assert m, name
    depth, i = 1, m.end()
    while depth:
        depth += {"(": 1, ")": -1}.get(text[i], 0)
        i += 1
    body = " ".join(text[m.end():i - 1].split())
    return [] if body in ("", "void") else [p.strip() for p in body.split(",")]


def test_binding_signatures_match_header(sv):
    """Every ctypes signature the binding sets has the header's parameter count
    and, position by position, a matching kind: pointers for pointers, and the
    same width for int32_t, int64_t and size_t."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "sv.h")).read(), flags=re.S)
    scalar = {"int32_t": C.c_int32, "int64_t": C.c_int64, "size_t": C.c_size_t}
    for name, args in sv._SIGS.items():
        params = _prototype_params(text, name)
        assert len(params) == len(args), f"{name}: header {len(params)} parameters, binding {len(args)}"
        for k, (decl, ct) in enumerate(zip(params, args)):
            if "*" in decl:
                assert ct is C.c_void_p or issubclass(ct, C._Pointer), f"{name} parameter {k}: {decl} vs {ct}"
            else:
                base = decl.split()[0]
                assert scalar.get(base) is ct, f"{name} parameter {k}: {decl} vs {ct}"
