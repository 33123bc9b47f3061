"""The C-ABI library without a GPU: it loads, exports exactly what
include/*.h declares, its argument structs match the binding's layouts, and
the host-side argument checks return before any HIP call."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

import rejection_sampling_verify_08_amd as R
from rejection_sampling_verify_08_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"SPEC_VERIFY_API\s+[\w\s\*]+?\b(spec_verify_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = R.load_library()
    names = declared_functions()
    assert names == sorted(binding.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", R.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = sorted(set(re.findall(r"\bT (spec_verify_\w+)", out)))
    assert exported == names
    # nothing but the C ABI leaks out of the library
    assert not re.search(r"\bT _Z", out)


def test_args_struct_layout_matches_header(tmp_path):
    fields = [f for f, _ in binding.Args._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(
        f'  printf("{f} %zu\\n", offsetof(spec_verify_args, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "spec_verify.h"\n'
                   'int main(void){\n' + body +
                   '\n  printf("sizeof %zu\\n", sizeof(spec_verify_args));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), "-o", str(exe),
                    str(src)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                 check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(binding.Args, f).offset, f
    assert int(got["sizeof"]) == ctypes.sizeof(binding.Args)


def test_tree_args_layout_matches_header(tmp_path):
    fields = [f for f, _ in binding.TreeArgs._fields_]
    src = tmp_path / "layout3.c"
    body = "\n".join(
        f'  printf("{f} %zu\\n", offsetof(spec_verify_tree_args, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "spec_verify.h"\n'
                   'int main(void){\n' + body +
                   '\n  printf("sizeof %zu\\n", sizeof(spec_verify_tree_args));\n  return 0;\n}\n')
    exe = tmp_path / "layout3"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), "-o", str(exe),
                    str(src)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                 check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(binding.TreeArgs, f).offset, f
    assert int(got["sizeof"]) == ctypes.sizeof(binding.TreeArgs)


def test_adapt_params_layout_matches_header(tmp_path):
    fields = [f for f, _ in binding.AdaptParams._fields_]
    src = tmp_path / "layout2.c"
    body = "\n".join(
        f'  printf("{f} %zu\\n", offsetof(spec_verify_adapt_params, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "spec_verify_adapt.h"\n'
                   'int main(void){\n' + body +
                   '\n  printf("sizeof %zu\\n", sizeof(spec_verify_adapt_params));\n  return 0;\n}\n')
    exe = tmp_path / "layout2"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), "-o", str(exe),
                    str(src)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                 check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(binding.AdaptParams, f).offset, f
    assert int(got["sizeof"]) == ctypes.sizeof(binding.AdaptParams)


def test_header_compiles_as_c_and_cpp(tmp_path):
    for comp, ext in (("gcc", "c"), ("g++", "cpp")):
        src = tmp_path / f"h.{ext}"
        src.write_text('#include "spec_verify.h"\n#include "spec_verify_adapt.h"\n'
                       'int main(void){return SPEC_VERIFY_OK;}\n')
        subprocess.run([comp, "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        "-o", str(tmp_path / f"h_{ext}"), str(src)], check=True)


def test_status_strings():
    lib = R.load_library()
    for code in (0, -1, -2, -3, -4):
        s = lib.spec_verify_status_string(code)
        assert s and s != b"unknown status"
    assert lib.spec_verify_status_string(12345) == b"unknown status"


def test_host_side_argument_checks_without_a_device():
    lib = R.load_library()
    ctx = ctypes.c_void_p(123)
    ws = ctypes.c_size_t(7)
    bc = ctypes.byref
    # rejected before the HIP runtime is queried
    assert lib.spec_verify_create(None, 0, 1000, 1, 1, 1, 0, bc(ws)) == binding.EINVAL
    assert lib.spec_verify_create(bc(ctx), 0, 1000, 7, 1, 1, 0, bc(ws)) == binding.EUNSUPPORTED
    assert ctx.value is None
    assert lib.spec_verify_create(bc(ctx), 0, 0, 1, 1, 1, 0, bc(ws)) == binding.EUNSUPPORTED
    assert lib.spec_verify_create(bc(ctx), 0, (1 << 21) + 1, 1, 1, 1, 0, bc(ws)) == binding.EUNSUPPORTED
    assert lib.spec_verify_create(bc(ctx), 0, 1000, 1, -1, 1, 0, bc(ws)) == binding.EINVAL
    assert lib.spec_verify_create(bc(ctx), 0, 1000, 1, 1, -1, 0, bc(ws)) == binding.EINVAL
    assert lib.spec_verify_create(bc(ctx), 0, 1000, 1, 1, 1, 0x80, bc(ws)) == binding.EINVAL
    assert lib.spec_verify_run(None, None, None) == binding.EINVAL
    assert lib.spec_verify_run_greedy(None, None, None) == binding.EINVAL
    assert lib.spec_verify_run_point_drafts(None, None, None) == binding.EINVAL
    assert lib.spec_verify_tree_run_greedy(None, None, None) == binding.EINVAL
    assert lib.spec_verify_tree_run_point(None, None, None) == binding.EINVAL
    assert lib.spec_verify_destroy(None) == binding.OK
    assert lib.spec_verify_workspace_size(None) == 0
    assert lib.spec_verify_num_kernels(None) == 0
    # the read probe: null pointers, sizes that are not whole 8 KB wave spans,
    # misalignment and half an event pair are refused on the host
    P = ctypes.c_void_p
    assert lib.spec_verify_read_probe(None, 8192, 1, P(256), None, None, None) == binding.EINVAL
    assert lib.spec_verify_read_probe(P(256), 8192, 1, None, None, None, None) == binding.EINVAL
    assert lib.spec_verify_read_probe(P(256), 0, 1, P(256), None, None, None) == binding.EINVAL
    assert lib.spec_verify_read_probe(P(256), 8000, 1, P(256), None, None, None) == binding.EINVAL
    assert lib.spec_verify_read_probe(P(264), 8192, 1, P(256), None, None, None) == binding.EINVAL
    assert lib.spec_verify_read_probe(P(256), 8192, 1, P(256), None, P(8), None) == binding.EINVAL


def test_binding_fails_loudly_without_the_library(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(ImportError, match="no fallback"):
        binding.load_library(str(tmp_path / "missing.so"))


@pytest.mark.parametrize("V,B,R_d", [(1, 1, 0), (1000, 1, 4), (4097, 7, 33),
                                     (128256, 128, 1024), (152064, 512, 2048),
                                     (8, 1_000_000, 3_000_000)])
def test_workspace_covers_every_row_partial_and_tile(V, B, R_d):
    """The workspace must hold one 16-byte partial per 4096 logits of all
    R_t + R_d = B + 2 R_d rows the statistics pass reads, four doubles per
    2048-logit tile per sequence (the residual's tile sums) and one counter
    per sequence."""
    lib = R.load_library()
    ws = ctypes.c_size_t()
    assert lib.spec_verify_query_workspace(V, B, R_d, ctypes.byref(ws)) == binding.OK
    rows = B + 2 * R_d
    need = rows * -(-V // 4096) * 16 + B * -(-V // 2048) * 4 * 8 + B * 4
    assert ws.value >= need
    assert ws.value % 256 == 0
    assert lib.spec_verify_query_workspace(0, B, R_d, ctypes.byref(ws)) == binding.EUNSUPPORTED
    assert lib.spec_verify_query_workspace(V, -1, R_d, ctypes.byref(ws)) == binding.EINVAL
