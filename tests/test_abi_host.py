"""Host-side checks of the C-ABI library that need no GPU.

The library must load, export every entry point that include/specv.h declares
(and the binding must name the same ones), agree with the header on status
codes, and reject bad arguments that are caught before any HIP call.
"""

import ctypes
import os
import re

import pytest

import speculative_sampling_verification_specv_amd as specv
from speculative_sampling_verification_specv_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "specv.h")


def _header_text():
    with open(HEADER) as f:
        return f.read()


def _declared_functions():
    return re.findall(r"SPECV_API\s+[\w\s\*]+?\b(specv_\w+)\s*\(", _header_text())


def test_header_declares_the_boundary():
    assert set(_declared_functions()) == {"specv_create", "specv_verify", "specv_row_stats", "specv_destroy",
                                          "specv_strerror", "specv_set_timing", "specv_last_timings",
                                          "specv_stage_name", "specv_set_wait_limit",
                                          "specv_verify_static", "specv_sample", "specv_kv_commit",
                                          "specv_acceptance_rates", "specv_verify_lazy"}


def test_library_exports_every_declared_symbol():
    lib = specv.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_declared_functions()) == set(_lib._SIGNATURES)


def test_status_codes_match_header():
    text = _header_text()
    for name in ("SPECV_OK", "SPECV_EINVAL", "SPECV_ENOMEM", "SPECV_EHIP", "SPECV_EALIGN", "SPECV_ESTATE", "SPECV_ERANGE",
                 "SPECV_F32", "SPECV_BF16"):
        m = re.search(rf"\b{name}\s*=\s*(-?\d+)", text)
        assert m, name
        assert int(m.group(1)) == getattr(_lib, name), name
    m = re.search(r"#define\s+SPECV_MAX_DRAFT\s+(\d+)", text)
    assert int(m.group(1)) == _lib.SPECV_MAX_DRAFT
    m = re.search(r"#define\s+SPECV_MAX_VOCAB\s+(\d+)", text)
    assert int(m.group(1)) == _lib.SPECV_MAX_VOCAB


def test_strerror_covers_codes():
    seen = set()
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = specv.specv_strerror(code)
        assert s and s not in seen
        seen.add(s)
    assert "unknown" in specv.specv_strerror(-99)


def test_argument_errors_before_any_device_call():
    lib = specv.load_library()
    h = ctypes.c_void_p()
    assert lib.specv_create(None, 1, 1, 16, 0, 0) == _lib.SPECV_EINVAL
    for args in ((0, 4, 16, 0), (1, 0, 16, 0), (1, 65, 16, 0), (1, 4, 0, 0), (1, 4, _lib.SPECV_MAX_VOCAB + 1, 0),
                 (1, 4, 16, 2), (1, 4, 16, -1)):
        assert lib.specv_create(ctypes.byref(h), *args, 0) == _lib.SPECV_EINVAL, args
        assert h.value is None
    null = [None] * 9
    assert lib.specv_verify(None, 1, 1, *null) == _lib.SPECV_EINVAL
    assert lib.specv_verify_lazy(None, 1, 1, *null) == _lib.SPECV_EINVAL
    assert lib.specv_row_stats(None, None, None, None) == _lib.SPECV_EINVAL
    assert lib.specv_sample(None, 1, None, None, None, None, None) == _lib.SPECV_EINVAL
    assert lib.specv_acceptance_rates(None, 1, 1, *([None] * 7)) == _lib.SPECV_EINVAL
    # KV commit: sizes and alignment are checked before any device call.
    kv = lambda *a: lib.specv_kv_commit(*a)  # noqa: E731
    p16 = ctypes.c_void_p(4096)
    p4 = ctypes.c_void_p(4100)
    assert kv(-1, 1, 1, 8, 16, p16, 0, 0, p16, 0, 0, p4, p4, p4, None) == _lib.SPECV_EINVAL
    assert kv(1, 1, 0, 8, 16, p16, 0, 0, p16, 0, 0, p4, p4, p4, None) == _lib.SPECV_EINVAL
    assert kv(1, 1, 1, 8, 8, p16, 0, 0, p16, 0, 0, p4, p4, p4, None) == _lib.SPECV_EINVAL
    assert kv(1, 1, 1, 8, 24, p16, 0, 0, p16, 0, 0, p4, p4, p4, None) == _lib.SPECV_EALIGN
    assert kv(1, 1, 1, 8, 16, p4, 0, 0, p16, 0, 0, p4, p4, p4, None) == _lib.SPECV_EALIGN
    assert kv(1, 1, 1, 8, 16, p16, 8, 0, p16, 0, 0, p4, p4, p4, None) == _lib.SPECV_EALIGN
    assert kv(1, 1, 1, 8, 16, None, 0, 0, p16, 0, 0, p4, p4, p4, None) == _lib.SPECV_EINVAL
    assert kv(1, 0, 1, 8, 16, None, 0, 0, None, 0, 0, None, None, None, None) == _lib.SPECV_OK
    lib.specv_destroy(None)  # no-op
    assert lib.specv_set_timing(None, 1) == _lib.SPECV_EINVAL
    assert lib.specv_set_wait_limit(None, 10) == _lib.SPECV_EINVAL
    # The allocation-free entry point checks sizes before touching a device.
    nine = [None] * 9
    assert lib.specv_verify_static(-1, 1, 16, 0, *nine) == _lib.SPECV_EINVAL
    assert lib.specv_verify_static(1, 0, 16, 0, *nine) == _lib.SPECV_EINVAL
    assert lib.specv_verify_static(1, 1, 16, 2, *nine) == _lib.SPECV_EINVAL
    assert lib.specv_verify_static(257, 1, 16, 0, *nine) == _lib.SPECV_ERANGE
    assert lib.specv_verify_static(1, 17, 16, 0, *nine) == _lib.SPECV_ERANGE
    assert lib.specv_verify_static(1, 1, _lib.SPECV_MAX_VOCAB + 1, 1, *nine) == _lib.SPECV_ERANGE
    assert lib.specv_verify_static(0, 1, 16, 0, *nine) == _lib.SPECV_OK
    assert lib.specv_verify_static(1, 1, 16, 0, *nine) == _lib.SPECV_EINVAL  # null pointers
    n = ctypes.c_int()
    assert lib.specv_last_timings(None, (ctypes.c_float * 4)(), 4, ctypes.byref(n)) == _lib.SPECV_EINVAL
    assert specv.specv_stage_name(0) == "verify"
    assert specv.specv_stage_name(1) is None


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load_library(str(tmp_path / "libspecv.so"))


def test_header_is_c_and_links(tmp_path):
    """include/specv.h compiles as strict C11, a C program links every declared
    entry point from libspecv.so, and its host-side argument checks answer
    from C as they do through the binding."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    specv.load_library()  # the built library must exist (fails loudly otherwise)
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    names = _declared_functions()
    src = tmp_path / "abi.c"
    src.write_text("\n".join([
        "#include <stdio.h>",
        "#include \"specv.h\"",
        "typedef void (*any_fn)(void);",
        "static any_fn const entry_points[] = {",
        *[f"  (any_fn){n}," for n in names],
        "};",
        "int main(void) {",
        "  specv_handle h = NULL;",
        "  int bad = 0;",
        "  bad |= specv_create(&h, 0, 1, 16, SPECV_F32, 0) != SPECV_EINVAL || h != NULL;",
        "  bad |= specv_create(&h, 1, SPECV_MAX_DRAFT + 1, 16, SPECV_BF16, 0) != SPECV_EINVAL;",
        "  bad |= specv_verify(NULL, 1, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != SPECV_EINVAL;",
        "  bad |= specv_verify_static(257, 1, 16, SPECV_F32, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL)",
        "         != SPECV_ERANGE;",
        "  bad |= specv_strerror(SPECV_OK) == NULL;",
        "  specv_destroy(NULL);",
        "  printf(\"%d entry points, checks %s\\n\", (int)(sizeof entry_points / sizeof entry_points[0]),",
        "         bad ? \"failed\" : \"passed\");",
        "  return bad;",
        "}",
        "",
    ]))
    exe = tmp_path / "abi"
    cmd = [cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.dirname(HEADER), str(src), "-L", lib_dir, "-lspecv", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stdout + proc.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert f"{len(names)} entry points, checks passed" in run.stdout
