"""The C-ABI library loads, exports every function include/uno.h declares, and
rejects invalid arguments on the host before touching the GPU."""
import ctypes
import os
import re

import pytest

from lossless_diffusion_drafted_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "uno.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uno_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libuno.so is not built (run python -m lossless_diffusion_drafted_amd.build)")
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _header_functions()
    assert "uno_verify_block" in names and "uno_gated_lora_linear" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_status_strings_and_version(lib):
    assert lib.uno_status_string(0) == b"UNO_OK"
    assert lib.uno_status_string(3) == b"UNO_ERR_WORKSPACE"
    assert lib.uno_abi_version() >= 100


def _verify(lib, S=1, b=8, V=1024, dtype=1, sp=None, ws=1 << 20, null_ws=False, p=1):
    sp = sp or _lib.SamplingParams(1.0, 0.95, 50, 0)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    return lib.uno_verify_block(fake if p else None, fake, dtype, fake, fake, fake, S, b, V, sp,
                                fake, fake, fake, None, None,
                                None if null_ws else fake, ws, None)


def test_verify_argument_validation(lib):
    assert _verify(lib, b=0) == _lib.UNO_ERR_INVALID_ARG
    assert _verify(lib, b=65) == _lib.UNO_ERR_INVALID_ARG
    assert _verify(lib, V=0) == _lib.UNO_ERR_INVALID_ARG
    assert _verify(lib, dtype=7) == _lib.UNO_ERR_INVALID_ARG
    assert _verify(lib, p=0) == _lib.UNO_ERR_INVALID_ARG
    assert b"null" in lib.uno_last_error()
    assert _verify(lib, sp=_lib.SamplingParams(1.0, 0.0, 50, 0)) == _lib.UNO_ERR_INVALID_ARG
    assert _verify(lib, sp=_lib.SamplingParams(float("nan"), 0.9, 50, 0)) == _lib.UNO_ERR_INVALID_ARG
    assert _verify(lib, ws=16) == _lib.UNO_ERR_WORKSPACE
    assert _verify(lib, null_ws=True) == _lib.UNO_ERR_WORKSPACE
    assert b"workspace" in lib.uno_last_error()
    # S == 0 is a valid empty call that launches nothing
    assert _verify(lib, S=0) == _lib.UNO_OK


def test_workspace_sizes(lib):
    assert lib.uno_verify_block_workspace(64, 16, 151936) >= 64 * 4 + 64 * 16 * 8
    assert lib.uno_verify_block_workspace(0, 16, 151936) >= 0


def test_product_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "lossless_diffusion_drafted_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", src, re.M), f
                assert "oracle/" not in src, f


def _tv(lib, R=4, V=1024, dtype=1, T=1.0, loss=True, ws=1 << 24, null_ws=False):
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    return lib.uno_tv_loss_fwd_bwd(fake, fake, dtype, fake, R, V, T, fake if loss else None, None, None,
                                   None if null_ws else fake, ws, None)


def test_tv_argument_validation(lib):
    assert _tv(lib, R=-1) == _lib.UNO_ERR_INVALID_ARG
    assert _tv(lib, V=0) == _lib.UNO_ERR_INVALID_ARG
    assert _tv(lib, T=0.0) == _lib.UNO_ERR_INVALID_ARG
    assert _tv(lib, T=float("nan")) == _lib.UNO_ERR_INVALID_ARG
    assert _tv(lib, T=float("inf")) == _lib.UNO_ERR_INVALID_ARG
    assert _tv(lib, dtype=5) == _lib.UNO_ERR_INVALID_ARG
    assert _tv(lib, loss=False) == _lib.UNO_ERR_INVALID_ARG
    assert _tv(lib, ws=64) == _lib.UNO_ERR_WORKSPACE
    assert _tv(lib, null_ws=True) == _lib.UNO_ERR_WORKSPACE
    assert lib.uno_tv_loss_workspace(32768, 151936) >= 32768 * 8


def test_sampling_params_layout_matches_the_header(tmp_path):
    """The ctypes mirror of uno_sampling_params has the size and field offsets that a
    C compiler gives the struct declared in include/uno.h."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f for f, _ in _lib.SamplingParams._fields_]
    body = " ".join(f'printf(" %zu", offsetof(uno_sampling_params, {f}));' for f in fields)
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "uno.h"\n'
                   'int main(void) { printf("%zu", sizeof(uno_sampling_params)); '
                   + body + ' printf("\\n"); return 0; }\n')
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(_lib.SamplingParams)] + [getattr(_lib.SamplingParams, f).offset for f in fields]
    assert got == want, (got, want)


def test_noalloc_verify_rejects_sizes_beyond_its_scratch(lib):
    """Checked on the host before any HIP call: 4096 x 64 slots need more than the
    library's 1310720-byte verify scratch."""
    sp = _lib.SamplingParams(1.0, 0.95, 50, 0)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    st = lib.uno_verify_block_noalloc(fake, fake, 1, fake, fake, fake, 4096, 64, 1024, sp,
                                      fake, fake, fake, None, None, None)
    assert st == _lib.UNO_ERR_UNSUPPORTED
    assert b"scratch" in lib.uno_last_error()
    st = lib.uno_verify_block_noalloc(fake, fake, 1, fake, fake, fake, 4, 0, 1024, sp,
                                      fake, fake, fake, None, None, None)
    assert st == _lib.UNO_ERR_INVALID_ARG
