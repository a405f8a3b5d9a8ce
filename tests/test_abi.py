"""The C-ABI library loads on a machine without a GPU and exports every
function include/lora_gemm.h declares (no compute call is made here)."""
import ctypes
import os
import re

import heterogeneous_adapter_gemm_amd as hg
from heterogeneous_adapter_gemm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "lora_gemm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^(?!\s*typedef)\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_named_entry_points():
    names = declared_functions()
    for n in ("lora_pool_create", "lora_pool_page_in", "lora_linear_decode", "lora_linear_prefill", "base_gemm"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding covers every one of them, under the same name
    assert sorted(_lib.EXPORTED) == declared_functions()
    assert hg.lora_version().startswith("hagemm")


def test_error_codes_match_header():
    src = open(os.path.join(ROOT, "include", "lora_gemm.h")).read()
    for name, val in re.findall(r"(LORA_E\w+|LORA_OK)\s*=\s*(-?\d+)", src):
        assert getattr(_lib, name) == int(val), name


def test_probes_reject_bad_arguments_before_any_launch():
    """The measurement probes check their arguments on the host (no GPU needed)."""
    lib = _lib.library()
    fake = ctypes.c_void_p(16)   # never dereferenced: every call below fails its host-side check
    assert lib.lora_probe_read(None, 1 << 20, fake, 4, fake, None) == _lib.LORA_EINVAL
    assert lib.lora_probe_read(fake, 4096, fake, 4, fake, None) == _lib.LORA_EINVAL    # less than one chunk
    assert lib.lora_probe_read(fake, 1 << 20, fake, 0, fake, None) == _lib.LORA_EINVAL  # no chunks
    assert b"buf_bytes" in lib.lora_last_error()
    assert lib.lora_probe_mfma(8, 1, 1, fake, None, None) == _lib.LORA_EINVAL           # shape 16 or 32 only
    assert lib.lora_probe_mfma(16, 0, 1, fake, None, None) == _lib.LORA_EINVAL
