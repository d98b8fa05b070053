"""The C-ABI library loads, exports what include/fa.h declares, and rejects bad
arguments on the host.  CPU only: no call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

from exact_io_aware_57_amd import binding
from exact_io_aware_57_amd.build import LIB_PATH, build_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FAKE = 0x10000  # an aligned non-null address; validation must reject before any use of it


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        build_library()
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["fa_fwd", "fa_fwd_f32", "fa_fwd_gqa", "fa_fwd_gqa_f32", "fa_status_str"]
    assert tuple(declared_functions()) == tuple(sorted(binding.EXPORTED_SYMBOLS))


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name


def test_library_is_built_for_gfx950():
    # The fat binary that hipcc embeds names its device target triple.
    data = open(LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def test_status_strings(lib):
    for code in (binding.FA_OK, binding.FA_ERR_INVALID_ARG, binding.FA_ERR_UNSUPPORTED, binding.FA_ERR_MISALIGNED,
                 binding.FA_ERR_NO_DEVICE, binding.FA_ERR_LAUNCH):
        s = binding.fa_status_str(code)
        assert s and s != "unknown fa_status"
    assert binding.fa_status_str(12345) == "unknown fa_status"


ARGS = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64, scale=0.125, causal=0, seqlens=None,
            stream=None)


def call(fn, **over):
    a = dict(ARGS)
    a.update(over)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
              a["seqlens"], a["stream"])


@pytest.mark.parametrize("fn", [binding.fa_fwd, binding.fa_fwd_f32], ids=["bf16", "f32"])
def test_invalid_arguments_are_rejected_on_the_host(lib, fn):
    E = binding
    for name in ("q", "k", "v", "o"):
        assert call(fn, **{name: None}) == E.FA_ERR_INVALID_ARG, name
    for name in ("B", "H", "N"):
        assert call(fn, **{name: 0}) == E.FA_ERR_INVALID_ARG, name
        assert call(fn, **{name: -3}) == E.FA_ERR_INVALID_ARG, name
    for scale in (0.0, -1.0, float("nan"), float("inf")):
        assert call(fn, scale=scale) == E.FA_ERR_INVALID_ARG, scale
    for d in (0, 32, 96, 256):
        assert call(fn, d=d) == E.FA_ERR_UNSUPPORTED, d
    for name in ("q", "k", "v", "o"):
        assert call(fn, **{name: FAKE + 8}) == E.FA_ERR_MISALIGNED, name
    assert call(fn, lse=FAKE + 2) == E.FA_ERR_MISALIGNED
    assert call(fn, seqlens=FAKE + 1) == E.FA_ERR_MISALIGNED
    # element count past 2^40 or a grid past int32
    assert call(fn, B=1 << 20, H=1 << 10, N=1 << 10) == E.FA_ERR_INVALID_ARG


def _no_gpu_visible():
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_gpu_visible(), reason="a GPU is visible: valid arguments with fake pointers would launch")
def test_no_device_is_reported(lib):
    assert call(binding.fa_fwd) == binding.FA_ERR_NO_DEVICE
    assert call(binding.fa_fwd_f32) == binding.FA_ERR_NO_DEVICE
    assert call_gqa(binding.fa_fwd_gqa) == binding.FA_ERR_NO_DEVICE
    assert call_gqa(binding.fa_fwd_gqa_f32) == binding.FA_ERR_NO_DEVICE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        binding.load()


def test_ctypes_signatures(lib):
    assert lib.fa_fwd.restype is ctypes.c_int
    assert len(lib.fa_fwd.argtypes) == 13 and len(lib.fa_fwd_f32.argtypes) == 13
    assert len(lib.fa_fwd_gqa.argtypes) == 14 and len(lib.fa_fwd_gqa_f32.argtypes) == 14


GQA_ARGS = dict(ARGS, H=4, H_kv=2)


def call_gqa(fn, **over):
    a = dict(GQA_ARGS)
    a.update(over)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"], a["N"], a["d"], a["scale"], a["causal"],
              a["seqlens"], a["stream"])


@pytest.mark.parametrize("fn", [binding.fa_fwd_gqa, binding.fa_fwd_gqa_f32], ids=["bf16", "f32"])
def test_grouped_head_counts_are_checked_on_the_host(lib, fn):
    E = binding
    for H, H_kv in ((4, 0), (4, -1), (4, 3), (4, 8), (6, 4)):
        assert call_gqa(fn, H=H, H_kv=H_kv) == E.FA_ERR_INVALID_ARG, (H, H_kv)
    assert call_gqa(fn, q=None) == E.FA_ERR_INVALID_ARG
    assert call_gqa(fn, d=96) == E.FA_ERR_UNSUPPORTED
    assert call_gqa(fn, k=FAKE + 4) == E.FA_ERR_MISALIGNED
