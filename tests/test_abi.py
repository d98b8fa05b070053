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
    assert declared_functions() == ["fa_bwd", "fa_bwd_workspace_size", "fa_clock_sample", "fa_decode",
                                    "fa_decode_noalloc", "fa_decode_workspace_size", "fa_fwd", "fa_fwd_f32",
                                    "fa_fwd_fp8", "fa_fwd_gqa", "fa_fwd_gqa_f32", "fa_status_str"]
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
                 binding.FA_ERR_NO_DEVICE, binding.FA_ERR_LAUNCH, binding.FA_ERR_SCRATCH_TOO_SMALL):
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
    for d in (0, 32, 96, 192, 512):
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


DEC = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=2, H=8, H_kv=2, Nq=1, Nk=1000, d=128, scale=0.1, causal=0,
           seqlens=None, num_splits=0, workspace=FAKE, workspace_size=1 << 30, stream=None)


def call_dec(**over):
    a = dict(DEC)
    a.update(over)
    return binding.fa_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"], a["Nq"], a["Nk"], a["d"],
                             a["scale"], a["causal"], a["seqlens"], a["num_splits"], a["workspace"], a["workspace_size"],
                             a["stream"])


def test_decode_workspace_size(lib):
    f = binding.fa_decode_workspace_size
    # rows * splits * (d + 1) floats
    assert f(2, 8, 2, 1, 1000, 128, 3) == 2 * 8 * 1 * 3 * 129 * 4
    assert f(1, 1, 1, 4, 64, 64, 1) == 4 * 65 * 4
    auto = f(2, 8, 2, 1, 100000, 128, 0)
    assert auto > 0 and auto % (2 * 8 * 129 * 4) == 0
    for bad in [dict(H_kv=3), dict(d=96), dict(Nq=0), dict(Nk=0), dict(num_splits=-1)]:
        a = dict(B=2, H=8, H_kv=2, Nq=1, Nk=1000, d=128, num_splits=0)
        a.update(bad)
        assert f(**a) == 0, bad


def test_decode_arguments_are_checked_on_the_host(lib):
    E = binding
    for name in ("q", "k", "v", "o", "workspace"):
        assert call_dec(**{name: None}) == E.FA_ERR_INVALID_ARG, name
    for over in (dict(B=0), dict(Nq=0), dict(Nk=-1), dict(H_kv=3), dict(H_kv=16), dict(num_splits=-2), dict(scale=0.0),
                 dict(workspace_size=16)):
        assert call_dec(**over) == E.FA_ERR_INVALID_ARG, over
    assert call_dec(d=256) == E.FA_ERR_UNSUPPORTED
    assert call_dec(workspace=FAKE + 4) == E.FA_ERR_MISALIGNED
    assert call_dec(q=FAKE + 8) == E.FA_ERR_MISALIGNED


BWD = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dout=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=2, H=8, H_kv=2, N=1000,
           d=128, scale=0.1, causal=1, seqlens=None, workspace=FAKE, workspace_size=1 << 30, stream=None)


def call_bwd(**over):
    a = dict(BWD)
    a.update(over)
    return binding.fa_bwd(*(a[n] for n in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "B", "H", "H_kv", "N",
                                            "d", "scale", "causal", "seqlens", "workspace", "workspace_size",
                                            "stream")))


def test_bwd_workspace_size(lib):
    f = binding.fa_bwd_workspace_size
    # two floats per query row, rows of each head padded to a multiple of 128
    assert f(2, 8, 1000) == 2 * 2 * 8 * 1024 * 4
    assert f(1, 1, 128) == 2 * 128 * 4
    assert f(1, 1, 129) == 2 * 256 * 4
    assert f(1, 1, 1) == 2 * 128 * 4
    assert f(0, 1, 1) == 0 and f(1, 0, 1) == 0 and f(1, 1, 0) == 0


def test_bwd_arguments_are_checked_on_the_host(lib):
    E = binding
    for name in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "workspace"):
        assert call_bwd(**{name: None}) == E.FA_ERR_INVALID_ARG, name
    for over in (dict(B=0), dict(N=0), dict(H=-1), dict(H_kv=3), dict(H_kv=16), dict(scale=0.0),
                 dict(scale=float("nan")), dict(workspace_size=16)):
        assert call_bwd(**over) == E.FA_ERR_INVALID_ARG, over
    for d in (32, 96, 256):
        assert call_bwd(d=d) == E.FA_ERR_UNSUPPORTED, d
    # a head of 4 GiB or more (N * d * 2 bytes >= 2^32) is refused: the kernels
    # address a head's rows by 32-bit offsets; one row less still passes on
    big = dict(B=1, H=1, H_kv=1, workspace_size=1 << 40)
    assert call_bwd(N=(1 << 24) + 1, d=128, **big) == E.FA_ERR_UNSUPPORTED
    assert call_bwd(N=(1 << 25) + 1, d=64, **big) == E.FA_ERR_UNSUPPORTED
    assert call_bwd(N=(1 << 24) - 1, d=128, **big) == E.FA_ERR_NO_DEVICE
    for name in ("q", "k", "v", "o", "dout", "dq", "dk", "dv", "workspace"):
        assert call_bwd(**{name: FAKE + 8}) == E.FA_ERR_MISALIGNED, name
    assert call_bwd(lse=FAKE + 2) == E.FA_ERR_MISALIGNED
    assert call_bwd(seqlens=FAKE + 1) == E.FA_ERR_MISALIGNED
    # valid arguments reach the device check (no GPU here)
    assert call_bwd() == E.FA_ERR_NO_DEVICE


F8 = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=2, H=8, H_kv=2, N=1000, d=128, scale=0.1, sq=0.01, sk=0.02,
          sv=0.03, causal=1, seqlens=None, stream=None)


def call_fp8(**over):
    a = dict(F8)
    a.update(over)
    return binding.fa_fwd_fp8(*(a[n] for n in ("q", "k", "v", "o", "lse", "B", "H", "H_kv", "N", "d", "scale", "sq", "sk",
                                                "sv", "causal", "seqlens", "stream")))


def test_fp8_arguments_are_checked_on_the_host(lib):
    E = binding
    for name in ("q", "k", "v", "o"):
        assert call_fp8(**{name: None}) == E.FA_ERR_INVALID_ARG, name
    for over in (dict(B=0), dict(N=0), dict(H_kv=3), dict(scale=0.0), dict(sq=0.0), dict(sk=-1.0),
                 dict(sv=float("inf")), dict(sq=float("nan"))):
        assert call_fp8(**over) == E.FA_ERR_INVALID_ARG, over
    for d in (32, 96, 256):
        assert call_fp8(d=d) == E.FA_ERR_UNSUPPORTED, d
    for name in ("q", "k", "v", "o"):
        assert call_fp8(**{name: FAKE + 8}) == E.FA_ERR_MISALIGNED, name
    assert call_fp8(lse=FAKE + 2) == E.FA_ERR_MISALIGNED
    assert call_fp8() == E.FA_ERR_NO_DEVICE


def test_decode_noalloc_scratch_limit(lib):
    """fa_decode_noalloc refuses, on the host, a step whose partial results
    exceed its static scratch, and otherwise checks its arguments as fa_decode
    does (no call here reaches a launch: the pointers are fake)."""
    E = binding
    scratch = E.FA_DECODE_NOALLOC_SCRATCH_BYTES
    assert scratch == 16 << 20
    # 4096 query rows x 8 splits x (128 + 1) floats = 16.9 MB > 16 MiB
    big = (64, 64, 8, 1, 32768, 128)
    assert E.fa_decode_workspace_size(*big, 8) > scratch
    assert E.fa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, *big, 0.088, 1, None, 8, None) == E.FA_ERR_SCRATCH_TOO_SMALL
    # the same rows with 4 splits fit; on this host the call then stops at the device check
    assert E.fa_decode_workspace_size(*big, 4) <= scratch
    assert E.fa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, *big, 0.088, 1, None, 4, None) in (E.FA_ERR_NO_DEVICE,
                                                                                                 E.FA_ERR_UNSUPPORTED)
    assert E.fa_decode_noalloc(None, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 64, 64, 0.125, 0, None, 0, None) == \
        E.FA_ERR_INVALID_ARG
    assert E.fa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 64, 96, 0.125, 0, None, 0, None) == \
        E.FA_ERR_UNSUPPORTED
    assert E.fa_decode_noalloc(FAKE + 2, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 64, 64, 0.125, 0, None, 0, None) == \
        E.FA_ERR_MISALIGNED


def test_clock_sample_rejects_bad_pointers(lib):
    assert binding.fa_clock_sample(None, None) == binding.FA_ERR_INVALID_ARG
    assert binding.fa_clock_sample(FAKE + 4, None) == binding.FA_ERR_MISALIGNED
