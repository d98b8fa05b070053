"""Python binding of the C interface in include/fa.h (ctypes).

Argument marshalling only: every step of the attention forward pass runs in the
HIP kernels of libfa_mi355x.so.  ``fa_fwd``, ``fa_fwd_f32`` and
``fa_fwd_gqa``, ``fa_fwd_gqa_f32``, ``fa_fwd_fp8``, ``fa_bwd``, ``fa_bwd_workspace_size``, ``fa_decode``,
``fa_decode_noalloc``, ``fa_decode_workspace_size`` and ``fa_status_str`` mirror
the C entry points one to one (raw device pointers as
ints, a hipStream_t as an int or None).  ``attention_forward`` is a convenience
wrapper for torch device tensors: it checks shapes, dtypes and layout, takes
the pointers and the current stream, and raises ``FaError`` on a non-zero
status.  There is no fallback: if the library is missing, loading raises.
"""
import ctypes
import os
import threading

from .build import LIB_PATH

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_MISALIGNED = -3
FA_ERR_NO_DEVICE = -4
FA_ERR_LAUNCH = -5
FA_ERR_SCRATCH_TOO_SMALL = -6
FA_DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTED_SYMBOLS = ("fa_bwd", "fa_bwd_workspace_size", "fa_clock_sample", "fa_decode", "fa_decode_noalloc",
                    "fa_decode_workspace_size", "fa_fwd", "fa_fwd_f32", "fa_fwd_fp8", "fa_fwd_gqa", "fa_fwd_gqa_f32",
                    "fa_status_str")

_lock = threading.Lock()
_lib = None


class FaError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {fa_status_str(status)} ({status})")
        self.status = status


def library_path():
    return LIB_PATH


def load():
    """Load libfa_mi355x.so (once).  Raises RuntimeError if it has not been built.

    The environment variable FA_MI355X_LIB names another build of the same
    library to load instead (the kernel-candidate copies that the kernel-choice
    measurements use); it must exist as well."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = os.environ.get("FA_MI355X_LIB") or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP library {path} is missing: build it with `python -m exact_io_aware_57_amd.build` "
                "(or __graft_entry__.build()); there is no CPU fallback")
        lib = ctypes.CDLL(path)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        for name in ("fa_fwd", "fa_fwd_f32"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp]
            fn.restype = i32
        for name in ("fa_fwd_gqa", "fa_fwd_gqa_f32"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp]
            fn.restype = i32
        lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, f32, f32, f32, i32, vp, vp]
        lib.fa_fwd_fp8.restype = i32
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp,
                               ctypes.c_size_t, vp]
        lib.fa_bwd.restype = i32
        lib.fa_bwd_workspace_size.argtypes = [i32, i32, i32]
        lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
        lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp, i32, vp, ctypes.c_size_t, vp]
        lib.fa_decode.restype = i32
        lib.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp, i32, vp]
        lib.fa_decode_noalloc.restype = i32
        lib.fa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        lib.fa_decode_workspace_size.restype = ctypes.c_size_t
        lib.fa_clock_sample.argtypes = [vp, vp]
        lib.fa_clock_sample.restype = i32
        lib.fa_status_str.argtypes = [i32]
        lib.fa_status_str.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _ptr(x):
    return None if x is None or x == 0 else ctypes.c_void_p(int(x))


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check(name, t, shape, dtype):
    """t must be a contiguous torch tensor of this shape and dtype."""
    import torch

    _need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor, got {type(t).__name__}")
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _check_workspace(t, need):
    import torch

    _need(isinstance(t, torch.Tensor) and t.dtype == torch.uint8 and t.dim() == 1 and t.is_contiguous(),
          "workspace must be a contiguous 1-D uint8 tensor")
    _need(t.numel() >= need, f"workspace must hold at least {need} bytes, got {t.numel()}")


def _check_devices(ref, **tensors):
    """ref must be on a GPU, and every tensor given (not None) on ref's device:
    the kernels read and write these pointers directly."""
    _need(ref.is_cuda, f"tensors must be on a GPU device, got {ref.device}")
    for name, t in tensors.items():
        if t is not None:
            _need(t.device == ref.device, f"{name} must be on {ref.device}, got {t.device}")


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, seqlens, stream):
    """C fa_fwd with integer device pointers (lse, seqlens, stream may be None)."""
    return load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(N), int(d),
                         float(scale), int(bool(causal)), _ptr(seqlens), _ptr(stream))


def fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, seqlens, stream):
    """C fa_fwd_f32 with integer device pointers (lse, seqlens, stream may be None)."""
    return load().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(N), int(d),
                             float(scale), int(bool(causal)), _ptr(seqlens), _ptr(stream))


def fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, seqlens, stream):
    """C fa_fwd_gqa with integer device pointers (k, v have H_kv heads)."""
    return load().fa_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(H_kv), int(N), int(d),
                             float(scale), int(bool(causal)), _ptr(seqlens), _ptr(stream))


def fa_fwd_gqa_f32(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, seqlens, stream):
    """C fa_fwd_gqa_f32 with integer device pointers (k, v have H_kv heads)."""
    return load().fa_fwd_gqa_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(H_kv), int(N), int(d),
                                 float(scale), int(bool(causal)), _ptr(seqlens), _ptr(stream))


def fa_fwd_fp8(q, k, v, o, lse, B, H, H_kv, N, d, scale, q_descale, k_descale, v_descale, causal, seqlens, stream):
    """C fa_fwd_fp8 with integer device pointers."""
    return load().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(H_kv), int(N), int(d),
                             float(scale), float(q_descale), float(k_descale), float(v_descale), int(bool(causal)),
                             _ptr(seqlens), _ptr(stream))


def attention_forward_fp8(q8, k8, v8, descale, scale, causal=False, seqlens=None, out=None, lse=None, stream=None,
                          want_lse=True):
    """O (bf16) and LSE for uint8 device tensors of e4m3 codes q8 [B, H, N, d],
    k8, v8 [B, H_kv, N, d] standing for descale[i] * value(code)."""
    import torch

    if q8.dim() != 4 or k8.dim() != 4 or k8.shape != v8.shape or k8.shape[0] != q8.shape[0] or k8.shape[2:] != q8.shape[2:]:
        raise ValueError(f"need q8 [B, H, N, d] and k8, v8 [B, H_kv, N, d], got {tuple(q8.shape)}, {tuple(k8.shape)}")
    B, H, N, d = q8.shape
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _check(name, t, t.shape, torch.uint8)
    _need(len(descale) == 3, "descale must hold three scales (q, k, v)")
    if out is not None:
        _check("out", out, (B, H, N, d), torch.bfloat16)
    if lse is not None:
        _check("lse", lse, (B, H, N), torch.float32)
    if seqlens is not None:
        _check("seqlens", seqlens, (B,), torch.int32)
    _check_devices(q8, k8=k8, v8=v8, out=out, lse=lse, seqlens=seqlens)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if want_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    if stream is None:
        stream = torch.cuda.current_stream(q8.device).cuda_stream
    st = fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(), None if lse is None else lse.data_ptr(),
                    B, H, k8.shape[1], N, d, scale, descale[0], descale[1], descale[2], causal,
                    None if seqlens is None else seqlens.data_ptr(), stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8")
    return out, lse


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale, causal, seqlens, workspace, workspace_size,
           stream):
    """C fa_bwd with integer device pointers."""
    return load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), int(B),
                         int(H), int(H_kv), int(N), int(d), float(scale), int(bool(causal)), _ptr(seqlens),
                         _ptr(workspace), int(workspace_size), _ptr(stream))


def fa_bwd_workspace_size(B, H, N):
    """Bytes of workspace fa_bwd needs (0 for invalid arguments)."""
    return int(load().fa_bwd_workspace_size(int(B), int(H), int(N)))


def attention_backward(q, k, v, o, lse, dout, scale, causal=False, seqlens=None, dq=None, dk=None, dv=None,
                       workspace=None, stream=None):
    """(dq, dk, dv) for torch bf16 device tensors q, o, dout [B, H, N, d], k, v
    [B, H_kv, N, d] and the forward pass's float32 lse [B, H, N].  Outputs and
    the workspace are allocated with torch when not given."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]:
        raise ValueError(f"need q [B, H, N, d] and k, v [B, H_kv, N, d], got {tuple(q.shape)}, {tuple(k.shape)}")
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    bf = torch.bfloat16
    for name, t, shape in (("q", q, q.shape), ("k", k, k.shape), ("v", v, k.shape), ("o", o, q.shape),
                           ("dout", dout, q.shape)):
        _check(name, t, shape, bf)
    _check("lse", lse, (B, H, N), torch.float32)
    for name, t, shape in (("dq", dq, q.shape), ("dk", dk, k.shape), ("dv", dv, k.shape)):
        if t is not None:
            _check(name, t, shape, bf)
    if seqlens is not None:
        _check("seqlens", seqlens, (B,), torch.int32)
    need = fa_bwd_workspace_size(B, H, N)
    if workspace is not None:
        _check_workspace(workspace, need)
    _check_devices(q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, seqlens=seqlens, workspace=workspace)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                dk.data_ptr(), dv.data_ptr(), B, H, H_kv, N, d, scale, causal,
                None if seqlens is None else seqlens.data_ptr(), workspace.data_ptr(), workspace.numel(), stream)
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def fa_decode(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal, seqlens, num_splits, workspace, workspace_size,
              stream):
    """C fa_decode with integer device pointers."""
    return load().fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(H_kv), int(Nq), int(Nk),
                            int(d), float(scale), int(bool(causal)), _ptr(seqlens), int(num_splits), _ptr(workspace),
                            int(workspace_size), _ptr(stream))


def fa_decode_noalloc(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal, seqlens, num_splits, stream):
    """C fa_decode_noalloc with integer device pointers (no workspace: the
    library's static per-GPU scratch holds the partial results)."""
    return load().fa_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(H_kv), int(Nq),
                                    int(Nk), int(d), float(scale), int(bool(causal)), _ptr(seqlens), int(num_splits),
                                    _ptr(stream))


def fa_decode_workspace_size(B, H, H_kv, Nq, Nk, d, num_splits=0):
    """Bytes of workspace fa_decode needs (0 for invalid arguments)."""
    return int(load().fa_decode_workspace_size(int(B), int(H), int(H_kv), int(Nq), int(Nk), int(d), int(num_splits)))


def decode_forward(q, k, v, scale, causal=False, seqlens=None, num_splits=0, out=None, lse=None, workspace=None,
                   stream=None, want_lse=True):
    """O (and LSE) of a decode step for torch bf16 device tensors q [B, H, Nq, d]
    and k, v [B, H_kv, Nk, d].  The workspace (a uint8 device tensor) is
    allocated with torch when not given.  Returns (out, lse or None)."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError(f"need q [B, H, Nq, d] and k, v [B, H_kv, Nk, d], got {tuple(q.shape)}, {tuple(k.shape)}")
    B, H, Nq, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, t.shape, torch.bfloat16)
    if out is not None:
        _check("out", out, q.shape, torch.bfloat16)
    if lse is not None:
        _check("lse", lse, (B, H, Nq), torch.float32)
    if seqlens is not None:
        _check("seqlens", seqlens, (B,), torch.int32)
    need = fa_decode_workspace_size(B, H, H_kv, Nq, Nk, d, num_splits)
    if workspace is not None:
        _check_workspace(workspace, need)
    _check_devices(q, k=k, v=v, out=out, lse=lse, seqlens=seqlens, workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), None if lse is None else lse.data_ptr(),
                   B, H, H_kv, Nq, Nk, d, scale, causal, None if seqlens is None else seqlens.data_ptr(), num_splits,
                   workspace.data_ptr(), workspace.numel(), stream)
    if st != FA_OK:
        raise FaError(st, "fa_decode")
    return out, lse


FA_CLOCK_SAMPLE_UNITS = 256


def fa_clock_sample(out, stream):
    """C fa_clock_sample: out is the device address of 3 * FA_CLOCK_SAMPLE_UNITS uint64 values."""
    return load().fa_clock_sample(_ptr(out), _ptr(stream))


def clock_mhz_by_unit(first, second):
    """Average core clock (MHz) of each compute unit between two fa_clock_sample
    results (3 * FA_CLOCK_SAMPLE_UNITS integers each), paired by the unit's
    place; units that held more than one sampling workgroup are left out:
    {place: MHz}."""
    def by_unit(v):
        seen, out = set(), {}
        for w in range(len(v) // 3):
            key = int(v[3 * w + 2])
            if key in seen:
                out.pop(key, None)
                continue
            seen.add(key)
            out[key] = (int(v[3 * w]), int(v[3 * w + 1]))
        return out
    a, b = by_unit(first), by_unit(second)
    res = {}
    for key in sorted(set(a) & set(b)):
        cyc, ticks = b[key][0] - a[key][0], b[key][1] - a[key][1]
        if cyc > 0 and ticks > 0:
            res[key] = 100.0 * cyc / ticks
    return res


def fa_status_str(status):
    return load().fa_status_str(int(status)).decode()


def attention_forward(q, k, v, scale, causal=False, seqlens=None, out=None, lse=None, stream=None, want_lse=True):
    """O (and LSE) for torch device tensors q [B, H, N, d] and k, v [B, H_kv, N, d].

    H_kv = H goes to fa_fwd / fa_fwd_f32 (bf16 / float32 tensors), a smaller
    H_kv (dividing H: grouped or multi-query attention) to fa_fwd_gqa /
    fa_fwd_gqa_f32.  ``out``/``lse``
    may be given (they must have the right shape, dtype and be contiguous);
    otherwise they are allocated with torch.  ``stream`` defaults to torch's
    current stream.  Returns (out, lse or None).
    """
    import torch

    if (q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]
            or k.shape[1] < 1 or q.shape[1] % k.shape[1]):
        raise ValueError(f"need q [B, H, N, d] and k, v [B, H_kv, N, d] with H_kv dividing H, got "
                         f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, t.shape, q.dtype)
    if out is not None:
        _check("out", out, q.shape, q.dtype)
    if lse is not None:
        _check("lse", lse, (B, H, N), torch.float32)
    if seqlens is not None:
        _check("seqlens", seqlens, (B,), torch.int32)
    _check_devices(q, k=k, v=v, out=out, lse=lse, seqlens=seqlens)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    H_kv = k.shape[1]
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), None if lse is None else lse.data_ptr())
    tail = (N, d, scale, causal, None if seqlens is None else seqlens.data_ptr(), stream)
    if H_kv == H:
        fn = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
        st = fn(*args, B, H, *tail)
    else:
        fn = fa_fwd_gqa if q.dtype == torch.bfloat16 else fa_fwd_gqa_f32
        st = fn(*args, B, H, H_kv, *tail)
    if st != FA_OK:
        raise FaError(st, fn.__name__)
    return out, lse
