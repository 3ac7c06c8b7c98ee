"""Relative-position-bias attention on MI355X (gfx950): Python binding of librelbias_attn.so.

The binding only marshals arguments (shapes, dtypes, device pointers, the
current HIP stream) into the C ABI declared in include/relbias_attn.h; every
step of the computation runs in the library's HIP kernels.  PyTorch supplies
device memory and streams.  If the library is not built, every call raises.

  fwd(q, k, v, ...)                      prefill, q [B,S,Hq,D], k/v [B,S,Hkv,D]
  decode(q, k_cache, v_cache, kv_len, ...)  one new token per sequence
  decode_workspace_size(...)             scratch bytes decode needs
  decode_noalloc(q, k_cache, v_cache, kv_len, ...)  decode with the library's fixed scratch
  decode_paged(q, k_pages, v_pages, block_table, kv_lens, max_kv_len, ...)
                                         decode over a paged cache, one length per sequence

Bias modes: "none", "table" (table [Hq, bias_range] fp32), "rproj"
(r [.., Hq, R] in the activation dtype, E [Hq, R, bias_range] fp32) and
"rproj_shared" (the same r, one bank E [R, bias_range] for every head).
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = ["fwd", "bwd", "decode", "decode_noalloc", "decode_paged", "decode_fp4",
           "kv_quantize_fp4", "DECODE_NOALLOC_SCRATCH_BYTES",
           "decode_workspace_size", "last_error", "version",
           "library_path",
           "load_library", "RBA_OK", "RBA_EINVAL", "RBA_ENOTSUP", "RBA_EHIP", "MODES",
           "LibraryError"]

RBA_OK, RBA_EINVAL, RBA_ENOTSUP, RBA_EHIP = 0, 1, 2, 3
DECODE_NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024   # RBA_DECODE_NOALLOC_SCRATCH_BYTES
RBA_F32, RBA_BF16 = 0, 1
MODES = {"none": 0, "table": 1, "rproj": 2, "rproj_shared": 3}

_LIB = None


class LibraryError(RuntimeError):
    """A non-OK status from the C ABI (the message is relbias_attn_last_error())."""

    def __init__(self, status, message):
        super().__init__(f"[status {status}] {message}")
        self.status = status


def library_path() -> str:
    """The in-tree librelbias_attn.so, or the build named by RBA_LIBRARY (for instance the
    sanitizer build the CPU tests load)."""
    return os.environ.get("RBA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "librelbias_attn.so")


def load_library():
    """Load librelbias_attn.so (built in-tree); raise if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -m transformer_attention_learned_amd.build` "
            "(hipcc, gfx950) first; there is no fallback implementation")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.relbias_attn_fwd.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, vp, i,
                                     f, i, vp, sz, vp]
    lib.relbias_attn_fwd.restype = i
    lib.relbias_attn_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i, i, i, i, f]
    lib.relbias_attn_fwd_workspace_size.restype = sz
    lib.relbias_attn_decode.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, vp, vp,
                                        vp, i, f, i, vp, sz, vp]
    lib.relbias_attn_decode.restype = i
    lib.relbias_attn_decode_noalloc.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i,
                                                vp, vp, vp, i, f, i, vp]
    lib.relbias_attn_decode_noalloc.restype = i
    lib.relbias_attn_decode_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.relbias_attn_decode_workspace_size.restype = sz
    lib.relbias_attn_decode_paged.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                              i, i, i, vp, vp, vp, i, f, i, vp, sz, vp]
    lib.relbias_attn_decode_paged.restype = i
    lib.relbias_attn_decode_paged_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.relbias_attn_decode_paged_workspace_size.restype = sz
    lib.relbias_attn_bwd.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i,
                                     i, i, i, i, vp, vp, vp, i, f, i, vp, sz, vp]
    lib.relbias_attn_bwd.restype = i
    lib.relbias_attn_bwd_workspace_size.argtypes = [i, i, i, i, i]
    lib.relbias_attn_bwd_workspace_size.restype = sz
    lib.relbias_attn_kv_quantize_fp4.argtypes = [vp, vp, vp, ctypes.c_longlong, i, vp]
    lib.relbias_attn_kv_quantize_fp4.restype = i
    lib.relbias_attn_decode_fp4.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i,
                                            vp, vp, vp, i, f, i, vp, sz, vp]
    lib.relbias_attn_decode_fp4.restype = i
    lib.relbias_attn_decode_fp4_paged.argtypes = [vp] * 9 + [i] * 11 + [vp, vp, vp, i, f, i, vp,
                                                                          sz, vp]
    lib.relbias_attn_decode_fp4_paged.restype = i
    lib.relbias_attn_last_error.argtypes = []
    lib.relbias_attn_last_error.restype = ctypes.c_char_p
    lib.relbias_attn_version.argtypes = []
    lib.relbias_attn_version.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def last_error() -> str:
    return load_library().relbias_attn_last_error().decode()


def version() -> str:
    return load_library().relbias_attn_version().decode()


def _ptr(t):
    # a plain int: the c_void_p argtypes convert it (and None to NULL) without a wrapper object
    return None if t is None else t.data_ptr()


def _dtype_id(t):
    import torch
    if t.dtype == torch.bfloat16:
        return RBA_BF16
    if t.dtype == torch.float32:
        return RBA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _check(t, name, *, dtype=None, ndim=None, device=None):
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    # device check by index (get_device: -1 on the host), cheaper than comparing device objects
    if device is not None and t.get_device() != (-1 if device.index is None else device.index):
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream_handle(device, stream):
    import torch
    if stream is not None:
        return stream.cuda_stream
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None and device.index is not None:
        return raw(device.index)   # the current stream's handle, without a Stream object
    return torch.cuda.current_stream(device).cuda_stream


def _bias_args(mode, table, r, E, Hq, act_dtype, dev, bias_range):
    """Bias mode id and R; checks the exact shapes of the bias parameters (the C ABI can not:
    a table or bank shorter than bias_range or with fewer heads would be read past its end)."""
    import torch
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    if m not in (0, 1, 2, 3):
        raise ValueError(f"unknown bias mode {mode!r}")
    R = 0
    Rb = int(bias_range)
    if m == 1:
        if table is None:
            raise ValueError("mode 'table' needs table [Hq, bias_range]")
        _check(table, "table", dtype=torch.float32, ndim=2, device=dev)
        if tuple(table.shape) != (Hq, Rb):
            raise ValueError(f"table must be [Hq, bias_range] = {(Hq, Rb)}, got {tuple(table.shape)}")
    elif m in (2, 3):
        if r is None or E is None:
            raise ValueError("rproj modes need r and E")
        _check(E, "E", dtype=torch.float32, ndim=3 if m == 2 else 2, device=dev)
        _check(r, "r", dtype=act_dtype, device=dev)
        R = int(E.shape[1] if m == 2 else E.shape[0])
        want = (Hq, R, Rb) if m == 2 else (R, Rb)
        if tuple(E.shape) != want:
            raise ValueError(f"E must be {'[Hq, R, bias_range]' if m == 2 else '[R, bias_range]'} = "
                             f"{want}, got {tuple(E.shape)}")
        if r.shape[-1] != R or r.shape[-2] != Hq:
            raise ValueError(f"r must end in [Hq={Hq}, R={R}], got {tuple(r.shape)}")
    return m, R


def fwd_workspace_size(B, S, Hq, Hkv, D, *, dtype="bf16", window=0, bias_range=0, mode="none",
                       R=0, scale=None):
    """Workspace bytes fwd needs for these sizes (relbias_attn_fwd_workspace_size)."""
    lib = load_library()
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dt = RBA_BF16 if dtype in ("bf16", "bfloat16") else RBA_F32
    return int(lib.relbias_attn_fwd_workspace_size(dt, B, S, Hq, Hkv, D, int(window), int(bias_range),
                                                   m, int(R), float(scale)))


def fwd(q, k, v, *, window=0, bias_range=0, mode="none", table=None, r=None, E=None,
        scale=None, temp_len=0, out=None, lse=None, return_lse=False, workspace=None, stream=None):
    """Prefill attention with a relative-position bias (relbias_attn_fwd).

    q [B,S,Hq,D], k/v [B,S,Hkv,D] (bf16 or fp32, contiguous, on one GPU).
    temp_len: context-length temperature threshold (0: none; 131072 for the 128k form).
    workspace: optional uint8 device tensor of at least fwd_workspace_size(...) bytes; allocated
    here when needed and not given.
    Returns o [B,S,Hq,D] (and lse [B,Hq,S] fp32 when return_lse or lse is given).
    """
    import torch
    lib = load_library()
    dev = q.device
    _check(q, "q", ndim=4)
    _check(k, "k", dtype=q.dtype, ndim=4, device=dev)
    _check(v, "v", dtype=q.dtype, ndim=4, device=dev)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, S, Hkv, D) or tuple(v.shape) != (B, S, Hkv, D):
        raise ValueError(f"k/v must be [B,S,Hkv,D] = {(B, S, Hkv, D)}")
    m, R = _bias_args(mode, table, r, E, Hq, q.dtype, dev, bias_range)
    if m in (2, 3) and tuple(r.shape) != (B, S, Hq, R):
        raise ValueError(f"r must be [B,S,Hq,R] = {(B, S, Hq, R)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", dtype=q.dtype, ndim=4, device=dev)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    _check(lse, "lse", dtype=torch.float32, device=dev)
    need = int(lib.relbias_attn_fwd_workspace_size(_dtype_id(q), B, S, Hq, Hkv, D, int(window),
                                                   int(bias_range), m, R, float(scale)))
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(workspace, "workspace", dtype=torch.uint8, device=dev)
    st = lib.relbias_attn_fwd(_dtype_id(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                              B, S, Hq, Hkv, D, int(window), int(bias_range), m,
                              _ptr(table if m == 1 else None), _ptr(r if m in (2, 3) else None),
                              _ptr(E if m in (2, 3) else None), R, float(scale), int(temp_len),
                              _ptr(workspace), workspace.numel() if workspace is not None else 0,
                              _stream_handle(dev, stream))
    if st != RBA_OK:
        raise LibraryError(st, last_error())
    return (out, lse) if (return_lse or lse is not None) else out


def bwd(q, k, v, o, lse, dout, *, window=0, bias_range=0, mode="none", table=None, r=None,
        E=None, scale=None, temp_len=0, workspace=None, stream=None):
    """Backward of fwd (relbias_attn_bwd): gradients for an upstream gradient dout on o.

    q, k, v, window, bias_range, mode, table, r, E, scale, temp_len: as passed to fwd;
    o and lse [B,Hq,S] fp32: fwd's outputs.  bf16 (D 64 / 128) or fp32 (D 32 / 64 / 128).
    Returns a dict with dq, dk, dv and dtable (mode "table") or dr and dE (modes "rproj",
    "rproj_shared").
    """
    import torch
    lib = load_library()
    dev = q.device
    _check(q, "q", ndim=4)
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check(t, n, dtype=q.dtype, ndim=4, device=dev)
    _check(lse, "lse", dtype=torch.float32, ndim=3, device=dev)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, S, Hkv, D) or tuple(v.shape) != (B, S, Hkv, D):
        raise ValueError(f"k/v must be [B,S,Hkv,D] = {(B, S, Hkv, D)}")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    if tuple(lse.shape) != (B, Hq, S):
        raise ValueError(f"lse must be [B,Hq,S] = {(B, Hq, S)}")
    m, R = _bias_args(mode, table, r, E, Hq, q.dtype, dev, bias_range)
    if m in (2, 3) and tuple(r.shape) != (B, S, Hq, R):
        raise ValueError(f"r must be [B,S,Hq,R] = {(B, S, Hq, R)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v)}
    if m == 1:
        out["dtable"] = torch.empty_like(table)
    if m in (2, 3):
        out["dr"] = torch.empty_like(r)
        out["dE"] = torch.empty_like(E)
    need = lib.relbias_attn_bwd_workspace_size(B, S, Hq, m, int(bias_range))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.relbias_attn_bwd(
        _dtype_id(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(out["dq"]),
        _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out.get("dtable")), _ptr(out.get("dr")),
        _ptr(out.get("dE")), B, S, Hq, Hkv, D, int(window), int(bias_range), m,
        _ptr(table if m == 1 else None), _ptr(r if m in (2, 3) else None),
        _ptr(E if m in (2, 3) else None), R, float(scale), int(temp_len), _ptr(workspace), wbytes,
        _stream_handle(dev, stream))
    if st != RBA_OK:
        raise LibraryError(st, last_error())
    return out


def kv_quantize_fp4(x, stream=None):
    """MXFP4 quantisation (relbias_attn_kv_quantize_fp4) of bf16 x [..., D] (D % 32 == 0).

    Returns (codes uint8 [..., D / 2], scales uint8 [..., D / 32]) on x's device.
    """
    import torch
    lib = load_library()
    _check(x, "x", dtype=torch.bfloat16)
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    codes = torch.empty(x.shape[:-1] + (D // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (D // 32,), dtype=torch.uint8, device=x.device)
    st = lib.relbias_attn_kv_quantize_fp4(_ptr(x), _ptr(codes), _ptr(scales), rows, D,
                                          _stream_handle(x.device, stream))
    if st != RBA_OK:
        raise LibraryError(st, last_error())
    return codes, scales


def decode_fp4(q, k_codes, k_scales, v_codes, v_scales, kv_len, *, window=0, bias_range=0,
               mode="none", table=None, r=None, E=None, scale=None, temp_len=0, out=None,
               lse=None, workspace=None, return_lse=False, stream=None):
    """One decode step over MXFP4 caches (relbias_attn_decode_fp4).

    q [B,Hq,D] bf16; k_codes / v_codes uint8 [B,L_max,Hkv,D/2]; k_scales / v_scales uint8
    [B,L_max,Hkv,D/32] (as kv_quantize_fp4 writes them).  Other arguments as in decode.
    """
    import torch
    lib = load_library()
    dev = q.device
    _check(q, "q", dtype=torch.bfloat16, ndim=3)
    for t, n in ((k_codes, "k_codes"), (k_scales, "k_scales"), (v_codes, "v_codes"),
                 (v_scales, "v_scales")):
        _check(t, n, dtype=torch.uint8, ndim=4, device=dev)
    B, Hq, D = q.shape
    L_max, Hkv = k_codes.shape[1], k_codes.shape[2]
    if (tuple(k_codes.shape) != (B, L_max, Hkv, D // 2) or v_codes.shape != k_codes.shape or
            tuple(k_scales.shape) != (B, L_max, Hkv, D // 32) or v_scales.shape != k_scales.shape):
        raise ValueError("codes must be [B,L_max,Hkv,D/2] and scales [B,L_max,Hkv,D/32]")
    m, R = _bias_args(mode, table, r, E, Hq, q.dtype, dev, bias_range)
    if m in (2, 3) and tuple(r.shape) != (B, Hq, R):
        raise ValueError(f"r must be [B,Hq,R] = {(B, Hq, R)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = lib.relbias_attn_decode_workspace_size(B, Hq, Hkv, D, int(kv_len), int(window))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.relbias_attn_decode_fp4(
        _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales), _ptr(out),
        _ptr(lse), B, L_max, int(kv_len), Hq, Hkv, D, int(window), int(bias_range), m,
        _ptr(table if m == 1 else None), _ptr(r if m in (2, 3) else None),
        _ptr(E if m in (2, 3) else None), R, float(scale), int(temp_len), _ptr(workspace), wbytes,
        _stream_handle(dev, stream))
    if st != RBA_OK:
        raise LibraryError(st, last_error())
    return (out, lse) if (return_lse or lse is not None) else out


def decode_fp4_paged(q, k_codes, k_scales, v_codes, v_scales, block_table, kv_lens, max_kv_len,
                     *, window=0, bias_range=0, mode="none", table=None, r=None, E=None,
                     scale=None, temp_len=0, out=None, lse=None, workspace=None,
                     return_lse=False, stream=None):
    """One decode step over MXFP4 page pools (relbias_attn_decode_fp4_paged).

    k_codes / v_codes uint8 [num_pages, page_size, Hkv, D/2]; k_scales / v_scales uint8
    [num_pages, page_size, Hkv, D/32]; block_table, kv_lens and max_kv_len as in decode_paged.
    """
    import torch
    lib = load_library()
    dev = q.device
    _check(q, "q", dtype=torch.bfloat16, ndim=3)
    for t, n in ((k_codes, "k_codes"), (k_scales, "k_scales"), (v_codes, "v_codes"),
                 (v_scales, "v_scales")):
        _check(t, n, dtype=torch.uint8, ndim=4, device=dev)
    _check(block_table, "block_table", dtype=torch.int32, ndim=2, device=dev)
    _check(kv_lens, "kv_lens", dtype=torch.int32, ndim=1, device=dev)
    B, Hq, D = q.shape
    num_pages, page_size, Hkv = k_codes.shape[0], k_codes.shape[1], k_codes.shape[2]
    if (tuple(k_codes.shape) != (num_pages, page_size, Hkv, D // 2) or v_codes.shape != k_codes.shape
            or tuple(k_scales.shape) != (num_pages, page_size, Hkv, D // 32)
            or v_scales.shape != k_scales.shape):
        raise ValueError("codes must be [num_pages,page_size,Hkv,D/2] and scales "
                         "[num_pages,page_size,Hkv,D/32]")
    if block_table.shape[0] != B or kv_lens.shape[0] != B:
        raise ValueError("block_table [B, max_pages] and kv_lens [B] must match q's batch")
    m, R = _bias_args(mode, table, r, E, Hq, q.dtype, dev, bias_range)
    if m in (2, 3) and tuple(r.shape) != (B, Hq, R):
        raise ValueError(f"r must be [B,Hq,R] = {(B, Hq, R)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = lib.relbias_attn_decode_paged_workspace_size(B, Hq, Hkv, D, int(max_kv_len), int(window))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.relbias_attn_decode_fp4_paged(
        _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales), _ptr(block_table),
        _ptr(kv_lens), _ptr(out), _ptr(lse), B, num_pages, page_size, int(block_table.shape[1]),
        int(max_kv_len), Hq, Hkv, D, int(window), int(bias_range), m,
        _ptr(table if m == 1 else None), _ptr(r if m in (2, 3) else None),
        _ptr(E if m in (2, 3) else None), R, float(scale), int(temp_len), _ptr(workspace), wbytes,
        _stream_handle(dev, stream))
    if st != RBA_OK:
        raise LibraryError(st, last_error())
    return (out, lse) if (return_lse or lse is not None) else out


def decode_workspace_size(B, Hq, Hkv, D, kv_len, window=0) -> int:
    return int(load_library().relbias_attn_decode_workspace_size(B, Hq, Hkv, D, kv_len, window))


def decode(q, k_cache, v_cache, kv_len, *, window=0, bias_range=0, mode="none", table=None,
           r=None, E=None, scale=None, temp_len=0, out=None, lse=None, workspace=None,
           return_lse=False, stream=None):
    """One decode step (relbias_attn_decode): q [B,Hq,D] at position kv_len-1.

    k_cache/v_cache [B,L_max,Hkv,D]; rows [0, kv_len) are valid and row kv_len-1
    holds the new token.  workspace: optional uint8 device buffer (allocated
    here when needed and not given).
    """
    import torch
    lib = load_library()
    dev = q.device
    _check(q, "q", ndim=3)
    _check(k_cache, "k_cache", dtype=q.dtype, ndim=4, device=dev)
    _check(v_cache, "v_cache", dtype=q.dtype, ndim=4, device=dev)
    B, Hq, D = q.shape
    L_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, L_max, Hkv, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [B,L_max,Hkv,D] matching q")
    m, R = _bias_args(mode, table, r, E, Hq, q.dtype, dev, bias_range)
    if m in (2, 3) and tuple(r.shape) != (B, Hq, R):
        raise ValueError(f"r must be [B,Hq,R] = {(B, Hq, R)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = lib.relbias_attn_decode_workspace_size(B, Hq, Hkv, D, int(kv_len), int(window))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.relbias_attn_decode(_dtype_id(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                 _ptr(lse), B, L_max, int(kv_len), Hq, Hkv, D, int(window),
                                 int(bias_range), m, _ptr(table if m == 1 else None),
                                 _ptr(r if m in (2, 3) else None), _ptr(E if m in (2, 3) else None), R,
                                 float(scale), int(temp_len), _ptr(workspace), wbytes,
                                 _stream_handle(dev, stream))
    if st != RBA_OK:
        raise LibraryError(st, last_error())
    return (out, lse) if (return_lse or lse is not None) else out


def decode_noalloc(q, k_cache, v_cache, kv_len, *, window=0, bias_range=0, mode="none",
                   table=None, r=None, E=None, scale=None, temp_len=0, out=None, lse=None,
                   return_lse=False, stream=None):
    """decode through relbias_attn_decode_noalloc: no workspace, the split partials go to the
    library's fixed per-GPU scratch (bf16).  Calls that overlap on one GPU race; out (and lse)
    are allocated here when not given, so a caller that must not allocate passes them."""
    import torch
    lib = load_library()
    dev = q.device
    _check(q, "q", dtype=torch.bfloat16, ndim=3)
    _check(k_cache, "k_cache", dtype=q.dtype, ndim=4, device=dev)
    _check(v_cache, "v_cache", dtype=q.dtype, ndim=4, device=dev)
    B, Hq, D = q.shape
    L_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, L_max, Hkv, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache must be [B,L_max,Hkv,D] matching q")
    m, R = _bias_args(mode, table, r, E, Hq, q.dtype, dev, bias_range)
    if m in (2, 3) and tuple(r.shape) != (B, Hq, R):
        raise ValueError(f"r must be [B,Hq,R] = {(B, Hq, R)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", dtype=q.dtype, ndim=3, device=dev)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _check(lse, "lse", dtype=torch.float32, device=dev)
    st = lib.relbias_attn_decode_noalloc(RBA_BF16, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                         _ptr(lse), B, L_max, int(kv_len), Hq, Hkv, D, int(window),
                                         int(bias_range), m, _ptr(table if m == 1 else None),
                                         _ptr(r if m in (2, 3) else None),
                                         _ptr(E if m in (2, 3) else None), R, float(scale),
                                         int(temp_len), _stream_handle(dev, stream))
    if st != RBA_OK:
        raise LibraryError(st, last_error())
    return (out, lse) if (return_lse or lse is not None) else out


def decode_paged(q, k_pages, v_pages, block_table, kv_lens, max_kv_len, *, window=0,
                 bias_range=0, mode="none", table=None, r=None, E=None, scale=None, temp_len=0,
                 out=None, lse=None, workspace=None, return_lse=False, stream=None):
    """One decode step over a paged cache (relbias_attn_decode_paged).

    q [B,Hq,D] bf16; k_pages/v_pages [num_pages, page_size, Hkv, D]; block_table int32
    [B, max_pages] and kv_lens int32 [B] on the device; max_kv_len: host bound of kv_lens.
    Sequence b's row j is row j % page_size of page block_table[b, j // page_size].
    """
    import torch
    lib = load_library()
    dev = q.device
    _check(q, "q", ndim=3)
    _check(k_pages, "k_pages", dtype=q.dtype, ndim=4, device=dev)
    _check(v_pages, "v_pages", dtype=q.dtype, ndim=4, device=dev)
    _check(block_table, "block_table", dtype=torch.int32, ndim=2, device=dev)
    _check(kv_lens, "kv_lens", dtype=torch.int32, ndim=1, device=dev)
    B, Hq, D = q.shape
    num_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if tuple(k_pages.shape) != (num_pages, page_size, Hkv, D) or v_pages.shape != k_pages.shape:
        raise ValueError("k_pages/v_pages must be [num_pages, page_size, Hkv, D] matching q")
    if block_table.shape[0] != B or kv_lens.shape[0] != B:
        raise ValueError("block_table [B, max_pages] and kv_lens [B] must match q's batch")
    m, R = _bias_args(mode, table, r, E, Hq, q.dtype, dev, bias_range)
    if m in (2, 3) and tuple(r.shape) != (B, Hq, R):
        raise ValueError(f"r must be [B,Hq,R] = {(B, Hq, R)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = lib.relbias_attn_decode_paged_workspace_size(B, Hq, Hkv, D, int(max_kv_len), int(window))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.relbias_attn_decode_paged(
        _dtype_id(q), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(kv_lens),
        _ptr(out), _ptr(lse), B, num_pages, page_size, int(block_table.shape[1]), int(max_kv_len),
        Hq, Hkv, D, int(window), int(bias_range), m, _ptr(table if m == 1 else None),
        _ptr(r if m in (2, 3) else None), _ptr(E if m in (2, 3) else None), R, float(scale),
        int(temp_len), _ptr(workspace), wbytes, _stream_handle(dev, stream))
    if st != RBA_OK:
        raise LibraryError(st, last_error())
    return (out, lse) if (return_lse or lse is not None) else out
