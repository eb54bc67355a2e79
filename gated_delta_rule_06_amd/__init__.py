"""Python binding of libmuir: channel-wise gated delta-rule linear attention with
matched-filter readout (Muir), hand-written HIP kernels for AMD CDNA4 (gfx950).

The binding only marshals arguments: it checks tensor dtypes, shapes and devices,
allocates outputs and the workspace with PyTorch, passes raw device pointers and the
current HIP stream to the C ABI declared in ``include/muir.h``, and raises
``MuirError`` with the library's message on a non-zero status. Every step of the
computation runs in the library's kernels; there is no fallback. Importing works
without a GPU (argument validation can be exercised on the CPU), but the library
itself must be built (``python -m gated_delta_rule_06_amd._build``).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MuirError", "lib", "chunk_fwd", "chunk_fwd_workspace_size", "chunk_fwd_prepare",
    "chunk_fwd_scan", "chunk_fwd_scalar_erase", "chunk_fwd_scalar_erase_workspace_size",
    "chunk_fwd_scalar_erase_solve",
    "chunk_fwd_scalar_erase_scan", "lowrank_gates", "chunk_fwd_lowrank", "decode_step",
    "chunk_bwd", "chunk_bwd_workspace_size", "BWD_GRADS",
    "status_string", "last_error", "version", "MUIR_F32", "MUIR_BF16", "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuir.so")

MUIR_F32, MUIR_BF16 = 0, 1
STATUS = {0: "MUIR_OK", 1: "MUIR_ERR_NULL", 2: "MUIR_ERR_SHAPE", 3: "MUIR_ERR_UNSUPPORTED",
          4: "MUIR_ERR_WORKSPACE", 5: "MUIR_ERR_ALIAS", 6: "MUIR_ERR_HIP"}


class MuirError(RuntimeError):
    """A libmuir call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded ``libmuir.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m gated_delta_rule_06_amd._build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.muir_chunk_fwd_workspace_size.argtypes = [i] * 6 + [i]
        L.muir_chunk_fwd_workspace_size.restype = sz
        L.muir_chunk_fwd.argtypes = [vp] * 11 + [i] * 7 + [vp, sz, vp]
        L.muir_chunk_fwd.restype = i
        L.muir_chunk_fwd_noalloc.argtypes = [vp] * 11 + [i] * 7 + [vp]
        L.muir_chunk_fwd_noalloc.restype = i
        L.muir_chunk_fwd_noalloc_max_workspace.argtypes = []
        L.muir_chunk_fwd_noalloc_max_workspace.restype = sz
        L.muir_chunk_fwd_prepare.argtypes = [vp] * 5 + [i] * 6 + [vp, sz, vp]
        L.muir_chunk_fwd_prepare.restype = i
        L.muir_chunk_fwd_scan.argtypes = [vp] * 6 + [i] * 7 + [vp, sz, vp]
        L.muir_chunk_fwd_scan.restype = i
        L.muir_chunk_fwd_gated.argtypes = [vp] * 12 + [i] * 7 + [vp, sz, vp]
        L.muir_chunk_fwd_gated.restype = i
        L.muir_chunk_fwd_scan_gated.argtypes = [vp] * 7 + [i] * 7 + [vp, sz, vp]
        L.muir_chunk_fwd_scan_gated.restype = i
        L.muir_chunk_fwd_scalar_erase.argtypes = [vp] * 11 + [i] * 7 + [vp, sz, vp]
        L.muir_chunk_fwd_scalar_erase.restype = i
        L.muir_chunk_fwd_scalar_erase_workspace_size.argtypes = [i] * 6
        L.muir_chunk_fwd_scalar_erase_workspace_size.restype = sz
        L.muir_chunk_fwd_scalar_erase_solve.argtypes = [vp] * 3 + [i] * 6 + [vp, sz, vp]
        L.muir_chunk_fwd_scalar_erase_solve.restype = i
        L.muir_chunk_fwd_scalar_erase_scan.argtypes = [vp] * 3 + [i] * 7 + [vp, sz, vp]
        L.muir_chunk_fwd_scalar_erase_scan.restype = i
        L.muir_chunk_fwd_lowrank_workspace_size.argtypes = [i] * 6
        L.muir_chunk_fwd_lowrank_workspace_size.restype = sz
        L.muir_chunk_fwd_lowrank.argtypes = [vp] * 16 + [i] * 7 + [vp, sz, vp]
        L.muir_chunk_fwd_lowrank.restype = i
        L.muir_lowrank_gates.argtypes = [vp] * 13 + [i] * 4 + [vp]
        L.muir_lowrank_gates.restype = i
        L.muir_lowrank_output_gate.argtypes = [vp] * 4 + [i] * 4 + [vp]
        L.muir_lowrank_output_gate.restype = i
        L.muir_chunk_fwd_lowrank_gated_workspace_size.argtypes = [i] * 6
        L.muir_chunk_fwd_lowrank_gated_workspace_size.restype = sz
        L.muir_chunk_fwd_lowrank_gated.argtypes = [vp] * 18 + [i] * 7 + [vp, sz, vp]
        L.muir_chunk_fwd_lowrank_gated.restype = i
        L.muir_chunk_bwd_workspace_size.argtypes = [i] * 7
        L.muir_chunk_bwd_workspace_size.restype = sz
        L.muir_chunk_bwd.argtypes = [vp] * 20 + [i] * 7 + [vp, sz, vp]
        L.muir_chunk_bwd.restype = i
        L.muir_decode_step.argtypes = [vp] * 10 + [i] * 5 + [vp]
        L.muir_decode_step.restype = i
        L.muir_status_string.argtypes = [i]
        L.muir_status_string.restype = ctypes.c_char_p
        L.muir_last_error.argtypes = []
        L.muir_last_error.restype = ctypes.c_char_p
        L.muir_version.argtypes = []
        L.muir_version.restype = i
        L.muir_state_bytes.argtypes = [i] * 4
        L.muir_state_bytes.restype = sz
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().muir_status_string(int(status)).decode()


def last_error() -> str:
    return lib().muir_last_error().decode()


def version() -> int:
    return int(lib().muir_version())


def state_bytes(B: int, H: int, dk: int, dv: int) -> int:
    """Bytes of the fp32 recurrent state of B sequences x H heads (``muir_state_bytes``)."""
    return int(lib().muir_state_bytes(B, H, dk, dv))


def _check(status: int):
    if status != 0:
        raise MuirError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    if device.type != "cuda":
        return None
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return MUIR_F32
    if t.dtype == torch.bfloat16:
        return MUIR_BF16
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _require(t, name, dtype=None, shape=None, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (the library has no host path)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def chunk_fwd_workspace_size(B: int, T: int, H: int, dk: int, dv: int, chunk: int,
                             dtype_code: int) -> int:
    return int(lib().muir_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, dtype_code))


def chunk_fwd(q, k, v, a, g, e, w, r, s0=None, *, chunk: int = 64, o=None, s_out=None,
              return_state: bool = True, workspace=None, og=None):
    """Chunkwise forward over whole sequences (``muir_chunk_fwd``).

    q, k [B,T,H,dk] and v [B,T,H,dv] in float32 or bfloat16 (same dtype); a, g
    [B,T,H,dk], e, w [B,T,H,dv] and r [H,dk] float32; s0 [B,H,dk,dv] float32 or None.
    Returns (o, s_out): o [B,T,H,dv] in the q/k/v dtype and the final state (or None
    with ``return_state=False``). ``s_out`` may be passed (it may be ``s0`` itself for
    an in-place update); ``workspace`` may be a pre-allocated uint8 device tensor.
    With ``og`` ([B,T,H,dv] float32) the output-gate epilogue runs
    (``muir_chunk_fwd_gated``): o is multiplied by og elementwise as it is stored.
    """
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, q.dtype, (B, T, H, dk if name != "v" else dv), dev)
    for name, t, d in (("a", a, dk), ("g", g, dk), ("e", e, dv), ("w", w, dv)):
        _require(t, name, torch.float32, (B, T, H, d), dev)
    _require(r, "r", torch.float32, (H, dk), dev)
    if s0 is not None:
        _require(s0, "s0", torch.float32, (B, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    else:
        _require(o, "o", q.dtype, (B, T, H, dv), dev)
    if s_out is None and return_state:
        s_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif s_out is not None:
        _require(s_out, "s_out", torch.float32, (B, H, dk, dv), dev)
    need = chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _require(workspace, "workspace", torch.uint8, None, dev)
    if og is None:
        status = lib().muir_chunk_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(g), _ptr(e), _ptr(w), _ptr(r), _ptr(s0),
            _ptr(o), _ptr(s_out), B, T, H, dk, dv, chunk, code, _ptr(workspace),
            workspace.numel(), _stream(dev))
    else:
        _require(og, "og", torch.float32, (B, T, H, dv), dev)
        status = lib().muir_chunk_fwd_gated(
            _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(g), _ptr(e), _ptr(w), _ptr(og), _ptr(r),
            _ptr(s0), _ptr(o), _ptr(s_out), B, T, H, dk, dv, chunk, code, _ptr(workspace),
            workspace.numel(), _stream(dev))
    _check(status)
    return o, s_out


def chunk_bwd_workspace_size(B: int, T: int, H: int, dk: int, dv: int, chunk: int,
                            dtype_code: int) -> int:
    return int(lib().muir_chunk_bwd_workspace_size(B, T, H, dk, dv, chunk, dtype_code))


BWD_GRADS = ("q", "k", "v", "la", "g", "e", "w", "r", "s0")


def chunk_bwd(q, k, v, a, g, e, w, r, s0=None, *, do, ds_out=None, chunk: int = 64,
              workspace=None, out=None):
    """Backward pass of ``chunk_fwd`` (``muir_chunk_bwd``).

    Inputs as for ``chunk_fwd``, plus ``do`` (dL/do, [B,T,H,dv], the q/k/v dtype) and
    ``ds_out`` (dL/ds_out, [B,H,dk,dv] float32 or None). Returns a dict of float32
    gradients keyed by ``BWD_GRADS``: "la" is a * dL/da, "r" is [H,dk], "s0" is
    [B,H,dk,dv]. ``out`` may hold pre-allocated tensors under those keys.
    """
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        _require(t, name, q.dtype, (B, T, H, dk if name in ("q", "k") else dv), dev)
    for name, t, d in (("a", a, dk), ("g", g, dk), ("e", e, dv), ("w", w, dv)):
        _require(t, name, torch.float32, (B, T, H, d), dev)
    _require(r, "r", torch.float32, (H, dk), dev)
    for name, t in (("s0", s0), ("ds_out", ds_out)):
        if t is not None:
            _require(t, name, torch.float32, (B, H, dk, dv), dev)
    shapes = {n: (B, T, H, dk if n in ("q", "k", "la", "g") else dv) for n in BWD_GRADS}
    shapes["r"] = (H, dk)
    shapes["s0"] = (B, H, dk, dv)
    out = dict(out or {})
    for n, shp in shapes.items():
        if n in out:
            _require(out[n], "d" + n, torch.float32, shp, dev)
        else:
            out[n] = torch.empty(shp, dtype=torch.float32, device=dev)
    need = chunk_bwd_workspace_size(B, T, H, dk, dv, chunk, code)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _require(workspace, "workspace", torch.uint8, None, dev)
    status = lib().muir_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(g), _ptr(e), _ptr(w), _ptr(r), _ptr(s0),
        _ptr(do), _ptr(ds_out), *[_ptr(out[n]) for n in BWD_GRADS],
        B, T, H, dk, dv, chunk, code, _ptr(workspace), workspace.numel(), _stream(dev))
    _check(status)
    return out


def chunk_fwd_prepare(q, k, a, g, r, *, chunk: int, workspace):
    """Parallel phase of the chunk forward (``muir_chunk_fwd_prepare``) into ``workspace``."""
    import torch
    B, T, H, dk = q.shape
    dev = q.device
    code = _dtype_code(q)
    _require(q, "q", q.dtype, (B, T, H, dk), dev)
    _require(k, "k", q.dtype, (B, T, H, dk), dev)
    for name, t in (("a", a), ("g", g)):
        _require(t, name, torch.float32, (B, T, H, dk), dev)
    _require(r, "r", torch.float32, (H, dk), dev)
    _require(workspace, "workspace", torch.uint8, None, dev)
    _check(lib().muir_chunk_fwd_prepare(
        _ptr(q), _ptr(k), _ptr(a), _ptr(g), _ptr(r), B, T, H, dk, chunk, code,
        _ptr(workspace), workspace.numel(), _stream(dev)))


def chunk_fwd_scan(v, e, w, s0=None, *, chunk: int, workspace, o, s_out=None, og=None):
    """Sequential phase of the chunk forward (``muir_chunk_fwd_scan``) from ``workspace``;
    with ``og`` the output-gate epilogue (``muir_chunk_fwd_scan_gated``)."""
    import torch
    B, T, H, dv = v.shape
    dev = v.device
    code = _dtype_code(v)
    for name, t in (("e", e), ("w", w)):
        _require(t, name, torch.float32, (B, T, H, dv), dev)
    _require(o, "o", v.dtype, (B, T, H, dv), dev)
    if s0 is not None:
        _require(s0, "s0", torch.float32, (B, H, dv, dv), dev)
    if s_out is not None:
        _require(s_out, "s_out", torch.float32, (B, H, dv, dv), dev)
    _require(workspace, "workspace", torch.uint8, None, dev)
    if og is None:
        _check(lib().muir_chunk_fwd_scan(
            _ptr(v), _ptr(e), _ptr(w), _ptr(s0), _ptr(o), _ptr(s_out), B, T, H, dv, dv, chunk,
            code, _ptr(workspace), workspace.numel(), _stream(dev)))
    else:
        _require(og, "og", torch.float32, (B, T, H, dv), dev)
        _check(lib().muir_chunk_fwd_scan_gated(
            _ptr(v), _ptr(e), _ptr(w), _ptr(og), _ptr(s0), _ptr(o), _ptr(s_out), B, T, H, dv,
            dv, chunk, code, _ptr(workspace), workspace.numel(), _stream(dev)))


def chunk_fwd_scalar_erase_workspace_size(B: int, T: int, H: int, dk: int, dv: int,
                                          chunk: int) -> int:
    return int(lib().muir_chunk_fwd_scalar_erase_workspace_size(B, T, H, dk, dv, chunk))


def chunk_fwd_scalar_erase(q, k, v, a, g, e, w, r, s0=None, *, chunk: int = 256, o=None,
                           s_out=None, return_state: bool = True, workspace=None):
    """Chunk forward with one erase strength per token (``muir_chunk_fwd_scalar_erase``).

    As :func:`chunk_fwd` (bfloat16 q/k/v only) except ``e`` is [B,T,H] float32: the
    result equals the channel-wise forward with e broadcast over the value channels.
    Returns (o, s_out). ``workspace`` (uint8, at least
    :func:`chunk_fwd_scalar_erase_workspace_size` bytes) may be passed.
    """
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, q.dtype, (B, T, H, dk if name != "v" else dv), dev)
    for name, t, d in (("a", a, dk), ("g", g, dk), ("w", w, dv)):
        _require(t, name, torch.float32, (B, T, H, d), dev)
    _require(e, "e", torch.float32, (B, T, H), dev)
    _require(r, "r", torch.float32, (H, dk), dev)
    if s0 is not None:
        _require(s0, "s0", torch.float32, (B, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    else:
        _require(o, "o", q.dtype, (B, T, H, dv), dev)
    if s_out is None and return_state:
        s_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif s_out is not None:
        _require(s_out, "s_out", torch.float32, (B, H, dk, dv), dev)
    need = chunk_fwd_scalar_erase_workspace_size(B, T, H, dk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _require(workspace, "workspace", torch.uint8, None, dev)
    _check(lib().muir_chunk_fwd_scalar_erase(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(g), _ptr(e), _ptr(w), _ptr(r), _ptr(s0),
        _ptr(o), _ptr(s_out), B, T, H, dk, dv, chunk, code, _ptr(workspace),
        workspace.numel(), _stream(dev)))
    return o, s_out


def chunk_fwd_scalar_erase_solve(v, e, w, *, chunk: int, workspace):
    """The chunk-parallel phase (``muir_chunk_fwd_scalar_erase_solve``) on a workspace that
    :func:`chunk_fwd_prepare` (bf16 q/k/v) filled: the inverse, then the per-chunk products.
    Run it once per prepare."""
    import torch
    B, T, H, dv = v.shape
    dev = v.device
    _require(v, "v", torch.bfloat16, (B, T, H, dv), dev)
    _require(e, "e", torch.float32, (B, T, H), dev)
    _require(w, "w", torch.float32, (B, T, H, dv), dev)
    _require(workspace, "workspace", torch.uint8, None, dev)
    _check(lib().muir_chunk_fwd_scalar_erase_solve(
        _ptr(v), _ptr(e), _ptr(w), B, T, H, dv, chunk, MUIR_BF16, _ptr(workspace),
        workspace.numel(), _stream(dev)))


def chunk_fwd_scalar_erase_scan(s0=None, *, B: int, T: int, H: int, d: int, chunk: int,
                                workspace, o, s_out=None):
    """The sequential phase and the readout (``muir_chunk_fwd_scalar_erase_scan``) from a
    solved workspace; o [B,T,H,d] bfloat16 is written."""
    import torch
    dev = o.device
    _require(o, "o", torch.bfloat16, (B, T, H, d), dev)
    if s0 is not None:
        _require(s0, "s0", torch.float32, (B, H, d, d), dev)
    if s_out is not None:
        _require(s_out, "s_out", torch.float32, (B, H, d, d), dev)
    _require(workspace, "workspace", torch.uint8, None, dev)
    _check(lib().muir_chunk_fwd_scalar_erase_scan(
        _ptr(s0), _ptr(o), _ptr(s_out), B, T, H, d, d, chunk, MUIR_BF16, _ptr(workspace),
        workspace.numel(), _stream(dev)))


def lowrank_gates(z, U, c, *, H: int, d: int, which=("a", "e", "w", "g"), out=None):
    """Gates from the fused low-rank projection (``muir_lowrank_gates``).

    z [B,T,512] bfloat16; U a dict of up-projections {"decay": [H,d,64], "erase": [H,d,64],
    "write": [H,d,128], "read": [H,d,128]} bfloat16 and c the matching offsets [H,d]
    float32. Returns a dict of the requested gates among a (decay), e, w, g, each
    [B,T,H,d] float32 (``out`` may supply them)."""
    import torch
    B, T, R = z.shape
    dev = z.device
    _require(z, "z", torch.bfloat16, (B, T, 512), dev)
    names = {"a": ("decay", 64), "e": ("erase", 64), "w": ("write", 128), "g": ("read", 128)}
    out = dict(out or {})
    args = []
    for gname in ("a", "e", "w", "g"):
        n, r = names[gname]
        if gname in which:
            _require(U[n], "U_" + n, torch.bfloat16, (H, d, r), dev)
            _require(c[n], "c_" + n, torch.float32, (H, d), dev)
            if gname not in out:
                out[gname] = torch.empty((B, T, H, d), dtype=torch.float32, device=dev)
            _require(out[gname], gname, torch.float32, (B, T, H, d), dev)
            args.append((U[n], c[n], out[gname]))
        else:
            args.append((None, None, None))
    _check(lib().muir_lowrank_gates(
        _ptr(z), *[_ptr(x[0]) for x in args], *[_ptr(x[1]) for x in args],
        *[_ptr(x[2]) for x in args], B, T, H, d, _stream(dev)))
    return {k: v for k, v in out.items() if k in which}


def _chunk_fwd_lowrank(q, k, v, z, U, c, r, s0, chunk, o, s_out, return_state, workspace,
                       gated: bool):
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, torch.bfloat16, (B, T, H, dk if name != "v" else dv), dev)
    _require(z, "z", torch.bfloat16, (B, T, 512), dev)
    names = ("decay", "erase", "write", "read") + (("output",) if gated else ())
    for n in names:
        _require(U[n], "U_" + n, torch.bfloat16, (H, dk, 64 if n in ("decay", "erase") else 128), dev)
        _require(c[n], "c_" + n, torch.float32, (H, dk), dev)
    _require(r, "r", torch.float32, (H, dk), dev)
    if s0 is not None:
        _require(s0, "s0", torch.float32, (B, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    if s_out is None and return_state:
        s_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    size = (lib().muir_chunk_fwd_lowrank_gated_workspace_size if gated
            else lib().muir_chunk_fwd_lowrank_workspace_size)
    need = int(size(B, T, H, dk, dv, chunk))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ups = [_ptr(U[n]) for n in ("decay", "erase", "write", "read")]
    offs = [_ptr(c[n]) for n in ("decay", "erase", "write", "read")]
    tail = (_ptr(r), _ptr(s0), _ptr(o), _ptr(s_out), B, T, H, dk, dv, chunk, MUIR_BF16,
            _ptr(workspace), workspace.numel(), _stream(dev))
    if gated:
        _check(lib().muir_chunk_fwd_lowrank_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(z), *ups,
                                                  _ptr(U["output"]), *offs, _ptr(c["output"]), *tail))
    else:
        _check(lib().muir_chunk_fwd_lowrank(_ptr(q), _ptr(k), _ptr(v), _ptr(z), *ups, *offs, *tail))
    return o, s_out


def chunk_fwd_lowrank(q, k, v, z, U, c, r, s0=None, *, chunk: int = 256, o=None, s_out=None,
                      return_state: bool = True, workspace=None):
    """Chunk forward with the gates made from the low-rank gate projection inside the call
    (``muir_chunk_fwd_lowrank``). q, k, v bfloat16 as for :func:`chunk_fwd`; z, U, c as for
    :func:`lowrank_gates` (all four gates). Returns (o, s_out)."""
    return _chunk_fwd_lowrank(q, k, v, z, U, c, r, s0, chunk, o, s_out, return_state, workspace,
                              False)


def chunk_fwd_lowrank_gated(q, k, v, z, U, c, r, s0=None, *, chunk: int = 256, o=None,
                            s_out=None, return_state: bool = True, workspace=None):
    """As :func:`chunk_fwd_lowrank` with the output gate too (``muir_chunk_fwd_lowrank_gated``):
    U and c also hold "output" ([H, d, 128] bf16, [H, d] fp32); the readout is o * og."""
    return _chunk_fwd_lowrank(q, k, v, z, U, c, r, s0, chunk, o, s_out, return_state, workspace,
                              True)


def lowrank_output_gate(z, Uo, co, *, out=None):
    """The output gate og [B, T, H, d] fp32 from z's output slice (``muir_lowrank_output_gate``):
    z [B, T, 512] bf16, Uo [H, d, 128] bf16, co [H, d] fp32."""
    import torch
    B, T, _ = z.shape
    H, d, _ = Uo.shape
    dev = z.device
    _require(z, "z", torch.bfloat16, (B, T, 512), dev)
    _require(Uo, "Uo", torch.bfloat16, (H, d, 128), dev)
    _require(co, "co", torch.float32, (H, d), dev)
    if out is None:
        out = torch.empty((B, T, H, d), dtype=torch.float32, device=dev)
    _require(out, "og", torch.float32, (B, T, H, d), dev)
    _check(lib().muir_lowrank_output_gate(_ptr(z), _ptr(Uo), _ptr(co), _ptr(out), B, T, H, d,
                                          _stream(dev)))
    return out


def decode_step(q, k, v, a, g, e, w, r, state, *, o=None):
    """One recurrent step per (batch, head), updating ``state`` in place.

    q, k [B,H,dk], v [B,H,dv] (float32 or bfloat16); a, g [B,H,dk], e, w [B,H,dv],
    r [H,dk] float32; state [B,H,dk,dv] float32. Returns o [B,H,dv] (q/k/v dtype).
    """
    import torch
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    code = _dtype_code(q)
    for name, t, d in (("q", q, dk), ("k", k, dk), ("v", v, dv)):
        _require(t, name, q.dtype, (B, H, d), dev)
    for name, t, d in (("a", a, dk), ("g", g, dk), ("e", e, dv), ("w", w, dv)):
        _require(t, name, torch.float32, (B, H, d), dev)
    _require(r, "r", torch.float32, (H, dk), dev)
    _require(state, "state", torch.float32, (B, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    else:
        _require(o, "o", q.dtype, (B, H, dv), dev)
    status = lib().muir_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(g), _ptr(e), _ptr(w), _ptr(r),
        _ptr(state), _ptr(o), B, H, dk, dv, code, _stream(dev))
    _check(status)
    return o
