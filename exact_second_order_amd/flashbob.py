"""Python binding of the C ABI in include/flashbob.h (argument marshalling only).

Every step of the computation runs in the HIP kernels of libflashbob.so; torch
only provides device memory and the current stream. If the library is not
built, loading fails loudly: there is no fallback path.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflashbob.so")

FLASHBOB_F32 = 0
FLASHBOB_BF16 = 1
FLASHBOB_CAUSAL = 1
FLASHBOB_FIRST_BACKWARD = 2
FLASHBOB_SAVED_LSE = 4
FLASHBOB_BF16_OUTPUTS = 8
# static buffer of flashbob_bob_noalloc (the header's FLASHBOB_NOALLOC_* macros)
FLASHBOB_NOALLOC_MAX_ROWS = 1 << 20
FLASHBOB_NOALLOC_SCRATCH_BYTES = 16 << 20
STAGE_BITS = {"pass1": 1, "pass2_query": 2, "pass2_key": 4}

ERRORS = {
    0: "OK",
    -1: "ERR_NULL",
    -2: "ERR_SHAPE",
    -3: "ERR_UNSUPPORTED_D",
    -4: "ERR_UNSUPPORTED_N",
    -5: "ERR_DTYPE",
    -6: "ERR_ALIGN",
    -7: "ERR_WORKSPACE",
    -8: "ERR_ALIAS",
    -9: "ERR_SCALE",
    -10: "ERR_FLAGS",
    -11: "ERR_SCRATCH",
    -100: "ERR_HIP",
}

EXPORTS = (
    "flashbob_workspace_bytes",
    "flashbob_bob",
    "flashbob_bob_pass1",
    "flashbob_bob_pass2_query",
    "flashbob_bob_pass2_key",
    "flashbob_rowstats",
    "flashbob_bob_ex",
    "flashbob_bob_noalloc",
    "flashbob_rowstats_ex",
    "flashbob_strerror",
    "flashbob_version",
)

_lib = None

# the kernels of one BoB call, in launch order
STAGES = {"pass1": "flashbob_bob_pass1", "pass2_query": "flashbob_bob_pass2_query",
          "pass2_key": "flashbob_bob_pass2_key"}


class FlashBoBError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"flashbob error {code} ({ERRORS.get(code, '?')}): {msg}")
        self.code = code


def load_library(path=LIB_PATH):
    """Load libflashbob.so and declare the C signatures."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m exact_second_order_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.flashbob_workspace_bytes.argtypes = [i, i, i, i]
    lib.flashbob_workspace_bytes.restype = sz
    lib.flashbob_bob.argtypes = [vp] * 7 + [vp] * 4 + [i, i, i, i, f, i, vp, sz, vp]
    lib.flashbob_bob.restype = i
    for name in STAGES.values():
        fn = getattr(lib, name)
        fn.argtypes = [vp] * 7 + [vp] * 4 + [i, i, i, i, f, i, vp, sz, vp]
        fn.restype = i
    lib.flashbob_rowstats.argtypes = [vp] * 7 + [vp] * 4 + [i, i, i, i, f, i, vp]
    lib.flashbob_rowstats.restype = i
    lib.flashbob_bob_ex.argtypes = [vp] * 7 + [vp] * 8 + [i, i, i, i, i, f, i, i, i, vp, sz, vp]
    lib.flashbob_bob_ex.restype = i
    lib.flashbob_bob_noalloc.argtypes = [vp] * 7 + [vp] * 4 + [i, i, i, i, f, i, vp]
    lib.flashbob_bob_noalloc.restype = i
    lib.flashbob_rowstats_ex.argtypes = [vp] * 7 + [vp] * 4 + [i, i, i, i, i, f, i, i, vp]
    lib.flashbob_rowstats_ex.restype = i
    lib.flashbob_strerror.argtypes = [i]
    lib.flashbob_strerror.restype = ctypes.c_char_p
    lib.flashbob_version.argtypes = []
    lib.flashbob_version.restype = i
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(code):
    if code != 0:
        msg = load_library().flashbob_strerror(code).decode()
        raise FlashBoBError(code, msg)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return FLASHBOB_BF16
    if dt == torch.float32:
        return FLASHBOB_F32
    raise TypeError(f"unsupported dtype {dt}; use torch.bfloat16 or torch.float32")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream_handle(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _inputs(Q, K, V, dO, gQ, gK, gV):
    """Checks shapes; returns the inputs and the key/value head count."""
    ins = (Q, K, V, dO, gQ, gK, gV)
    if Q.dim() != 4:
        raise ValueError("inputs must be [B, H, N, d]")
    B, H, N, d = Q.shape
    for k, t in enumerate(ins):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError("all inputs must be device tensors")
        if t.dtype != Q.dtype or t.device != Q.device:
            raise ValueError("all inputs need the same dtype and device")
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous [B, H, N, d]")
        want = Q.shape if k in (0, 3, 4) else K.shape  # Q, dO, gQ | K, V, gK, gV
        if t.shape != want:
            raise ValueError("Q, dO, gQ need one shape and K, V, gK, gV another")
    if K.dim() != 4 or K.shape[0] != B or K.shape[2:] != Q.shape[2:] or K.shape[1] < 1 or H % K.shape[1]:
        raise ValueError("K, V, gK, gV must be [B, H_kv, N, d] with H a multiple of H_kv")
    return ins, K.shape[1]


def shapes_of(B, H, Hkv, N, d):
    """Shapes of (gradQ, gradK, gradV, graddO); dQ, dK, dV follow the first three."""
    return ((B, H, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, H, N, d))


def workspace_bytes(B, H, N, d):
    return int(load_library().flashbob_workspace_bytes(B, H, N, d))


def _check_out(tensors, shapes, device, what, dtype=torch.float32):
    """Caller-given outputs: `dtype` (float32, or bfloat16 with the bf16-output
    flag), contiguous, on the inputs' device, of the expected shapes (the C ABI
    sees only pointers and trusts the sizes)."""
    tensors = tuple(tensors)
    if len(tensors) != len(shapes):
        raise ValueError(f"{what}: expected {len(shapes)} tensors, got {len(tensors)}")
    for t, s in zip(tensors, shapes):
        if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device != device:
            raise TypeError(f"{what}: outputs must be {dtype} tensors on {device}")
        if tuple(t.shape) != tuple(s) or not t.is_contiguous():
            raise ValueError(f"{what}: expected contiguous {tuple(s)}, got {tuple(t.shape)}")
    return tensors


def _check_lse(lse, B, H, N, device):
    """A saved log-sum-exp: float32 [B, H, N] on the inputs' device."""
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or lse.device != device:
        raise TypeError(f"lse must be a float32 tensor on {device}")
    if tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError(f"lse must be contiguous ({B}, {H}, {N}), got {tuple(lse.shape)}")
    return lse


def _out_dtype(dt):
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError(f"unsupported output dtype {dt}; use torch.float32 or torch.bfloat16")
    return dt


def _call_ex(lib, ins, out, first, lse, B, H, Hkv, N, d, scale, dtype, causal, stages, workspace, stream):
    flags = ((FLASHBOB_CAUSAL if causal else 0) | (FLASHBOB_FIRST_BACKWARD if first is not None else 0)
             | (FLASHBOB_SAVED_LSE if lse is not None else 0)
             | (FLASHBOB_BF16_OUTPUTS if out[0].dtype == torch.bfloat16 else 0))
    fb = first if first is not None else (None, None, None)
    return lib.flashbob_bob_ex(*[_ptr(t) for t in ins], *[_ptr(t) for t in out], *[_ptr(t) for t in fb],
                               _ptr(lse), B, H, Hkv, N, d, ctypes.c_float(scale), _dtype_code(dtype), flags,
                               stages, _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                               stream)


def _check_workspace(ws, B, H, N, d, device):
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise TypeError(f"workspace must be a contiguous tensor on {device}")
    if ws.numel() * ws.element_size() < workspace_bytes(B, H, N, d):
        raise ValueError(f"workspace needs {workspace_bytes(B, H, N, d)} bytes")
    return ws


def bob_stage(stage, Q, K, V, dO, gQ, gK, gV, out, workspace, scale=None, stream=None, causal=False,
              first=None, lse=None):
    """Run one kernel of bob(): stage in STAGES ("pass1", "pass2_query", "pass2_key").

    first: None, or the (dQ, dK, dV) float32 tensors that the pass-2 stages
    also fill with the first backward (flag FLASHBOB_FIRST_BACKWARD).
    lse: None, or the rows' saved log-sum-exp [B, H, N] that pass 1 starts
    from (flag FLASHBOB_SAVED_LSE).
    The outputs' dtype (float32, or bfloat16: flag FLASHBOB_BF16_OUTPUTS) is
    that of out[0]; every output must have it.
    """
    lib = load_library()
    ins, Hkv = _inputs(Q, K, V, dO, gQ, gK, gV)
    B, H, N, d = Q.shape
    if scale is None:
        scale = d ** -0.5
    shapes = shapes_of(B, H, Hkv, N, d)
    out = tuple(out)
    odt = _out_dtype(out[0].dtype if out and isinstance(out[0], torch.Tensor) else torch.float32)
    out = _check_out(out, shapes, Q.device, "out", odt)
    _check_workspace(workspace, B, H, N, d, Q.device)
    if first is not None:
        first = _check_out(first, shapes[:3], Q.device, "first", odt)
    if lse is not None:
        _check_lse(lse, B, H, N, Q.device)
    if causal or Hkv != H or first is not None or lse is not None or odt != torch.float32:
        rc = _call_ex(lib, ins, out, first, lse, B, H, Hkv, N, d, scale, Q.dtype, causal, STAGE_BITS[stage],
                      workspace, _stream_handle(Q.device, stream))
    else:
        fn = getattr(lib, STAGES[stage])
        rc = fn(*[_ptr(t) for t in ins], *[_ptr(t) for t in out], B, H, N, d, ctypes.c_float(scale),
                _dtype_code(Q.dtype), _ptr(workspace),
                ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                _stream_handle(Q.device, stream))
    _check(rc)


def bob_noalloc(Q, K, V, dO, gQ, gK, gV, scale=None, out=None, stream=None):
    """flashbob_bob_noalloc: BoB with the library's static row-scalar buffer
    instead of a workspace (plain multi-head, non-causal, float32 outputs;
    B*H*N <= 2^20). With `out` given the call allocates nothing. Calls that
    overlap on one GPU share the buffer and race."""
    lib = load_library()
    ins, Hkv = _inputs(Q, K, V, dO, gQ, gK, gV)
    if Hkv != Q.shape[1]:
        raise ValueError("bob_noalloc takes H_kv = H")
    B, H, N, d = Q.shape
    if scale is None:
        scale = d ** -0.5
    shapes = shapes_of(B, H, Hkv, N, d)
    if out is None:
        out = tuple(torch.empty(sh, dtype=torch.float32, device=Q.device) for sh in shapes)
    out = _check_out(out, shapes, Q.device, "out", torch.float32)
    _check(lib.flashbob_bob_noalloc(*[_ptr(t) for t in ins], *[_ptr(t) for t in out], B, H, N, d,
                                    ctypes.c_float(scale), _dtype_code(Q.dtype), _stream_handle(Q.device, stream)))
    return out


def bob(Q, K, V, dO, gQ, gK, gV, scale=None, out=None, workspace=None, stream=None, causal=False,
        first_backward=False, first_out=None, lse=None, out_dtype=torch.float32):
    """Exact BoB of softmax attention: (gradQ, gradK, gradV, graddO).

    Inputs [B, H, N, d] bf16 or fp32 device tensors; `scale` defaults to
    1/sqrt(d). `out` (four tensors of dtype out_dtype, shapes as returned)
    and `workspace` (a device tensor of at least workspace_bytes(B, H, N, d)
    bytes) may be given; with them (and first_out) the call allocates nothing.
    causal=True masks key j > query i (flashbob_bob_ex with FLASHBOB_CAUSAL).
    K, V, gK, gV may have fewer heads than Q (grouped-query attention): then
    gradK, gradV have their shape and sum over each group's query heads.
    first_backward=True also returns the first backward (dQ, dK, dV) of the
    same attention, float32, computed in the same passes: the result is then
    (gradQ, gradK, gradV, graddO, dQ, dK, dV). `first_out` may hold the three
    output tensors.
    lse ([B, H, N] float32) is a saved log-sum-exp of the rows (as a forward
    pass keeps it): pass 1 then starts from it instead of tracking a running
    maximum (flag FLASHBOB_SAVED_LSE; the outputs do not depend on it beyond
    rounding).
    out_dtype=torch.bfloat16 stores every output as bf16 (the float32 results
    rounded to nearest even; flag FLASHBOB_BF16_OUTPUTS).
    """
    lib = load_library()
    ins, Hkv = _inputs(Q, K, V, dO, gQ, gK, gV)
    B, H, N, d = Q.shape
    if scale is None:
        scale = d ** -0.5
    shapes = shapes_of(B, H, Hkv, N, d)
    odt = _out_dtype(out_dtype)
    if out is None:
        out = tuple(torch.empty(s, dtype=odt, device=Q.device) for s in shapes)
    out = _check_out(out, shapes, Q.device, "out", odt)
    nws = lib.flashbob_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=Q.device)
    _check_workspace(workspace, B, H, N, d, Q.device)
    first = None
    if first_backward:
        first = first_out
        if first is None:
            first = tuple(torch.empty(s, dtype=odt, device=Q.device) for s in shapes[:3])
        first = _check_out(first, shapes[:3], Q.device, "first_out", odt)
    if lse is not None:
        _check_lse(lse, B, H, N, Q.device)
    if causal or Hkv != H or first is not None or lse is not None or odt != torch.float32:
        rc = _call_ex(lib, ins, out, first, lse, B, H, Hkv, N, d, scale, Q.dtype, causal, 7, workspace,
                      _stream_handle(Q.device, stream))
    else:
        rc = lib.flashbob_bob(*[_ptr(t) for t in ins], *[_ptr(t) for t in out], B, H, N, d,
                              ctypes.c_float(scale), _dtype_code(Q.dtype), _ptr(workspace),
                              ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                              _stream_handle(Q.device, stream))
    _check(rc)
    return tuple(out) + (tuple(first) if first is not None else ())


def rowstats(Q, K, V, dO, gQ, gK, gV, scale=None, stream=None, causal=False):
    """Pass 1 alone: (LSE, D, c, r) per query row, each [B, H, N] float32."""
    lib = load_library()
    ins, Hkv = _inputs(Q, K, V, dO, gQ, gK, gV)
    B, H, N, d = Q.shape
    if scale is None:
        scale = d ** -0.5
    outs = tuple(torch.empty((B, H, N), dtype=torch.float32, device=Q.device) for _ in range(4))
    rc = lib.flashbob_rowstats_ex(*[_ptr(t) for t in ins], *[_ptr(t) for t in outs], B, H, Hkv, N, d,
                                  ctypes.c_float(scale), _dtype_code(Q.dtype),
                                  FLASHBOB_CAUSAL if causal else 0, _stream_handle(Q.device, stream))
    _check(rc)
    return outs


def raw_bob(ptrs_in, ptrs_out, B, H, N, d, scale, dtype_code, ws_ptr, ws_bytes, stream_ptr=0):
    """Direct C-ABI call with integer pointers; returns the integer status code."""
    lib = load_library()
    return lib.flashbob_bob(*[ctypes.c_void_p(p) for p in ptrs_in], *[ctypes.c_void_p(p) for p in ptrs_out],
                            B, H, N, d, ctypes.c_float(scale), dtype_code, ctypes.c_void_p(ws_ptr),
                            ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream_ptr))
