"""Python binding of libflashgau.so (include/flashgau.h): argument marshalling only.

Every step of the layer runs in the HIP kernels of the library; this module checks tensor
metadata, allocates the output and the workspace with torch (caller-owned device memory, the
library itself never allocates) and passes raw pointers and torch's current stream. There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libflashgau.so")

F32 = 0
BF16 = 1

OK = 0
ERR_NULL_PTR = -1
ERR_BAD_SHAPE = -2
ERR_UNSUPPORTED = -3
ERR_MISALIGNED = -4
ERR_WORKSPACE = -5
ERR_ALIASING = -6
ERR_HIP = -7
ERR_TOO_LARGE = -8

# Order of the workspace buffers (FLASHGAU_WS_* in include/flashgau.h).
WS_NAMES = ("WCAT_T", "WO_T", "VT", "QQ", "KQ", "QL", "KLT", "P", "ST", "Y", "CARRY")

# Order of the decoding-state buffers (FLASHGAU_DS_* in include/flashgau.h).
DS_NAMES = ("S", "KQ", "KL", "V", "U", "QQ", "QL", "Y")

EXPORTS = ("flashgau_workspace_size", "flashgau_workspace_bytes", "flashgau_workspace_offsets", "flashgau_state_groups",
           "flash_gau_forward", "flash_gau_forward_packed", "flash_gau_forward_noalloc",
           "flashgau_noalloc_scratch_bytes",
           "flash_gau_forward_rope", "flash_gau_forward_timed",
           "flashgau_packed_weights_size",
           "flashgau_pack_weights", "flashgau_decode_state_size", "flashgau_decode_state_offsets",
           "flash_gau_decode_step", "flashgau_backward_workspace_size", "flash_gau_backward",
           "flash_gau_forward_train", "flash_gau_backward_saved", "flashgau_strerror")

# Kernels of one forward call, in launch order (FLASHGAU_NUM_STAGES in include/flashgau.h).
STAGES = ("pack", "proj", "scores_states", "carry", "mix", "out")

_lib = None


class FlashGauError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def lib() -> ctypes.CDLL:
    """Load libflashgau.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(python -m efficient_transformer_attention_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    i64, sz = ctypes.c_int64, ctypes.c_size_t
    L.flashgau_workspace_size.argtypes = [i64] * 6 + [ctypes.c_int, ctypes.c_int, ctypes.POINTER(sz)]
    L.flashgau_workspace_size.restype = ctypes.c_int
    L.flashgau_workspace_bytes.argtypes = [i64] * 6 + [ctypes.c_int, ctypes.c_int]
    L.flashgau_workspace_bytes.restype = sz
    L.flashgau_workspace_offsets.argtypes = [i64] * 6 + [ctypes.c_int, ctypes.c_int, ctypes.POINTER(sz)]
    L.flashgau_workspace_offsets.restype = ctypes.c_int
    L.flashgau_state_groups.argtypes = [i64] * 6 + [ctypes.c_int, ctypes.c_int, ctypes.POINTER(i64)]
    L.flashgau_state_groups.restype = ctypes.c_int
    vp = ctypes.c_void_p
    L.flash_gau_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, ctypes.c_int,
                                    i64, i64, i64, i64, i64, ctypes.c_int, vp, vp, sz, vp]
    L.flash_gau_forward.restype = ctypes.c_int
    L.flash_gau_forward_packed.argtypes = [vp, vp, sz, vp, vp, i64, ctypes.c_int, i64, i64, i64, i64,
                                           i64, ctypes.c_int, vp, vp, sz, vp]
    L.flash_gau_forward_packed.restype = ctypes.c_int
    L.flash_gau_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, ctypes.c_int,
                                            i64, i64, i64, i64, i64, ctypes.c_int, vp, vp]
    L.flash_gau_forward_noalloc.restype = ctypes.c_int
    L.flashgau_noalloc_scratch_bytes.argtypes = []
    L.flashgau_noalloc_scratch_bytes.restype = sz
    L.flash_gau_forward_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, ctypes.c_int, ctypes.c_float,
                                         i64, i64, i64, i64, i64, ctypes.c_int, vp, vp, sz, vp]
    L.flash_gau_forward_rope.restype = ctypes.c_int
    L.flash_gau_forward_timed.argtypes = L.flash_gau_forward.argtypes + [ctypes.POINTER(vp), ctypes.c_int]
    L.flash_gau_forward_timed.restype = ctypes.c_int
    L.flashgau_packed_weights_size.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(sz)]
    L.flashgau_packed_weights_size.restype = ctypes.c_int
    L.flashgau_pack_weights.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp, sz, vp]
    L.flashgau_pack_weights.restype = ctypes.c_int
    L.flashgau_decode_state_size.argtypes = [i64] * 5 + [ctypes.c_int, ctypes.POINTER(sz)]
    L.flashgau_decode_state_size.restype = ctypes.c_int
    L.flashgau_decode_state_offsets.argtypes = [i64] * 5 + [ctypes.c_int, ctypes.POINTER(sz)]
    L.flashgau_decode_state_offsets.restype = ctypes.c_int
    L.flash_gau_decode_step.argtypes = [vp, vp, sz, vp, vp, i64, i64, i64, ctypes.c_float, i64, i64,
                                        i64, i64, ctypes.c_int, vp, vp, sz, vp]
    L.flash_gau_decode_step.restype = ctypes.c_int
    L.flashgau_backward_workspace_size.argtypes = [i64] * 6 + [ctypes.c_int, ctypes.c_int, ctypes.POINTER(sz)]
    L.flashgau_backward_workspace_size.restype = ctypes.c_int
    L.flash_gau_backward.argtypes = [vp] * 8 + [i64, ctypes.c_int, ctypes.c_float] + [i64] * 5 + \
        [ctypes.c_int] + [vp] * 7 + [vp, sz, vp]
    L.flash_gau_backward.restype = ctypes.c_int
    L.flash_gau_backward_saved.argtypes = L.flash_gau_backward.argtypes
    L.flash_gau_backward_saved.restype = ctypes.c_int
    L.flash_gau_forward_train.argtypes = L.flash_gau_forward_rope.argtypes
    L.flash_gau_forward_train.restype = ctypes.c_int
    L.flashgau_strerror.argtypes = [ctypes.c_int]
    L.flashgau_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def strerror(code: int) -> str:
    return lib().flashgau_strerror(int(code)).decode()


def workspace_size(B, n, d, e, s, chunk, causal, dtype) -> int:
    out = ctypes.c_size_t(0)
    rc = lib().flashgau_workspace_size(B, n, d, e, s, chunk, int(bool(causal)), dtype, ctypes.byref(out))
    if rc != OK:
        raise FlashGauError(rc, "flashgau_workspace_size")
    return out.value


def workspace_bytes(B, n, d, e, s, chunk, causal, dtype) -> int:
    """flashgau_workspace_bytes: the workspace size, 0 for an empty or an invalid problem."""
    return int(lib().flashgau_workspace_bytes(B, n, d, e, s, chunk, int(bool(causal)), dtype))


def workspace_offsets(B, n, d, e, s, chunk, causal, dtype) -> dict:
    arr = (ctypes.c_size_t * len(WS_NAMES))()
    rc = lib().flashgau_workspace_offsets(B, n, d, e, s, chunk, int(bool(causal)), dtype, arr)
    if rc != OK:
        raise FlashGauError(rc, "flashgau_workspace_offsets")
    return dict(zip(WS_NAMES, list(arr)))


def state_groups(B, n, d, e, s, chunk, causal, dtype) -> int:
    out = ctypes.c_int64(0)
    rc = lib().flashgau_state_groups(B, n, d, e, s, chunk, int(bool(causal)), dtype, ctypes.byref(out))
    if rc != OK:
        raise FlashGauError(rc, "flashgau_state_groups")
    return out.value


def forward_raw(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, B, n, d, e, s, dtype, O,
                workspace, workspace_bytes, stream) -> int:
    """Direct call of flash_gau_forward with integer addresses; returns the library's code."""
    return lib().flash_gau_forward(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, int(bool(causal)),
                                   B, n, d, e, s, dtype, O, workspace, workspace_bytes, stream)


def forward_packed_raw(X, packed, packed_bytes, gamma, beta, chunk, causal, B, n, d, e, s, dtype, O,
                       workspace, workspace_bytes, stream) -> int:
    """Direct call of flash_gau_forward_packed with integer addresses; returns the library's code."""
    return lib().flash_gau_forward_packed(X, packed, packed_bytes, gamma, beta, chunk, int(bool(causal)),
                                          B, n, d, e, s, dtype, O, workspace, workspace_bytes, stream)


def forward_noalloc_raw(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, B, n, d, e, s, dtype, O,
                        stream) -> int:
    """Direct call of flash_gau_forward_noalloc with integer addresses; returns the library's code."""
    return lib().flash_gau_forward_noalloc(X, W_u, W_v, W_z, gamma, beta, W_o, chunk,
                                           int(bool(causal)), B, n, d, e, s, dtype, O, stream)


def noalloc_scratch_bytes() -> int:
    return int(lib().flashgau_noalloc_scratch_bytes())


def forward_rope_raw(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, rope_base, B, n, d, e, s,
                     dtype, O, workspace, workspace_bytes, stream) -> int:
    """Direct call of flash_gau_forward_rope with integer addresses; returns the library's code."""
    return lib().flash_gau_forward_rope(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, int(bool(causal)),
                                        float(rope_base), B, n, d, e, s, dtype, O, workspace,
                                        workspace_bytes, stream)


def forward_timed_raw(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, B, n, d, e, s, dtype, O,
                      workspace, workspace_bytes, stream, events) -> int:
    """flash_gau_forward_timed with integer addresses; ``events`` is a sequence of hipEvent_t
    handles (integers): len(STAGES) + 1 stage boundaries, or 2 * len(STAGES) start/stop pairs,
    one pair per kernel."""
    arr = (ctypes.c_void_p * len(events))(*events)
    return lib().flash_gau_forward_timed(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, int(bool(causal)),
                                         B, n, d, e, s, dtype, O, workspace, workspace_bytes, stream,
                                         arr, len(events))


def _dtype_code(t):
    import torch
    if t == torch.bfloat16:
        return BF16
    if t == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t}; use torch.bfloat16 or torch.float32")


def _check_inputs(X, W_u, W_v, W_z, gamma, beta, W_o, extra=()):
    """Shape, dtype, device and layout checks of the layer's inputs (and of `extra`: (name, tensor,
    shape) triples in X's dtype). Returns B, n, d, e, s, the dtype code and the device."""
    import torch
    if X.dim() != 3:
        raise ValueError(f"X must be [B, n, d], got shape {tuple(X.shape)}")
    B, n, d = X.shape
    if W_u.dim() != 2 or W_z.dim() != 2:
        raise ValueError("W_u and W_z must be matrices")
    e = W_u.shape[1]
    s = W_z.shape[1]
    dt = _dtype_code(X.dtype)
    for name, t, shape in (("W_u", W_u, (d, e)), ("W_v", W_v, (d, e)), ("W_z", W_z, (d, s)),
                           ("W_o", W_o, (e, d))) + tuple(extra):
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != X.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from X dtype {X.dtype}")
    for name, t in (("gamma", gamma), ("beta", beta)):
        if tuple(t.shape) != (4, s) or t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 [4, {s}]")
    tensors = (X, W_u, W_v, W_z, gamma, beta, W_o) + tuple(t for _, t, _ in extra)
    dev = X.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors):
        raise ValueError("all tensors must be on the same GPU")
    if any(not t.is_contiguous() for t in tensors):
        raise ValueError("all tensors must be contiguous (row-major)")
    return B, n, d, e, s, dt, dev


def _check_output(t, name, shape, dtype, dev):
    """A caller-supplied output buffer: exact shape and dtype, on the call's device, contiguous
    (the library writes through its raw address and cannot check any of this)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} dtype {t.dtype}, expected {dtype}")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(ws, nbytes, dev):
    """A caller-supplied workspace: a contiguous uint8 tensor of at least nbytes on the device."""
    import torch
    if ws.dtype != torch.uint8:
        raise TypeError(f"workspace must be uint8, got {ws.dtype}")
    if ws.device != dev:
        raise ValueError(f"workspace is on {ws.device}, expected {dev}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if ws.numel() < nbytes:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {nbytes} needed")


def _hold_for_stream(tensors, stream, dev):
    """Tensors that a call allocated from torch's caching allocator (which ties them to the
    current stream) but whose memory the library uses on ``stream``: when that is another stream,
    each is recorded on it, so that the allocator hands the memory out again only after the work
    queued there has finished (a workspace freed on return could otherwise be reused while the
    kernels still read it)."""
    import torch
    if not tensors or stream == torch.cuda.current_stream(dev).cuda_stream:
        return
    ext = torch.cuda.ExternalStream(stream, device=dev)
    for t in tensors:
        t.record_stream(ext)


def flash_gau_forward(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, out=None, workspace=None,
                      stream=None, rope_base=None):
    """One FLASH layer forward on the GPU. X [B, n, d]; W_u, W_v [d, e]; W_z [d, s]; gamma, beta
    [4, s] float32 (heads Q_quad, K_quad, Q_lin, K_lin); W_o [e, d]. X and the weights share one
    dtype (bfloat16 or float32). Returns O [B, n, d] of that dtype. ``workspace`` (uint8, on the
    same device) receives the intermediates; it is allocated when not given. ``rope_base`` (e.g.
    10000.0) selects flash_gau_forward_rope: the heads are rotated at their positions."""
    import torch
    B, n, d, e, s, dt, dev = _check_inputs(X, W_u, W_v, W_z, gamma, beta, W_o)
    nbytes = workspace_size(B, n, d, e, s, chunk, causal, dt)
    made = []
    if out is None:
        out = torch.empty((B, n, d), dtype=X.dtype, device=dev)
        made.append(out)
    else:
        _check_output(out, "out", (B, n, d), X.dtype, dev)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
        made.append(workspace)
    else:
        _check_workspace(workspace, nbytes, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    _hold_for_stream(made, stream, dev)
    ptrs = (X.data_ptr(), W_u.data_ptr(), W_v.data_ptr(), W_z.data_ptr(), gamma.data_ptr(),
            beta.data_ptr(), W_o.data_ptr())
    if rope_base is None:
        rc = forward_raw(*ptrs, chunk, causal, B, n, d, e, s, dt, out.data_ptr(), workspace.data_ptr(),
                         workspace.numel(), stream)
    else:
        rc = forward_rope_raw(*ptrs, chunk, causal, rope_base, B, n, d, e, s, dt, out.data_ptr(),
                              workspace.data_ptr(), workspace.numel(), stream)
    if rc != OK:
        raise FlashGauError(rc, "flash_gau_forward" if rope_base is None else "flash_gau_forward_rope")
    return out


def workspace_views(workspace, B, n, d, e, s, chunk, causal, dtype):
    """Typed views of the intermediates inside a workspace filled by flash_gau_forward, with the
    layouts documented in include/flashgau.h (for stage-by-stage checks)."""
    import torch
    tdt = torch.bfloat16 if dtype == BF16 else torch.float32
    esz = 2 if dtype == BF16 else 4
    off = workspace_offsets(B, n, d, e, s, chunk, causal, dtype)
    G = n // chunk
    M = B * n
    shapes = {
        "WCAT_T": (2 * e + s, d), "WO_T": (d, e), "VT": (B * G, e, chunk),
        "QQ": (M, s), "KQ": (M, s), "QL": (M, s), "KLT": (B * G, s, chunk),
        "P": (B * G, chunk, chunk), "ST": ((B * G) if causal else B, e, s), "Y": (M, e),
        "CARRY": (B, state_groups(B, n, d, e, s, chunk, causal, dtype), e, s),
    }
    views = {}
    for name, shape in shapes.items():
        count = 1
        for x in shape:
            count *= x
        raw = workspace[off[name]: off[name] + count * esz]
        views[name] = raw.view(tdt).view(shape)
    return views


# ------------------------------------------------------------------------------ decoding


def packed_weights_size(d, e, s, dtype) -> int:
    out = ctypes.c_size_t(0)
    rc = lib().flashgau_packed_weights_size(d, e, s, dtype, ctypes.byref(out))
    if rc != OK:
        raise FlashGauError(rc, "flashgau_packed_weights_size")
    return out.value


def decode_state_size(B, d, e, s, chunk, dtype) -> int:
    out = ctypes.c_size_t(0)
    rc = lib().flashgau_decode_state_size(B, d, e, s, chunk, dtype, ctypes.byref(out))
    if rc != OK:
        raise FlashGauError(rc, "flashgau_decode_state_size")
    return out.value


def decode_state_offsets(B, d, e, s, chunk, dtype) -> dict:
    arr = (ctypes.c_size_t * len(DS_NAMES))()
    rc = lib().flashgau_decode_state_offsets(B, d, e, s, chunk, dtype, arr)
    if rc != OK:
        raise FlashGauError(rc, "flashgau_decode_state_offsets")
    return dict(zip(DS_NAMES, list(arr)))


def pack_weights_raw(W_u, W_v, W_z, W_o, d, e, s, dtype, packed, packed_bytes, stream) -> int:
    """Direct call of flashgau_pack_weights with integer addresses; returns the library's code."""
    return lib().flashgau_pack_weights(W_u, W_v, W_z, W_o, d, e, s, dtype, packed, packed_bytes, stream)


def decode_step_raw(x, packed, packed_bytes, gamma, beta, chunk, t, n, rope_base, B, d, e, s, dtype, o,
                    state, state_bytes, stream) -> int:
    """Direct call of flash_gau_decode_step with integer addresses; returns the library's code."""
    return lib().flash_gau_decode_step(x, packed, packed_bytes, gamma, beta, chunk, t, n, float(rope_base),
                                       B, d, e, s, dtype, o, state, state_bytes, stream)


def pack_weights(W_u, W_v, W_z, W_o, stream=None):
    """Packs the weights for decoding (one transpose launch): returns a uint8 device tensor."""
    import torch
    d, e = W_u.shape
    s = W_z.shape[1]
    dt = _dtype_code(W_u.dtype)
    for name, t, shape in (("W_v", W_v, (d, e)), ("W_z", W_z, (d, s)), ("W_o", W_o, (e, d))):
        if tuple(t.shape) != shape or t.dtype != W_u.dtype:
            raise ValueError(f"{name} must be {W_u.dtype} {shape}")
    if any(not t.is_contiguous() or t.device != W_u.device for t in (W_u, W_v, W_z, W_o)):
        raise ValueError("weights must be contiguous and on one GPU")
    nbytes = packed_weights_size(d, e, s, dt)
    packed = torch.empty((nbytes,), dtype=torch.uint8, device=W_u.device)
    if stream is None:
        stream = torch.cuda.current_stream(W_u.device).cuda_stream
    _hold_for_stream([packed], stream, W_u.device)
    rc = pack_weights_raw(W_u.data_ptr(), W_v.data_ptr(), W_z.data_ptr(), W_o.data_ptr(), d, e, s, dt,
                          packed.data_ptr(), nbytes, stream)
    if rc != OK:
        raise FlashGauError(rc, "flashgau_pack_weights")
    return packed


class DecodeState:
    """Caller-owned decoding state of B sequences (one uint8 device buffer, layout in
    include/flashgau.h). The step at t = 0 clears the linear state itself."""

    def __init__(self, B, d, e, s, chunk, dtype, device):
        import torch
        self.B, self.d, self.e, self.s, self.chunk = B, d, e, s, chunk
        self.dt = _dtype_code(dtype)
        self.nbytes = decode_state_size(B, d, e, s, chunk, self.dt)
        self.buf = torch.empty((max(self.nbytes, 1),), dtype=torch.uint8, device=device)

    def views(self):
        """Typed views of the state's buffers."""
        import torch
        tdt = torch.bfloat16 if self.dt == BF16 else torch.float32
        esz = 2 if self.dt == BF16 else 4
        off = decode_state_offsets(self.B, self.d, self.e, self.s, self.chunk, self.dt)
        B, e, s, c = self.B, self.e, self.s, self.chunk
        shapes = {"S": (B, s, e), "KQ": (B, c, s), "KL": (B, c, s), "V": (B, c, e), "U": (B, e),
                  "QQ": (B, s), "QL": (B, s), "Y": (B, e)}
        views = {}
        for name, shape in shapes.items():
            count = 1
            for x in shape:
                count *= x
            if name == "S":
                views[name] = self.buf[off[name]: off[name] + count * 4].view(torch.float32).view(shape)
            else:
                views[name] = self.buf[off[name]: off[name] + count * esz].view(tdt).view(shape)
        return views


def flash_gau_decode_step(x, packed, gamma, beta, chunk, t, n, state, out=None, stream=None,
                          rope_base=0.0):
    """One causal decoding step on the GPU: x [B, d] holds token t of each sequence; returns
    o [B, d]. ``packed`` comes from pack_weights, ``state`` is a DecodeState advanced in place.
    ``rope_base`` > 0 rotates the heads at position t (as flash_gau_forward(rope_base=...))."""
    import torch
    B, d = x.shape
    if (B, d) != (state.B, state.d) or _dtype_code(x.dtype) != state.dt:
        raise ValueError("x does not match the decoding state")
    if not x.is_contiguous() or any(not g.is_contiguous() or g.dtype != torch.float32 for g in (gamma, beta)):
        raise ValueError("x must be contiguous; gamma and beta contiguous float32 [4, s]")
    if x.device.type != "cuda" or any(t.device != x.device for t in (packed, gamma, beta, state.buf)):
        raise ValueError("x, the packed weights, gamma, beta and the state must be on one GPU")
    if tuple(gamma.shape) != (4, state.s) or tuple(beta.shape) != (4, state.s):
        raise ValueError(f"gamma and beta must be float32 [4, {state.s}]")
    if packed.dtype != torch.uint8 or not packed.is_contiguous():
        raise ValueError("packed must be the contiguous uint8 tensor pack_weights returned")
    made = []
    if out is None:
        out = torch.empty((B, d), dtype=x.dtype, device=x.device)
        made.append(out)
    else:
        _check_output(out, "out", (B, d), x.dtype, x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    _hold_for_stream(made, stream, x.device)
    rc = decode_step_raw(x.data_ptr(), packed.data_ptr(), packed.numel(), gamma.data_ptr(),
                         beta.data_ptr(), chunk, t, n, rope_base, B, d, state.e, state.s, state.dt,
                         out.data_ptr(), state.buf.data_ptr(), state.buf.numel(), stream)
    if rc != OK:
        raise FlashGauError(rc, "flash_gau_decode_step")
    return out


# ------------------------------------------------------------------------------------- backward

GRAD_NAMES = ("dX", "dW_u", "dW_v", "dW_z", "dgamma", "dbeta", "dW_o")


def backward_workspace_size(B, n, d, e, s, chunk, causal, dtype) -> int:
    out = ctypes.c_size_t(0)
    rc = lib().flashgau_backward_workspace_size(B, n, d, e, s, chunk, int(bool(causal)), dtype,
                                               ctypes.byref(out))
    if rc != OK:
        raise FlashGauError(rc, "flashgau_backward_workspace_size")
    return out.value


def backward_raw(X, W_u, W_v, W_z, gamma, beta, W_o, dO, chunk, causal, rope_base, B, n, d, e, s,
                 dtype, dX, dW_u, dW_v, dW_z, dgamma, dbeta, dW_o, workspace, workspace_bytes,
                 stream) -> int:
    """Direct call of flash_gau_backward with integer addresses; returns the library's code."""
    return lib().flash_gau_backward(X, W_u, W_v, W_z, gamma, beta, W_o, dO, chunk, int(bool(causal)),
                                    float(rope_base), B, n, d, e, s, dtype, dX, dW_u, dW_v, dW_z,
                                    dgamma, dbeta, dW_o, workspace, workspace_bytes, stream)


def forward_train_raw(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, rope_base, B, n, d, e, s,
                      dtype, O, workspace, workspace_bytes, stream) -> int:
    """Direct call of flash_gau_forward_train with integer addresses; returns the library's code."""
    return lib().flash_gau_forward_train(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, int(bool(causal)),
                                         float(rope_base), B, n, d, e, s, dtype, O, workspace,
                                         workspace_bytes, stream)


def backward_saved_raw(X, W_u, W_v, W_z, gamma, beta, W_o, dO, chunk, causal, rope_base, B, n, d, e,
                       s, dtype, dX, dW_u, dW_v, dW_z, dgamma, dbeta, dW_o, workspace,
                       workspace_bytes, stream) -> int:
    """Direct call of flash_gau_backward_saved with integer addresses; returns the library's code."""
    return lib().flash_gau_backward_saved(X, W_u, W_v, W_z, gamma, beta, W_o, dO, chunk,
                                          int(bool(causal)), float(rope_base), B, n, d, e, s, dtype,
                                          dX, dW_u, dW_v, dW_z, dgamma, dbeta, dW_o, workspace,
                                          workspace_bytes, stream)


def flash_gau_forward_train(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, workspace,
                            rope_base=0.0, out=None, stream=None):
    """flash_gau_forward that also leaves in ``workspace`` (uint8, at least
    backward_workspace_size() bytes) what flash_gau_backward_saved reads. Returns O."""
    import torch
    B, n, d, e, s, dt, dev = _check_inputs(X, W_u, W_v, W_z, gamma, beta, W_o)
    nbytes = backward_workspace_size(B, n, d, e, s, chunk, causal, dt)
    _check_workspace(workspace, nbytes, dev)
    made = []
    if out is None:
        out = torch.empty((B, n, d), dtype=X.dtype, device=dev)
        made.append(out)
    else:
        _check_output(out, "out", (B, n, d), X.dtype, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    _hold_for_stream(made, stream, dev)
    tensors = (X, W_u, W_v, W_z, gamma, beta, W_o)
    rc = forward_train_raw(*(t.data_ptr() for t in tensors), chunk, causal, rope_base or 0.0, B, n,
                           d, e, s, dt, out.data_ptr(), workspace.data_ptr(), workspace.numel(), stream)
    if rc != OK:
        raise FlashGauError(rc, "flash_gau_forward_train")
    return out


def flash_gau_backward(X, W_u, W_v, W_z, gamma, beta, W_o, dO, chunk, causal, rope_base=0.0,
                       workspace=None, stream=None, out=None, saved=False):
    """Gradients of Σ O ⊙ dO for O = flash_gau_forward(X, ..., chunk, causal, rope_base) on the
    GPU. Arguments as flash_gau_forward, plus dO [B, n, d] of X's dtype. Returns a dict with dX
    [B, n, d], dW_u, dW_v [d, e], dW_z [d, s], dW_o [e, d] (X's dtype) and dgamma, dbeta [4, s]
    (float32). ``out`` may hold preallocated tensors under those names; ``workspace`` (uint8) is
    allocated when not given. ``saved=True`` calls flash_gau_backward_saved: ``workspace`` must then
    be the one a flash_gau_forward_train of the same inputs filled."""
    import torch
    if X.dim() != 3:
        raise ValueError(f"X must be [B, n, d], got shape {tuple(X.shape)}")
    B, n, d, e, s, dt, dev = _check_inputs(X, W_u, W_v, W_z, gamma, beta, W_o,
                                           extra=(("dO", dO, tuple(X.shape)),))
    tensors = (X, W_u, W_v, W_z, gamma, beta, W_o, dO)
    shapes = dict(dX=((B, n, d), X.dtype), dW_u=((d, e), X.dtype), dW_v=((d, e), X.dtype),
                  dW_z=((d, s), X.dtype), dgamma=((4, s), torch.float32),
                  dbeta=((4, s), torch.float32), dW_o=((e, d), X.dtype))
    grads = dict(out or {})
    unknown = set(grads) - set(shapes)
    if unknown:
        raise ValueError(f"unknown gradient names {sorted(unknown)}")
    made = []
    for k, (shape, tdt) in shapes.items():
        if k not in grads:
            grads[k] = torch.empty(shape, dtype=tdt, device=dev)
            made.append(grads[k])
        else:
            _check_output(grads[k], k, shape, tdt, dev)
    nbytes = backward_workspace_size(B, n, d, e, s, chunk, causal, dt)
    if saved and workspace is None:
        raise ValueError("saved=True needs the workspace of a flash_gau_forward_train call")
    if workspace is None:
        workspace = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
        made.append(workspace)
    else:
        _check_workspace(workspace, nbytes, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    _hold_for_stream(made, stream, dev)
    call = backward_saved_raw if saved else backward_raw
    rc = call(*(t.data_ptr() for t in tensors), chunk, causal, rope_base or 0.0, B, n, d, e,
              s, dt, *(grads[k].data_ptr() for k in GRAD_NAMES), workspace.data_ptr(),
              workspace.numel(), stream)
    if rc != OK:
        raise FlashGauError(rc, "flash_gau_backward_saved" if saved else "flash_gau_backward")
    return grads
