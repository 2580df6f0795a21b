"""Python binding of libexl3.so (include/exl3.h): argument marshalling only.

Every step of the EXL3 linear runs in the library's HIP kernels; this module
turns torch tensors into device pointers and torch streams into hipStream_t
handles, and turns error codes into exceptions. There is no CPU fallback: if
the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libexl3.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "exl3.h")

EXL3_OK = 0
EXL3_EINVAL = -1
EXL3_EALIGN = -2
EXL3_ERANGE = -3
EXL3_EBITS = -4
EXL3_EWORKSPACE = -5
EXL3_EGROUP = -6
EXL3_EHIP = -7
EXL3_ESCRATCH = -8
STATIC_SCRATCH_BYTES = 64 << 20
STATIC_COUNTER_BYTES = 256 << 10
WIDE_BLOCKS = 64


class exl3_weight_t(ctypes.Structure):
    _fields_ = [("words", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("suh", ctypes.c_void_p),
                ("svh", ctypes.c_void_p), ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("block_stride", ctypes.c_int64), ("bits", ctypes.c_int32), ("flags", ctypes.c_int32)]


class exl3_plan_t(ctypes.Structure):
    _fields_ = [("splits", ctypes.c_int32), ("waves", ctypes.c_int32), ("chunks", ctypes.c_int64),
                ("n_blocks", ctypes.c_int64)]


class exl3_workspace_t(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("bytes", ctypes.c_size_t), ("counter_bytes", ctypes.c_size_t)]


class Exl3Error(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        lib = _LIB
        msg = lib.exl3_strerror(code).decode() if lib is not None else str(code)
        if code == EXL3_EHIP and lib is not None:
            msg += f" (hip error {lib.exl3_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{code}]")


_LIB = None
P = ctypes.c_void_p
I64 = ctypes.c_int64
I32 = ctypes.c_int32
PP = ctypes.POINTER(ctypes.c_void_p)
W_P = ctypes.POINTER(exl3_weight_t)

_SIGNATURES = {
    "exl3_plan": (ctypes.c_int, [I64, I64, I32, ctypes.POINTER(exl3_plan_t)]),
    "exl3_weight_columns": (ctypes.c_int, [W_P, I64, I64, W_P]),
    "exl3_workspace_need": (ctypes.c_int, [I32, ctypes.POINTER(W_P), I64, ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.POINTER(ctypes.c_size_t)]),
    "exl3_workspace_grow": (ctypes.c_int, [ctypes.POINTER(exl3_workspace_t), P, ctypes.c_size_t, ctypes.c_size_t, P]),
    "exl3_workspace_reset": (ctypes.c_int, [ctypes.POINTER(exl3_workspace_t), P]),
    "exl3_linear": (ctypes.c_int, [W_P, P, I64, I64, P, I64, ctypes.POINTER(exl3_workspace_t), P]),
    "exl3_linear_group": (ctypes.c_int, [I32, ctypes.POINTER(W_P), P, I64, I64, PP, ctypes.POINTER(I64),
                                         ctypes.POINTER(exl3_workspace_t), P]),
    "exl3_linear_group_static": (ctypes.c_int, [I32, ctypes.POINTER(W_P), P, I64, I64, PP, ctypes.POINTER(I64), P]),
    "exl3_rotate": (ctypes.c_int, [I32, ctypes.POINTER(W_P), P, I64, I64, ctypes.POINTER(exl3_workspace_t), P]),
    "exl3_linear_rotated": (ctypes.c_int, [I32, ctypes.POINTER(W_P), I64, PP, ctypes.POINTER(I64),
                                           ctypes.POINTER(exl3_workspace_t), P]),
    "exl3_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "exl3_last_hip_error": (ctypes.c_int, []),
    "exl3_test_dequant": (ctypes.c_int, [W_P, P, P]),
    "exl3_test_codebook": (ctypes.c_int, [P, P, I64, P]),
    "exl3_test_rot_in": (ctypes.c_int, [W_P, P, I64, I64, P, P]),
    "exl3_set_prompt_arithmetic": (ctypes.c_int, [I32]),
    "exl3_test_force": (ctypes.c_int, [I32, I32, I32]),
    "exl3_test_fuse_rotation": (ctypes.c_int, [I32, I32]),
    "exl3_test_last_form": (ctypes.c_int, [ctypes.c_char_p, I64]),
    "exl3_test_mock": (ctypes.c_int, [I32]),
    "exl3_test_mock_counts": (ctypes.c_int, [ctypes.POINTER(I64), ctypes.POINTER(I64), ctypes.POINTER(I64), PP]),
}


def lib():
    """Load libexl3.so (built in-tree by __graft_entry__.build()); raise if absent.

    torch is imported first: it ships its own HIP runtime whose soname
    (libamdhip64.so.7) then satisfies libexl3.so's dependency, so the process
    holds one HIP runtime and torch's streams and pointers are valid in the
    library. Loaded the other way round, two runtimes would coexist.
    """
    global _LIB
    if _LIB is None:
        import torch  # noqa: F401  (loads the HIP runtime torch was built with)
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def _check(code: int, where: str):
    if code != EXL3_OK:
        raise Exl3Error(code, where)


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _torch_stream(stream):
    """The torch stream object for a stream argument (None: the current one)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


class Weight:
    """An EXL3 weight (or column view) whose tensors live on the device.

    Holds references to its tensors (or to its parent) so the raw pointers in
    the descriptor stay valid.
    """

    def __init__(self, words, scales, suh, svh, K: int, N: int, bits: int,
                 block_stride: Optional[int] = None, _desc: Optional[exl3_weight_t] = None, _parent=None):
        self.words, self.scales, self.suh, self.svh = words, scales, suh, svh
        self.K, self.N, self.bits = int(K), int(N), int(bits)
        self.parent = _parent
        if _desc is None:
            bs = block_stride if block_stride is not None else 16 * self.K * self.bits
            _desc = exl3_weight_t(_ptr(words), _ptr(scales), _ptr(suh), _ptr(svh), self.K, self.N, int(bs),
                                  self.bits, 0)
        self.desc = _desc
        self.block_stride = int(_desc.block_stride)

    @classmethod
    def from_host(cls, layer, device="cuda"):
        """Upload a synth.LayerInputs (raw bit patterns) to the device."""
        import torch
        words = torch.from_numpy(layer.words.copy()).to(device)
        as16 = lambda a: torch.from_numpy(a.view("int16").copy()).to(device)
        return cls(words, as16(layer.scales), as16(layer.suh), as16(layer.svh), layer.K, layer.N, layer.bits)

    def columns(self, col_from: int, n_cols: int) -> "Weight":
        return exl3_weight_columns(self, col_from, n_cols)


def exl3_plan(K: int, N: int, bits: int) -> exl3_plan_t:
    out = exl3_plan_t()
    _check(lib().exl3_plan(K, N, bits, ctypes.byref(out)), "exl3_plan")
    return out


def exl3_weight_columns(parent: Weight, col_from: int, n_cols: int) -> Weight:
    view = exl3_weight_t()
    _check(lib().exl3_weight_columns(ctypes.byref(parent.desc), col_from, n_cols, ctypes.byref(view)),
           "exl3_weight_columns")
    return Weight(None, None, None, None, parent.K, n_cols, parent.bits, _desc=view, _parent=parent)


def _wlist(weights: Sequence[Weight]):
    arr = (W_P * len(weights))(*[ctypes.pointer(w.desc) for w in weights])
    return arr


def exl3_workspace_need(weights: Sequence[Weight], M: int):
    b, cb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().exl3_workspace_need(len(weights), _wlist(weights), M, ctypes.byref(b), ctypes.byref(cb)),
           "exl3_workspace_need")
    return int(b.value), int(cb.value)


class Workspace:
    """Caller-side workspace: device memory that grows, never shrinks.

    `reserve` sizes it for some members up to `max_rows` rows; growth
    allocates a new buffer and lets the library zero its counters once on the
    given stream. Linear calls themselves never allocate.

    A replaced buffer is handed back to torch's allocator marked as in use by
    the growth's stream (record_stream), so its memory is reused only after
    the work queued there before the growth has finished. Calls on other
    streams must be ordered before the growth by the caller. With
    keep_retired=True replaced buffers are kept instead (for HIP graphs
    captured before a growth, which hold the old address) until
    release_retired().
    """

    def __init__(self, device="cuda", keep_retired: bool = False):
        self.device = device
        self.ws = exl3_workspace_t(None, 0, 0)
        self.buf = None
        self.keep_retired = keep_retired
        self.retired = []

    def release_retired(self):
        """Drop buffers kept by keep_retired=True (once nothing uses them)."""
        self.retired = []

    def reserve(self, weights: Sequence[Weight], max_rows: int, stream=None):
        import torch
        need, need_cb = exl3_workspace_need(weights, max_rows)
        rest = need - need_cb
        cur_cb = int(self.ws.counter_bytes)
        cur_rest = int(self.ws.bytes) - cur_cb
        if need_cb <= cur_cb and rest <= cur_rest:
            return self
        cb = max(cur_cb, need_cb)
        total = cb + max(rest, cur_rest)
        buf = torch.empty(total, dtype=torch.uint8, device=self.device)
        _check(lib().exl3_workspace_grow(ctypes.byref(self.ws), _ptr(buf), total, cb, _stream_handle(stream)),
               "exl3_workspace_grow")
        if self.buf is not None:
            if self.keep_retired:
                self.retired.append(self.buf)
            else:
                self.buf.record_stream(_torch_stream(stream))
        self.buf = buf
        return self

    def reset(self, stream=None):
        _check(lib().exl3_workspace_reset(ctypes.byref(self.ws), _stream_handle(stream)), "exl3_workspace_reset")

    def counters(self):
        """The counter region as a uint32-valued int64 tensor copy (for tests)."""
        import torch
        n = int(self.ws.counter_bytes) // 4
        return self.buf[: 4 * n].view(torch.int32).clone()


def exl3_linear(w: Weight, x, y, ws: Workspace, stream=None, M: Optional[int] = None):
    """y[:M, :N] = linear(x[:M, :K]); x and y are bf16 tensors with unit column stride."""
    M = x.shape[0] if M is None else M
    _check(lib().exl3_linear(ctypes.byref(w.desc), _ptr(x), x.stride(0), M, _ptr(y), y.stride(0),
                             ctypes.byref(ws.ws), _stream_handle(stream)), "exl3_linear")
    return y


def exl3_linear_group(weights: Sequence[Weight], x, ys, ws: Workspace, stream=None, M: Optional[int] = None):
    M = x.shape[0] if M is None else M
    n = len(weights)
    yp = (ctypes.c_void_p * n)(*[_ptr(y) for y in ys])
    ld = (I64 * n)(*[y.stride(0) for y in ys])
    _check(lib().exl3_linear_group(n, _wlist(weights), _ptr(x), x.stride(0), M, yp, ld, ctypes.byref(ws.ws),
                                   _stream_handle(stream)), "exl3_linear_group")
    return ys


def exl3_linear_group_static(weights: Sequence[Weight], x, ys, stream=None, M: Optional[int] = None):
    """exl3_linear_group in the library's static scratch (no workspace)."""
    M = x.shape[0] if M is None else M
    n = len(weights)
    yp = (ctypes.c_void_p * n)(*[_ptr(y) for y in ys])
    ld = (I64 * n)(*[y.stride(0) for y in ys])
    _check(lib().exl3_linear_group_static(n, _wlist(weights), _ptr(x), x.stride(0), M, yp, ld,
                                          _stream_handle(stream)), "exl3_linear_group_static")
    return ys


def exl3_rotate(weights: Sequence[Weight], x, ws: Workspace, stream=None, M: Optional[int] = None):
    """First launch of the group call: rotate x for every member into ws."""
    M = x.shape[0] if M is None else M
    _check(lib().exl3_rotate(len(weights), _wlist(weights), _ptr(x), x.stride(0), M, ctypes.byref(ws.ws),
                             _stream_handle(stream)), "exl3_rotate")


def exl3_linear_rotated(weights: Sequence[Weight], ys, ws: Workspace, M: int, stream=None):
    """Second launch: the linear on the rotated input held by ws."""
    n = len(weights)
    yp = (ctypes.c_void_p * n)(*[_ptr(y) for y in ys])
    ld = (I64 * n)(*[y.stride(0) for y in ys])
    _check(lib().exl3_linear_rotated(n, _wlist(weights), M, yp, ld, ctypes.byref(ws.ws), _stream_handle(stream)),
           "exl3_linear_rotated")
    return ys


def exl3_test_dequant(w: Weight, out, stream=None):
    _check(lib().exl3_test_dequant(ctypes.byref(w.desc), _ptr(out), _stream_handle(stream)), "exl3_test_dequant")
    return out


def exl3_test_codebook(states, out, stream=None):
    _check(lib().exl3_test_codebook(_ptr(states), _ptr(out), states.numel(), _stream_handle(stream)),
           "exl3_test_codebook")
    return out


def exl3_test_rot_in(w: Weight, x, out, stream=None, M: Optional[int] = None):
    M = x.shape[0] if M is None else M
    _check(lib().exl3_test_rot_in(ctypes.byref(w.desc), _ptr(x), x.stride(0), M, _ptr(out),
                                  _stream_handle(stream)), "exl3_test_rot_in")
    return out


def exl3_set_prompt_arithmetic(mode: int):
    """0: bit-stable prompt rows (default); 1: opt-in single-chain prompt tiles
    above 128 rows (faster, other bits)."""
    _check(lib().exl3_set_prompt_arithmetic(mode), "exl3_set_prompt_arithmetic")


def exl3_test_force(m_tiles: int = -1, chained: int = -1, splits: int = 0):
    _check(lib().exl3_test_force(m_tiles, chained, splits), "exl3_test_force")


def exl3_test_fuse_rotation(on: bool, spin_limit: int = -1):
    """on: rotate the input inside the linear launch at up to 32 rows (off by
    default); spin_limit: flag polls before a wave rotates a chunk itself
    (-1: the default)."""
    _check(lib().exl3_test_fuse_rotation(1 if on else 0, spin_limit), "exl3_test_fuse_rotation")


def exl3_test_last_form() -> str:
    """The kernel form of the last linear launch (issued or mock-recorded)."""
    buf = ctypes.create_string_buffer(128)
    _check(lib().exl3_test_last_form(buf, 128), "exl3_test_last_form")
    return buf.value.decode()


def exl3_test_mock(on: bool):
    _check(lib().exl3_test_mock(1 if on else 0), "exl3_test_mock")


def exl3_test_mock_counts():
    a, b, c = I64(), I64(), I64()
    s = ctypes.c_void_p()
    lib().exl3_test_mock_counts(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c), ctypes.byref(s))
    return int(a.value), int(b.value), int(c.value), s.value
