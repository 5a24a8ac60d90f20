"""Python binding of libgsi (include/gsi.h): argument marshalling only.

Every operation runs in the HIP kernels of libgsi.so; this module only turns
torch tensors into device pointers and status codes into exceptions.  If the
library is not built the first call raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_size_t, c_uint8, c_void_p

import torch

# GSI_LIBRARY names another build of the same library (the host-sanitizer
# build of build.build_sanitized, for the CPU-side argument tests).
LIB_PATH = os.environ.get("GSI_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgsi.so")

GSI_FP32, GSI_BF16 = 0, 1
GATED, FORCE_FAST, FORCE_SLOW = 0, 1, 2
PHASE_PROJECT, PHASE_APPLY = 1, 2
GSI_OK = 0

_DTYPES = {torch.float32: GSI_FP32, torch.bfloat16: GSI_BF16}


class GsiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


class GsiMapStruct(ctypes.Structure):
    _fields_ = [("d", c_int32), ("d_out", c_int32), ("k", c_int32), ("dtype", c_int32),
                ("W", c_void_p), ("V", c_void_p), ("M", c_void_p), ("G", c_void_p)]


class GsiCallStruct(ctypes.Structure):
    _fields_ = [("map", GsiMapStruct), ("x", c_void_p), ("y", c_void_p), ("eps", c_float),
                ("wave", c_int32), ("rho", c_void_p), ("slow", c_void_p)]


class GsiCalibStruct(ctypes.Structure):
    _fields_ = [("n", c_int32), ("d", c_int32), ("k", c_int32), ("dtype", c_int32),
                ("A", c_void_p), ("V0", c_void_p), ("V", c_void_p), ("iters", c_int32),
                ("reserved", c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgsi.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libgsi.so not built at {LIB_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.gsi_abi_version.restype = c_int32
        L.gsi_status_str.restype = ctypes.c_char_p
        L.gsi_status_str.argtypes = [c_int32]
        L.gsi_image_bytes.restype = c_size_t
        L.gsi_image_bytes.argtypes = [c_int32, c_int32, c_int32]
        L.gsi_gram_bytes.restype = c_size_t
        L.gsi_gram_bytes.argtypes = [c_int32, c_int32]
        L.gsi_prepare.restype = c_int32
        L.gsi_prepare.argtypes = [POINTER(GsiMapStruct), c_void_p]
        L.gsi_linear_workspace.restype = c_size_t
        L.gsi_linear_workspace.argtypes = [POINTER(GsiMapStruct), c_int32]
        L.gsi_linear.restype = c_int32
        L.gsi_linear.argtypes = [POINTER(GsiMapStruct), c_void_p, c_void_p, c_int32, c_float,
                                 c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.gsi_stack_plan_bytes.restype = c_size_t
        L.gsi_stack_plan_bytes.argtypes = [POINTER(GsiCallStruct), c_int32]
        L.gsi_stack_plan.restype = c_int32
        L.gsi_stack_plan.argtypes = [POINTER(GsiCallStruct), c_int32, c_void_p, c_size_t]
        L.gsi_stack_workspace.restype = c_size_t
        L.gsi_stack_workspace.argtypes = [c_void_p]
        L.gsi_stack.restype = c_int32
        L.gsi_stack.argtypes = [c_void_p, c_void_p, c_int32, c_void_p, c_size_t, c_void_p]
        L.gsi_stack_status_offset.restype = c_size_t
        L.gsi_stack_status_offset.argtypes = [c_void_p]
        L.gsi_calibrate_workspace.restype = c_size_t
        L.gsi_calibrate_workspace.argtypes = [POINTER(GsiCalibStruct)]
        L.gsi_calibrate_status_offset.restype = c_size_t
        L.gsi_calibrate_status_offset.argtypes = []
        L.gsi_calibrate.restype = c_int32
        L.gsi_calibrate.argtypes = [POINTER(GsiCalibStruct), c_void_p, c_size_t, c_void_p]
        L.gsi_static_scratch_bytes.restype = c_size_t
        L.gsi_static_scratch_bytes.argtypes = []
        L.gsi_linear_static.restype = c_int32
        L.gsi_linear_static.argtypes = [POINTER(GsiMapStruct), c_void_p, c_void_p, c_int32, c_float,
                                        c_int32, c_void_p, c_void_p, c_void_p]
        L.gsi_stack_phase.restype = c_int32
        L.gsi_stack_phase.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_size_t,
                                      c_void_p]
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().gsi_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != GSI_OK:
        raise GsiError(status, where)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def gsi_abi_version() -> int:
    return int(lib().gsi_abi_version())


def gsi_image_bytes(d_out: int, k: int, dtype: int) -> int:
    return int(lib().gsi_image_bytes(d_out, k, dtype))


class Map:
    """A linear map W [d_out][d] with basis V [d][k], its cached image M and,
    with exact_rho, the cached E = V^T V - I that makes its gates use the
    exact residual ratio of the stored basis."""

    def __init__(self, W: torch.Tensor, V: torch.Tensor, M: torch.Tensor | None = None,
                 exact_rho: bool = False):
        if W.dim() != 2 or V.dim() != 2 or W.shape[1] != V.shape[0]:
            raise ValueError(f"shapes W {tuple(W.shape)} and V {tuple(V.shape)} do not chain")
        if W.dtype != V.dtype:
            raise TypeError("W and V must share a dtype")
        if not (W.is_contiguous() and V.is_contiguous()):
            raise ValueError("W and V must be contiguous")
        self.W, self.V = W, V
        self.d_out, self.d = W.shape
        self.k = V.shape[1]
        self.dtype = _dtype_code(W)
        nbytes = gsi_image_bytes(self.d_out, self.k, self.dtype)
        if M is None:
            M = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=W.device)
        self.M = M
        self.G = None
        if exact_rho:
            self.G = torch.empty(max(int(lib().gsi_gram_bytes(self.k, self.dtype)), 16), dtype=torch.uint8,
                                 device=W.device)
        self.struct = GsiMapStruct(self.d, self.d_out, self.k, self.dtype,
                                   _ptr(W), _ptr(V), _ptr(M), _ptr(self.G))

    def gram(self) -> torch.Tensor:
        """E = V^T V - I as built by gsi_prepare ([k][k], storage dtype)."""
        return self.G[: self.k * self.k * self.W.element_size()].view(self.W.dtype).view(self.k, self.k)

    def image_rows(self) -> torch.Tensor:
        """The image M as a [d_out][k] tensor (un-tiles the library layout)."""
        el = self.W.dtype
        vw = 16 // self.W.element_size()
        tiles = (self.d_out + 63) // 64
        m = self.M[: tiles * 64 * self.k * self.W.element_size()].view(el)
        m = m.view(tiles, self.k // vw, 64, vw).permute(0, 2, 1, 3).reshape(tiles * 64, self.k)
        return m[: self.d_out]


def gsi_prepare(m: Map, stream=None) -> Map:
    """Build M = W V_k into m.M."""
    _check(lib().gsi_prepare(ctypes.byref(m.struct), _stream(stream)), "gsi_prepare")
    return m


def gsi_linear_workspace(m: Map, T: int) -> int:
    return int(lib().gsi_linear_workspace(ctypes.byref(m.struct), int(T)))


def workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled workspace buffer (zero before first use, as gsi.h requires)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def gsi_linear(m: Map, x: torch.Tensor, eps: float, mode: int = GATED, y=None, rho=None,
               slow=None, ws=None, stream=None):
    """Gated map on x [T][d]; returns (y [T][d_out], rho [T], slow [T] uint8)."""
    if x.dim() == 1:
        x = x[None]
    T = x.shape[0]
    if x.dtype != m.W.dtype or not x.is_contiguous() or x.shape[1] != m.d:
        raise ValueError("x must be a contiguous [T][d] tensor in the map's dtype")
    dev = x.device
    if y is None:
        y = torch.empty((T, m.d_out), dtype=x.dtype, device=dev)
    if rho is None:
        rho = torch.empty(T, dtype=torch.float32, device=dev)
    if slow is None:
        slow = torch.empty(T, dtype=torch.uint8, device=dev)
    need = gsi_linear_workspace(m, T)
    if ws is None:
        ws = workspace(need, dev)
    st = lib().gsi_linear(ctypes.byref(m.struct), _ptr(x), _ptr(y), int(T), float(eps), int(mode),
                          _ptr(rho), _ptr(slow), _ptr(ws), ws.numel() * ws.element_size(),
                          _stream(stream))
    _check(st, "gsi_linear")
    return y, rho, slow


def gsi_linear_static(m: Map, x: torch.Tensor, eps: float, mode: int = GATED, y=None, rho=None,
                      slow=None, stream=None):
    """gsi_linear with the library's own device scratch (no workspace, no
    allocation by the library); y, rho and slow are allocated here only if
    not given."""
    if x.dim() == 1:
        x = x[None]
    T = x.shape[0]
    if x.dtype != m.W.dtype or not x.is_contiguous() or x.shape[1] != m.d:
        raise ValueError("x must be a contiguous [T][d] tensor in the map's dtype")
    dev = x.device
    if y is None:
        y = torch.empty((T, m.d_out), dtype=x.dtype, device=dev)
    if rho is None:
        rho = torch.empty(T, dtype=torch.float32, device=dev)
    if slow is None:
        slow = torch.empty(T, dtype=torch.uint8, device=dev)
    st = lib().gsi_linear_static(ctypes.byref(m.struct), _ptr(x), _ptr(y), int(T), float(eps), int(mode),
                                 _ptr(rho), _ptr(slow), _stream(stream))
    _check(st, "gsi_linear_static")
    return y, rho, slow


def gsi_static_scratch_bytes() -> int:
    return int(lib().gsi_static_scratch_bytes())


class Stack:
    """A stack plan over batch-1 calls, with its device copy.

    calls: list of (Map, x [d], y [d_out], eps, rho (1 float) or None,
    slow (1 byte) or None[, wave]).  Calls of one wave are independent; a
    call may read the y of a call of an earlier wave.  Tensors must stay
    alive as long as the plan.
    """

    def __init__(self, calls, device=None):
        self._keep = calls
        n = len(calls)
        arr = (GsiCallStruct * max(n, 1))()
        for i, call in enumerate(calls):
            m, x, y, eps, rho, slow = call[:6]
            wave = int(call[6]) if len(call) > 6 else 0
            arr[i] = GsiCallStruct(m.struct, _ptr(x), _ptr(y), float(eps), wave, _ptr(rho), _ptr(slow))
        self._arr = arr
        nbytes = int(lib().gsi_stack_plan_bytes(arr, n))
        if n > 0 and nbytes == 0:
            # run the full check to get the failing status
            _check(lib().gsi_stack_plan(arr, n, None, 0), "gsi_stack_plan")
            raise GsiError(7, "gsi_stack_plan_bytes")
        self.host = torch.zeros(max(nbytes, 256), dtype=torch.uint8)
        _check(lib().gsi_stack_plan(arr, n, _ptr(self.host), self.host.numel()), "gsi_stack_plan")
        self.n = n
        self.ws_bytes = int(lib().gsi_stack_workspace(_ptr(self.host)))
        dev = device if device is not None else (calls[0][1].device if n else "cpu")
        self.dev = self.host.to(dev) if n else None
        self.status_offset = int(lib().gsi_stack_status_offset(_ptr(self.host)))

    def status(self, ws: torch.Tensor) -> int:
        """The device status word of this plan's runs in `ws` (0 = every run completed)."""
        o = self.status_offset
        return int(ws[o:o + 4].cpu().view(torch.int32)[0])

    def run(self, mode: int = GATED, ws=None, stream=None, check: bool = False):
        """Enqueue the plan's launch; with check=True wait for the stream and
        raise StackIncomplete if the launch left its status word set."""
        if ws is None:
            ws = workspace(self.ws_bytes, self.dev.device)
        gsi_stack(self, mode, ws, stream, check=check)
        return ws


class StackIncomplete(RuntimeError):
    """A stack launch ended with a device-side wait that ran out of its bound:
    the outputs of that run are incomplete (include/gsi.h, gsi_stack)."""

    def __init__(self, word: int):
        self.word = word
        super().__init__(f"gsi_stack: a device-side wait ran out (status word {word:#x}); outputs incomplete")


def gsi_stack(plan: Stack, mode: int, ws: torch.Tensor, stream=None, check: bool = False):
    """Run a plan (one launch).  gsi_stack returns GSI_OK once the launch is
    enqueued; whether every device-side wait finished is only known from the
    workspace's status word after the stream has run, which check=True
    reads (synchronising the stream) and turns into StackIncomplete."""
    st = lib().gsi_stack(_ptr(plan.host), _ptr(plan.dev), int(mode), _ptr(ws),
                         ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "gsi_stack")
    if check:
        if stream is None:
            torch.cuda.current_stream().synchronize()
        elif hasattr(stream, "synchronize"):
            stream.synchronize()
        else:
            torch.cuda.synchronize()
        word = plan.status(ws)
        if word != 0:
            raise StackIncomplete(word)


def gsi_stack_phase(plan: Stack, mode: int, phase: int, ws: torch.Tensor, stream=None):
    st = lib().gsi_stack_phase(_ptr(plan.host), _ptr(plan.dev), int(mode), int(phase), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "gsi_stack_phase")


def gsi_calibrate(A: torch.Tensor, V0: torch.Tensor, iters: int, V=None, ws=None, stream=None):
    """Basis of the dominant k-dim subspace of the samples A [n][d] after
    `iters` sweeps of subspace iteration from V0 [d][k] (random: a cold
    start; the previous layer's basis: the cascade).  Returns (V, status)
    where status is the device status word (0 = good) as a 1-element tensor."""
    if A.dim() != 2 or V0.dim() != 2 or A.shape[1] != V0.shape[0]:
        raise ValueError("A [n][d] and V0 [d][k] do not chain")
    if A.dtype != V0.dtype or not (A.is_contiguous() and V0.is_contiguous()):
        raise ValueError("A and V0 must be contiguous and share a dtype")
    n, d = A.shape
    k = V0.shape[1]
    if V is None:
        V = torch.empty_like(V0)
    c = GsiCalibStruct(n, d, k, _dtype_code(A), _ptr(A), _ptr(V0), _ptr(V), int(iters), 0)
    need = int(lib().gsi_calibrate_workspace(ctypes.byref(c)))
    if ws is None:
        ws = workspace(need, A.device)
    _check(lib().gsi_calibrate(ctypes.byref(c), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "gsi_calibrate")
    o = int(lib().gsi_calibrate_status_offset())
    return V, ws[o:o + 4].view(torch.int32)
