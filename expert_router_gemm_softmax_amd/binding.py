"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
of libmoe.so.  Tensors are passed as device pointers (``data_ptr()``) and
the stream is torch's current HIP stream unless one is given.  There is no
fallback: if libmoe.so is missing or fails to load, importing this module
raises ``MoeLibraryError``.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_double, c_float, c_int, c_int32, \
    c_int64, c_size_t, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK = 0
MOE_ERR_ARG = -1
MOE_ERR_DTYPE = -2
MOE_ERR_SHAPE = -3
MOE_ERR_ALIGN = -4
MOE_ERR_WORKSPACE = -5
MOE_ERR_LAUNCH = -6
MOE_ERR_UNIMPLEMENTED = -7

MOE_FP32 = 0
MOE_BF16 = 1
MOE_NO_CAPACITY = -1
MOE_FLAG_RECOMPUTE = 1
MOE_FLAG_RENORM = 2
MOE_FLAG_SLOT_PRIORITY = 4
MOE_FLAG_DROP_IDENTITY = 8

KERNELS = dict(ROUTE=0, PERMUTE_COUNT=1, PERMUTE_SCAN=2, PERMUTE_SCATTER=3,
               GEMM_UP=4, GEMM_DOWN=5, COMBINE=6, COMBINE_BWD=7, GEMM_DH=8,
               GEMM_DX=9, GEMM_DW2=10, GEMM_DW1=11, UNPERMUTE_BWD=12,
               ROUTE_BWD_DZ=13, ROUTE_BWD_DX=14, ROUTE_BWD_DW=15, SCHEDULE=16,
               ROUTE_PREP=17, PERMUTE_COPY=18, ROUTE_LOGITS=19, ROUTE_AUX=20,
               GEMM_RECOMPUTE=21, GEMM_FIXUP=22)


class MoeLibraryError(ImportError):
    pass


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        detail = lib.moe_last_error().decode() if status == MOE_ERR_LAUNCH else ""
        super().__init__(f"{fn} failed: {status} ({status_str(status)}) {detail}".rstrip())
        self.status = status


class MoeProbe(ctypes.Structure):
    _fields_ = [("kernel_id", c_int32), ("capacity", c_int32), ("count", c_int32),
                ("reserved_", c_int32), ("begin", POINTER(c_void_p)), ("end", POINTER(c_void_p))]


class MoeCfg(ctypes.Structure):
    _fields_ = [("T", c_int64), ("d", c_int32), ("E", c_int32), ("k", c_int32),
                ("f", c_int32), ("dtype", c_int32), ("capacity", c_int64),
                ("route_margin", c_float), ("flags", c_uint32), ("aux_coeff", c_float),
                ("probe", c_void_p)]

    def __copy__(self):
        # ctypes cannot pickle a structure holding a pointer: copy field by field
        return MoeCfg(**{n: getattr(self, n) for n, _ in self._fields_})

    def __repr__(self):
        return (f"MoeCfg(T={self.T}, d={self.d}, E={self.E}, k={self.k}, f={self.f}, "
                f"dtype={self.dtype}, capacity={self.capacity}, aux_coeff={self.aux_coeff})")


class MoeWeights(ctypes.Structure):
    _fields_ = [("Wr", c_void_p), ("b", c_void_p), ("W1", c_void_p), ("W2", c_void_p)]


class MoeCtx(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("probs", "idx", "gate", "counts", "offsets",
                                         "row_of", "src_of", "x_perm", "A", "H", "Y",
                                         "aux")]


class MoeGrads(ctypes.Structure):
    _fields_ = [("dWr", c_void_p), ("db", c_void_p), ("dW1", c_void_p), ("dW2", c_void_p)]


_P = c_void_p
_CFG = POINTER(MoeCfg)
_SIGS = {
    "moe_capacity": (c_int64, [c_int64, c_int32, c_int32, c_double]),
    "moe_rows_max": (c_int64, [_CFG]),
    "moe_workspace_bytes": (c_size_t, [_CFG]),
    "moe_status_str": (c_char_p, [c_int]),
    "moe_check_cfg": (c_int, [_CFG]),
    "moe_last_error": (c_char_p, []),
    "moe_route": (c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "moe_permute": (c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "moe_permute_noalloc": (c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_ffn": (c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "moe_combine": (c_int, [_CFG, _P, _P, _P, _P, _P, _P]),
    "moe_combine_bwd": (c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_ffn_bwd": (c_int, [_CFG] + [_P] * 11 + [c_size_t, _P]),
    "moe_unpermute_bwd": (c_int, [_CFG, _P, _P, _P, _P, _P, _P]),
    "moe_router_aux": (c_int, [_CFG, _P, _P, _P, _P, _P, c_size_t, _P]),
    "moe_route_bwd": (c_int, [_CFG] + [_P] * 12 + [c_size_t, _P]),
    "moe_layer_fwd": (c_int, [_CFG, POINTER(MoeWeights), _P, _P, POINTER(MoeCtx), _P,
                              c_size_t, _P]),
    "moe_layer_bwd": (c_int, [_CFG, POINTER(MoeWeights), _P, _P, POINTER(MoeCtx), _P,
                              POINTER(MoeGrads), _P, c_size_t, _P]),
}


def _hip_runtimes():
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def _load():
    # Device pointers and streams come from torch's HIP runtime; load it
    # first so that libmoe.so's libamdhip64.so.7 resolves to that same
    # runtime (by soname) instead of mapping a second one.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise MoeLibraryError(
            f"{LIB_PATH} is missing: build it with "
            "`python expert_router_gemm_softmax_amd/build.py`")
    try:
        lib = ctypes.CDLL(LIB_PATH)
    except OSError as e:
        raise MoeLibraryError(f"cannot load {LIB_PATH}: {e}") from e
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    rts = _hip_runtimes()
    if len(rts) > 1:
        raise MoeLibraryError(
            "two HIP runtimes are mapped into this process (" + ", ".join(rts) + "); "
            "import torch before anything that loads libamdhip64")
    return lib


lib = _load()


# ------------------------------------------------------------------ helpers
def status_str(status: int) -> str:
    return lib.moe_status_str(int(status)).decode()


def _check(fn: str, rc: int):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def _ptr(t):
    """Device address of a tensor (None for None or an empty tensor); an int
    passes through as a raw address.  The kernels read every tensor as a dense
    row-major buffer in GPU memory, so a host tensor or a strided view is
    refused here instead of faulting or giving wrong results in a kernel."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if t.device.type != "cuda":
        raise ValueError(f"tensor on {t.device}: the library reads GPU memory only")
    if not t.is_contiguous():
        raise ValueError(f"tensor of strides {tuple(t.stride())}: the library reads "
                         "dense row-major buffers")
    return t.data_ptr() or None


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_cfg(T, d, E, k, f, dtype="bf16", capacity=None, route_margin=0.0,
             aux_coeff=0.0, recompute=False, renorm=False, priority="token",
             fallback="none") -> MoeCfg:
    """capacity: None = no limit, else an int >= 0; aux_coeff: weight of the
    load-balancing loss (0 = none); recompute: keep A and H out of the saved
    state and recompute them in backward (MOE_FLAG_RECOMPUTE); renorm: gates
    renormalised over the selected experts (MOE_FLAG_RENORM); priority:
    'token' or 'slot' capacity walk (MOE_FLAG_SLOT_PRIORITY); fallback: 'none'
    or 'identity' for dropped assignments (MOE_FLAG_DROP_IDENTITY)."""
    if priority not in ("token", "slot"):
        raise ValueError(f"priority must be 'token' or 'slot', not {priority!r}")
    if fallback not in ("none", "identity"):
        raise ValueError(f"fallback must be 'none' or 'identity', not {fallback!r}")
    dt = {"bf16": MOE_BF16, "f32": MOE_FP32, MOE_BF16: MOE_BF16, MOE_FP32: MOE_FP32}[dtype]
    return MoeCfg(T=int(T), d=int(d), E=int(E), k=int(k), f=int(f), dtype=dt,
                  capacity=MOE_NO_CAPACITY if capacity is None else int(capacity),
                  route_margin=float(route_margin),
                  flags=((MOE_FLAG_RECOMPUTE if recompute else 0)
                         | (MOE_FLAG_RENORM if renorm else 0)
                         | (MOE_FLAG_SLOT_PRIORITY if priority == "slot" else 0)
                         | (MOE_FLAG_DROP_IDENTITY if fallback == "identity" else 0)),
                  aux_coeff=float(aux_coeff))


def moe_capacity(T, k, E, cf) -> int:
    return int(lib.moe_capacity(int(T), int(k), int(E), float(cf)))


def moe_rows_max(cfg: MoeCfg) -> int:
    return int(lib.moe_rows_max(byref(cfg)))


def moe_workspace_bytes(cfg: MoeCfg) -> int:
    return int(lib.moe_workspace_bytes(byref(cfg)))


def moe_check_cfg(cfg: MoeCfg) -> int:
    return int(lib.moe_check_cfg(byref(cfg)))


# ------------------------------------------------------------------ entry points
def moe_route(cfg, x, Wr, b, probs, idx, gate, ws, stream=None):
    _check("moe_route", lib.moe_route(
        byref(cfg), _ptr(x), _ptr(Wr), _ptr(b), _ptr(probs), _ptr(idx), _ptr(gate),
        _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_permute(cfg, x, idx, counts, offsets, row_of, src_of, x_perm, ws, stream=None):
    _check("moe_permute", lib.moe_permute(
        byref(cfg), _ptr(x), _ptr(idx), _ptr(counts), _ptr(offsets), _ptr(row_of),
        _ptr(src_of), _ptr(x_perm), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_permute_noalloc(cfg, x, idx, counts, offsets, row_of, src_of, x_perm, stream=None):
    _check("moe_permute_noalloc", lib.moe_permute_noalloc(
        byref(cfg), _ptr(x), _ptr(idx), _ptr(counts), _ptr(offsets), _ptr(row_of),
        _ptr(src_of), _ptr(x_perm), _stream(stream)))


def moe_grouped_ffn(cfg, x_perm, offsets, W1, W2, A, H, Y, ws, stream=None):
    _check("moe_grouped_ffn", lib.moe_grouped_ffn(
        byref(cfg), _ptr(x_perm), _ptr(offsets), _ptr(W1), _ptr(W2), _ptr(A), _ptr(H),
        _ptr(Y), _ptr(ws), _nbytes(ws), _stream(stream)))


def moe_combine(cfg, Y, row_of, gate, out, x=None, stream=None):
    """x: only read under the identity fallback (MOE_FLAG_DROP_IDENTITY)."""
    _check("moe_combine", lib.moe_combine(
        byref(cfg), _ptr(Y), _ptr(row_of), _ptr(gate), _ptr(x), _ptr(out), _stream(stream)))


def moe_combine_bwd(cfg, dOut, Y, row_of, gate, dYp, dgate, x=None, stream=None):
    """x: only read under the identity fallback (MOE_FLAG_DROP_IDENTITY)."""
    _check("moe_combine_bwd", lib.moe_combine_bwd(
        byref(cfg), _ptr(dOut), _ptr(Y), _ptr(row_of), _ptr(gate), _ptr(x), _ptr(dYp),
        _ptr(dgate), _stream(stream)))


def moe_grouped_ffn_bwd(cfg, x_perm, offsets, W1, W2, A, H, dYp, dXp, dW1, dW2, ws,
                        stream=None):
    _check("moe_grouped_ffn_bwd", lib.moe_grouped_ffn_bwd(
        byref(cfg), _ptr(x_perm), _ptr(offsets), _ptr(W1), _ptr(W2), _ptr(A), _ptr(H),
        _ptr(dYp), _ptr(dXp), _ptr(dW1), _ptr(dW2), _ptr(ws), _nbytes(ws),
        _stream(stream)))


def moe_unpermute_bwd(cfg, dXp, row_of, dXe, gate=None, dOut=None, stream=None):
    """gate, dOut: only read under the identity fallback."""
    _check("moe_unpermute_bwd", lib.moe_unpermute_bwd(
        byref(cfg), _ptr(dXp), _ptr(row_of), _ptr(gate), _ptr(dOut), _ptr(dXe),
        _stream(stream)))


def moe_router_aux(cfg, probs, counts, offsets, aux, ws, stream=None):
    _check("moe_router_aux", lib.moe_router_aux(
        byref(cfg), _ptr(probs), _ptr(counts), _ptr(offsets), _ptr(aux), _ptr(ws),
        _nbytes(ws), _stream(stream)))


def moe_route_bwd(cfg, x, Wr, probs, idx, row_of, counts, dgate, dXe, dX, dWr, db, ws,
                  stream=None):
    """dXe: the fp32 unpermute-sum written by moe_unpermute_bwd; counts may be
    None when cfg.aux_coeff is 0."""
    _check("moe_route_bwd", lib.moe_route_bwd(
        byref(cfg), _ptr(x), _ptr(Wr), _ptr(probs), _ptr(idx), _ptr(row_of), _ptr(counts),
        _ptr(dgate), _ptr(dXe), _ptr(dX), _ptr(dWr), _ptr(db), _ptr(ws), _nbytes(ws),
        _stream(stream)))


def moe_layer_fwd(cfg, weights: MoeWeights, x, out, ctx: MoeCtx, ws, stream=None):
    _check("moe_layer_fwd", lib.moe_layer_fwd(
        byref(cfg), byref(weights), _ptr(x), _ptr(out), byref(ctx), _ptr(ws), _nbytes(ws),
        _stream(stream)))


def moe_layer_bwd(cfg, weights: MoeWeights, x, dOut, ctx: MoeCtx, dX, grads: MoeGrads, ws,
                  stream=None):
    _check("moe_layer_bwd", lib.moe_layer_bwd(
        byref(cfg), byref(weights), _ptr(x), _ptr(dOut), byref(ctx), _ptr(dX),
        byref(grads), _ptr(ws), _nbytes(ws), _stream(stream)))


class KernelProbe:
    """Kernel timing through moe_cfg.probe: HIP events created here with the
    process's HIP runtime (torch's), recorded by the library around the
    launches of one kernel made with a cfg that carries the probe, and read
    here after the caller has synchronised.  All state is this object's."""

    def __init__(self, kernel, capacity: int):
        self._hip = ctypes.CDLL(_hip_runtimes()[0])
        self._hip.hipEventCreate.argtypes = [POINTER(c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [POINTER(c_float), c_void_p, c_void_p]
        self._hip.hipEventSynchronize.argtypes = [c_void_p]
        self._hip.hipEventDestroy.argtypes = [c_void_p]
        n = max(int(capacity), 0)
        self._begin = (c_void_p * max(n, 1))()
        self._end = (c_void_p * max(n, 1))()
        for arr in (self._begin, self._end):
            for i in range(n):
                ev = c_void_p()
                if self._hip.hipEventCreate(byref(ev)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = ev
        self._n = n
        kid = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
        self.struct = MoeProbe(kernel_id=kid, capacity=n, count=0, reserved_=0,
                               begin=ctypes.cast(self._begin, POINTER(c_void_p)),
                               end=ctypes.cast(self._end, POINTER(c_void_p)))

    def attach(self, cfg: MoeCfg) -> MoeCfg:
        cfg.probe = ctypes.addressof(self.struct)
        return cfg

    @staticmethod
    def detach(cfg: MoeCfg) -> MoeCfg:
        cfg.probe = None
        return cfg

    def reset(self):
        self.struct.count = 0

    def read(self):
        """(summed ms, launches, per-launch ms) of the recorded launches."""
        times = []
        for i in range(self.struct.count):
            if self._hip.hipEventSynchronize(self._end[i]) != 0:
                raise RuntimeError("hipEventSynchronize failed")
            ms = c_float(0.0)
            if self._hip.hipEventElapsedTime(byref(ms), self._begin[i], self._end[i]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            times.append(float(ms.value))
        return sum(times), len(times), times

    def close(self):
        for arr in (self._begin, self._end):
            for i in range(self._n):
                if arr[i]:
                    self._hip.hipEventDestroy(arr[i])
                    arr[i] = None
        self._n = 0
