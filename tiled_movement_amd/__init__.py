"""Python binding of libswz.so: swizzled LDS tile movement on gfx950.

Argument marshalling only.  Every step of the path runs in the HIP kernels of
libswz.so; there is no Python or CPU fallback, and importing this package
raises if the library has not been built (``python tiled_movement_amd/build.py``).

Functions take torch tensors (or raw device addresses as ints) and the
library's enum values; they run on the current torch stream unless a stream
is given, and raise ``SwzError`` on a negative status.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswz.so")

# enum values of include/swz.h
SWZ_OK, SWZ_EINVAL, SWZ_EUNSUPPORTED, SWZ_EHIP = 0, -1, -2, -3
LAYOUT_SWIZZLE, LAYOUT_PAD, LAYOUT_PLAIN, LAYOUT_SWIZZLE_DIRECT = 0, 1, 2, 3
READ_AUTO, READ_SCALAR_COL, READ_B64_4X4, READ_B128_8X8, READ_MFMA_16X16X32, READ_B64_TR16, READ_B64_TR8 = (
    -1, 0, 1, 2, 3, 4, 5)
READ_NARROW1, READ_NARROW2, READ_NARROW4, READ_NARROW8, READ_NARROW16 = 6, 7, 8, 9, 10
READ_HNARROW1, READ_HNARROW2, READ_HNARROW4, READ_HNARROW8, READ_HNARROW16, READ_HNARROW32 = 11, 12, 13, 14, 15, 16
READ_BNARROW1, READ_BNARROW2, READ_BNARROW4, READ_BNARROW8, READ_BNARROW16, READ_BNARROW32, READ_BNARROW64 = (
    17, 18, 19, 20, 21, 22, 23)
READ_ROWS = 24
FRAG_MFMA_F32_16X16X32_BF16 = 0
ORDER_DIAGONAL, ORDER_HALF_DIAGONAL, ORDER_COLUMNS, ORDER_STEEP_DIAGONAL = 0, 1, 2, 3
ORDER_SLOPE_8, ORDER_SLOPE_16, ORDER_SLOPE_32 = 4, 5, 6
ORDERS = tuple(range(7))
C_F32, C_BF16 = 0, 1
LAYOUTS = {"swizzle": LAYOUT_SWIZZLE, "pad": LAYOUT_PAD, "plain": LAYOUT_PLAIN, "direct": LAYOUT_SWIZZLE_DIRECT}

EXPORTS = (
    "swz_map",
    "swz_map_batch",
    "swz_transpose",
    "swz_convert_layout",
    "swz_set_tile_order",
    "swz_get_tile_order",
    "swz_tune_tile_order",
    "swz_stage_operand",
    "swz_stage_operands",
    "swz_gemm_frag",
    "swz_gemm",
    "swz_gemm_ex",
    "swz_fold",
    "swz_choose",
    "swz_predict_conflicts",
    "swz_kernel_accesses",
    "swz_bank_model_get",
    "swz_plan",
    "swz_strerror",
    "swz_lds_probe",
    "swz_copy",
)


class SwzError(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__(f"{call}: {strerror(status)} ({status})")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("M", ctypes.c_int32), ("S", ctypes.c_int32)]

    def tuple(self) -> Tuple[int, int, int]:
        return (self.B, self.M, self.S)


class BankModelInfo(ctypes.Structure):
    _fields_ = [
        ("n_banks", (ctypes.c_int32 * 3) * 2),
        ("bank_bytes", (ctypes.c_int32 * 3) * 2),
        ("phase", ((ctypes.c_uint8 * 64) * 3) * 2),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("read_kind", ctypes.c_int32),
        ("tile_rows", ctypes.c_int32),
        ("tile_cols", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("params", Params),
        ("pad_elems", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32),
        ("vec_bytes", ctypes.c_int32),
        ("aligned", ctypes.c_int32),
        ("threads", ctypes.c_int32),
        ("interior_tiles", ctypes.c_int32),
    ]

    def as_dict(self):
        return {
            "read_kind": self.read_kind,
            "tile": (self.tile_rows, self.tile_cols),
            "layout": self.layout,
            "params": self.params.tuple(),
            "pad_elems": self.pad_elems,
            "lds_bytes": self.lds_bytes,
            "vec_bytes": self.vec_bytes,
            "aligned": bool(self.aligned),
            "threads": self.threads,
            "interior_tiles": self.interior_tiles,
        }


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python tiled_movement_amd/build.py` "
            "(there is no fallback path)"
        )
    try:  # bind to the HIP runtime torch already loaded, if torch is present
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    P = ctypes.POINTER
    lib.swz_map.argtypes = [vp, vp, i64, Params, vp]
    lib.swz_map_batch.argtypes = [vp, vp, i64, vp, i32, vp]
    lib.swz_transpose.argtypes = [vp, vp, i64, i64, i32, i32, i32, P(Params), vp]
    lib.swz_convert_layout.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, P(Params), vp]
    lib.swz_set_tile_order.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.swz_get_tile_order.argtypes = [i64, i64, i64, i32, i32, P(ctypes.c_int32)]
    lib.swz_tune_tile_order.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, P(Params), i32, P(ctypes.c_int32), vp]
    lib.swz_stage_operand.argtypes = [vp, vp, i64, i64, i32, i32, i32, P(Params), vp]
    lib.swz_stage_operands.argtypes = [vp, vp, i64, vp, vp, i64, i64, i32, i32, i32, P(Params), vp]
    lib.swz_gemm_frag.argtypes = [vp, vp, vp, i64, i64, i64, i32, vp]
    lib.swz_gemm.argtypes = [vp, vp, vp, i64, i64, i64, i32, P(Params), vp]
    lib.swz_gemm_ex.argtypes = [vp, vp, vp, i64, i64, i64, i32, P(Params), i32, vp]
    lib.swz_fold.argtypes = [P(Params), ctypes.c_uint32, ctypes.c_uint32, P(ctypes.c_uint32), P(ctypes.c_uint32),
                             P(i64)]
    lib.swz_choose.argtypes = [i32, i32, i32, i32, i32, P(Params)]
    lib.swz_predict_conflicts.argtypes = [i32, i32, P(Params), P(i64), P(i64)]
    lib.swz_kernel_accesses.argtypes = [i32, i32, P(Params), i32, P(i32), i32, P(i32), P(i32)]
    lib.swz_bank_model_get.argtypes = [P(BankModelInfo)]
    lib.swz_plan.argtypes = [i32, i64, i64, i32, i32, i32, P(Params), P(PlanInfo)]
    lib.swz_strerror.argtypes = [ctypes.c_int]
    lib.swz_strerror.restype = ctypes.c_char_p
    lib.swz_copy.argtypes = [vp, vp, i64, vp]
    lib.swz_lds_probe.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp]
    for name in EXPORTS:
        if name != "swz_strerror":
            getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.swz_strerror(status).decode()


def _check(status: int, call: str) -> None:
    if status != SWZ_OK:
        raise SwzError(status, call)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _buf(call: str, **bufs) -> None:
    """Check the device buffers of one call before it reaches the library:
    every tensor is a contiguous CUDA tensor, all on the current device, and
    holds at least the bytes the call reads or writes there (name=(tensor, bytes)).
    Raw integer addresses and None pass unchecked (the library checks what
    it can: NULL, alignment, overlap).  Raises ValueError."""
    device = None
    for name, (t, need) in bufs.items():
        if t is None or isinstance(t, int):
            continue
        if not getattr(t, "is_cuda", False):
            raise ValueError(f"{call}: {name} must be a CUDA tensor (got {type(t).__name__} on "
                             f"{getattr(t, 'device', 'the host')})")
        if not t.is_contiguous():
            raise ValueError(f"{call}: {name} must be contiguous (a strided view is not its own bytes)")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{call}: {name} is on {t.device}, the other buffers on {device}")
        have = t.numel() * t.element_size()
        if have < max(int(need), 0):
            raise ValueError(f"{call}: {name} holds {have} bytes, the call needs {int(need)}")
    if device is not None and device.index is not None:
        import torch

        # the library launches on, and creates its events on, the current device
        cur = torch.cuda.current_device()
        if device.index != cur:
            raise ValueError(f"{call}: the buffers are on {device}, the current device is cuda:{cur} "
                             f"(call inside torch.cuda.device({device.index}))")


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if hasattr(t, "is_cuda") and t.is_cuda:
            import torch

            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _params(p) -> Optional[ctypes.pointer]:
    if p is None:
        return None
    if isinstance(p, Params):
        return ctypes.pointer(p)
    B, M, S = p
    return ctypes.pointer(Params(B, M, S))


def _layout(layout) -> int:
    return LAYOUTS[layout] if isinstance(layout, str) else int(layout)


def swz_map(inp, out, n: int, params, stream=None) -> None:
    B, M, S = params
    _buf("swz_map", inp=(inp, 4 * n), out=(out, 4 * n))
    _check(lib.swz_map(_ptr(inp), _ptr(out), n, Params(B, M, S), _stream(stream, inp, out)), "swz_map")


def swz_set_tile_order(batch: int, rows: int, cols: int, elem_bytes: int, read_kind: int = READ_AUTO,
                       order: int = ORDER_DIAGONAL) -> None:
    _check(lib.swz_set_tile_order(batch, rows, cols, elem_bytes, read_kind, order), "swz_set_tile_order")


def swz_get_tile_order(batch: int, rows: int, cols: int, elem_bytes: int, read_kind: int = READ_AUTO) -> int:
    order = ctypes.c_int32(-1)
    _check(lib.swz_get_tile_order(batch, rows, cols, elem_bytes, read_kind, ctypes.byref(order)),
           "swz_get_tile_order")
    return order.value


def swz_tune_tile_order(src, dst, batch: int, rows: int, cols: int, elem_bytes: int, layout="swizzle",
                        read_kind: int = READ_AUTO, params=None, reps: int = 10, stream=None) -> int:
    """Time every tile order on this conversion, pin the fastest and return it."""
    chosen = ctypes.c_int32(-1)
    nbytes = batch * rows * cols * elem_bytes
    _buf("swz_tune_tile_order", src=(src, nbytes), dst=(dst, nbytes))
    _check(lib.swz_tune_tile_order(_ptr(src), _ptr(dst), batch, rows, cols, elem_bytes, _layout(layout), read_kind,
                                   _params(params), reps, ctypes.byref(chosen), _stream(stream, src, dst)),
           "swz_tune_tile_order")
    return chosen.value


def swz_map_batch(inp, out, n: int, params_list, stream=None) -> None:
    """out[j][i] = Swizzle(params_list[j])(inp[i]); out holds len(params_list) rows of n."""
    arr = (Params * max(len(params_list), 1))(*[Params(*p) for p in params_list])
    _buf("swz_map_batch", inp=(inp, 4 * n), out=(out, 4 * n * len(params_list)))
    _check(lib.swz_map_batch(_ptr(inp), _ptr(out), n, ctypes.addressof(arr), len(params_list),
                             _stream(stream, inp, out)), "swz_map_batch")


def swz_transpose(src, dst, rows: int, cols: int, elem_bytes: int, layout="swizzle", read_kind: int = READ_AUTO,
                  params=None, stream=None) -> None:
    _buf("swz_transpose", src=(src, rows * cols * elem_bytes), dst=(dst, rows * cols * elem_bytes))
    _check(lib.swz_transpose(_ptr(src), _ptr(dst), rows, cols, elem_bytes, _layout(layout), read_kind,
                             _params(params), _stream(stream, src, dst)), "swz_transpose")


def swz_convert_layout(src, dst, batch: int, rows: int, cols: int, elem_bytes: int, layout="swizzle",
                       read_kind: int = READ_AUTO, params=None, stream=None) -> None:
    nbytes = batch * rows * cols * elem_bytes
    _buf("swz_convert_layout", src=(src, nbytes), dst=(dst, nbytes))
    _check(lib.swz_convert_layout(_ptr(src), _ptr(dst), batch, rows, cols, elem_bytes, _layout(layout), read_kind,
                                  _params(params), _stream(stream, src, dst)), "swz_convert_layout")


def swz_stage_operand(src, frag, mn: int, k: int, elem_bytes: int = 2, frag_kind: int = FRAG_MFMA_F32_16X16X32_BF16,
                      layout="swizzle", params=None, stream=None) -> None:
    _buf("swz_stage_operand", src=(src, mn * k * elem_bytes), frag=(frag, mn * k * elem_bytes))
    _check(lib.swz_stage_operand(_ptr(src), _ptr(frag), mn, k, elem_bytes, frag_kind, _layout(layout),
                                 _params(params), _stream(stream, src, frag)), "swz_stage_operand")


def swz_stage_operands(a, fa, m: int, bt, fb, n: int, k: int, elem_bytes: int = 2,
                       frag_kind: int = FRAG_MFMA_F32_16X16X32_BF16, layout="swizzle", params=None,
                       stream=None) -> None:
    """Stage A [m][k] into fa and B^T [n][k] into fb in one launch."""
    _buf("swz_stage_operands", a=(a, m * k * elem_bytes), fa=(fa, m * k * elem_bytes), bt=(bt, n * k * elem_bytes),
         fb=(fb, n * k * elem_bytes))
    _check(lib.swz_stage_operands(_ptr(a), _ptr(fa), m, _ptr(bt), _ptr(fb), n, k, elem_bytes, frag_kind,
                                  _layout(layout), _params(params), _stream(stream, a, fa, bt, fb)),
           "swz_stage_operands")


def swz_gemm_frag(fa, fb, c, m: int, n: int, k: int, frag_kind: int = FRAG_MFMA_F32_16X16X32_BF16,
                  stream=None) -> None:
    _buf("swz_gemm_frag", fa=(fa, 2 * m * k), fb=(fb, 2 * n * k), c=(c, 4 * m * n))
    _check(lib.swz_gemm_frag(_ptr(fa), _ptr(fb), _ptr(c), m, n, k, frag_kind, _stream(stream, fa, fb, c)),
           "swz_gemm_frag")


def swz_gemm(a, bt, c, m: int, n: int, k: int, layout: str = "swizzle", params=None, stream=None) -> None:
    _buf("swz_gemm", a=(a, 2 * m * k), bt=(bt, 2 * n * k), c=(c, 4 * m * n))
    _check(lib.swz_gemm(_ptr(a), _ptr(bt), _ptr(c), m, n, k, _layout(layout), _params(params),
                        _stream(stream, a, bt, c)), "swz_gemm")


def swz_gemm_ex(a, bt, c, m: int, n: int, k: int, layout: str = "swizzle", params=None, c_type: int = C_F32,
                stream=None) -> None:
    _buf("swz_gemm_ex", a=(a, 2 * m * k), bt=(bt, 2 * n * k), c=(c, (2 if c_type == C_BF16 else 4) * m * n))
    _check(lib.swz_gemm_ex(_ptr(a), _ptr(bt), _ptr(c), m, n, k, _layout(layout), _params(params), c_type,
                           _stream(stream, a, bt, c)), "swz_gemm_ex")


def swz_fold(params, base: int, active: int):
    """(collision, folded_base or None, strides dict {bit: stride} or None)."""
    c, fb = ctypes.c_uint32(), ctypes.c_uint32()
    st = (ctypes.c_int64 * 32)()
    rc = lib.swz_fold(ctypes.byref(Params(*params)), base, active, ctypes.byref(c), ctypes.byref(fb), st)
    if rc == SWZ_EUNSUPPORTED:
        return c.value, None, None
    _check(rc, "swz_fold")
    return c.value, fb.value, {b: st[b] for b in range(32) if (active >> b) & 1}


def swz_choose(elem_bytes: int, vec_bytes: int, tile_rows: int, tile_cols: int, read_kind: int) -> Tuple[int, int, int]:
    out = Params()
    _check(lib.swz_choose(elem_bytes, vec_bytes, tile_rows, tile_cols, read_kind, ctypes.byref(out)), "swz_choose")
    return out.tuple()


def swz_predict_conflicts(read_kind: int, layout="swizzle", params=None) -> Tuple[int, int]:
    w, r = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.swz_predict_conflicts(read_kind, _layout(layout), _params(params), ctypes.byref(w), ctypes.byref(r)),
           "swz_predict_conflicts")
    return w.value, r.value


def swz_kernel_accesses(read_kind: int, layout="swizzle", params=None, is_write: int = 0):
    """List of (addresses[64], width) for one tile of the kernel; -1 = idle lane."""
    n, w = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.swz_kernel_accesses(read_kind, _layout(layout), _params(params), is_write, None, 0, ctypes.byref(n),
                                   ctypes.byref(w)), "swz_kernel_accesses")
    buf = (ctypes.c_int32 * (64 * max(n.value, 1)))()
    _check(lib.swz_kernel_accesses(read_kind, _layout(layout), _params(params), is_write, buf, n.value,
                                   ctypes.byref(n), ctypes.byref(w)), "swz_kernel_accesses")
    flat = list(buf)
    return [(flat[64 * i:64 * i + 64], w.value) for i in range(n.value)]


def swz_bank_model_get() -> dict:
    """The built-in bank model, keyed by (direction, bytes per lane) with
    direction "read" or "write": banks, bytes per bank and the phase number
    of every lane."""
    m = BankModelInfo()
    _check(lib.swz_bank_model_get(ctypes.byref(m)), "swz_bank_model_get")
    out = {}
    for d, dname in enumerate(("read", "write")):
        for w, width in enumerate((4, 8, 16)):
            out[(dname, width)] = {
                "n_banks": m.n_banks[d][w],
                "bank_bytes": m.bank_bytes[d][w],
                "phase": list(m.phase[d][w]),
            }
    return out


def swz_plan(op: int, rows: int, cols: int, elem_bytes: int, layout="swizzle", read_kind: int = READ_AUTO,
             params=None) -> dict:
    out = PlanInfo()
    _check(lib.swz_plan(op, rows, cols, elem_bytes, _layout(layout), read_kind, _params(params), ctypes.byref(out)),
           "swz_plan")
    return out.as_dict()


def swz_strerror(status: int) -> str:
    return strerror(status)


def swz_lds_probe(addrs, masks, n_patterns: int, width_bytes: int, is_write: int, iters: int, waves: int, cycles,
                  stream=None) -> None:
    _buf("swz_lds_probe", addrs=(addrs, 4 * 64 * n_patterns), masks=(masks, 8 * n_patterns),
         cycles=(cycles, 8 * n_patterns * waves))
    _check(lib.swz_lds_probe(_ptr(addrs), _ptr(masks), n_patterns, width_bytes, is_write, iters, waves,
                             _ptr(cycles), _stream(stream, addrs, masks, cycles)), "swz_lds_probe")


def swz_copy(src, dst, nbytes: int, stream=None) -> None:
    _buf("swz_copy", src=(src, nbytes), dst=(dst, nbytes))
    _check(lib.swz_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream, src, dst)), "swz_copy")


# Status-returning raw entry points, for callers that test error paths.
raw = lib
