"""Mixed-precision Tile-CSC Conjugate Gradient for AMD MI355X (gfx950).

Python binding of libmpcg.so. Every function here only marshals arguments:
the layout builder is host C++, and every step of SpMV and CG runs in the
library's HIP kernels. torch is used for device memory and streams only.

Functions carry the C ABI's names (include/mpcg.h). The two classes
:class:`TileCSC` and :class:`Solver` own the library objects.
"""

from __future__ import annotations

import ctypes as ct

import numpy as np

from . import _lib
from ._lib import (CG_BF16, CG_BREAKDOWN, CG_EDEVICE, CG_EINVAL, CG_ENOMEM, CG_FP32, CG_FP64,  # noqa: F401
                   CG_NOT_CONVERGED, CG_OK, CG_P1_COLUMN_SCALE, CG_P1_PAD_COLUMNS, CG_P1_ROUND_VECTOR,
                   CGError, check)

__all__ = [
    "TileCSC", "Solver", "cg_tilecsc_from_csr", "cg_create", "cg_spmv", "cg_solve", "cg_tune_row_height",
    "cg_version", "library_path", "CGError", "cg_stream_read", "cg_stream_copy", "cg_stream_mix",
]

STATUS = {CG_OK: "converged", CG_NOT_CONVERGED: "maxit", CG_BREAKDOWN: "breakdown"}


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ct.c_void_p)


def _dev_ptr(t) -> int:
    import torch

    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError("expected a torch tensor on a GPU")
    if t.dtype != torch.float64 or not t.is_contiguous():
        raise TypeError("expected a contiguous float64 tensor")
    return t.data_ptr()


def _vec_ptr(t, n: int, device: int, name: str) -> int:
    """Device pointer of a float64 vector the library reads or writes n entries of: it must be
    on the handle's GPU and hold at least n entries (the library cannot check either)."""
    p = _dev_ptr(t)
    if t.numel() < n:
        raise ValueError(f"{name} has {t.numel()} entries; the handle needs {n}")
    if t.device.index != device:
        raise ValueError(f"{name} is on cuda:{t.device.index}; the handle lives on cuda:{device}")
    return p


def _stream(stream) -> int:
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def library_path() -> str:
    return _lib.LIB_PATH


def cg_version() -> int:
    return _lib.load().cg_version()


class TileCSC:
    """Host canonical Tile-CSC matrix (owns a ``cg_tilecsc``)."""

    def __init__(self, handle: int):
        self._h = ct.c_void_p(handle)
        v = _lib.cg_tilecsc_view()
        check(_lib.load().cg_tilecsc_get_view(self._h, ct.byref(v)))
        self.n, self.T, self.nnz, self.R, self.C = int(v.n), int(v.T), int(v.nnz), int(v.R), int(v.C)
        self._view = v

    def _arr(self, ptr, count, dtype):
        if count == 0:
            return np.zeros(0, dtype=dtype)
        return np.ctypeslib.as_array(ptr, shape=(count,)).view(dtype).copy()

    @property
    def tile_row_ptr(self):
        return self._arr(self._view.tile_row_ptr, -(-self.n // self.R) + 1, np.int64)

    @property
    def tile_col_idx(self):
        return self._arr(self._view.tile_col_idx, self.T, np.int32)

    @property
    def tile_nnz_ptr(self):
        return self._arr(self._view.tile_nnz_ptr, self.T + 1, np.int64)

    @property
    def row_idx(self):
        return self._arr(self._view.row_idx, self.nnz, np.uint16)

    @property
    def col_local(self):
        return self._arr(self._view.col_local, self.nnz, np.uint8)

    @property
    def val(self):
        return self._arr(self._view.val, self.nnz, np.float64)

    def col_ptr(self) -> np.ndarray:
        out = np.empty(self.T * (self.C + 1), dtype=np.int32)
        check(_lib.load().cg_tilecsc_col_ptr(self._h, _ptr(out)))
        return out.reshape(self.T, self.C + 1)

    def perm(self) -> np.ndarray:
        out = np.empty(self.nnz, dtype=np.int64)
        check(_lib.load().cg_tilecsc_perm(self._h, _ptr(out)))
        return out

    def close(self):
        if self._h:
            _lib.load().cg_tilecsc_free(self._h)
            self._h = ct.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def cg_tilecsc_from_csr(n, indptr, indices, data, R, C) -> TileCSC:
    indptr = np.ascontiguousarray(indptr, dtype=np.int64)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    data = np.ascontiguousarray(data, dtype=np.float64)
    out = ct.c_void_p()
    check(_lib.load().cg_tilecsc_from_csr(int(n), _ptr(indptr), _ptr(indices), _ptr(data), int(R),
                                          int(C), ct.byref(out)))
    return TileCSC(out.value)


class Solver:
    """Device-resident solver handle (owns a ``cg_handle``)."""

    def __init__(self, A: TileCSC, precision_map=None, jacobi=False, window=0, use_graph=-1,
                 p1=0, col_slices=0, single_block=0, stage_x=0, stream=None):
        lib = _lib.load()
        opt = _lib.cg_options()
        opt.jacobi = 1 if jacobi else 0
        opt.window = int(window)
        opt.use_graph = int(use_graph)
        opt.p1 = int(p1)
        opt.col_slices = int(col_slices)
        opt.single_block = int(single_block)
        opt.stage_x = int(stage_x)
        pm = None
        if precision_map is not None:
            pm = np.ascontiguousarray(precision_map, dtype=np.uint8)
            if pm.size != A.T:
                raise ValueError("precision_map must have one entry per non-empty tile")
        out = ct.c_void_p()
        check(lib.cg_create(A._h, _ptr(pm) if pm is not None else None, ct.byref(opt),
                            ct.c_void_p(_stream(stream)), ct.byref(out)))
        self._h = out
        n, T, nnz = ct.c_int64(), ct.c_int64(), ct.c_int64()
        check(lib.cg_get_sizes(self._h, ct.byref(n), ct.byref(T), ct.byref(nnz), None, None))
        # nnz counts the padding sentinels when CG_P1_PAD_COLUMNS is set
        self.n, self.T, self.nnz, self.R, self.C = n.value, T.value, nnz.value, A.R, A.C
        import torch

        self.device = torch.cuda.current_device()
        self.jacobi = bool(jacobi)
        self.p1 = int(p1)

    # -- maps and schedules ------------------------------------------------
    def cg_set_precision_map(self, prec_map):
        pm = np.ascontiguousarray(prec_map, dtype=np.uint8)
        if pm.size != self.T:
            raise ValueError("map must have one entry per non-empty tile")
        check(_lib.load().cg_set_precision_map(self._h, _ptr(pm), 0))

    def cg_get_active_map(self) -> np.ndarray:
        out = np.empty(self.T, dtype=np.uint8)
        check(_lib.load().cg_get_active_map(self._h, _ptr(out)))
        return out

    def cg_map_from_magnitude(self, t_bf16: float, t_fp32: float):
        check(_lib.load().cg_map_from_magnitude(self._h, float(t_bf16), float(t_fp32)))

    def cg_set_schedule_residual(self, thresholds, prec):
        th = np.ascontiguousarray(thresholds, dtype=np.float64)
        pr = np.ascontiguousarray(prec, dtype=np.uint8)
        if pr.size < 1 or th.size != pr.size - 1:
            raise ValueError("need one precision per stage and one threshold fewer than precisions")
        check(_lib.load().cg_set_schedule_residual(self._h, int(pr.size), _ptr(th), _ptr(pr)))

    def cg_set_schedule_tile_rule(self, period, scores, hi, lo):
        sc = np.ascontiguousarray(scores, dtype=np.float64)
        if sc.size != self.T:
            raise ValueError("scores must have one entry per non-empty tile")
        check(_lib.load().cg_set_schedule_tile_rule(self._h, int(period), _ptr(sc), float(hi),
                                                    float(lo)))

    def cg_set_schedule_pmag(self, lo, hi, period=1):
        """Per-segment max|p| rule, evaluated every `period` iterations (see include/mpcg.h)."""
        check(_lib.load().cg_set_schedule_pmag(self._h, float(lo), float(hi), int(period)))

    def cg_record_column_codes(self, enable=True):
        check(_lib.load().cg_record_column_codes(self._h, 1 if enable else 0))

    def cg_get_column_codes(self, cap=100000):
        """Recorded column-block codes of the last solve, uint8[evaluations][ceil(n/C)]."""
        ncb = -(-self.n // self.C)
        n = check(_lib.load().cg_get_column_codes(self._h, 0, None))
        out = np.empty((min(n, cap), ncb), dtype=np.uint8)
        check(_lib.load().cg_get_column_codes(self._h, int(out.shape[0]), _ptr(out)))
        return out

    def cg_record_window_maps(self, cap):
        check(_lib.load().cg_record_window_maps(self._h, int(cap)))

    def cg_get_window_maps(self, cap=100000):
        """Tile-rule maps of the last solve's windows, uint8[windows][T] (canonical tile order)."""
        n = check(_lib.load().cg_get_window_maps(self._h, 0, None))
        out = np.empty((min(n, cap), self.T), dtype=np.uint8)
        check(_lib.load().cg_get_window_maps(self._h, int(out.shape[0]), _ptr(out)))
        return out

    def cg_eval_tile_rule(self, rho):
        check(_lib.load().cg_eval_tile_rule(self._h, float(rho)))

    def cg_clear_schedule(self):
        check(_lib.load().cg_clear_schedule(self._h))

    # -- compute -------------------------------------------------------------
    def _vec(self, t, name):
        return _vec_ptr(t, self.n, self.device, name)

    def cg_spmv(self, x, y, stream=None):
        check(_lib.load().cg_spmv(self._h, ct.c_void_p(self._vec(x, "x")), ct.c_void_p(self._vec(y, "y")),
                                  ct.c_void_p(_stream(stream))))

    def cg_solve(self, b, x, tol, maxit, x0=None, stream=None):
        """Returns (status string, iterations, residual history as a numpy array)."""
        hist = np.empty(int(maxit) + 1, dtype=np.float64)
        it = ct.c_int32()
        rc = check(_lib.load().cg_solve(self._h, ct.c_void_p(self._vec(b, "b")),
                                        ct.c_void_p(self._vec(x0, "x0")) if x0 is not None else None,
                                        float(tol), int(maxit), ct.c_void_p(self._vec(x, "x")),
                                        ct.byref(it), _ptr(hist), ct.c_void_p(_stream(stream))))
        return STATUS[rc], int(it.value), hist[: it.value + 1].copy()

    def cg_true_residual(self, b, x, stream=None) -> float:
        """||b - A x|| / ||b|| with the exact FP64 values (device vectors in, host float out)."""
        out = ct.c_double()
        check(_lib.load().cg_true_residual(self._h, ct.c_void_p(self._vec(b, "b")), ct.c_void_p(self._vec(x, "x")),
                                           ct.byref(out), ct.c_void_p(_stream(stream))))
        return float(out.value)

    def cg_true_residual_noalloc(self, b, x, out, stream=None):
        """The same value as cg_true_residual, written into the device float64 tensor `out`
        (first entry) on the stream, with no allocation and no synchronisation."""
        check(_lib.load().cg_true_residual_noalloc(self._h, ct.c_void_p(self._vec(b, "b")),
                                                   ct.c_void_p(self._vec(x, "x")),
                                                   ct.c_void_p(_vec_ptr(out, 1, self.device, "out")),
                                                   ct.c_void_p(_stream(stream))))

    def cg_get_map_trace(self, cap=100000):
        ks = np.empty(cap, dtype=np.int32)
        cnt = np.empty(3 * cap, dtype=np.int64)
        n = check(_lib.load().cg_get_map_trace(self._h, int(cap), _ptr(ks), _ptr(cnt)))
        m = min(n, cap)
        return ks[:m].copy(), cnt[: 3 * m].reshape(m, 3).copy()

    def cg_export_layout(self):
        nrb = -(-self.n // self.R)
        out = dict(tile_row_ptr=np.empty(nrb + 1, np.int64), tile_col_idx=np.empty(self.T, np.int32),
                   tile_nnz_ptr=np.empty(self.T + 1, np.int64), row_idx=np.empty(self.nnz, np.uint16),
                   col_local=np.empty(self.nnz, np.uint8), val64=np.empty(self.nnz, np.float64),
                   val32=np.empty(self.nnz, np.float32), bf16=np.empty(self.nnz, np.uint16))
        check(_lib.load().cg_export_layout(self._h, *[_ptr(out[k]) for k in (
            "tile_row_ptr", "tile_col_idx", "tile_nnz_ptr", "row_idx", "col_local", "val64", "val32",
            "bf16")]))
        return out

    def cg_export_column_scale(self) -> np.ndarray:
        out = np.empty(self.n, dtype=np.int32)
        check(_lib.load().cg_export_column_scale(self._h, _ptr(out)))
        return out

    def device_bytes(self) -> int:
        return int(_lib.load().cg_device_bytes(self._h))

    def cg_get_options(self) -> dict:
        """The options the handle runs with, after its automatic choices (cg_get_options)."""
        o = _lib.cg_options()
        check(_lib.load().cg_get_options(self._h, ct.byref(o)))
        return {k: int(getattr(o, k)) for k in ("jacobi", "window", "use_graph", "p1", "col_slices",
                                                 "single_block", "stage_x")}

    def close(self):
        if self._h:
            _lib.load().cg_destroy(self._h)
            self._h = ct.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def cg_create(A: TileCSC, precision_map=None, **kw) -> Solver:
    return Solver(A, precision_map, **kw)


def cg_spmv(h: Solver, x, y, stream=None):
    h.cg_spmv(x, y, stream)


def cg_tune_row_height(n, indptr, indices, C, max_R=16384, min_row_blocks=1024):
    """Tuned row-block height and the per-candidate table (see ``cg_tune_row_height`` in mpcg.h).

    Returns ``(R, rows)`` with one dict per candidate height: R, row_blocks,
    tiles, cv, max_ratio, admissible.
    """
    indptr = np.ascontiguousarray(indptr, dtype=np.int64)
    indices = np.ascontiguousarray(indices, dtype=np.int32)
    cap = 10
    cR = np.empty(cap, np.int32)
    cnrb, cT = np.empty(cap, np.int64), np.empty(cap, np.int64)
    ccv, cmx = np.empty(cap, np.float64), np.empty(cap, np.float64)
    cok = np.empty(cap, np.uint8)
    R = ct.c_int32()
    m = check(_lib.load().cg_tune_row_height(int(n), _ptr(indptr), _ptr(indices), int(C), int(max_R),
                                             int(min_row_blocks), ct.byref(R), cap, _ptr(cR), _ptr(cnrb),
                                             _ptr(cT), _ptr(ccv), _ptr(cmx), _ptr(cok)))
    rows = [dict(R=int(cR[i]), row_blocks=int(cnrb[i]), tiles=int(cT[i]), cv=float(ccv[i]),
                 max_ratio=float(cmx[i]), admissible=bool(cok[i])) for i in range(min(m, cap))]
    return R.value, rows


def cg_select_reuse_interval(codes, max_fraction=0.1):
    """K* from a per-iteration record of column-block codes; returns (K*, [(K, fraction), ...])."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    if c.ndim != 2:
        raise ValueError("codes must be [records][column blocks]")
    kstar = ct.c_int32()
    cap = 40
    iv = np.empty(cap, dtype=np.int32)
    fr = np.empty(cap, dtype=np.float64)
    n = check(_lib.load().cg_select_reuse_interval(_ptr(c), int(c.shape[0]), int(c.shape[1]),
                                                   float(max_fraction), ct.byref(kstar), cap,
                                                   _ptr(iv), _ptr(fr)))
    return int(kstar.value), [(int(iv[i]), float(fr[i])) for i in range(min(n, cap))]


def cg_solve(h: Solver, b, x0, tol, maxit, x, stream=None):
    return h.cg_solve(b, x, tol, maxit, x0=x0, stream=stream)


def _bytes_ptr(t):
    import torch

    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
        raise TypeError("expected a contiguous torch tensor on a GPU")
    return t.data_ptr(), t.numel() * t.element_size()


def _check_sink(sink, blocks):
    import torch

    if not isinstance(sink, torch.Tensor) or sink.dtype != torch.float64 or sink.numel() < int(blocks):
        raise ValueError("sink must be a float64 tensor of at least `blocks` entries")


def cg_stream_read(src, sink, blocks, stream=None):
    """Bandwidth reference: read all of src once (sink: float64 tensor of at least `blocks` entries)."""
    p, nbytes = _bytes_ptr(src)
    _check_sink(sink, blocks)
    check(_lib.load().cg_stream_read(ct.c_void_p(p), nbytes, ct.c_void_p(_dev_ptr(sink)), int(blocks),
                                     ct.c_void_p(_stream(stream))))


def cg_stream_mix(src, dst, sink, blocks, stream=None):
    """Bandwidth reference: read all of src once and, interleaved in proportion, write all of dst
    (sink: float64 tensor of at least `blocks` entries; it receives the block sums of src)."""
    p, rbytes = _bytes_ptr(src)
    q, wbytes = _bytes_ptr(dst)
    _check_sink(sink, blocks)
    check(_lib.load().cg_stream_mix(ct.c_void_p(p), rbytes, ct.c_void_p(q), wbytes, ct.c_void_p(_dev_ptr(sink)),
                                    int(blocks), ct.c_void_p(_stream(stream))))


def cg_stream_copy(src, dst, blocks, stream=None):
    """Bandwidth reference: copy src into dst (same byte size)."""
    p, nbytes = _bytes_ptr(src)
    q, nb2 = _bytes_ptr(dst)
    if nb2 != nbytes:
        raise ValueError("src and dst must have the same size")
    check(_lib.load().cg_stream_copy(ct.c_void_p(p), ct.c_void_p(q), nbytes, int(blocks),
                                     ct.c_void_p(_stream(stream))))
