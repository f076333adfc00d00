"""ctypes wrapper of the fp64 C oracle (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this module.  Inputs are the raw storage arrays of a Workload (host numpy):
bf16 as uint16 bit patterns, e4m3 as uint8 codes, scales as stored.  Every
result is float64.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_DT = {"f32": 0, "bf16": 1, "e4m3": 2, "mxfp8": 2, "e4m3_128": 2}
_SCALE_NONE, _SCALE_F32, _SCALE_E8M0 = 0, 1, 2
#: storage format -> (scale kind, elements per scale)
_SCALES = {"f32": (_SCALE_NONE, 0), "bf16": (_SCALE_NONE, 0), "e4m3": (_SCALE_F32, 128),
           "e4m3_128": (_SCALE_F32, 128), "mxfp8": (_SCALE_E8M0, 32)}
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        p, i32, i64, d = C.c_void_p, C.c_int, C.c_int64, C.c_double
        L.oracle_bf16_to_f64.restype = d
        L.oracle_bf16_to_f64.argtypes = [C.c_uint16]
        L.oracle_e4m3_to_f64.restype = d
        L.oracle_e4m3_to_f64.argtypes = [C.c_uint8]
        L.oracle_e8m0_to_f64.restype = d
        L.oracle_e8m0_to_f64.argtypes = [C.c_uint8]
        L.oracle_dequant.argtypes = [p, i32, p, i32, i32, i32, i64, p]
        L.oracle_indexer_scores.argtypes = [i32, i32, p, p, i32, i32, i64,
                                            p, i32, p, i32, i32, i32, i32, p,
                                            p, i32, p, i32, i32, p, i32, p, i64]
        L.oracle_topk.argtypes = [i32, p, p, i64, i32, p]
        attn = [i32, i32, p, p, i32, i32, i64, p, i32, i32, i32, i32, p, i32, p, i32, i32]
        L.oracle_sparse_attn.argtypes = attn + [p, i32, d, p, i32, p, p]
        L.oracle_dense_attn.argtypes = attn + [d, p, i32, p, p]
        L.oracle_f32_to_e4m3.restype = C.c_uint8
        L.oracle_f32_to_e4m3.argtypes = [C.c_float]
        L.oracle_cache_append.argtypes = [i32, i32, p, p, i32, i32, i64, p, i32, i32, i32, i32, i32, p, p]
        L.oracle_cache_append.restype = i32
        L.oracle_e4m3_encode.argtypes = [p, i64, p]
        L.oracle_indexer_prolog.argtypes = [i32, i32, p, p, p, p, p, d, i32, i32, p, p, p]
        L.oracle_num_threads.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def bf16_to_f64(h: int) -> float:
    return lib().oracle_bf16_to_f64(h)


def e4m3_to_f64(c: int) -> float:
    return lib().oracle_e4m3_to_f64(c)


def e8m0_to_f64(b: int) -> float:
    return lib().oracle_e8m0_to_f64(b)


def dequant(data, dtype: str, scales=None, scale_kind: str = "none", group: int = 0):
    """Dequantize an array whose last axis is the vector width; returns float64."""
    data = _c(data)
    width = data.shape[-1]
    n = data.size // width
    out = np.empty(data.shape, np.float64)
    kind = {"none": _SCALE_NONE, "f32": _SCALE_F32, "e8m0": _SCALE_E8M0}[scale_kind]
    lib().oracle_dequant(_ptr(data), _DT[dtype], _ptr(_c(scales)), kind, group, width, n, _ptr(out))
    return out


def _rows_arg(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, np.int32))
    return r, int(r.size)


def indexer_scores(wl, rows=None, ld=None):
    """I[r, s] (float64) for the listed rows (all when None); NaN for s >= L_r."""
    r, n = _rows_arg(rows)
    n_rows = wl.rows if r is None else n
    ld = wl.max_seq_len if ld is None else ld
    out = np.empty((n_rows, max(ld, 1)), np.float64)
    seq, tab = _c(wl.seq_lens, np.int32), _c(wl.block_table, np.int32)
    qi, kp, hw = _c(wl.q_idx), _c(wl.k_pool), _c(wl.head_w, np.float32)
    qs, ks = _c(wl.q_idx_scale), _c(wl.k_scale)
    kind, grp = _SCALES[wl.idx_dtype]
    lib().oracle_indexer_scores(wl.batch, wl.n_q, _ptr(seq), _ptr(tab), wl.max_blocks, 64,
                                wl.num_blocks, _ptr(qi), _DT[wl.idx_dtype], _ptr(qs), kind, grp,
                                wl.H_I, wl.d_I, _ptr(hw), _ptr(kp), _DT[wl.idx_dtype], _ptr(ks),
                                kind, grp, _ptr(r), n, _ptr(out), out.shape[1])
    return out


def topk(scores, row_len, top_k: int):
    """Per row: the min(top_k, L) best positions, ties to the lowest, ascending, -1 padded."""
    s = _c(scores, np.float64)
    rl = _c(np.asarray(row_len), np.int32)
    out = np.empty((s.shape[0], top_k), np.int32)
    lib().oracle_topk(s.shape[0], _ptr(rl), _ptr(s), s.shape[1], top_k, _ptr(out))
    return out


def _kv_args(wl):
    kind, grp = _SCALES[wl.kv_dtype]
    return _c(wl.kv_pool), _DT[wl.kv_dtype], _c(wl.kv_scale), kind, grp


def sparse_attn(wl, indices, rows=None, top_k=None):
    """out [n, H, d_v] and lse [n, H] (float64) over the index lists of all rows_total rows."""
    r, n = _rows_arg(rows)
    n_rows = wl.rows if r is None else n
    idx = _c(indices, np.int32)
    top_k = idx.shape[1] if top_k is None else top_k
    out = np.empty((n_rows, wl.H, wl.d_v), np.float64)
    lse = np.empty((n_rows, wl.H), np.float64)
    seq, tab, q = _c(wl.seq_lens, np.int32), _c(wl.block_table, np.int32), _c(wl.q)
    kv, kvd, kvs, kind, grp = _kv_args(wl)
    lib().oracle_sparse_attn(wl.batch, wl.n_q, _ptr(seq), _ptr(tab), wl.max_blocks, 64,
                             wl.num_blocks, _ptr(q), _DT[wl.q_dtype], wl.H, wl.d_qk, wl.d_v,
                             _ptr(kv), kvd, _ptr(kvs), kind, grp, _ptr(idx), top_k,
                             float(wl.sm_scale), _ptr(r), n, _ptr(out), _ptr(lse))
    return out, lse


def dense_attn(wl, rows=None):
    """Dense causal attention over every s < L_r: out [n, H, d_v], lse [n, H] (float64)."""
    r, n = _rows_arg(rows)
    n_rows = wl.rows if r is None else n
    out = np.empty((n_rows, wl.H, wl.d_v), np.float64)
    lse = np.empty((n_rows, wl.H), np.float64)
    seq, tab, q = _c(wl.seq_lens, np.int32), _c(wl.block_table, np.int32), _c(wl.q)
    kv, kvd, kvs, kind, grp = _kv_args(wl)
    lib().oracle_dense_attn(wl.batch, wl.n_q, _ptr(seq), _ptr(tab), wl.max_blocks, 64,
                            wl.num_blocks, _ptr(q), _DT[wl.q_dtype], wl.H, wl.d_qk, wl.d_v,
                            _ptr(kv), kvd, _ptr(kvs), kind, grp, float(wl.sm_scale),
                            _ptr(r), n, _ptr(out), _ptr(lse))
    return out, lse


def forward(wl, rows=None):
    """The whole stage on the listed rows: (scores, indices, out, lse)."""
    rows_l = np.arange(wl.rows, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    sc = indexer_scores(wl, rows_l)
    idx_rows = topk(sc, wl.row_lens()[rows_l], wl.top_k)
    full = np.full((wl.rows, wl.top_k), -1, np.int32)
    full[rows_l] = idx_rows
    out, lse = sparse_attn(wl, full, rows_l)
    return sc, idx_rows, out, lse


def f32_to_e4m3(x: float) -> int:
    """The oracle's OCP e4m3 code of one float (nearest, ties to even, saturating)."""
    return int(lib().oracle_f32_to_e4m3(float(x)))


def cache_append(wl, x_new, fmt: str, pool, scales):
    """Write rows x_new [rows, width] into `pool` (and `scales`) in place, as storage
    format `fmt` ("f32", "bf16", "e4m3" = fp32 per 128, "e4m3_128", "mxfp8").  An f32
    pool takes float32 rows; every other pool takes bf16 rows, as uint16 bit patterns
    (a bf16 pool copies them bit for bit)."""
    kind, grp = _SCALES[fmt]
    if fmt == "f32":
        x, xdt = _c(x_new, np.float32), _DT["f32"]
    else:
        x = np.ascontiguousarray(x_new)
        assert x.dtype == np.uint16, "bf16 rows as uint16 bit patterns"
        xdt = _DT["bf16"]
    seq, tab = _c(wl.seq_lens, np.int32), _c(wl.block_table, np.int32)
    assert pool.flags.c_contiguous and (scales is None or scales.flags.c_contiguous)
    st = lib().oracle_cache_append(wl.batch, wl.n_q, _ptr(seq), _ptr(tab), wl.max_blocks, 64, wl.num_blocks,
                                   _ptr(x), xdt, x.shape[1], _DT[fmt], kind, grp, _ptr(pool), _ptr(scales))
    if st != 0:
        raise ValueError(f"oracle_cache_append: unsupported pairing of {fmt} pool and {x.dtype} rows")


def e4m3_encode(x):
    """The oracle's e4m3 codes (uint8) of a float32 array, elementwise."""
    v = _c(x, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3_encode(_ptr(v), v.size, _ptr(out))
    return out


def indexer_prolog(p):
    """q [rows, H_I, d_I], head_w [rows, H_I] and k_norm [rows, d_I] (float64) of the
    prolog inputs `p` (bf16 bit arrays x, w_q, w_h, k; fp32 gain; eps)."""
    x, wq, wh, k = _c(p.x), _c(p.w_q), _c(p.w_h), _c(p.k)
    gain = _c(p.gain, np.float32)
    q = np.empty((p.rows, p.H_I, p.d_I), np.float64)
    hw = np.empty((p.rows, p.H_I), np.float64)
    kn = np.empty((p.rows, p.d_I), np.float64)
    lib().oracle_indexer_prolog(p.rows, p.d_x, _ptr(x), _ptr(wq), _ptr(wh), _ptr(k), _ptr(gain),
                                float(p.eps), p.H_I, p.d_I, _ptr(q), _ptr(hw), _ptr(kn))
    return q, hw, kn
