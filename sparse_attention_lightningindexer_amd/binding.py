"""Thin ctypes binding of libdsa.so (include/dsa.h): argument marshalling only.

Every step of the DSA stage runs in the library's HIP kernels; this module
only turns torch device tensors into the ABI's structs and pointers, passes
torch's current HIP stream, and raises on a non-OK status.  There is no CPU
fallback: if libdsa.so is missing, loading fails loudly.

Functions with the C names:
    dsa_indexer_scores(dev, scores=None)          -> scores  fp32 [rows, ld]
    dsa_topk(dev, scores, top_k=None)             -> indices int32 [rows, top_k]
    dsa_sparse_attn(dev, indices, top_k=None)     -> (out, lse)
    dsa_forward(dev, top_k=None, indices_out=...) -> (out, lse, indices)
    dsa_forward_noalloc(dev, top_k=None, indices_out=None) -> (out, lse, indices_out)
    dsa_cache_append(dev, k_new, kv_new)
    dsa_indexer_prolog(pd, q_fmt)                 -> (q, q_scale, head_w, k_norm)
and their *_workspace_bytes queries, where `dev` is a DeviceInputs (device
copies of a Workload plus the ABI structs that point at them).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch  # must be imported before libdsa.so so both share one HIP runtime

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

DSA_OK, DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(6)
DSA_F32, DSA_BF16, DSA_E4M3 = 0, 1, 2
DSA_SCALE_NONE, DSA_SCALE_F32, DSA_SCALE_E8M0 = 0, 1, 2


class DsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib().dsa_status_string(status).decode()}")


class dsa_batch(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q", C.c_int32), ("seq_lens", C.c_void_p),
                ("block_table", C.c_void_p), ("max_blocks", C.c_int32), ("block_size", C.c_int32),
                ("max_seq_len", C.c_int32)]


class dsa_cache(C.Structure):
    """A paged pool; strides are in elements (of the data, then of the scales), 0 = dense."""
    _fields_ = [("data", C.c_void_p), ("scales", C.c_void_p), ("dtype", C.c_int),
                ("scale_kind", C.c_int), ("group", C.c_int32), ("width", C.c_int32),
                ("num_blocks", C.c_int64), ("block_stride", C.c_int64), ("row_stride", C.c_int64),
                ("scale_block_stride", C.c_int64), ("scale_row_stride", C.c_int64)]


class dsa_indexer_args(C.Structure):
    _fields_ = [("q", C.c_void_p), ("dtype", C.c_int), ("q_scale", C.c_void_p),
                ("n_heads", C.c_int32), ("head_dim", C.c_int32), ("head_w", C.c_void_p),
                ("k", dsa_cache)]


class dsa_attn_args(C.Structure):
    _fields_ = [("q", C.c_void_p), ("dtype", C.c_int), ("n_heads", C.c_int32), ("d_v", C.c_int32),
                ("sm_scale", C.c_float), ("kv", dsa_cache), ("out", C.c_void_p), ("lse", C.c_void_p)]


class dsa_prolog_args(C.Structure):
    _fields_ = [("rows", C.c_int32), ("d_x", C.c_int32), ("n_heads", C.c_int32), ("head_dim", C.c_int32),
                ("x", C.c_void_p), ("w_q", C.c_void_p), ("w_h", C.c_void_p), ("k", C.c_void_p),
                ("k_gain", C.c_void_p), ("eps", C.c_float), ("q_dtype", C.c_int), ("q_out", C.c_void_p),
                ("q_scale_out", C.c_void_p), ("head_w_out", C.c_void_p), ("k_out", C.c_void_p)]


_lib = None

#: every entry point include/dsa.h declares
EXPORTS = ("dsa_status_string", "dsa_version", "dsa_indexer_scores", "dsa_topk_workspace_bytes",
           "dsa_topk", "dsa_sparse_attn_workspace_bytes", "dsa_sparse_attn",
           "dsa_forward_workspace_bytes", "dsa_forward", "dsa_forward_noalloc", "dsa_forward_noalloc_max_bytes",
           "dsa_cache_append", "dsa_indexer_prolog")


def lib():
    """The loaded libdsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        P, S = C.POINTER, C.c_size_t
        L.dsa_status_string.restype = C.c_char_p
        L.dsa_status_string.argtypes = [C.c_int]
        L.dsa_version.restype = C.c_int32
        L.dsa_indexer_scores.restype = C.c_int
        L.dsa_indexer_scores.argtypes = [P(dsa_batch), P(dsa_indexer_args), C.c_void_p, C.c_int64, C.c_void_p]
        L.dsa_topk_workspace_bytes.restype = S
        L.dsa_topk_workspace_bytes.argtypes = [P(dsa_batch), C.c_int32]
        L.dsa_topk.restype = C.c_int
        L.dsa_topk.argtypes = [P(dsa_batch), C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p, S,
                               C.c_void_p]
        L.dsa_sparse_attn_workspace_bytes.restype = S
        L.dsa_sparse_attn_workspace_bytes.argtypes = [P(dsa_batch), P(dsa_attn_args), C.c_int32]
        L.dsa_sparse_attn.restype = C.c_int
        L.dsa_sparse_attn.argtypes = [P(dsa_batch), P(dsa_attn_args), C.c_void_p, C.c_int32, C.c_void_p, S,
                                      C.c_void_p]
        L.dsa_forward_workspace_bytes.restype = S
        L.dsa_forward_workspace_bytes.argtypes = [P(dsa_batch), P(dsa_indexer_args), P(dsa_attn_args),
                                                  C.c_int32]
        L.dsa_cache_append.restype = C.c_int
        L.dsa_cache_append.argtypes = [P(dsa_batch), C.c_void_p, C.c_void_p, C.c_int, P(dsa_cache), P(dsa_cache),
                                       C.c_void_p]
        L.dsa_indexer_prolog.restype = C.c_int
        L.dsa_indexer_prolog.argtypes = [P(dsa_prolog_args), C.c_void_p]
        L.dsa_forward.restype = C.c_int
        L.dsa_forward.argtypes = [P(dsa_batch), P(dsa_indexer_args), P(dsa_attn_args), C.c_int32, C.c_void_p,
                                  C.c_void_p, S, C.c_void_p]
        L.dsa_forward_noalloc.restype = C.c_int
        L.dsa_forward_noalloc.argtypes = [P(dsa_batch), P(dsa_indexer_args), P(dsa_attn_args), C.c_int32,
                                          C.c_void_p, C.c_void_p]
        L.dsa_forward_noalloc_max_bytes.restype = S
        L.dsa_forward_noalloc_max_bytes.argtypes = []
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != DSA_OK:
        raise DsaError(status, where)


def _stream(stream):
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


_DT = {"f32": DSA_F32, "bf16": DSA_BF16, "e4m3": DSA_E4M3, "mxfp8": DSA_E4M3, "e4m3_128": DSA_E4M3}
#: storage format name -> (element dtype, scale kind, elements per scale)
_FMT = {"f32": (DSA_F32, DSA_SCALE_NONE, 0), "bf16": (DSA_BF16, DSA_SCALE_NONE, 0),
        "e4m3": (DSA_E4M3, DSA_SCALE_F32, 128), "e4m3_128": (DSA_E4M3, DSA_SCALE_F32, 128),
        "mxfp8": (DSA_E4M3, DSA_SCALE_E8M0, 32)}


def _dev(a, device):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceInputs:
    """Device copies of a Workload's inputs, the output buffers, and the ABI structs."""

    def __init__(self, wl, device="cuda"):
        self.wl = wl
        self.rows = wl.rows
        self.top_k = wl.top_k
        d = device
        self.seq_lens = _dev(wl.seq_lens.astype(np.int32), d)
        self.block_table = _dev(wl.block_table.astype(np.int32), d)
        self.q_idx = _dev(wl.q_idx, d)
        self.q_idx_scale = _dev(wl.q_idx_scale, d)
        self.head_w = _dev(wl.head_w.astype(np.float32), d)
        self.k_pool = _dev(wl.k_pool, d)
        self.k_scale = _dev(wl.k_scale, d)
        self.q = _dev(wl.q, d)
        self.kv_pool = _dev(wl.kv_pool, d)
        self.kv_scale = _dev(wl.kv_scale, d)
        out_dt = torch.float32 if wl.out_dtype == "f32" else torch.bfloat16
        self.out = torch.empty((wl.rows, wl.H, wl.d_v), dtype=out_dt, device=d)
        self.lse = torch.empty((wl.rows, wl.H), dtype=torch.float32, device=d)
        self.ld = int(max(1, wl.max_seq_len))
        self.batch = dsa_batch(wl.batch, wl.n_q, self.seq_lens.data_ptr() if wl.batch else None,
                               self.block_table.data_ptr() if wl.batch else None, wl.max_blocks, 64,
                               wl.max_seq_len)
        idt, ikind, igroup = _FMT[wl.idx_dtype]
        idx_scaled = ikind != DSA_SCALE_NONE
        kcache = dsa_cache(self.k_pool.data_ptr(), self.k_scale.data_ptr() if idx_scaled else None,
                           idt, ikind, igroup, wl.d_I, wl.num_blocks)
        self.idx = dsa_indexer_args(self.q_idx.data_ptr(), idt,
                                    self.q_idx_scale.data_ptr() if idx_scaled else None, wl.H_I, wl.d_I,
                                    self.head_w.data_ptr(), kcache)
        kdt, kkind, kgroup = _FMT[wl.kv_dtype]
        kv_scaled = kkind != DSA_SCALE_NONE
        kvcache = dsa_cache(self.kv_pool.data_ptr(), self.kv_scale.data_ptr() if kv_scaled else None,
                            kdt, kkind, kgroup, wl.d_qk, wl.num_blocks)
        self.attn = dsa_attn_args(self.q.data_ptr(), _DT[wl.q_dtype], wl.H, wl.d_v, float(wl.sm_scale),
                                  kvcache, self.out.data_ptr(), self.lse.data_ptr())

    def set_outputs(self, out, lse):
        """Point the attention outputs at other tensors (lse may be None)."""
        self.out, self.lse = out, lse
        self.attn.out = out.data_ptr()
        self.attn.lse = None if lse is None else lse.data_ptr()


def dsa_indexer_scores(dev: DeviceInputs, scores=None, ld=None, stream=None):
    ld = dev.ld if ld is None else ld
    if scores is None:
        scores = torch.full((dev.rows, ld), float("nan"), dtype=torch.float32, device=dev.q.device)
    _check(lib().dsa_indexer_scores(C.byref(dev.batch), C.byref(dev.idx), _ptr(scores), ld, _stream(stream)),
           "dsa_indexer_scores")
    return scores


def dsa_topk_workspace_bytes(dev: DeviceInputs, top_k=None) -> int:
    return int(lib().dsa_topk_workspace_bytes(C.byref(dev.batch), dev.top_k if top_k is None else top_k))


def dsa_topk(dev: DeviceInputs, scores, top_k=None, indices=None, ld=None, ws=None, stream=None):
    top_k = dev.top_k if top_k is None else top_k
    ld = scores.shape[1] if ld is None else ld
    if indices is None:
        indices = torch.empty((dev.rows, top_k), dtype=torch.int32, device=scores.device)
    nws = dsa_topk_workspace_bytes(dev, top_k)
    if ws is None and nws:
        ws = torch.empty(nws, dtype=torch.uint8, device=scores.device)
    _check(lib().dsa_topk(C.byref(dev.batch), _ptr(scores), ld, top_k, _ptr(indices), _ptr(ws), nws,
                          _stream(stream)), "dsa_topk")
    return indices


def dsa_sparse_attn_workspace_bytes(dev: DeviceInputs, top_k=None) -> int:
    return int(lib().dsa_sparse_attn_workspace_bytes(C.byref(dev.batch), C.byref(dev.attn),
                                                     dev.top_k if top_k is None else top_k))


def dsa_sparse_attn(dev: DeviceInputs, indices, top_k=None, ws=None, stream=None):
    top_k = indices.shape[1] if top_k is None else top_k
    nws = dsa_sparse_attn_workspace_bytes(dev, top_k)
    if ws is None and nws:
        ws = torch.empty(nws, dtype=torch.uint8, device=indices.device)
    _check(lib().dsa_sparse_attn(C.byref(dev.batch), C.byref(dev.attn), _ptr(indices), top_k, _ptr(ws),
                                 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "dsa_sparse_attn")
    return dev.out, dev.lse


def dsa_forward_workspace_bytes(dev: DeviceInputs, top_k=None) -> int:
    return int(lib().dsa_forward_workspace_bytes(C.byref(dev.batch), C.byref(dev.idx), C.byref(dev.attn),
                                                 dev.top_k if top_k is None else top_k))


def dsa_forward(dev: DeviceInputs, top_k=None, indices_out=None, ws=None, stream=None, want_indices=True):
    top_k = dev.top_k if top_k is None else top_k
    if indices_out is None and want_indices:
        indices_out = torch.empty((dev.rows, top_k), dtype=torch.int32, device=dev.q.device)
    nws = dsa_forward_workspace_bytes(dev, top_k)
    if ws is None:
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev.q.device)
    _check(lib().dsa_forward(C.byref(dev.batch), C.byref(dev.idx), C.byref(dev.attn), top_k, _ptr(indices_out),
                             _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "dsa_forward")
    return dev.out, dev.lse, indices_out


def dsa_forward_noalloc(dev: DeviceInputs, top_k=None, indices_out=None, stream=None):
    """dsa_forward in the library's per-GPU scratch array (no workspace argument);
    indices_out may be None."""
    top_k = dev.top_k if top_k is None else top_k
    _check(lib().dsa_forward_noalloc(C.byref(dev.batch), C.byref(dev.idx), C.byref(dev.attn), top_k,
                                     _ptr(indices_out), _stream(stream)), "dsa_forward_noalloc")
    return dev.out, dev.lse, indices_out


def dsa_cache_append(dev: DeviceInputs, k_new, kv_new, stream=None):
    """Write rows k_new [rows, d_I] and kv_new [rows, d_qk] (bf16, or fp32 for fp32 pools)
    into dev's pools (and scales) at each row's own position."""
    new_dt = DSA_F32 if k_new.dtype == torch.float32 else DSA_BF16
    _check(lib().dsa_cache_append(C.byref(dev.batch), _ptr(k_new), _ptr(kv_new), new_dt, C.byref(dev.idx.k),
                                  C.byref(dev.attn.kv), _stream(stream)), "dsa_cache_append")


class PrologDevice:
    """Device copies of the indexer prolog's inputs (a PrologInputs)."""

    def __init__(self, p, device="cuda"):
        self.p = p
        self.x = _dev(p.x, device)
        self.w_q = _dev(p.w_q, device)
        self.w_h = _dev(p.w_h, device)
        self.k = _dev(p.k, device)
        self.gain = _dev(p.gain.astype(np.float32), device)


def dsa_indexer_prolog(pd: PrologDevice, q_fmt: str = "bf16", outs=None, stream=None):
    """q [rows, H_I, d_I] (bf16 bits as int16, or e4m3 codes as uint8 for q_fmt "mxfp8"),
    q_scale (E8M0 bytes [rows, H_I, d_I/32], or None), head_w fp32 [rows, H_I] and
    k_norm (bf16 bits as int16) [rows, d_I].  `outs` reuses those four tensors."""
    p, dev = pd.p, pd.x.device
    mx = q_fmt == "mxfp8"
    if q_fmt not in ("bf16", "mxfp8"):
        raise ValueError(f"prolog query format {q_fmt!r}: bf16 or mxfp8")
    if outs is None:
        q = torch.empty((p.rows, p.H_I, p.d_I), dtype=torch.uint8 if mx else torch.int16, device=dev)
        qs = torch.empty((p.rows, p.H_I, p.d_I // 32), dtype=torch.uint8, device=dev) if mx else None
        hw = torch.empty((p.rows, p.H_I), dtype=torch.float32, device=dev)
        kn = torch.empty((p.rows, p.d_I), dtype=torch.int16, device=dev)
    else:
        q, qs, hw, kn = outs
    args = dsa_prolog_args(p.rows, p.d_x, p.H_I, p.d_I, pd.x.data_ptr(), pd.w_q.data_ptr(), pd.w_h.data_ptr(),
                           pd.k.data_ptr(), pd.gain.data_ptr(), float(p.eps), DSA_E4M3 if mx else DSA_BF16,
                           q.data_ptr(), None if qs is None else qs.data_ptr(), hw.data_ptr(), kn.data_ptr())
    _check(lib().dsa_indexer_prolog(C.byref(args), _stream(stream)), "dsa_indexer_prolog")
    return q, qs, hw, kn
