"""Seeded synthetic inputs for the DSA stage, shared by the HIP path and the oracle.

This module draws random tensors, rounds them to the storage dtype, quantizes
them, and scatters them into a paged pool.  It holds none of the method's
arithmetic: no scoring, no selection, no attention.

Recipe (every tensor has its own counter-keyed stream, so tensors are
independent of each other and of the draw order):

    rng(tensor, chunk) = numpy.random.default_rng([seed, rotation, tensor_id, chunk])

* lengths   -- fixed per workload, or for the skewed decode workload drawn
               uniformly from the integers [4096, 131072] (both ends included);
               a sequence's length counts this step's n_q query tokens.
* paging    -- 64-token blocks.  Sequence b owns ceil(L_b/64) logical blocks.
               "permuted": one global random permutation of the pool's blocks;
               "identity": block j of the (single) sequence is pool block j.
               One extra pool block (the last) is never referenced by a valid
               table entry; spare table entries point at it.
* values    -- standard normal float32 times sqrt(var): q_I and k_I use
               var = 1/d_I, head weights 1/H_I, q and kv 1/d_qk.  They are then
               rounded to nearest-even into the storage dtype.
* fp32-scaled e4m3 -- one fp32 scale per 128 elements: scale = amax/448 (1
               when amax = 0), code = e4m3(x/scale).  The fp8 decode workload
               stores q_I and k_I this way; the pages' assignment (workload 6)
               stores the latent KV this way, a 576 row in groups 0..4 of 128
               (the last one covering the 64 rope channels).
* MXFP8     -- e4m3 codes with one E8M0 scale per 32 elements:
               e = floor(log2(amax)) - 8, code = e4m3(clamp(x/2^e, +-448)),
               scale byte = e + 127.  The fp8 decode workload stores the
               latent KV this way; workload 6 stores q_I and k_I this way.
* prolog    -- the indexer prolog's inputs (make_prolog): hidden states x ~
               N(0, 1), the index-key rows k ~ N(0, 1) before normalization,
               projection weights W_q ~ N(0, 1/(d_I*d_x)) and W_h ~
               N(0, 1/(H_I*d_x)), so that the projections have the variances
               of the indexer inputs above, all rounded to bf16; an fp32
               normalization gain 1 + N(0, 0.01).  The hidden width d_x is not
               given by the pages; the decode prolog workload takes 7168.
* poison    -- when requested, every pool element that no valid position maps
               to (the tail of each sequence's last block, and the spare block)
               is NaN, so a kernel that reads outside the history shows it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK = 64

# tensor ids of the counter-keyed streams
_T_LENS, _T_PERM, _T_QI, _T_KI, _T_W, _T_Q, _T_KV = 1, 2, 3, 4, 5, 6, 7
_T_X, _T_WQ, _T_WH, _T_KNEW, _T_GAIN = 8, 9, 10, 11, 12

#: The workloads: the tiny fp32 prefill, decode B=32 at 8k, prefill 32k,
#: skewed long-context decode with 2 verify tokens, and fp8 decode B=64 at 16k.
CONFIGS = {
    1: dict(name="tiny_fp32_prefill_t256", batch=1, n_q=256, lens=256, H_I=4, d_I=32,
            H=8, d_qk=80, d_v=64, top_k=64, idx_dtype="f32", kv_dtype="f32",
            q_dtype="f32", out_dtype="f32", paging="identity", seed=0),
    2: dict(name="decode_bf16_b32_ctx8192", batch=32, n_q=1, lens=8192, H_I=64, d_I=128,
            H=128, d_qk=576, d_v=512, top_k=2048, idx_dtype="bf16", kv_dtype="bf16",
            q_dtype="bf16", out_dtype="bf16", paging="permuted", seed=2),
    3: dict(name="prefill_bf16_t32768", batch=1, n_q=32768, lens=32768, H_I=64, d_I=128,
            H=128, d_qk=576, d_v=512, top_k=2048, idx_dtype="bf16", kv_dtype="bf16",
            q_dtype="bf16", out_dtype="bf16", paging="identity", seed=1),
    4: dict(name="skewed_decode_bf16_b8_nq2_ctx4k_128k", batch=8, n_q=2, lens="skewed",
            H_I=64, d_I=128, H=128, d_qk=576, d_v=512, top_k=2048, idx_dtype="bf16",
            kv_dtype="bf16", q_dtype="bf16", out_dtype="bf16", paging="permuted", seed=4),
    5: dict(name="fp8_decode_b64_ctx16384", batch=64, n_q=1, lens=16384, H_I=64, d_I=128,
            H=128, d_qk=576, d_v=512, top_k=2048, idx_dtype="e4m3", kv_dtype="mxfp8",
            q_dtype="bf16", out_dtype="bf16", paging="permuted", seed=5),
    # the pages' own assignment: MXFP8 indexer q/k (E8M0 per 32) and an fp8
    # KV cache with an fp32 scale per 128 channels
    6: dict(name="fp8_pages_decode_b64_ctx16384", batch=64, n_q=1, lens=16384, H_I=64, d_I=128,
            H=128, d_qk=576, d_v=512, top_k=2048, idx_dtype="mxfp8", kv_dtype="e4m3_128",
            q_dtype="bf16", out_dtype="bf16", paging="permuted", seed=6),
}

_CHUNK = 1 << 22  # elements per drawn chunk, keeps host memory bounded
_POOL = None


def _threads():
    global _POOL
    if _POOL is None:
        import os
        from concurrent.futures import ThreadPoolExecutor
        n = min(16, len(os.sched_getaffinity(0)))
        _POOL = ThreadPoolExecutor(max_workers=n)
    return _POOL


def _rng(seed, rotation, tid, chunk=0):
    return np.random.default_rng([seed, rotation, tid, chunk])


def _normal(shape, var, seed, rotation, tid, convert=None, out_dtype=np.float32):
    """N(0, var) of `shape`, drawn as float32 in fixed-size chunks along the first
    axis (chunk ci from stream rng(tid, ci)); `convert` (float32 chunk -> storage
    dtype chunk) is applied per chunk.  Chunks are drawn on a thread pool; the
    result does not depend on the number of threads."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, out_dtype)
    flat = out.reshape(shape[0], -1) if len(shape) > 1 else out.reshape(-1, 1)
    per = max(1, _CHUNK // max(1, flat.shape[1]))
    sd = np.float32(math.sqrt(var))

    def job(ci, r0):
        r1 = min(flat.shape[0], r0 + per)
        x = _rng(seed, rotation, tid, ci).standard_normal((r1 - r0, flat.shape[1]), np.float32)
        x *= sd
        flat[r0:r1] = x if convert is None else convert(x)

    futs = [_threads().submit(job, ci, r0) for ci, r0 in enumerate(range(0, flat.shape[0], per))]
    for f in futs:
        f.result()
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even); returns the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to OCP e4m3 (nearest-even, saturating at +-448); uint8 codes."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def quantize_e4m3_f32scale(x: np.ndarray, group: int):
    """Per-group (last axis) e4m3 codes with an fp32 scale amax/448 per group.

    When `group` does not divide the last axis, the last group is shorter
    (zero padding changes no amax); there are ceil(n/group) scales."""
    shp = x.shape
    n = shp[-1]
    ng = (n + group - 1) // group
    if ng * group != n:
        pad = np.zeros((*shp[:-1], ng * group - n), np.float32)
        codes, scale = quantize_e4m3_f32scale(np.concatenate([x.astype(np.float32), pad], axis=-1), group)
        return np.ascontiguousarray(codes[..., :n]), scale
    g = x.reshape(*shp[:-1], shp[-1] // group, group)
    amax = np.abs(g).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = f32_to_e4m3_bits(g / scale[..., None]).reshape(shp)
    return codes, scale


def quantize_mxfp8(x: np.ndarray, group: int = 32):
    """Per-group (last axis) MXFP8: e4m3 codes with an E8M0 power-of-two scale.

    floor(log2 amax) is taken exactly from the binary exponent (frexp), and the
    division by 2^e is exact in float32, so the codes are the RNE e4m3 rounding
    of x/2^e, clamped to +-448."""
    shp = x.shape
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).reshape(-1, group)
    amax = t.abs().amax(dim=1)
    _, ex = torch.frexp(amax)                       # amax = m * 2^ex, m in [0.5, 1)
    e = torch.where(amax > 0, ex - 1 - 8, torch.full_like(ex, -127)).clamp(-127, 127)
    inv = torch.exp2((-e).to(torch.float32))        # exact powers of two
    codes = (t * inv[:, None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return (codes.numpy().reshape(shp),
            (e + 127).to(torch.uint8).numpy().reshape(*shp[:-1], shp[-1] // group))


_NAN_BITS = {"f32": None, "bf16": np.uint16(0x7FC0), "e4m3": np.uint8(0x7F), "mxfp8": np.uint8(0x7F),
             "e4m3_128": np.uint8(0x7F)}


@dataclass
class Workload:
    """One batch of DSA inputs in host memory (numpy), in the layouts the library takes.

    Rows are query tokens r = b*n_q + i; row r sees L_r = seq_lens[b] - n_q + i + 1
    positions.  Pools are [num_blocks, 64, width]; scale pools follow the data.
    """
    cfg: dict
    batch: int
    n_q: int
    H_I: int
    d_I: int
    H: int
    d_qk: int
    d_v: int
    top_k: int
    sm_scale: float
    seq_lens: np.ndarray          # int32 [batch]
    block_table: np.ndarray       # int32 [batch, max_blocks]
    num_blocks: int
    idx_dtype: str                # "f32" | "bf16" | "e4m3" (fp32 per 128) | "mxfp8" (E8M0 per 32)
    kv_dtype: str                 # "f32" | "bf16" | "mxfp8" (E8M0 per 32) | "e4m3_128" (fp32 per 128)
    q_dtype: str
    out_dtype: str
    q_idx: np.ndarray             # [rows, H_I, d_I]  f32 | uint16(bf16) | uint8(e4m3)
    q_idx_scale: np.ndarray | None  # f32 [rows, H_I] (per 128) | uint8 [rows, H_I, 4] (per 32) | None
    head_w: np.ndarray            # f32 [rows, H_I]
    k_pool: np.ndarray            # [num_blocks, 64, d_I]
    k_scale: np.ndarray | None    # f32 [num_blocks, 64] | uint8 e8m0 [num_blocks, 64, 4]
    q: np.ndarray                 # [rows, H, d_qk]
    kv_pool: np.ndarray           # [num_blocks, 64, d_qk]
    kv_scale: np.ndarray | None   # uint8 e8m0 [num_blocks, 64, d_qk/32] | f32 [num_blocks, 64, 5]
    extra: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.batch * self.n_q

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.batch else 0

    def row_lens(self) -> np.ndarray:
        b = np.arange(self.rows) // self.n_q
        i = np.arange(self.rows) % self.n_q
        return np.maximum(self.seq_lens[b] - self.n_q + i + 1, 0).astype(np.int32)


def make_workload(cfg_id: int, *, seed: int | None = None, rotation: int = 0,
                  batch: int | None = None, n_q: int | None = None, lens=None,
                  top_k: int | None = None, paging: str | None = None,
                  poison: bool = False, spare_table_blocks: int = 1,
                  idx_dtype: str | None = None) -> Workload:
    """Build the inputs of workload `cfg_id` (1..6), optionally reshaped for small tests.

    `lens` may be an int (all sequences), a sequence of ints, or None (the
    workload's own).  `spare_table_blocks` extra columns are added to the
    block table; they point at the never-valid spare block.  `idx_dtype`
    stores the indexer's q/k in another format; the drawn values are the same.
    """
    cfg = dict(CONFIGS[cfg_id])
    seed = cfg["seed"] if seed is None else seed
    B = cfg["batch"] if batch is None else batch
    nq = cfg["n_q"] if n_q is None else n_q
    paging = cfg["paging"] if paging is None else paging
    K = cfg["top_k"] if top_k is None else top_k
    H_I, d_I, H, d_qk, d_v = cfg["H_I"], cfg["d_I"], cfg["H"], cfg["d_qk"], cfg["d_v"]

    if lens is None:
        lens = cfg["lens"]
    if isinstance(lens, str):  # skewed long-context lengths
        L = _rng(seed, rotation, _T_LENS).integers(4096, 131072, size=B, endpoint=True)
    elif np.isscalar(lens):
        L = np.full(B, int(lens))
    else:
        L = np.asarray(lens, np.int64)
        assert L.shape == (B,)
    L = L.astype(np.int32)
    prefill = cfg["n_q"] == cfg["lens"]
    if prefill and n_q is None:
        assert (L == L[0]).all(), "prefill batches need equal lengths"
        nq = int(L[0])  # prefill: one query per position, row t sees t+1 positions

    nblk_seq = [(int(x) + BLOCK - 1) // BLOCK for x in L]
    n_used = int(sum(nblk_seq))
    num_blocks = n_used + 1  # + one spare block
    if paging == "identity":
        perm = np.arange(n_used, dtype=np.int64)
    else:
        perm = _rng(seed, rotation, _T_PERM).permutation(n_used)
    spare = num_blocks - 1
    max_blocks = max(nblk_seq) + spare_table_blocks if B else 1
    table = np.full((B, max_blocks), spare, np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk_seq[b]] = perm[off:off + nblk_seq[b]]
        off += nblk_seq[b]

    rows = B * nq
    if idx_dtype is not None:
        cfg["idx_dtype"] = idx_dtype
    idx_dtype, kv_dtype = cfg["idx_dtype"], cfg["kv_dtype"]

    def pooled(tid, width, var):
        """Logical [L_b, width] per sequence, scattered into a [num_blocks*64, width] pool."""
        pool = np.zeros((num_blocks * BLOCK, width), np.float32)
        valid = np.zeros(num_blocks * BLOCK, bool)
        for b in range(B):
            x = _normal((int(L[b]), width), var, seed, rotation, tid * 100003 + b)
            s = np.arange(int(L[b]))
            prow = table[b, s // BLOCK].astype(np.int64) * BLOCK + s % BLOCK
            pool[prow] = x
            valid[prow] = True
        return pool, valid

    kf, kvalid = pooled(_T_KI, d_I, 1.0 / d_I)
    kvf, kvvalid = pooled(_T_KV, d_qk, 1.0 / d_qk)
    if idx_dtype == "bf16":
        qif = _normal((rows, H_I, d_I), 1.0 / d_I, seed, rotation, _T_QI,
                      convert=f32_to_bf16_bits, out_dtype=np.uint16)
    else:
        qif = _normal((rows, H_I, d_I), 1.0 / d_I, seed, rotation, _T_QI)
    w = _normal((rows, H_I), 1.0 / H_I, seed, rotation, _T_W)
    if cfg["q_dtype"] == "f32":
        q = _normal((rows, H, d_qk), 1.0 / d_qk, seed, rotation, _T_Q)
    else:
        q = _normal((rows, H, d_qk), 1.0 / d_qk, seed, rotation, _T_Q,
                    convert=f32_to_bf16_bits, out_dtype=np.uint16)

    q_idx_scale = k_scale = kv_scale = None
    if idx_dtype == "f32":
        q_idx, k_pool = qif, kf
    elif idx_dtype == "bf16":
        q_idx, k_pool = qif, f32_to_bf16_bits(kf)
    elif idx_dtype == "e4m3":
        q_idx, qs = quantize_e4m3_f32scale(qif, 128)
        q_idx_scale = qs.reshape(rows, H_I * d_I // 128)
        k_pool, ks = quantize_e4m3_f32scale(kf, 128)
        k_scale = ks.reshape(num_blocks * BLOCK, d_I // 128)
    elif idx_dtype == "mxfp8":
        q_idx, q_idx_scale = quantize_mxfp8(qif, 32)   # [rows, H_I, d_I], [rows, H_I, d_I/32]
        k_pool, k_scale = quantize_mxfp8(kf, 32)       # [pool rows, d_I], [pool rows, d_I/32]
    else:
        raise ValueError(idx_dtype)

    if kv_dtype == "f32":
        kv_pool = kvf
    elif kv_dtype == "bf16":
        kv_pool = f32_to_bf16_bits(kvf)
    elif kv_dtype == "mxfp8":
        kv_pool, kv_scale = quantize_mxfp8(kvf, 32)
    elif kv_dtype == "e4m3_128":
        kv_pool, kv_scale = quantize_e4m3_f32scale(kvf, 128)  # scales [pool rows, 5]
    else:
        raise ValueError(kv_dtype)

    if poison:
        inv_k, inv_kv = ~kvalid, ~kvvalid
        if idx_dtype == "f32":
            k_pool[inv_k] = np.nan
        else:
            k_pool[inv_k] = _NAN_BITS[idx_dtype]
        if k_scale is not None:
            k_scale[inv_k] = np.uint8(0xFF) if k_scale.dtype == np.uint8 else np.nan
        if kv_dtype == "f32":
            kv_pool[inv_kv] = np.nan
        elif kv_dtype == "bf16":
            kv_pool[inv_kv] = _NAN_BITS["bf16"]
        else:
            kv_pool[inv_kv] = _NAN_BITS["e4m3"]
            kv_scale[inv_kv] = np.uint8(0xFF) if kv_scale.dtype == np.uint8 else np.nan

    def blocks(a):
        return None if a is None else np.ascontiguousarray(a.reshape(num_blocks, BLOCK, *a.shape[1:]))

    wl = Workload(
        cfg=cfg, batch=B, n_q=nq, H_I=H_I, d_I=d_I, H=H, d_qk=d_qk, d_v=d_v, top_k=K,
        sm_scale=1.0 / math.sqrt(d_qk), seq_lens=L, block_table=table, num_blocks=num_blocks,
        idx_dtype=idx_dtype, kv_dtype=kv_dtype, q_dtype=cfg["q_dtype"], out_dtype=cfg["out_dtype"],
        q_idx=np.ascontiguousarray(q_idx), q_idx_scale=q_idx_scale,
        head_w=np.ascontiguousarray(w), k_pool=blocks(k_pool),
        k_scale=(None if k_scale is None else np.ascontiguousarray(
            k_scale.reshape(num_blocks, BLOCK) if idx_dtype == "e4m3" else blocks(k_scale))),
        q=np.ascontiguousarray(q), kv_pool=blocks(kv_pool), kv_scale=blocks(kv_scale),
    )
    return wl


#: The indexer prolog of one decode step of the decode workload (32 query
#: tokens), from a hidden state of width 7168.
PROLOG = dict(name="prolog_decode_b32_dx7168", rows=32, d_x=7168, H_I=64, d_I=128, eps=1e-6, seed=7)


@dataclass
class PrologInputs:
    rows: int
    d_x: int
    H_I: int
    d_I: int
    eps: float
    x: np.ndarray      # uint16 bf16 bits [rows, d_x]
    w_q: np.ndarray    # uint16 bf16 bits [H_I*d_I, d_x]
    w_h: np.ndarray    # uint16 bf16 bits [H_I, d_x]
    k: np.ndarray      # uint16 bf16 bits [rows, d_I]
    gain: np.ndarray   # float32 [d_I]


def make_prolog(rows: int, d_x: int = 7168, H_I: int = 64, d_I: int = 128, *, seed: int = 7,
                rotation: int = 0, eps: float = 1e-6) -> PrologInputs:
    """Seeded inputs of the indexer prolog (recipe in the module docstring)."""
    bf = f32_to_bf16_bits
    x = _normal((rows, d_x), 1.0, seed, rotation, _T_X, bf, np.uint16)
    w_q = _normal((H_I * d_I, d_x), 1.0 / (d_I * d_x), seed, rotation, _T_WQ, bf, np.uint16)
    w_h = _normal((H_I, d_x), 1.0 / (H_I * d_x), seed, rotation, _T_WH, bf, np.uint16)
    k = _normal((rows, d_I), 1.0, seed, rotation, _T_KNEW, bf, np.uint16)
    gain = (1.0 + _normal((d_I,), 0.01, seed, rotation, _T_GAIN)).astype(np.float32)
    return PrologInputs(rows=rows, d_x=d_x, H_I=H_I, d_I=d_I, eps=eps, x=x.reshape(rows, d_x),
                        w_q=w_q, w_h=w_h, k=k.reshape(rows, d_I), gain=gain)
