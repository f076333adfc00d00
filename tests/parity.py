"""Comparison helpers for the GPU parity tests (oracle on the CPU, HIP path on the GPU).

Tolerances:
* indexer scores -- the fp32 forward error bound of the computation: products
  of the bf16/e4m3 inputs are exact in fp32, a dot of d_I terms and a weighted
  sum of H_I terms accumulate in fp32, so
      |I_gpu - I| <= 4 * (d_I + H_I + 4) * 2^-24 * sum_j |w_j| sum_c |q_jc k_c|
  (the factor 4 covers the two extra scale roundings of the fp8 path);
* indices -- bit-exact when the oracle selects from the GPU's own fp32 scores
  (both sides then take the decision in the kernel's precision); against the
  oracle's fp64 scores, a position may differ only if its score is within
  1e-3 relative of the k-th score, where the k-th score is the oracle's
  k_r-th largest fp64 score of the row (1e-3 of the row's largest magnitude
  when that score is 0);
* attention -- bf16 outputs: max |d| <= 2e-2 and ||d||_2 <= 1e-2 ||ref||_2;
  fp32 outputs: max |d| <= 1e-4 max |ref|; lse: |d| <= 1e-3 (+ 1e-4 relative
  for fp32).
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle as O
from sparse_attention_lightningindexer_amd import binding as B


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def dequant_np(a, dtype):
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()
    return torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()


def logical_rows(pool, wl, b, L):
    s = np.arange(L)
    flat = pool.reshape(-1, *pool.shape[2:])
    return flat[wl.block_table[b, s // 64].astype(np.int64) * 64 + s % 64]


def score_bound(wl, rows):
    """Forward error bound per (row, s) of the fp32 indexer, from |inputs|."""
    out = []
    for r in rows:
        b = r // wl.n_q
        L = int(wl.row_lens()[r])
        K = np.abs(dequant_np(logical_rows(wl.k_pool, wl, b, L), wl.idx_dtype))
        Q = np.abs(dequant_np(wl.q_idx[r], wl.idx_dtype))
        if wl.idx_dtype == "e4m3":  # one fp32 factor per 128-element vector
            Q = Q * wl.q_idx_scale[r][:, None].astype(np.float64)
            K = K * logical_rows(wl.k_scale[..., None], wl, b, L)[:, :1].astype(np.float64)
        elif wl.idx_dtype == "mxfp8":  # one E8M0 factor per 32 elements
            def e8m0(a):
                f = torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e8m0fnu).double().numpy()
                return np.repeat(f, 32, axis=-1)
            Q = Q * e8m0(wl.q_idx_scale[r])
            K = K * e8m0(logical_rows(wl.k_scale, wl, b, L))
        S = np.abs(wl.head_w[r]).astype(np.float64) @ (Q @ K.T)
        out.append(4 * (wl.d_I + wl.H_I + 4) * 2.0 ** -24 * S + 1e-30)
    return out


def check_scores(wl, gpu_scores: np.ndarray, ref_scores: np.ndarray, rows):
    bounds = score_bound(wl, rows)
    for i, r in enumerate(rows):
        L = int(wl.row_lens()[r])
        g, ref = gpu_scores[i, :L], ref_scores[i, :L]
        assert np.isfinite(g).all(), f"row {r}: non-finite GPU score"
        err = np.abs(g - ref)
        bad = err > bounds[i]
        assert not bad.any(), (f"row {r}: {bad.sum()} scores beyond the fp32 bound, worst "
                               f"{err[bad].max():.3e} vs bound {bounds[i][bad].min():.3e}")


def check_indices_exact(gpu_idx: np.ndarray, ref_idx: np.ndarray, rows=None):
    rows = range(gpu_idx.shape[0]) if rows is None else rows
    for i in rows:
        assert np.array_equal(gpu_idx[i], ref_idx[i]), (
            f"row {i}: indices differ at slots {np.nonzero(gpu_idx[i] != ref_idx[i])[0][:10]}")


def check_indices_band(gpu_idx_row, ref_idx_row, ref_scores_row, L, top_k, rtol=1e-3):
    """Set equality except positions whose oracle score lies within rtol of the k-th score."""
    k = min(top_k, L)
    g = gpu_idx_row[:k]
    assert (gpu_idx_row[k:] == -1).all() and (g >= 0).all() and (g < L).all()
    assert len(set(g.tolist())) == k and np.all(np.diff(g) > 0), "indices not unique ascending"
    if L <= top_k:
        assert g.tolist() == list(range(L))
        return 0
    sc = ref_scores_row[:L]
    kth = np.sort(sc)[::-1][k - 1]
    tol = rtol * (abs(kth) if kth != 0 else np.abs(sc).max())
    diff = set(g.tolist()) ^ set(ref_idx_row[:k].tolist())
    for p in diff:
        assert abs(sc[p] - kth) <= tol, f"position {p} score {sc[p]!r} outside the band of k-th {kth!r}"
    return len(diff)


def check_attention(wl, out_gpu: np.ndarray, lse_gpu: np.ndarray, out_ref: np.ndarray, lse_ref: np.ndarray,
                    what=""):
    assert np.isfinite(out_gpu).all(), f"{what}: non-finite output"
    d = np.abs(out_gpu - out_ref)
    if wl.out_dtype == "f32":
        assert d.max() <= 1e-4 * np.abs(out_ref).max() + 1e-30, f"{what}: max|d| {d.max():.3e}"
    else:
        assert d.max() <= 2e-2, f"{what}: max|d| {d.max():.3e}"
        nr = np.linalg.norm(out_ref)
        if nr > 0:
            assert np.linalg.norm(out_gpu - out_ref) <= 1e-2 * nr, (
                f"{what}: normwise {np.linalg.norm(out_gpu - out_ref) / nr:.3e}")
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse_gpu)), f"{what}: lse finiteness differs"
    assert (np.isneginf(lse_gpu[~fin])).all()
    tol = 1e-3 + (1e-4 * np.abs(lse_ref[fin]) if wl.out_dtype == "f32" else 0)
    assert (np.abs(lse_gpu[fin] - lse_ref[fin]) <= tol).all(), (
        f"{what}: lse max|d| {np.abs(lse_gpu[fin] - lse_ref[fin]).max():.3e}")
    empty = ~np.isfinite(lse_ref)
    if empty.any():
        assert (out_gpu[empty] == 0).all(), f"{what}: empty rows not zero"


def full_indices(wl, rows, idx_rows):
    full = np.full((wl.rows, idx_rows.shape[1]), -1, np.int32)
    full[np.asarray(rows)] = idx_rows
    return full


def gpu_all(wl, dev=None):
    """Unfused calls through the C ABI: (dev, scores, indices, out, lse) as host arrays."""
    dev = B.DeviceInputs(wl) if dev is None else dev
    sc = B.dsa_indexer_scores(dev)
    idx = B.dsa_topk(dev, sc)
    out, lse = B.dsa_sparse_attn(dev, idx)
    torch.cuda.synchronize()
    return dev, sc.cpu().numpy().astype(np.float64), idx.cpu().numpy(), f64(out), f64(lse)


# ------------------------------------------------------------ indexer prolog

_U = 2.0 ** -24


def _bf16_bits_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()


def _to_bf16_f64(v: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 of float32(v) (monotone in v), as float64."""
    return torch.from_numpy(np.ascontiguousarray(v, np.float64).astype(np.float32)).to(torch.bfloat16).double().numpy()


def prolog_bound(p) -> tuple:
    """Forward error bounds of the prolog's fp32 projections: along any path of the
    kernel's sums a result passes at most n = 32 (inside one MFMA) + 4*ceil(d_x/1024)
    (a wave's MFMA chain) + 8 (the waves' partials) + 4 additions, so
        |v_gpu - v| <= n * 2^-24 * sum_c |w_nc x_rc| + 2^-24 |v|."""
    x = np.abs(_bf16_bits_f64(p.x))
    n = 32 + 4 * -(-p.d_x // 1024) + 8 + 4
    sq = n * _U * (x @ np.abs(_bf16_bits_f64(p.w_q)).T)
    sh = n * _U * (x @ np.abs(_bf16_bits_f64(p.w_h)).T)
    return sq.reshape(p.rows, p.H_I, p.d_I), sh


def _mx_exponent(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) - 8, -127 for a = 0, clamped to [-127, 127] (monotone in a)."""
    m, e2 = np.frexp(a)
    e = np.where(a > 0, e2.astype(np.int64) - 1 - 8, -127)
    return np.clip(e, -127, 127)


def check_prolog(p, q_fmt, q_gpu, qs_gpu, hw_gpu, kn_gpu, ref):
    """GPU prolog outputs against the oracle's fp64 values: every stored value must be
    one that the kernel's rounding rule gives for some fp32 result within the forward
    error bound (an interval check: bf16 and e4m3 rounding are monotone), and the
    E8M0 exponent must lie between those of the bound's smallest and largest amax."""
    q64, hw64, kn64 = ref
    bq, bh = prolog_bound(p)
    lo, hi = q64 - bq - _U * np.abs(q64), q64 + bq + _U * np.abs(q64)
    # head weights, fp32
    d = np.abs(hw_gpu.astype(np.float64) - hw64)
    assert (d <= bh + 2 * _U * np.abs(hw64)).all(), f"head_w: worst excess {np.max(d - bh)}"
    # normalized keys, bf16: fp32 sum of squares, square root, division, two products
    kn = _bf16_bits_f64(kn_gpu)
    rel = (2 * p.d_I + 16) * _U
    klo, khi = kn64 - rel * np.abs(kn64), kn64 + rel * np.abs(kn64)
    assert ((kn >= _to_bf16_f64(klo)) & (kn <= _to_bf16_f64(khi))).all(), "k_norm outside its interval"
    if q_fmt == "bf16":
        qg = _bf16_bits_f64(q_gpu)
        ok = (qg >= _to_bf16_f64(lo)) & (qg <= _to_bf16_f64(hi))
        assert ok.all(), f"q (bf16): {np.count_nonzero(~ok)} values outside their interval"
        return
    # MXFP8: one exponent per 32 channels
    g = 32
    shp = (p.rows, p.H_I, p.d_I // g, g)
    lo_g, hi_g = lo.reshape(shp), hi.reshape(shp)
    amax_hi = np.maximum(np.abs(lo_g), np.abs(hi_g)).max(axis=-1)
    amin_each = np.where((lo_g <= 0) & (hi_g >= 0), 0.0, np.minimum(np.abs(lo_g), np.abs(hi_g)))
    amax_lo = amin_each.max(axis=-1)
    e_gpu = qs_gpu.astype(np.int64) - 127
    e_lo = _mx_exponent(amax_lo.astype(np.float32).astype(np.float64))
    e_hi = _mx_exponent(amax_hi.astype(np.float32).astype(np.float64))
    ok_e = (e_gpu >= e_lo) & (e_gpu <= e_hi)
    assert ok_e.all(), f"q scale: {np.count_nonzero(~ok_e)} E8M0 exponents outside their range"
    sc = np.ldexp(1.0, -e_gpu)[..., None]

    def enc(v):
        w = np.clip((v.astype(np.float32).astype(np.float64) * sc), -448, 448).astype(np.float32)
        return O.dequant(O.e4m3_encode(w).reshape(-1, 1), "e4m3")[:, 0].reshape(shp)

    got = O.dequant(np.ascontiguousarray(q_gpu).reshape(-1, 1), "e4m3")[:, 0].reshape(shp)
    ok = (got >= enc(lo_g)) & (got <= enc(hi_g))
    assert ok.all(), f"q (MXFP8): {np.count_nonzero(~ok)} codes outside their interval"
    # the interval check is tight: nearly every code equals the one of the fp64 value
    same = got == enc(q64.reshape(shp))
    assert same.mean() > 0.99, same.mean()
