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
  1e-3 relative of the k-th score (R8 of the readings in the design notes);
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
