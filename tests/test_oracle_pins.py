"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one part of the oracle to an independent fact: a hand-derived
worked example, a library routine that a special case reduces to (fp64
matmul, scaled_dot_product_attention, logsumexp, torch's dtype decoders),
brute force on tiny inputs, or an invariant the method must satisfy.  They are
chosen so that a dropped term, a wrong sign or index, or a transposed operand
anywhere in the oracle fails at least one of them.
"""
import copy
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightningindexer_amd.inputs import Workload, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ formats

def test_bf16_decoder_all_codes():
    codes = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = O.dequant(codes.reshape(-1, 1), "bf16")[:, 0]
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e4m3_decoder_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([O.e4m3_to_f64(int(c)) for c in codes])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.nanmax(np.abs(got)) == 448.0


def test_e8m0_decoder_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([O.e8m0_to_f64(int(c)) for c in codes])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


# ------------------------------------------------------- hand worked example

def _golden_workload(top_k):
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    T = 4
    k = np.zeros((2, 64, 2), np.float32)
    k[0, :T] = g["k_idx"]
    kv = np.zeros((2, 64, 2), np.float32)
    kv[0, :T] = g["kv"]
    wl = Workload(cfg={}, batch=1, n_q=T, H_I=2, d_I=2, H=1, d_qk=2, d_v=1, top_k=top_k,
                  sm_scale=1.0, seq_lens=np.array([T], np.int32),
                  block_table=np.array([[0, 1]], np.int32), num_blocks=2,
                  idx_dtype="f32", kv_dtype="f32", q_dtype="f32", out_dtype="f32",
                  q_idx=np.array(g["q_idx"], np.float32), q_idx_scale=None,
                  head_w=np.array(g["head_w"], np.float32), k_pool=k, k_scale=None,
                  q=np.array(g["q"], np.float32), kv_pool=kv, kv_scale=None)
    return wl, g


def test_worked_example_scores_and_indices():
    wl, g = _golden_workload(2)
    sc = O.indexer_scores(wl)
    for t, row in enumerate(g["scores"]):
        assert np.array_equal(sc[t, :t + 1], np.array(row, np.float64)), t
        assert np.isnan(sc[t, t + 1:]).all()
    assert O.topk(sc, wl.row_lens(), 2).tolist() == g["indices_top2"]
    assert O.topk(sc, wl.row_lens(), 1).tolist() == g["indices_top1"]


def test_worked_example_attention():
    wl, g = _golden_workload(2)
    out, lse = O.sparse_attn(wl, np.array(g["indices_top2"], np.int32))
    # q holds rounded ln values in fp32, so allow the float32 rounding of q
    np.testing.assert_allclose(out, np.array(g["out_top2"]), rtol=1e-6, atol=0)
    np.testing.assert_allclose(lse, np.array(g["lse_top2"]), rtol=1e-6, atol=0)


# ------------------------------------------------------------ indexer pins

def _f64(a, dtype):
    """Library decoding of a storage array to float64 (torch's own conversions)."""
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double().numpy()
    if dtype in ("e4m3", "mxfp8", "e4m3_128"):
        return torch.from_numpy(a).view(torch.float8_e4m3fn).double().numpy()
    raise ValueError(dtype)


def _scales_f64(sc, per: int, width: int):
    """Per-element float64 factors of a scale array [..., groups]: E8M0 bytes (torch's
    float8_e8m0fnu) or fp32; group g covers elements [g*per, (g+1)*per), cut at `width`."""
    if sc.dtype == np.uint8:
        f = torch.from_numpy(np.ascontiguousarray(sc)).view(torch.float8_e8m0fnu).double().numpy()
    else:
        f = sc.astype(np.float64)
    return np.repeat(f, per, axis=-1)[..., :width]


def _logical(pool, wl, b, L):
    """Logical rows 0..L-1 of sequence b gathered through the block table."""
    s = np.arange(L)
    return pool.reshape(-1, *pool.shape[2:])[wl.block_table[b, s // 64].astype(np.int64) * 64 + s % 64]


@pytest.mark.parametrize("cfg", [1, 2, 5, 6])
def test_indexer_one_hot_head_weight_is_relu_matmul(cfg):
    """w = e_j reduces the score to relu(q_j . K^T): one fp64 library matmul."""
    wl = make_workload(cfg, batch=2, n_q=3, lens=[150, 77]) if cfg != 1 else make_workload(1)
    rng = np.random.default_rng(7)
    for j in rng.choice(wl.H_I, size=min(3, wl.H_I), replace=False):
        w2 = copy.copy(wl)
        w2.head_w = np.zeros_like(wl.head_w)
        w2.head_w[:, j] = 1.0
        sc = O.indexer_scores(w2)
        for r in range(wl.rows):
            b = r // wl.n_q
            L = int(wl.row_lens()[r])
            K = _f64(_logical(wl.k_pool, wl, b, L), wl.idx_dtype)
            q = _f64(wl.q_idx[r, j], wl.idx_dtype)
            if wl.idx_dtype == "e4m3":  # one fp32 factor per 128-element vector
                q = q * np.float64(wl.q_idx_scale[r, j])
                kr = _logical(wl.k_scale[..., None], wl, b, L)[:, 0].astype(np.float64)
                K = K * kr[:, None]
            elif wl.idx_dtype == "mxfp8":  # one E8M0 factor per 32 elements
                q = q * _scales_f64(wl.q_idx_scale[r, j], 32, wl.d_I)
                K = K * _scales_f64(_logical(wl.k_scale, wl, b, L), 32, wl.d_I)
            ref = np.maximum(K @ q, 0.0)
            # forward error bound of an fp64 dot product of length d: gamma_d * sum |q_c k_c|
            bound = 2 * wl.d_I * 2.0 ** -53 * (np.abs(K) @ np.abs(q))
            assert (np.abs(sc[r, :L] - ref) <= bound).all()
            assert np.isnan(sc[r, L:]).all()


def test_indexer_head_weights_combine_linearly():
    """I(w1 + w2) = I(w1) + I(w2) and I(-w) = -I(w): the weighting is linear in w."""
    wl = make_workload(1)
    w2 = copy.copy(wl)
    rng = np.random.default_rng(3)
    a = rng.standard_normal(wl.head_w.shape).astype(np.float32)
    b = rng.standard_normal(wl.head_w.shape).astype(np.float32)
    w2.head_w = a
    Ia = O.indexer_scores(w2)
    w2.head_w = b
    Ib = O.indexer_scores(w2)
    w2.head_w = (a.astype(np.float64) + b).astype(np.float32)
    Iab = O.indexer_scores(w2)
    ok = ~np.isnan(Ia)
    ab_exact = (a.astype(np.float64) + b) == w2.head_w  # fp32 sum was exact
    rows = ab_exact.all(axis=1)
    np.testing.assert_allclose(Iab[rows][ok[rows]], (Ia + Ib)[rows][ok[rows]], rtol=1e-9, atol=1e-12)
    w2.head_w = -a
    np.testing.assert_array_equal(O.indexer_scores(w2)[ok], -Ia[ok])


def test_indexer_zero_query_gives_zero():
    wl = make_workload(1)
    w2 = copy.copy(wl)
    w2.q_idx = np.zeros_like(wl.q_idx)
    sc = O.indexer_scores(w2)
    L = wl.row_lens()
    for r in range(wl.rows):
        assert (sc[r, :L[r]] == 0).all()


def test_indexer_causal_mask_and_paging_invariance():
    wl = make_workload(2, batch=3, n_q=2, lens=[130, 64, 200], poison=True)
    sc = O.indexer_scores(wl)
    L = wl.row_lens()
    assert L.tolist() == [129, 130, 63, 64, 199, 200]   # query i of n_q sees L_b - n_q + i + 1
    for r in range(wl.rows):
        assert np.isfinite(sc[r, :L[r]]).all() and np.isnan(sc[r, L[r]:]).all()
    # identical logical data under a different (identity-like) block table
    w2 = copy.copy(wl)
    nb = wl.num_blocks
    newperm = np.random.default_rng(11).permutation(nb - 1)
    pool_k = np.full_like(wl.k_pool, 0x7FC0)
    table = wl.block_table.copy()
    for b in range(wl.batch):
        nblk = (int(wl.seq_lens[b]) + 63) // 64
        for j in range(nblk):
            old = wl.block_table[b, j]
            new = newperm[old]
            pool_k[new] = wl.k_pool[old]
            table[b, j] = new
    w2.k_pool, w2.block_table = pool_k, table
    assert np.array_equal(O.indexer_scores(w2), sc, equal_nan=True)


def test_indexer_later_positions_do_not_leak_into_earlier_rows():
    wl = make_workload(1)
    sc = O.indexer_scores(wl)
    w2 = copy.copy(wl)
    kp = wl.k_pool.copy().reshape(-1, wl.d_I)
    kp[200:] = np.random.default_rng(5).standard_normal(kp[200:].shape)
    w2.k_pool = kp.reshape(wl.k_pool.shape)
    sc2 = O.indexer_scores(w2)
    assert np.array_equal(sc2[:200], sc[:200], equal_nan=True)
    assert not np.array_equal(sc2[200:], sc[200:], equal_nan=True)


# -------------------------------------------------------------- top-k pins

def _topk_brute(vals, k):
    """Position p is kept iff fewer than k positions beat it, where q beats p when
    its score is larger, or equal with a lower position (then sorted ascending)."""
    L = len(vals)
    keep = []
    for p in range(L):
        beaten_by = sum(1 for q in range(L) if vals[q] > vals[p] or (vals[q] == vals[p] and q < p))
        if beaten_by < k:
            keep.append(p)
    return keep + [-1] * (k - len(keep))


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n_rows, ld, k = 12, 40, 9
    sc = rng.integers(-3, 4, size=(n_rows, ld)).astype(np.float64)
    sc[rng.random(sc.shape) < 0.2] = -0.0
    L = rng.integers(0, ld + 1, size=n_rows)
    L[0], L[1] = k, k - 1
    got = O.topk(sc, L, k)
    for i in range(n_rows):
        assert got[i].tolist() == _topk_brute(sc[i, :L[i]].tolist(), k), (i, L[i])


def test_topk_all_equal_scores_pick_lowest_positions():
    sc = np.full((3, 100), 0.25)
    got = O.topk(sc, [100, 50, 5], 10)
    assert got[0].tolist() == list(range(10))
    assert got[1].tolist() == list(range(10))
    assert got[2].tolist() == list(range(5)) + [-1] * 5


def test_topk_negative_zero_equals_positive_zero():
    sc = np.array([[-1.0, -0.0, 0.0, -0.0, -2.0]])
    assert O.topk(sc, [5], 2).tolist() == [[1, 2]]


def test_topk_duplicate_key_rows_straddling_the_cut():
    """Two positions with identical K_I rows score identically: the lower one wins the last slot."""
    wl = make_workload(1)
    w2 = copy.copy(wl)
    kp = wl.k_pool.copy().reshape(-1, wl.d_I)
    r = 255
    sc = O.indexer_scores(wl)[r]
    order = np.lexsort((np.arange(256), -sc[:256]))
    kth, nxt = order[wl.top_k - 1], order[wl.top_k]   # in, out
    lo, hi = min(kth, nxt), max(kth, nxt)
    kp[hi] = kp[lo]
    w2.k_pool = kp.reshape(wl.k_pool.shape)
    sc2 = O.indexer_scores(w2)
    idx = O.topk(sc2, w2.row_lens(), wl.top_k)[r]
    assert sc2[r, lo] == sc2[r, hi]
    assert lo in idx.tolist()


# --------------------------------------------------------- attention pins

def _sdpa_ref(wl, rows):
    """Dense causal attention from torch's scaled_dot_product_attention in fp64, K = kv,
    V = kv[..., :d_v], one shared latent row per position for all heads; lse from
    torch.logsumexp over the masked logits."""
    outs, lses = [], []
    for r in rows:
        b, i = r // wl.n_q, r % wl.n_q
        Lb = int(wl.seq_lens[b])
        kv = _f64(_logical(wl.kv_pool, wl, b, Lb), wl.kv_dtype)
        if wl.kv_scale is not None:  # E8M0 per 32, or fp32 per 128 (five groups of a 576 row)
            kv = kv * _scales_f64(_logical(wl.kv_scale, wl, b, Lb), 32 if wl.kv_dtype == "mxfp8" else 128,
                                  wl.d_qk)
        q = torch.from_numpy(_f64(wl.q[r], wl.q_dtype))[None, :, None, :]   # [1,H,1,d]
        K = torch.from_numpy(kv)[None, None].expand(1, wl.H, Lb, wl.d_qk)
        V = torch.from_numpy(np.ascontiguousarray(kv[:, :wl.d_v]))[None, None].expand(1, wl.H, Lb, wl.d_v)
        qpos = Lb - wl.n_q + i                     # absolute position of this query token
        mask = torch.arange(Lb)[None, :] <= qpos   # textbook causal mask
        o = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=wl.sm_scale)
        logits = (q[0, :, 0, :] @ torch.from_numpy(kv).T) * wl.sm_scale   # [H, Lb]
        logits = logits.masked_fill(~mask, float("-inf"))
        outs.append(o[0, :, 0, :].numpy())
        lses.append(torch.logsumexp(logits, dim=-1).numpy())
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("cfg,kw", [
    (1, {}),
    (2, dict(batch=2, n_q=1, lens=[70, 129])),
    (4, dict(batch=2, n_q=2, lens=[66, 130])),
    (5, dict(batch=2, n_q=1, lens=[100, 65])),
    (6, dict(batch=2, n_q=1, lens=[100, 65])),
])
def test_sparse_equals_dense_sdpa_when_topk_covers_history(cfg, kw):
    wl = make_workload(cfg, **kw)
    wl.top_k = int(wl.row_lens().max())
    idx = np.full((wl.rows, wl.top_k), -1, np.int32)
    perm_rng = np.random.default_rng(1)
    for r, L in enumerate(wl.row_lens()):
        idx[r, :L] = perm_rng.permutation(L)   # any order: only the set matters
    rows = list(range(wl.rows)) if wl.rows <= 8 else [0, 1, 63, 127, 200, 255]
    out, lse = O.sparse_attn(wl, idx, rows)
    ref_o, ref_l = _sdpa_ref(wl, rows)
    np.testing.assert_allclose(out, ref_o, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(lse, ref_l, rtol=1e-12, atol=0)
    dout, dlse = O.dense_attn(wl, rows)
    np.testing.assert_allclose(dout, ref_o, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dlse, ref_l, rtol=1e-12, atol=0)


def test_sharp_softmax_equals_sdpa():
    wl = make_workload(1)
    wl.q = (wl.q * 30).astype(np.float32)
    rows = [5, 64, 130, 255]
    wl.top_k = 256
    idx = np.full((wl.rows, 256), -1, np.int32)
    for r, L in enumerate(wl.row_lens()):
        idx[r, :L] = np.arange(L)
    out, lse = O.sparse_attn(wl, idx, rows)
    ref_o, ref_l = _sdpa_ref(wl, rows)
    np.testing.assert_allclose(out, ref_o, rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(lse, ref_l, rtol=1e-12)


def test_single_index_returns_that_value_row():
    wl = make_workload(2, batch=2, n_q=1, lens=[90, 300])
    idx = np.full((2, 16), -1, np.int32)
    idx[0, 3], idx[1, 0] = 17, 299
    out, lse = O.sparse_attn(wl, idx)
    for r, s in ((0, 17), (1, 299)):
        v = _f64(_logical(wl.kv_pool, wl, r, s + 1)[s], "bf16")
        assert np.array_equal(out[r], np.broadcast_to(v[:wl.d_v], out[r].shape))
        q = _f64(wl.q[r], "bf16")
        np.testing.assert_allclose(lse[r], (q @ v) * wl.sm_scale, rtol=1e-12)


def test_zero_query_gives_mean_of_selected_values():
    wl = make_workload(1)
    wl.q = np.zeros_like(wl.q)
    sel = [3, 40, 41, 200]
    idx = np.full((wl.rows, 8), -1, np.int32)
    idx[255, :4] = sel
    out, lse = O.sparse_attn(wl, idx, [255])
    v = _logical(wl.kv_pool, wl, 0, 256)[sel, :wl.d_v].astype(np.float64)
    np.testing.assert_allclose(out[0], np.broadcast_to(v.mean(0), out[0].shape), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(lse[0], math.log(4), rtol=1e-14)


def test_invalid_indices_are_skipped_and_empty_rows_are_zero():
    wl = make_workload(1)
    idx = np.full((wl.rows, 6), -1, np.int32)
    idx[10] = [2, -1, 11, 4000, 3, -7]       # 11 >= L_10 = 11 is outside the history
    idx[20, :] = -1                           # nothing to attend
    out, lse = O.sparse_attn(wl, idx, [10, 20])
    ref, rl = O.sparse_attn(wl, np.array([[2, 3]] * wl.rows, np.int32), [10])
    np.testing.assert_array_equal(out[0], ref[0])
    np.testing.assert_array_equal(lse[0], rl[0])
    assert (out[1] == 0).all() and np.isneginf(lse[1]).all()


def test_attention_depends_only_on_the_index_set():
    wl = make_workload(2, batch=1, n_q=1, lens=[500])
    rng = np.random.default_rng(2)
    sel = np.sort(rng.choice(500, 100, replace=False)).astype(np.int32)
    a, la = O.sparse_attn(wl, sel[None])
    b, lb = O.sparse_attn(wl, rng.permutation(sel)[None])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(la, lb, rtol=1e-14)


def test_mxfp8_cache_equals_its_dequantized_fp32_copy():
    """MXFP8 dequantization is exact in fp32, so the oracle on codes+scales must equal the
    oracle on the fp32 values that torch decodes (code * 2^(byte-127))."""
    wl = make_workload(5, batch=2, n_q=1, lens=[200, 97])
    codes = torch.from_numpy(wl.kv_pool).view(torch.float8_e4m3fn).float()
    scl = torch.from_numpy(wl.kv_scale).view(torch.float8_e8m0fnu).float()
    deq = (codes * scl.repeat_interleave(32, dim=-1)).numpy()
    w2 = copy.copy(wl)
    w2.kv_pool, w2.kv_scale, w2.kv_dtype = deq, None, "f32"
    idx = np.stack([np.arange(150), np.r_[np.arange(97), -np.ones(53)]]).astype(np.int32)
    a, la = O.sparse_attn(wl, idx)
    b, lb = O.sparse_attn(w2, idx)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_fp32_per_128_cache_dequantizes_with_a_short_last_group():
    """A 576 row with one fp32 factor per 128 channels has five groups, the last covering
    the 64 rope channels: the oracle's decoding equals torch's e4m3 decode times the
    factor of group c // 128, exactly (both in float64)."""
    wl = make_workload(6, batch=2, n_q=1, lens=[70, 64])
    assert wl.kv_scale.shape[-1] == 5 and wl.kv_scale.dtype == np.float32
    codes = wl.kv_pool.reshape(-1, wl.d_qk)[:200]
    scl = wl.kv_scale.reshape(-1, 5)[:200]
    got = O.dequant(codes, "e4m3", scl, "f32", 128)
    ref = _f64(codes, "e4m3") * np.repeat(scl.astype(np.float64), 128, axis=-1)[:, :576]
    assert np.array_equal(got, ref)
    assert not np.array_equal(got[:, 512:], _f64(codes, "e4m3")[:, 512:] * scl[:, 3:4])  # group 4 is its own


def test_quantized_inputs_round_trip_within_e4m3_rounding():
    """Codes times scales reproduce the values, clamped to +-448 times their scale, within
    half an e4m3 step (2^-4 relative for normals, 2^-10 times the scale below), for both
    scale formats of workload 6.  (The MX rule e = floor(log2 amax) - 8 puts amax/2^e in
    [256, 512), so the largest values of a group can saturate at 448.)"""
    from sparse_attention_lightningindexer_amd.inputs import quantize_e4m3_f32scale, quantize_mxfp8
    x = np.random.default_rng(3).standard_normal((64, 576)).astype(np.float32) / 24
    for codes, scl, kind, group in [(*quantize_e4m3_f32scale(x, 128), "f32", 128),
                                    (*quantize_mxfp8(x, 32), "e8m0", 32)]:
        deq = O.dequant(codes, "e4m3", scl, kind, group)
        f = _scales_f64(scl, group, 576)
        xc = np.clip(x.astype(np.float64), -448 * f, 448 * f)
        err = np.abs(deq - xc)
        assert (err <= np.maximum(np.abs(xc) * 2.0 ** -4, f * 2.0 ** -10) * (1 + 1e-12)).all()
        if kind == "f32":  # amax/448 scales never saturate (up to the rounding of the division)
            assert (np.abs(x) <= 448 * f * (1 + 2.0 ** -20)).all()


def test_forward_with_full_topk_is_dense_attention():
    """End to end: when top_k covers every history, selection keeps everything."""
    wl = make_workload(1)
    wl.top_k = 256
    sc, idx, out, lse = O.forward(wl)
    L = wl.row_lens()
    for r in (0, 17, 255):
        assert idx[r, :L[r]].tolist() == list(range(L[r]))
    dout, dlse = O.dense_attn(wl)
    np.testing.assert_allclose(out, dout, rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------ cache append pins

def test_e4m3_encoder_matches_torch_conversion():
    """The oracle's e4m3 encoder (written from the format's definition) against torch's
    float8_e4m3fn conversion: random magnitudes over the whole range, every code, every
    midpoint between neighbouring codes (the ties) and the subnormals."""
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.standard_normal(20000).astype(np.float32) * s for s in (1e-3, 0.05, 1, 30, 300)])
    codes = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()
    fin = np.sort(codes[np.isfinite(codes)])
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    vals = np.clip(np.concatenate([vals, fin, mids, -mids, np.float32([2.0 ** -10, 3 * 2.0 ** -10, -0.0])]),
                   -448, 448)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.f32_to_e4m3(v) for v in vals], np.uint8)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", ["e4m3_128", "mxfp8"])
def test_cache_append_quantizes_like_the_input_generator(fmt):
    """The oracle's append (C, fp32 decisions) and the seeded input generator's quantizers
    (numpy + torch) are independent implementations of one rule: the appended rows must
    hold the same codes and scales, bit for bit, and every other pool row stays unchanged."""
    from sparse_attention_lightningindexer_amd.inputs import quantize_e4m3_f32scale, quantize_mxfp8
    wl = make_workload(2, batch=3, n_q=2, lens=[300, 130, 65])
    x = (np.random.default_rng(5).standard_normal((wl.rows, 576)).astype(np.float32) / 24)
    xb = torch.from_numpy(x).to(torch.bfloat16)                          # bf16 inputs
    x = xb.float().numpy()
    nrows = wl.num_blocks * 64
    pool = np.zeros((nrows, 576), np.uint8)
    scl = np.zeros((nrows, 5), np.float32) if fmt == "e4m3_128" else np.zeros((nrows, 18), np.uint8)
    O.cache_append(wl, xb.view(torch.int16).numpy().view(np.uint16), fmt, pool, scl)
    codes, sref = quantize_e4m3_f32scale(x, 128) if fmt == "e4m3_128" else quantize_mxfp8(x, 32)
    touched = np.zeros(nrows, bool)
    for r in range(wl.rows):
        b = r // wl.n_q
        s = int(wl.row_lens()[r]) - 1
        pr = int(wl.block_table[b, s // 64]) * 64 + s % 64
        assert np.array_equal(pool[pr], codes[r]) and np.array_equal(scl[pr], sref[r])
        touched[pr] = True
    assert not pool[~touched].any() and not scl[~touched].any()


def test_cache_append_bf16_pool_copies_every_code():
    """A bf16 pool takes bf16 rows and stores their codes unchanged: every one of the
    65536 bf16 codes (NaN payloads, signalling and quiet, both infinities, -0 and the
    subnormals included) lands at its row's pool position, and nothing else is
    written; an fp32 pool copies fp32 rows, NaN payloads included."""
    wl = make_workload(2, batch=2, n_q=128, lens=[300, 700])  # 256 rows
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(wl.rows, 256)
    nrows = wl.num_blocks * 64
    pool = np.full((nrows, 256), 0x1234, np.uint16)
    O.cache_append(wl, codes, "bf16", pool, None)
    touched = np.zeros(nrows, bool)
    for r in range(wl.rows):
        b, s = r // wl.n_q, int(wl.row_lens()[r]) - 1
        pr = int(wl.block_table[b, s // 64]) * 64 + s % 64
        assert np.array_equal(pool[pr], codes[r])
        touched[pr] = True
    assert (pool[~touched] == 0x1234).all()
    # fp32: quiet and signalling NaN payloads and infinities survive the copy
    bits = np.array([0x7F800001, 0xFF800001, 0x7FC00000, 0x7FFFFFFF, 0x7F800000, 0xFF800000, 0x00000001,
                     0x80000000], np.uint32)
    x = np.tile(bits, (wl.rows, 32)).view(np.float32)
    pool32 = np.zeros((nrows, 256), np.float32)
    O.cache_append(wl, x, "f32", pool32, None)
    s0 = int(wl.row_lens()[0]) - 1                      # row 0's own position
    pr = int(wl.block_table[0, s0 // 64]) * 64 + s0 % 64
    assert np.array_equal(pool32[pr].view(np.uint32), np.tile(bits, 32))


def test_cache_append_rejects_unsupported_pairings():
    """The append takes fp32 rows into an fp32 pool and bf16 rows into every other pool."""
    wl = make_workload(2, batch=1, lens=[10])
    pool = np.zeros((wl.num_blocks * 64, 8), np.uint16)
    with pytest.raises(AssertionError):
        O.cache_append(wl, np.zeros((1, 8), np.float32), "bf16", pool, None)


# ------------------------------------------------------------ indexer prolog pins

def _bf16_f64(bits):
    """torch's bf16 decoder, independent of the oracle's."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def test_vector_e4m3_encoder_matches_torch_conversion():
    rng = np.random.default_rng(3)
    vals = np.clip(np.concatenate([rng.standard_normal(50000).astype(np.float32) * s for s in (0.01, 1, 100)]),
                   -448, 448)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(vals), ref)


def test_prolog_projections_match_fp64_matmul():
    """q and the head weights are fp64 matrix products of the decoded bf16 operands
    (numpy's matmul on torch-decoded values); q's channel n of the flat projection is
    head n // d_I, channel n % d_I."""
    from sparse_attention_lightningindexer_amd.inputs import make_prolog
    p = make_prolog(5, d_x=256, H_I=4, d_I=32, seed=11)
    q, hw, _ = O.indexer_prolog(p)
    x = _bf16_f64(p.x)
    qref = (x @ _bf16_f64(p.w_q).T).reshape(5, 4, 32)
    href = x @ _bf16_f64(p.w_h).T
    np.testing.assert_allclose(q, qref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hw, href, rtol=1e-12, atol=1e-14)


def test_prolog_one_hot_hidden_state_selects_weight_columns():
    """A hidden state that is the unit vector e_c projects to column c of each weight
    matrix, exactly."""
    from sparse_attention_lightningindexer_amd.inputs import make_prolog
    p = make_prolog(3, d_x=128, H_I=2, d_I=64, seed=12)
    cols = [0, 77, 127]
    p.x[:] = 0
    for r, c in enumerate(cols):
        p.x[r, c] = np.uint16(0x3F80)       # bf16 1.0
    q, hw, _ = O.indexer_prolog(p)
    wq, wh = _bf16_f64(p.w_q), _bf16_f64(p.w_h)
    for r, c in enumerate(cols):
        assert np.array_equal(q[r].reshape(-1), wq[:, c])
        assert np.array_equal(hw[r], wh[:, c])


def test_prolog_rmsnorm_worked_example():
    """k = (3, 4), gain (1, 2): the mean square is 12.5, so k_norm = (3, 8)/sqrt(12.5 + eps):
    (0.848528137423857, 2.262741699796952) at eps = 0 and
    (0.8320502943378437, 2.2188007849009166) at eps = 0.5."""
    from sparse_attention_lightningindexer_amd.inputs import make_prolog
    for eps, want in ((0.0, (0.848528137423857, 2.262741699796952)),
                      (0.5, (0.8320502943378437, 2.2188007849009166))):
        p = make_prolog(1, d_x=128, H_I=1, d_I=2, seed=13, eps=eps)
        p.k[0] = np.array([0x4040, 0x4080], np.uint16)      # bf16 3.0, 4.0
        p.gain[:] = (1.0, 2.0)
        _, _, kn = O.indexer_prolog(p)
        np.testing.assert_allclose(kn[0], want, rtol=1e-14)


def test_prolog_rmsnorm_invariants():
    """With gain 1: the output's mean square is ms/(ms + eps) (1 at eps = 0); doubling k
    (exact in bf16) or flipping its sign scales nothing but the sign; the gain multiplies
    channelwise."""
    from sparse_attention_lightningindexer_amd.inputs import make_prolog
    p = make_prolog(6, d_x=128, H_I=1, d_I=128, seed=14, eps=0.0)
    g = p.gain.copy()
    p.gain[:] = 1.0
    _, _, kn = O.indexer_prolog(p)
    np.testing.assert_allclose((kn ** 2).mean(axis=1), 1.0, rtol=1e-13)
    k = _bf16_f64(p.k)
    p2 = copy.deepcopy(p)
    p2.k = (p.k.astype(np.uint32) + (1 << 7)).astype(np.uint16)   # exponent + 1: k * 2
    p2.k[p.k & 0x7F80 == 0] = p.k[p.k & 0x7F80 == 0]               # leave zeros/subnormals alone
    assert np.array_equal(_bf16_f64(p2.k)[k != 0], 2 * k[k != 0])
    _, _, kn2 = O.indexer_prolog(p2)
    np.testing.assert_allclose(kn2, kn, rtol=1e-14, atol=1e-300)
    p3 = copy.deepcopy(p)
    p3.k = p.k ^ np.uint16(0x8000)
    _, _, kn3 = O.indexer_prolog(p3)
    assert np.array_equal(kn3, -kn)
    p4 = copy.deepcopy(p)
    p4.gain[:] = g
    _, _, kn4 = O.indexer_prolog(p4)
    np.testing.assert_allclose(kn4, kn * g.astype(np.float64), rtol=1e-14)
    p5 = copy.deepcopy(p)
    p5.eps = 0.25
    _, _, kn5 = O.indexer_prolog(p5)
    ms = (k ** 2).mean(axis=1)
    np.testing.assert_allclose((kn5 ** 2).mean(axis=1), ms / (ms + 0.25), rtol=1e-13)
