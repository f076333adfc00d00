"""The seeded input generator (CPU only): determinism, paging, quantizers."""
import numpy as np
import torch

from sparse_attention_lightningindexer_amd.inputs import (CONFIGS, make_workload,
                                                          quantize_e4m3_f32scale, quantize_mxfp8)


def test_same_seed_same_inputs_and_rotation_changes_them():
    a = make_workload(2, batch=3, lens=[100, 64, 1])
    b = make_workload(2, batch=3, lens=[100, 64, 1])
    c = make_workload(2, batch=3, lens=[100, 64, 1], rotation=1)
    for f in ("q_idx", "head_w", "k_pool", "q", "kv_pool", "block_table"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert not np.array_equal(a.q, c.q)


def test_paging_scatter_then_gather_is_identity():
    """The permuted pool holds, through the table, exactly the identity-paged logical rows."""
    p = make_workload(4, batch=2, lens=[300, 129])
    i = make_workload(4, batch=2, lens=[300, 129], paging="identity")
    for b in range(2):
        L = int(p.seq_lens[b])
        s = np.arange(L)
        def rows(w, pool):
            return pool.reshape(-1, pool.shape[-1])[w.block_table[b, s // 64].astype(np.int64) * 64 + s % 64]
        assert np.array_equal(rows(p, p.kv_pool), rows(i, i.kv_pool))
        assert np.array_equal(rows(p, p.k_pool), rows(i, i.k_pool))
    assert sorted(p.block_table[p.block_table != p.num_blocks - 1].tolist()) == list(range(p.num_blocks - 1))


def test_poison_marks_exactly_the_unused_slots():
    w = make_workload(2, batch=2, lens=[70, 64], poison=True)
    k = torch.from_numpy(w.k_pool.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan_rows = np.isnan(k).all(axis=-1).reshape(-1)
    assert nan_rows.sum() == w.num_blocks * 64 - (70 + 64)
    assert not np.isnan(k).any(axis=-1).reshape(-1)[~nan_rows].any()


def test_skewed_lengths_in_range_and_prefill_rows():
    w = make_workload(4)
    assert w.seq_lens.min() >= 4096 and w.seq_lens.max() <= 131072 and w.n_q == 2
    assert w.row_lens()[0] == w.seq_lens[0] - 1 and w.row_lens()[1] == w.seq_lens[0]
    p = make_workload(3, lens=130)
    assert p.n_q == 130 and p.row_lens().tolist() == list(range(1, 131))
    assert CONFIGS[3]["lens"] == 32768


def test_e4m3_blockscale_quantizer_error_bound():
    x = np.random.default_rng(0).standard_normal((50, 256)).astype(np.float32)
    codes, scale = quantize_e4m3_f32scale(x, 128)
    deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy().reshape(50, 2, 128) * scale[..., None]
    err = np.abs(deq.reshape(50, 256) - x)
    # half an e4m3 ulp: 2^-4 relative for normals, plus the subnormal spacing 2^-10 * scale
    bound = np.abs(x) * 2.0 ** -4 + np.repeat(scale, 128, axis=-1) * 2.0 ** -10
    assert (err <= bound + 1e-12).all()
    assert np.isclose(np.abs(deq).reshape(50, 2, 128).max(-1), np.abs(x).reshape(50, 2, 128).max(-1)).all()


def test_mxfp8_quantizer_error_bound_and_scale_rule():
    x = np.random.default_rng(1).standard_normal((40, 576)).astype(np.float32) / 24
    codes, e8 = quantize_mxfp8(x, 32)
    scale = torch.from_numpy(e8).view(torch.float8_e8m0fnu).double().numpy()
    deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy() * np.repeat(scale, 32, -1)
    amax = np.abs(x.reshape(40, 18, 32)).max(-1)
    assert (amax / scale >= 256).all() and (amax / scale < 512).all()   # e = floor(log2 amax) - 8
    bound = np.abs(x) * 2.0 ** -4 + np.repeat(scale, 32, -1) * 2.0 ** -9 + np.maximum(np.abs(x) - 448 * np.repeat(scale, 32, -1), 0)
    assert (np.abs(deq - x) <= bound + 1e-15).all()


def test_prolog_inputs_are_seeded_and_shaped():
    """make_prolog: same seed and rotation give the same bits, another rotation other
    bits; shapes, dtypes and the stated variances (projections with the indexer
    inputs' variances: var(W_q x) = 1/d_I, var(W_h x) = 1/H_I)."""
    from sparse_attention_lightningindexer_amd.inputs import make_prolog
    a, b, c = make_prolog(8, 1024, seed=3), make_prolog(8, 1024, seed=3), make_prolog(8, 1024, seed=3, rotation=1)
    for name in ("x", "w_q", "w_h", "k", "gain"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
        assert not np.array_equal(getattr(a, name), getattr(c, name)), name
    assert a.x.shape == (8, 1024) and a.x.dtype == np.uint16
    assert a.w_q.shape == (64 * 128, 1024) and a.w_h.shape == (64, 1024) and a.k.shape == (8, 128)
    assert a.gain.shape == (128,) and a.gain.dtype == np.float32
    f = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    wq = f(a.w_q)
    assert abs(wq.var() * 1024 * 128 - 1) < 0.02
    assert abs(f(a.x).var() - 1) < 0.05 and abs(a.gain.mean() - 1) < 0.03
