"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on an MI355X.

Small cases span several 64-position tiles, several 32-position attention
chunks and ragged tails, at every kernel's real head counts and widths; the
full workload sizes are checked on sampled rows in the launch configuration
the benchmark times.  Every input is NaN-poisoned outside the histories.
"""
import copy
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_attention_lightningindexer_amd import binding as B
from sparse_attention_lightningindexer_amd.inputs import make_workload

from parity import (check_attention, check_indices_band, check_indices_exact, check_scores, f64,
                    full_indices, gpu_all)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# (config, overrides): lengths chosen to leave ragged 64-tiles and 32-chunks
SMALL = {
    "tiny_fp32": (1, dict(poison=True)),
    "decode_bf16": (2, dict(batch=3, lens=[300, 1000, 453], top_k=128, poison=True)),
    "decode_bf16_dense": (2, dict(batch=2, lens=[200, 77], top_k=256, poison=True)),
    "skewed_nq2": (4, dict(batch=3, lens=[700, 1500, 1], top_k=256, poison=True)),
    "fp8_decode": (5, dict(batch=3, lens=[500, 900, 130], top_k=256, poison=True)),
    "fp8_pages_decode": (6, dict(batch=3, lens=[500, 900, 130], top_k=256, poison=True)),
    "fp8_pages_nq2": (6, dict(batch=2, n_q=2, lens=[700, 66], top_k=256, poison=True)),
    "prefill_bf16": (3, dict(lens=333, top_k=96, poison=True)),
    # several query tokens per sequence with batch > 1: the multi-row indexer
    # kernel then spans several sequences, each row with its own causal length
    "nq3_bf16": (2, dict(batch=2, n_q=3, lens=[300, 130], top_k=128, poison=True)),
    "nq4_mxfp8": (6, dict(batch=3, n_q=4, lens=[500, 64, 261], top_k=128, poison=True)),
    "nq8_bf16": (2, dict(batch=2, n_q=8, lens=[1000, 77], top_k=256, poison=True)),
    "nq8_mxfp8": (6, dict(batch=2, n_q=8, lens=[1000, 77], top_k=256, poison=True)),
    # the fp32-per-128 indexer with two query tokens per sequence
    "fp8_nq2": (5, dict(batch=3, n_q=2, lens=[700, 66, 1500], top_k=256, poison=True)),
    # chunked prefill: 100 new tokens on top of a longer history, and a sequence
    # shorter than the chunk (its first rows see nothing)
    "chunked_prefill_nq100": (2, dict(batch=2, n_q=100, lens=[700, 60], top_k=128, poison=True)),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_small_all_stages_match_oracle(case):
    cfg, kw = SMALL[case]
    say(f"[parity] {case}: cfg {cfg} {kw}")
    wl = make_workload(cfg, **kw)
    dev, sc, idx, out, lse = gpu_all(wl)
    rows = list(range(wl.rows))
    ref_sc = O.indexer_scores(wl, rows, ld=sc.shape[1])
    check_scores(wl, sc, ref_sc, rows)
    # Top-K: exact on the GPU's own fp32 scores; within the band on the oracle's
    ref_idx_own = O.topk(sc, wl.row_lens(), wl.top_k)
    check_indices_exact(idx, ref_idx_own)
    ref_idx = O.topk(ref_sc, wl.row_lens(), wl.top_k)
    for r in rows:
        check_indices_band(idx[r], ref_idx[r], ref_sc[r], int(wl.row_lens()[r]), wl.top_k)
    # attention on the GPU's (validated) indices
    ref_o, ref_l = O.sparse_attn(wl, idx)
    check_attention(wl, out, lse, ref_o, ref_l, case)
    # the fused entry point is the same computation, bit for bit
    dev2 = B.DeviceInputs(wl)
    out2, lse2, idx2 = B.dsa_forward(dev2)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), idx)
    assert np.array_equal(f64(out2), out) and np.array_equal(f64(lse2), lse)


@pytest.mark.parametrize("case", ["decode_bf16", "skewed_nq2", "fp8_decode", "nq4_mxfp8"])
def test_identity_and_permuted_paging_give_identical_outputs(case):
    cfg, kw = SMALL[case]
    a = make_workload(cfg, **kw)
    b = make_workload(cfg, paging="identity", **kw)
    _, sa, ia, oa, la = gpu_all(a)
    _, sb, ib, ob, lb = gpu_all(b)
    L = a.row_lens()
    for r in range(a.rows):
        assert np.array_equal(sa[r, :L[r]], sb[r, :L[r]])
    assert np.array_equal(ia, ib) and np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_sparse_attention_with_full_history_equals_dense_attention():
    wl = make_workload(2, batch=2, lens=[150, 700], top_k=1024, poison=True)
    dev = B.DeviceInputs(wl)
    idx = np.full((wl.rows, 1024), -1, np.int32)
    rng = np.random.default_rng(0)
    for r, L in enumerate(wl.row_lens()):
        idx[r, :L] = rng.permutation(L)          # unsorted on purpose
    out, lse = B.dsa_sparse_attn(dev, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    ref_o, ref_l = O.dense_attn(wl)
    check_attention(wl, f64(out), f64(lse), ref_o, ref_l, "dense")


def test_sharp_softmax_and_scattered_invalid_indices():
    wl = make_workload(2, batch=2, lens=[900, 400], top_k=512, poison=True)
    wl.q = (torch.from_numpy(wl.q.view(np.int16)).view(torch.bfloat16).float() * 30).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rng = np.random.default_rng(5)
    idx = rng.integers(-50, 1000, size=(wl.rows, 512)).astype(np.int32)   # includes -ve and >= L
    dev = B.DeviceInputs(wl)
    out, lse = B.dsa_sparse_attn(dev, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    ref_o, ref_l = O.sparse_attn(wl, idx)
    check_attention(wl, f64(out), f64(lse), ref_o, ref_l, "sharp")


def test_empty_histories_and_absent_blocks():
    # n_q = 2 and a sequence of length 1: its first query row sees nothing
    wl = make_workload(4, batch=3, lens=[1, 200, 300], top_k=64, poison=True)
    wl.block_table = wl.block_table.copy()
    wl.block_table[2, 1] = -1                 # positions 64..127 of sequence 2 are absent
    wl.block_table[1, 2] = wl.num_blocks + 5  # out-of-range entry: absent too
    dev, sc, idx, out, lse = gpu_all(wl)
    ref_sc = O.indexer_scores(wl, ld=sc.shape[1])
    L = wl.row_lens()
    assert L[0] == 0 and (idx[0] == -1).all()
    for r in range(wl.rows):
        assert np.array_equal(np.isneginf(sc[r, :L[r]]), np.isneginf(ref_sc[r, :L[r]]))
    ref_o, ref_l = O.sparse_attn(wl, idx)
    check_attention(wl, out, lse, ref_o, ref_l, "absent")
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()


def test_forward_with_the_topk_in_the_attention_at_256_rows():
    # 256 rows (64 sequences x 4 query tokens), the most the fused form takes:
    # one split per row, so each workgroup keeps all top_k places and its
    # head-half-0 workgroup writes the whole index row.
    wl = make_workload(2, batch=64, n_q=4, lens=[3000 + 37 * b for b in range(64)], top_k=2048)
    _, sc, idx, out, lse = gpu_all(wl)
    dev = B.DeviceInputs(wl)
    say("[parity] fused Top-K forward, 256 rows")
    out2, lse2, idx2 = B.dsa_forward(dev)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), idx)
    assert np.array_equal(f64(out2), out) and np.array_equal(f64(lse2), lse)
    check_indices_exact(idx, O.topk(sc, wl.row_lens(), wl.top_k))


@pytest.mark.parametrize("cfg", [2, 6])
def test_forward_with_the_topk_in_the_attention_matches_the_separate_calls(cfg):
    # dsa_forward selects each row's Top-K inside the attention kernel when the
    # rows are at most 8192 positions long and few: histories just below, at
    # and above top_k (the whole history, then a selection), the 8192 limit
    # and none; 22 splits of 96 slots, so every workgroup keeps
    # a narrow range of the row's places.  Indices, outputs and LSEs must equal
    # the three separate calls bit for bit.
    wl = make_workload(cfg, batch=6, lens=[2047, 2048, 2049, 8192, 1, 5000], top_k=2048, poison=True)
    wl.seq_lens = wl.seq_lens.copy()
    wl.seq_lens[4] = 0
    _, sc, idx, out, lse = gpu_all(wl)
    dev = B.DeviceInputs(wl)
    say(f"[parity] fused Top-K forward, cfg {cfg}")
    out2, lse2, idx2 = B.dsa_forward(dev)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), idx)
    assert np.array_equal(f64(out2), out) and np.array_equal(f64(lse2), lse)
    check_indices_exact(idx, O.topk(sc, wl.row_lens(), wl.top_k))
    assert (idx[4] == -1).all() and (idx[0][:2047] == np.arange(2047)).all() and idx[0][2047] == -1


@pytest.mark.parametrize("cfg", [2, 5])
def test_attention_history_too_long_for_the_table_in_lds(cfg):
    # A 470000-position history: 7344 table blocks, more than the 7168 whose
    # block-table row the attention's compaction stages in LDS, so the
    # compaction reads the table from memory per slot.  Logical blocks map
    # onto the 15 full physical blocks of a 1000-position sequence (two absent),
    # which is legal paging and keeps the pool small; the indices reach past
    # position 458752.
    wl = make_workload(cfg, batch=2, lens=[1000, 700], top_k=512, poison=True)
    own = wl.block_table[0, :15]             # the 15 full blocks of sequence 0's 1000 positions
    long_len, nbl = 470000, 7344
    table = np.full((2, nbl), -1, np.int32)
    table[0] = own[np.arange(nbl) % own.size]
    table[0, 7200] = -1                      # an absent block past the LDS window
    table[0, 100] = wl.num_blocks + 3        # an out-of-range entry: absent too
    table[1, :wl.block_table.shape[1]] = wl.block_table[1]
    wl.block_table = table
    wl.seq_lens = np.array([long_len, 700], np.int32)
    rng = np.random.default_rng(11)
    idx = np.full((wl.rows, 512), -1, np.int32)
    far = rng.choice(np.arange(458752, long_len), 200, replace=False)
    near = rng.choice(long_len, 300, replace=False)
    row0 = np.unique(np.concatenate([far, near, [7200 * 64 + 5, 100 * 64 + 1, long_len - 1]]))[:512]
    idx[0, :row0.size] = row0
    idx[1, :300] = np.sort(rng.choice(700, 300, replace=False))
    dev = B.DeviceInputs(wl)
    say(f"[parity] attention over a {long_len}-position history, cfg {cfg}")
    out, lse = B.dsa_sparse_attn(dev, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    ref_o, ref_l = O.sparse_attn(wl, idx)
    check_attention(wl, f64(out), f64(lse), ref_o, ref_l, f"long table cfg {cfg}")


def test_topk_ties_all_equal_scores_and_duplicate_keys():
    wl = make_workload(2, batch=2, lens=[1000, 333], top_k=100)
    dev = B.DeviceInputs(wl)
    scores = torch.zeros((wl.rows, 1000), dtype=torch.float32, device="cuda")
    scores[1] = -0.0                                   # -0 equals +0
    idx = B.dsa_topk(dev, scores).cpu().numpy()
    assert idx[0].tolist() == list(range(100)) and idx[1].tolist() == list(range(100))
    # random small-integer scores with many ties against the oracle, exactly
    rng = np.random.default_rng(1)
    s = rng.integers(-4, 5, size=(wl.rows, 1000)).astype(np.float32)
    idx = B.dsa_topk(dev, torch.from_numpy(s).cuda()).cpu().numpy()
    check_indices_exact(idx, O.topk(s.astype(np.float64), wl.row_lens(), 100))


@pytest.mark.parametrize("top_k", [1, 7, 2048, 4096])
def test_topk_extreme_k_and_long_rows(top_k):
    wl = make_workload(4, batch=2, lens=[131072, 5000], top_k=top_k)
    dev = B.DeviceInputs(wl)
    rng = np.random.default_rng(top_k)
    s = rng.standard_normal((wl.rows, 131072)).astype(np.float32)
    s[:, ::97] = s[:, 3:4]                                # ties across the row
    st = torch.from_numpy(s).cuda()
    idx = B.dsa_topk(dev, st).cpu().numpy()
    check_indices_exact(idx, O.topk(s.astype(np.float64), wl.row_lens(), top_k))


def test_topk_without_workspace_on_rows_beyond_the_segment_merge():
    """Rows whose segment candidates exceed what the merge keeps (9 segments of
    16384 positions x top_k 4096 > 32768) take the selection that re-reads the
    scores from memory; it needs no workspace and matches the oracle exactly."""
    wl = make_workload(4, batch=2, lens=[140000, 5000], top_k=4096)
    dev = B.DeviceInputs(wl)
    assert B.dsa_topk_workspace_bytes(dev) == 0
    rng = np.random.default_rng(140000)
    s = rng.standard_normal((wl.rows, 140000)).astype(np.float32)
    s[:, ::101] = s[:, 7:8]                               # ties across the row
    idx = B.dsa_topk(dev, torch.from_numpy(s).cuda()).cpu().numpy()
    check_indices_exact(idx, O.topk(s.astype(np.float64), wl.row_lens(), 4096))


@pytest.mark.parametrize("long_len,top_k", [(32768, 1), (32768, 2048), (20000, 4096), (16384, 7),
                                             (16384, 2048), (8192, 2047), (8192, 1)])
def test_topk_register_resident_lengths_with_ties(long_len, top_k):
    # rows up to 8192 / 16384 / 32768 positions take the register-resident kernel
    wl = make_workload(4, batch=2, lens=[long_len, long_len // 3 + 5], top_k=top_k)
    dev = B.DeviceInputs(wl)
    rng = np.random.default_rng(long_len + top_k)
    s = rng.standard_normal((wl.rows, long_len)).astype(np.float32)
    s[:, ::89] = s[:, 5:6]                                # ties across the row
    s[:, 1::13] = np.round(s[:, 1::13], 1)                # more ties near the cut
    st = torch.from_numpy(s).cuda()
    idx = B.dsa_topk(dev, st).cpu().numpy()
    check_indices_exact(idx, O.topk(s.astype(np.float64), wl.row_lens(), top_k))


@pytest.mark.parametrize("long_len", [8192, 32768, 100000, 140000])
def test_topk_nan_scores_still_give_valid_index_rows(long_len):
    """NaN scores have no specified order (dsa.h), but every row must still come
    out as k_r distinct ascending positions of its history, and the finite scores
    kept must be the largest finite ones: positive NaNs sort above +inf and
    negative NaNs below -inf, the all-ones NaN included (it shares the lowest
    real key)."""
    # 100000 x 4096: segments and merge; 140000 x 4096: no workspace
    top_k = 2048 if long_len < 100000 else 4096
    wl = make_workload(4, batch=2, lens=[long_len, long_len // 3 + 5], top_k=top_k)
    dev = B.DeviceInputs(wl)
    say(f"[parity] topk NaN rows {long_len}")
    rng = np.random.default_rng(long_len + 11)
    s = rng.standard_normal((wl.rows, long_len)).astype(np.float32)
    bits = s.view(np.uint32)
    bits[:, ::37] = 0x7FC00000                            # quiet NaN
    bits[:, 5::211] = 0xFFFFFFFF                          # the all-ones NaN (key 1)
    bits[:, 9::401] = 0xFF800001                          # negative signalling NaN
    bits[:, 11::503] = 0x7F800001                         # positive signalling NaN
    idx = B.dsa_topk(dev, torch.from_numpy(s).cuda()).cpu().numpy()
    for r, L in enumerate(wl.row_lens()):
        k = min(top_k, int(L))
        row, sel = s[r, :L], idx[r]
        assert (sel[k:] == -1).all(), r
        kept = sel[:k]
        assert (np.diff(kept) > 0).all() and kept[0] >= 0 and kept[-1] < L, r
        nan = np.isnan(row)
        pos_nan = nan & ((row.view(np.uint32) >> 31) == 0)
        # every positive NaN ranks above every finite score, every negative NaN below
        n_pos = int(pos_nan.sum())
        assert n_pos <= k  # by construction of the row
        assert np.isin(np.nonzero(pos_nan)[0], kept).all(), r
        fin_kept = kept[~nan[kept]]
        if n_pos < k and len(fin_kept):
            lo = row[fin_kept].min()
            fin = ~nan
            assert np.isin(np.nonzero(fin & (row > lo))[0], kept).all(), r


# ------------------------------------------------------- full workload sizes

@pytest.mark.parametrize("cfg", [1, 2, 4, 5, 6])
def test_full_size_every_row(cfg):
    """Every workload at its full size, in the launch configuration the benchmark
    times (dsa_forward into a workspace), checked on every row: scores within the
    fp32 bound, indices exact on the GPU's own scores and within the tie band on
    the oracle's fp64 scores, attention within the output tolerance."""
    say(f"[parity] full cfg {cfg}: generating")
    wl = make_workload(cfg)
    dev = B.DeviceInputs(wl)
    say(f"[parity] full cfg {cfg}: forward on GPU")
    ws = torch.empty(max(1, B.dsa_forward_workspace_bytes(dev)), dtype=torch.uint8, device="cuda")
    out, lse, idx = B.dsa_forward(dev, ws=ws)
    torch.cuda.synchronize()
    rows = list(range(wl.rows))
    ld = (wl.max_seq_len + 63) // 64 * 64
    sc_h = ws[: wl.rows * ld * 4].view(torch.float32).view(wl.rows, ld).cpu().numpy().astype(np.float64)
    idx_h = idx.cpu().numpy()
    say(f"[parity] full cfg {cfg}: oracle on all {len(rows)} rows")
    ref_sc = O.indexer_scores(wl, rows, ld=ld)
    check_scores(wl, sc_h, ref_sc, rows)
    check_indices_exact(idx_h, O.topk(sc_h, wl.row_lens(), wl.top_k))
    ref_idx = O.topk(ref_sc, wl.row_lens(), wl.top_k)
    nd = sum(check_indices_band(idx_h[r], ref_idx[r], ref_sc[r], int(wl.row_lens()[r]), wl.top_k) for r in rows)
    say(f"[parity] full cfg {cfg}: {nd} band swaps")
    ref_o, ref_l = O.sparse_attn(wl, idx_h)
    check_attention(wl, f64(out), f64(lse), ref_o, ref_l, f"full cfg {cfg}")


@pytest.mark.parametrize("cfg,batch,L", [(2, 32, 8192), (5, 64, 16384), (6, 64, 16384)])
def test_decode_indexer_long_wave_runs_with_ragged_lengths(cfg, batch, L):
    # One query row per sequence at the decode workloads' sizes, where each
    # indexer wave streams a run of 4 (bf16) or 8 (fp8, MXFP8) tiles.  Lengths
    # step down by 37 per sequence, so histories end inside tiles and inside
    # runs, and with permuted paging every table entry of a run matters.
    lens = [L - 37 * b for b in range(batch)]
    wl = make_workload(cfg, batch=batch, n_q=1, lens=lens, top_k=256, paging="permuted", poison=True)
    dev = B.DeviceInputs(wl)
    say(f"[parity] decode indexer runs, cfg {cfg}, batch {batch}: scores on GPU")
    sc = B.dsa_indexer_scores(dev)
    torch.cuda.synchronize()
    rows = sorted(set(range(0, batch, 5)) | {batch - 1})
    sc_h = sc[rows].cpu().numpy().astype(np.float64)
    ref_sc = O.indexer_scores(wl, rows, ld=sc.shape[1])
    check_scores(wl, sc_h, ref_sc, rows)
    # absent blocks inside a run: those positions score -inf, every other score
    # is unchanged to the bit
    wl2 = copy.copy(wl)
    wl2.block_table = wl.block_table.copy()
    wl2.block_table[0, 37] = -1
    wl2.block_table[5, 100] = wl.num_blocks + 5
    sc2 = B.dsa_indexer_scores(B.DeviceInputs(wl2))
    torch.cuda.synchronize()
    L = wl.row_lens()
    for r, blk in ((0, 37), (5, 100)):
        a, b_ = sc[r, :L[r]].cpu(), sc2[r, :L[r]].cpu()
        gone = torch.zeros(int(L[r]), dtype=torch.bool)
        gone[64 * blk:64 * blk + 64] = True
        assert torch.isneginf(b_[gone]).all(), r
        assert torch.equal(a[~gone].view(torch.int32), b_[~gone].view(torch.int32)), r
    others = [r for r in range(batch) if r not in (0, 5)]
    assert torch.equal(sc[others].view(torch.int32), sc2[others].view(torch.int32))


@pytest.mark.parametrize("cfg", [3, 5, 6])
def test_prefill_permuted_paging_across_table_windows(cfg):
    # 4500 causal rows: the prefill indexer kernel reads the block table in
    # windows of 64 tiles (4096 positions), so rows past 4096 use the second
    # window; permuted paging makes every window entry matter.  cfg 5 runs the
    # same rows with the fp8 indexer and the MXFP8 cache, cfg 6 with the MXFP8
    # indexer and the fp32-per-128 cache.
    wl = make_workload(cfg, batch=1, n_q=4500, lens=4500, top_k=256, paging="permuted", poison=True)
    dev = B.DeviceInputs(wl)
    say(f"[parity] prefill across table windows, cfg {cfg}: forward on GPU")
    out, lse, idx = B.dsa_forward(dev)
    sc = B.dsa_indexer_scores(dev)
    torch.cuda.synchronize()
    rows = [0, 63, 64, 4095, 4096, 4160, 4499]
    sc_h = sc[rows].cpu().numpy().astype(np.float64)
    idx_h = idx.cpu().numpy()
    ref_sc = O.indexer_scores(wl, rows, ld=sc.shape[1])
    check_scores(wl, sc_h, ref_sc, rows)
    check_indices_exact(idx_h[rows], O.topk(sc_h, wl.row_lens()[rows], wl.top_k))
    ref_o, ref_l = O.sparse_attn(wl, idx_h, rows)
    check_attention(wl, f64(out[rows]), f64(lse[rows]), ref_o, ref_l, f"prefill windows cfg {cfg}")


def prefill_check_rows(T, n_spread=200):
    """Rows of the full prefill checked against the oracle: n_spread rows evenly
    spread over the positions, the rows around the top_k boundary (2046..2049) and
    the last 64 rows."""
    return sorted(set(np.linspace(0, T - 1, n_spread).astype(int).tolist()) | {2046, 2047, 2048, 2049}
                  | set(range(T - 64, T)))


def test_full_prefill_rows_spread_over_positions():
    """The full prefill (32768 causal rows) in the benchmark's launch configuration:
    on 260+ rows spread over every position range, the scores are within the fp32
    bound, the indices exact on the GPU's own scores and within the tie band on the
    oracle's fp64 scores, and the attention within tolerance; on every row, the
    index list has k_r = min(2048, t+1) ascending unique positions < t+1."""
    say("[parity] full prefill: generating 32768 x 128 x 576 queries")
    wl = make_workload(3)
    dev = B.DeviceInputs(wl)
    say("[parity] full prefill: forward on GPU")
    ws = torch.empty(B.dsa_forward_workspace_bytes(dev), dtype=torch.uint8, device="cuda")
    out, lse, idx = B.dsa_forward(dev, ws=ws)
    torch.cuda.synchronize()
    rows = prefill_check_rows(wl.rows)
    ld = (wl.max_seq_len + 63) // 64 * 64
    sc_h = ws[: wl.rows * ld * 4].view(torch.float32).view(wl.rows, ld)[rows].cpu().numpy().astype(np.float64)
    idx_h = idx.cpu().numpy()
    say(f"[parity] full prefill: oracle on {len(rows)} rows")
    ref_sc = O.indexer_scores(wl, rows, ld=ld)
    check_scores(wl, sc_h, ref_sc, rows)
    Lr = wl.row_lens()[rows]
    check_indices_exact(idx_h[rows], O.topk(sc_h, Lr, wl.top_k))
    ref_idx = O.topk(ref_sc, Lr, wl.top_k)
    nd = sum(check_indices_band(idx_h[r], ref_idx[i], ref_sc[i], int(Lr[i]), wl.top_k) for i, r in enumerate(rows))
    say(f"[parity] full prefill: {nd} band swaps")
    ref_o, ref_l = O.sparse_attn(wl, idx_h, rows)
    check_attention(wl, f64(out[rows]), f64(lse[rows]), ref_o, ref_l, "full prefill")
    # property at every row: k_r = min(2048, t+1) ascending unique positions < t+1
    L = wl.row_lens()
    k = np.minimum(L, 2048)
    valid = idx_h >= 0
    assert (valid.sum(1) == k).all()
    assert (np.where(valid, idx_h, -1).max(1) < L).all()
    col = np.arange(idx_h.shape[1])[None, :]
    assert np.array_equal(valid, col < k[:, None])           # the k_r positions first, then -1
    inner = (col[:, 1:] < k[:, None])                        # consecutive pairs inside the prefix
    assert (np.diff(idx_h.astype(np.int64), axis=1)[inner] > 0).all()  # strictly ascending
    assert bool(torch.isfinite(out).all())


# (config, overrides): the pool formats of every workload, with n_q 1 and 2
APPEND = {
    "f32": (1, dict(batch=2, n_q=3, lens=[150, 80])),
    "bf16": (2, dict(batch=3, lens=[300, 1000, 453])),
    "fp8_mx_kv": (5, dict(batch=3, lens=[300, 1000, 453])),
    "mx_idx_fp32_kv": (6, dict(batch=2, n_q=2, lens=[700, 66])),
}


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def _append_both(wl, dev, k_new, kv_new):
    """The GPU's append (from device copies of the rows) and the oracle's (on host copies
    of the pools): (gpu pools and scales, oracle pools and scales).  Rows are float32
    for fp32 pools, bf16 bit patterns (uint16) otherwise."""
    def to_dev(a):
        return torch.from_numpy(a).cuda() if a.dtype == np.float32 else torch.from_numpy(a.view(np.int16)).view(
            torch.bfloat16).cuda()
    B.dsa_cache_append(dev, to_dev(k_new), to_dev(kv_new))
    torch.cuda.synchronize()
    kp, kvp = wl.k_pool.copy(), wl.kv_pool.copy()
    ks = None if wl.k_scale is None else wl.k_scale.copy()
    kvs = None if wl.kv_scale is None else wl.kv_scale.copy()
    O.cache_append(wl, k_new, wl.idx_dtype, kp, ks)
    O.cache_append(wl, kv_new, wl.kv_dtype, kvp, kvs)
    return [("k_pool", dev.k_pool, kp), ("kv_pool", dev.kv_pool, kvp), ("k_scale", dev.k_scale, ks),
            ("kv_scale", dev.kv_scale, kvs)]


def _assert_same_bytes(case, pairs):
    for name, got, ref in pairs:
        if ref is None:
            continue
        g = got.cpu().numpy().reshape(ref.shape)
        assert np.array_equal(g.view(np.uint8), np.ascontiguousarray(ref).view(np.uint8)), f"{case}: {name} differs"


@pytest.mark.parametrize("case", list(APPEND))
def test_cache_append_matches_oracle(case):
    """dsa_cache_append on the GPU writes the same pools and scales as the oracle's append
    (bit for bit), and leaves every other pool row as it was."""
    cfg, kw = APPEND[case]
    wl = make_workload(cfg, **kw)
    say(f"[parity] append {case}: cfg {cfg} {kw}")
    dev = B.DeviceInputs(wl)
    rng = np.random.default_rng(11)
    f32 = wl.idx_dtype == "f32"
    k_new = (rng.standard_normal((wl.rows, wl.d_I)) / np.sqrt(wl.d_I)).astype(np.float32)
    kv_new = (rng.standard_normal((wl.rows, wl.d_qk)) / np.sqrt(wl.d_qk)).astype(np.float32)
    if not f32:  # the new rows arrive in bf16
        k_new, kv_new = _bf16_bits(k_new), _bf16_bits(kv_new)
    pairs = _append_both(wl, dev, k_new, kv_new)
    assert not np.array_equal(pairs[1][2], wl.kv_pool)  # the append changed something
    _assert_same_bytes(case, pairs)


@pytest.mark.parametrize("case", ["f32", "bf16"])
def test_cache_append_copies_nan_payloads(case):
    """Unquantized pools are copies: rows of NaN payloads (signalling and quiet, both
    signs), infinities, -0 and subnormals land in the pools bit for bit."""
    cfg, kw = APPEND[case]
    wl = make_workload(cfg, **kw)
    say(f"[parity] append NaN payloads {case}")
    dev = B.DeviceInputs(wl)
    if case == "f32":
        pat = np.array([0x7F800001, 0xFF800001, 0x7FC00000, 0xFFC12345, 0x7FBFFFFF, 0x7F800000, 0xFF800000,
                        0x00000001, 0x80000000, 0x3F800000], np.uint32)
        mk = lambda w: np.resize(pat, (wl.rows, w)).view(np.float32)  # noqa: E731
    else:
        pat = np.array([0x7F81, 0xFF81, 0x7FC0, 0xFFC1, 0x7FBF, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x3F80], np.uint16)
        mk = lambda w: np.ascontiguousarray(np.resize(pat, (wl.rows, w)))  # noqa: E731
    _assert_same_bytes(case, _append_both(wl, dev, mk(wl.d_I), mk(wl.d_qk)))


# (rows, d_x, H_I, d_I, query format): one row and one k stage; ragged row tiles
# of every tile height (16, 32, 64 rows); fewer stages than the LDS ring holds;
# few heads (H_I 4, so few workgroups share out the normalized rows) and heads
# of 32, 64 and 256 channels (four values per lane in the normalization); four
# row tiles; the decode prolog workload (32 rows, d_x 7168) in both formats.
PROLOG = {
    "r1_dx256_mx": (1, 256, 64, 128, "mxfp8"),
    "r5_dx1024_bf16": (5, 1024, 64, 128, "bf16"),
    "r17_dx768_mx": (17, 768, 64, 128, "mxfp8"),
    "r70_dx1280_h4_mx": (70, 1280, 4, 32, "mxfp8"),
    "r130_dx256_h40_bf16": (130, 256, 40, 64, "bf16"),
    "r200_dx512_h8d256_mx": (200, 512, 8, 256, "mxfp8"),
    "decode_b32_dx7168_mx": (32, 7168, 64, 128, "mxfp8"),
    "decode_b32_dx7168_bf16": (32, 7168, 64, 128, "bf16"),
}


@pytest.mark.parametrize("case", list(PROLOG))
def test_indexer_prolog_matches_oracle(case):
    """dsa_indexer_prolog against the oracle's fp64 projections and normalization, by
    the interval rule of check_prolog; then the same call again into the same
    buffers gives the same bytes (no state kept between calls)."""
    from sparse_attention_lightningindexer_amd.inputs import make_prolog
    from parity import check_prolog
    rows, d_x, H_I, d_I, fmt = PROLOG[case]
    say(f"[parity] prolog {case}: rows {rows} d_x {d_x} H_I {H_I} d_I {d_I} {fmt}")
    p = make_prolog(rows, d_x, H_I, d_I, seed=21 + rows)
    pd = B.PrologDevice(p)
    outs = B.dsa_indexer_prolog(pd, fmt)
    torch.cuda.synchronize()
    host = [None if t is None else t.cpu().numpy() for t in outs]
    check_prolog(p, fmt, host[0].reshape(rows, H_I, d_I) if fmt == "bf16" else host[0],
                 None if host[1] is None else host[1], host[2], host[3], O.indexer_prolog(p))
    for t in outs:
        if t is not None:
            t.fill_(0x55)
    B.dsa_indexer_prolog(pd, fmt, outs=outs)
    torch.cuda.synchronize()
    for a, t in zip(host, outs):
        if t is not None:
            assert np.array_equal(a, t.cpu().numpy())


def test_indexer_prolog_zero_inputs_and_feeds_the_indexer():
    """A zero hidden state gives q = 0 (E8M0 byte 0, codes 0) and head weights 0; a zero
    key gives a zero normalized key.  The prolog's MXFP8 query and head weights then
    drive dsa_indexer_scores like the same values written by the input generator."""
    from sparse_attention_lightningindexer_amd.inputs import make_prolog
    say("[parity] prolog zero inputs and indexer hand-off")
    p = make_prolog(4, 256, 64, 128, seed=5)
    p.x[1] = 0
    p.k[2] = 0
    q, qs, hw, kn = B.dsa_indexer_prolog(B.PrologDevice(p), "mxfp8")
    torch.cuda.synchronize()
    assert not q[1].any() and not qs[1].any() and not hw[1].any()
    assert not kn[2].any()
    # hand-off: a decode workload of 4 sequences whose index query and head weights
    # are the prolog's outputs
    wl = make_workload(6, batch=4, lens=[300, 129, 64, 1000])
    wl.q_idx = q.cpu().numpy().reshape(wl.q_idx.shape)
    wl.q_idx_scale = qs.cpu().numpy().reshape(wl.q_idx_scale.shape)
    wl.head_w = hw.cpu().numpy().reshape(wl.head_w.shape)
    dev = B.DeviceInputs(wl)
    sc = B.dsa_indexer_scores(dev)
    torch.cuda.synchronize()
    rows = np.arange(wl.rows, dtype=np.int32)
    check_scores(wl, sc.cpu().numpy().astype(np.float64), O.indexer_scores(wl, rows), rows)


@pytest.mark.parametrize("case", ["fp8_mx_kv", "mx_idx_fp32_kv"])
def test_cache_append_edge_values_match_oracle(case):
    """Quantized appends of rows built from edge values: all-zero rows, -0.0, bf16
    subnormals, tiny and huge magnitudes in one group, and values a hair under the
    saturation point of their group; codes and scales bit-exact against the oracle."""
    cfg, kw = APPEND[case]
    wl = make_workload(cfg, **kw)
    say(f"[parity] append edge values {case}")
    dev = B.DeviceInputs(wl)
    rng = np.random.default_rng(12)
    specials = np.array([0.0, -0.0, 1e-39, -3e-39, 1e-30, 2.5e-20, 1.0, -1.0, 448.0, -447.0, 1e20, -3e30,
                         0.0625, 0.09375, 65504.0, 7.0e-3], np.float32)

    def rows(width):
        x = rng.choice(specials, size=(wl.rows, width)).astype(np.float32)
        x[0] = 0.0                                 # an all-zero row
        x[1] = -0.0
        x[2] = rng.standard_normal(width).astype(np.float32) * 1e-36  # subnormal-range row
        return torch.from_numpy(x).to(torch.bfloat16).float().numpy()

    k_new, kv_new = _bf16_bits(rows(wl.d_I)), _bf16_bits(rows(wl.d_qk))
    _assert_same_bytes(case, _append_both(wl, dev, k_new, kv_new))


def test_late_large_logit_takes_the_exact_second_pass():
    """A logit in a late chunk above its work item's first-chunk maximum by far more
    than the no-rescale slack (2^32 in probability): the work item runs again with
    the exact maximum.  One latent row's rope channels are aligned with head 0's
    query so that head's logit there is about 120 nats (173 in log2 units: without
    the second pass its probability would overflow fp32 and bf16); its value
    channels stay ordinary.  Output and lse match the oracle: 128 rows of 8 chunks
    (no split, the row in the last chunk) and 2 rows split 32 ways (the row in the
    second chunk of the last split)."""
    for batch, lens, top_k in ((128, 300, 256), (2, [3000, 2500], 2048)):
        wl = make_workload(2, batch=batch, lens=lens, top_k=top_k)
        say(f"[parity] late large logit: batch {batch}, top_k {top_k}")
        q = torch.from_numpy(wl.q.view(np.int16)).view(torch.bfloat16).double().numpy()
        s_star = top_k - 7
        marked = [0, batch - 1] + ([batch // 2] if batch > 2 else [])
        for b in marked:
            q0 = q[b, 0, 512:]                      # head 0 of row b (n_q = 1), rope channels
            beta = 120.0 / (wl.sm_scale * float(q0 @ q0))
            row = (beta * q0).astype(np.float32)
            blk = int(wl.block_table[b, s_star // 64])
            wl.kv_pool[blk, s_star % 64, 512:] = torch.from_numpy(row).to(torch.bfloat16).view(
                torch.int16).numpy().view(np.uint16)
        idx = np.tile(np.arange(top_k, dtype=np.int32), (wl.rows, 1))
        dev = B.DeviceInputs(wl)
        out, lse = B.dsa_sparse_attn(dev, torch.from_numpy(idx).cuda())
        torch.cuda.synchronize()
        ref_o, ref_l = O.sparse_attn(wl, idx)
        assert (ref_l[marked, 0] > 110).all()       # the late logit dominates head 0
        check_attention(wl, f64(out), f64(lse), ref_o, ref_l, f"late logit k={top_k}")


def test_side_stream_and_no_indices_out_give_the_same_bytes():
    """Every call runs on the stream it is given: dsa_forward on a second stream
    (default priority), with and without indices_out, gives the same output and lse
    bytes as on the current stream; the side stream's work is ordered after the
    inputs' copies by an event."""
    wl = make_workload(2, batch=4, lens=[5000, 700, 2049, 64])
    say("[parity] side stream, indices_out NULL")
    dev = B.DeviceInputs(wl)
    out0, lse0, idx0 = B.dsa_forward(dev)
    torch.cuda.synchronize()
    ref = (out0.clone(), lse0.clone(), idx0.clone())
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()
    ready.record(torch.cuda.current_stream())
    side.wait_event(ready)
    out_s = torch.empty_like(ref[0])
    lse_s = torch.empty_like(ref[1])
    dev.set_outputs(out_s, lse_s)
    with torch.cuda.stream(side):
        B.dsa_forward(dev, indices_out=None, want_indices=False, stream=side)
    side.synchronize()
    assert torch.equal(out_s, ref[0]) and torch.equal(lse_s, ref[1])
    # attention alone on the side stream, from the first call's indices
    out_a = torch.empty_like(ref[0])
    dev.set_outputs(out_a, None)
    with torch.cuda.stream(side):
        B.dsa_sparse_attn(dev, ref[2], stream=side)
    side.synchronize()
    assert torch.equal(out_a, ref[0])


def test_forward_replays_from_a_captured_graph():
    """dsa_forward captured into a HIP graph (workspace and outputs allocated
    beforehand; the library allocates nothing) replays to the eager bytes, three
    times, with eager work that clears the outputs between the replays."""
    wl = make_workload(2, batch=4, lens=[5000, 700, 2049, 64])
    say("[parity] graph capture and replay of dsa_forward")
    dev = B.DeviceInputs(wl)
    ws = torch.empty(max(1, B.dsa_forward_workspace_bytes(dev)), dtype=torch.uint8, device="cuda")
    idx = torch.empty((wl.rows, wl.top_k), dtype=torch.int32, device="cuda")
    B.dsa_forward(dev, indices_out=idx, ws=ws)
    torch.cuda.synchronize()
    ref = (dev.out.clone(), dev.lse.clone(), idx.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm call on the capture's side stream
        B.dsa_forward(dev, indices_out=idx, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.dsa_forward(dev, indices_out=idx, ws=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        dev.out.zero_()
        dev.lse.zero_()
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dev.out, ref[0]) and torch.equal(dev.lse, ref[1]) and torch.equal(idx, ref[2]), rep


# ------------------------------------------------------------ strided pools

def _strided(t, width, row_pad, block_pad, fill):
    """Device copy of pool tensor t ([num_blocks, 64, width] or [num_blocks, 64]) in a
    buffer whose rows are padded by row_pad elements and blocks by block_pad, the
    padding filled with `fill`: (buffer, block stride, row stride) in elements."""
    nb = t.shape[0]
    rs = width + row_pad
    bs = 64 * rs + block_pad
    flat = t.reshape(nb, 64, width)
    buf = torch.full((nb * bs,), 0, dtype=flat.dtype, device=flat.device)
    buf.fill_(fill)
    buf.as_strided((nb, 64, width), (bs, rs, 1)).copy_(flat)
    return buf, bs, rs


# pad sizes keep every row and block on the 16-byte grid the kernels read in
_PADS = {"f32": (4, 16), "bf16": (8, 128), "e4m3": (16, 128), "mxfp8": (16, 128), "e4m3_128": (16, 128)}
_FILL = {"f32": float("nan"), "bf16": 0x7FC0, "e4m3": 0x7F, "mxfp8": 0x7F, "e4m3_128": 0x7F}


def _use_strided_pools(dev):
    """Point dev's index-K and latent pools (and scales) at padded, NaN-filled copies
    with explicit strides; returns the buffers (kept alive by the caller)."""
    wl = dev.wl
    keep = []

    def fix(cache, data, scales, fmt, width):
        rp, bp = _PADS[fmt]
        buf, bs, rs = _strided(data, width, rp, bp, _FILL[fmt])
        keep.append(buf)
        cache.data, cache.block_stride, cache.row_stride = buf.data_ptr(), bs, rs
        if scales is not None:
            ng = 1 if scales.dim() == 2 else scales.shape[-1]
            sbuf, sbs, srs = _strided(scales, ng, 4, 8, float("nan") if scales.dtype == torch.float32 else 0xFF)
            keep.append(sbuf)
            cache.scales, cache.scale_block_stride, cache.scale_row_stride = sbuf.data_ptr(), sbs, srs

    fix(dev.idx.k, dev.k_pool, dev.k_scale, wl.idx_dtype, wl.d_I)
    fix(dev.attn.kv, dev.kv_pool, dev.kv_scale, wl.kv_dtype, wl.d_qk)
    return keep


STRIDED = {
    "tiny_fp32": (1, dict(poison=True)),
    "decode_bf16": (2, dict(batch=3, lens=[300, 1000, 453], top_k=128, poison=True)),
    "nq8_bf16_multirow_indexer": (2, dict(batch=2, n_q=8, lens=[1000, 77], top_k=256, poison=True)),
    "fp8_decode": (5, dict(batch=3, lens=[500, 900, 130], top_k=256, poison=True)),
    "fp8_pages_nq2": (6, dict(batch=2, n_q=2, lens=[700, 66], top_k=256, poison=True)),
    "nq8_mxfp8_multirow_indexer": (6, dict(batch=2, n_q=8, lens=[1000, 77], top_k=256, poison=True)),
}


@pytest.mark.parametrize("case", list(STRIDED))
def test_strided_pools_give_the_dense_results(case):
    """Pools with padded rows and blocks (the padding NaN) and explicit strides, for the
    data and the scales, give the same scores, indices, output and lse bytes as the
    dense layout, through every kernel that reads a pool (decode and multi-row
    indexers, every attention format)."""
    cfg, kw = STRIDED[case]
    wl = make_workload(cfg, **kw)
    say(f"[parity] strided pools {case}")
    _, sc, idx, out, lse = gpu_all(wl)
    dev = B.DeviceInputs(wl)
    keep = _use_strided_pools(dev)
    _, sc2, idx2, out2, lse2 = gpu_all(wl, dev)
    L = wl.row_lens()
    for r in range(wl.rows):
        assert np.array_equal(sc[r, :L[r]], sc2[r, :L[r]]), f"row {r}: scores differ"
    assert np.array_equal(idx, idx2) and np.array_equal(out, out2) and np.array_equal(lse, lse2)
    del keep


@pytest.mark.parametrize("case", list(APPEND))
def test_cache_append_into_strided_pools(case):
    """The append writes the same rows and scales into padded pools as into dense ones,
    and leaves the padding untouched."""
    cfg, kw = APPEND[case]
    wl = make_workload(cfg, **kw)
    say(f"[parity] append into strided pools {case}")
    rng = np.random.default_rng(13)
    f32 = wl.idx_dtype == "f32"
    k_new = (rng.standard_normal((wl.rows, wl.d_I)) / np.sqrt(wl.d_I)).astype(np.float32)
    kv_new = (rng.standard_normal((wl.rows, wl.d_qk)) / np.sqrt(wl.d_qk)).astype(np.float32)
    dt = torch.float32 if f32 else torch.bfloat16
    kt, kvt = torch.from_numpy(k_new).to(dt).cuda(), torch.from_numpy(kv_new).to(dt).cuda()
    dense = B.DeviceInputs(wl)
    B.dsa_cache_append(dense, kt, kvt)
    dev = B.DeviceInputs(wl)
    keep = _use_strided_pools(dev)
    B.dsa_cache_append(dev, kt, kvt)
    torch.cuda.synchronize()
    # the strided buffers, viewed back as dense pools, equal the dense append
    i = 0
    for cache, ref, scales in ((dev.idx.k, dense.k_pool, dense.k_scale), (dev.attn.kv, dense.kv_pool, dense.kv_scale)):
        for t, bs, rs in ((ref, cache.block_stride, cache.row_stride),
                          (scales, cache.scale_block_stride, cache.scale_row_stride)):
            if t is None:
                continue
            nb, width = t.shape[0], (1 if t.dim() == 2 else t.shape[-1])
            buf = keep[i]
            i += 1
            view = buf.as_strided((nb, 64, width), (bs, rs, 1))
            assert torch.equal(view.reshape(t.shape).view(torch.uint8) if t.dtype != torch.float32 else
                               view.reshape(t.shape).view(torch.int32),
                               t.view(torch.uint8) if t.dtype != torch.float32 else t.view(torch.int32)), case
            mask = torch.ones(buf.numel(), dtype=torch.bool, device=buf.device)
            mask.view(-1).as_strided((nb, 64, width), (bs, rs, 1)).fill_(False)
            pad = buf[mask]
            if pad.dtype == torch.float32:
                assert bool(torch.isnan(pad).all()), f"{case}: padding written"
            else:
                assert bool((pad == pad.flatten()[0]).all()), f"{case}: padding written"
