"""The C ABI on the host (CPU only): loading, exported symbols, validation, sizes.

No call here reaches a kernel launch: each one either is a pure host query or
fails validation first, which the ABI promises happens before anything is
enqueued.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

from sparse_attention_lightningindexer_amd import binding as B
from sparse_attention_lightningindexer_amd.inputs import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_entry_point():
    lib = B.lib()
    decl = _declared()
    assert set(decl) == set(B.EXPORTS), decl
    for name in decl:
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = B.lib()
    for s in range(6):
        assert lib.dsa_status_string(s).decode().startswith(["DSA_OK", "DSA_ERR_NULL", "DSA_ERR_SHAPE",
                                                             "DSA_ERR_UNSUPPORTED", "DSA_ERR_WORKSPACE",
                                                             "DSA_ERR_HIP"][s])
    assert lib.dsa_version() >= 100


def _fake_structs(wl):
    """ABI structs over fake (never dereferenced) device addresses."""
    fake = 0x10000
    batch = B.dsa_batch(wl.batch, wl.n_q, fake, fake, wl.max_blocks, 64, wl.max_seq_len)
    kc = B.dsa_cache(fake, None, B._DT[wl.idx_dtype], 0, 0, wl.d_I, wl.num_blocks)
    idx = B.dsa_indexer_args(fake, B._DT[wl.idx_dtype], None, wl.H_I, wl.d_I, fake, kc)
    kvc = B.dsa_cache(fake, None, B._DT[wl.kv_dtype], 0, 0, wl.d_qk, wl.num_blocks)
    attn = B.dsa_attn_args(fake, B._DT[wl.q_dtype], wl.H, wl.d_v, wl.sm_scale, kvc, fake, None)
    return batch, idx, attn


def test_validation_errors_are_returned_before_any_launch():
    lib = B.lib()
    wl = make_workload(2, batch=2, lens=[100, 50])
    batch, idx, attn = _fake_structs(wl)
    ref = C.byref
    assert lib.dsa_indexer_scores(None, ref(idx), 0x10000, 128, None) == B.DSA_ERR_NULL
    assert lib.dsa_indexer_scores(ref(batch), ref(idx), None, 128, None) == B.DSA_ERR_NULL
    assert lib.dsa_indexer_scores(ref(batch), ref(idx), 0x10000, 10, None) == B.DSA_ERR_SHAPE  # ld < max_seq_len
    bad = B.dsa_batch.from_buffer_copy(batch)
    bad.block_size = 32
    assert lib.dsa_indexer_scores(ref(bad), ref(idx), 0x10000, 128, None) == B.DSA_ERR_SHAPE
    for nb, nq in ((65536, 1), (1 << 12, (1 << 12) + 1)):  # more sequences than a grid dimension; too many rows
        bad = B.dsa_batch.from_buffer_copy(batch)
        bad.batch, bad.n_q = nb, nq
        assert lib.dsa_indexer_scores(ref(bad), ref(idx), 0x10000, 128, None) == B.DSA_ERR_SHAPE
    bad = B.dsa_batch.from_buffer_copy(batch)
    bad.max_seq_len = bad.max_blocks * 64 + 1
    assert lib.dsa_topk(ref(bad), 0x10000, 10**6, 16, 0x10000, None, 0, None) == B.DSA_ERR_SHAPE
    i2 = B.dsa_indexer_args.from_buffer_copy(idx)
    i2.n_heads = 32
    assert lib.dsa_indexer_scores(ref(batch), ref(i2), 0x10000, 128, None) == B.DSA_ERR_UNSUPPORTED
    i2 = B.dsa_indexer_args.from_buffer_copy(idx)
    i2.dtype = B.DSA_E4M3   # k pool still bf16
    assert lib.dsa_indexer_scores(ref(batch), ref(i2), 0x10000, 128, None) == B.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk(ref(batch), 0x10000, 128, 0, 0x10000, None, 0, None) == B.DSA_ERR_SHAPE
    assert lib.dsa_topk(ref(batch), 0x10000, 128, 4097, 0x10000, None, 0, None) == B.DSA_ERR_SHAPE
    assert lib.dsa_topk(ref(batch), None, 128, 16, 0x10000, None, 0, None) == B.DSA_ERR_NULL
    a2 = B.dsa_attn_args.from_buffer_copy(attn)
    a2.d_v = 256
    assert lib.dsa_sparse_attn(ref(batch), ref(a2), 0x10000, 16, None, 0, None) == B.DSA_ERR_UNSUPPORTED
    # 2 rows -> split partials are needed, so a missing workspace is refused
    need = lib.dsa_sparse_attn_workspace_bytes(ref(batch), ref(attn), 2048)
    assert need > 0
    assert lib.dsa_sparse_attn(ref(batch), ref(attn), 0x10000, 2048, None, 0, None) == B.DSA_ERR_WORKSPACE
    assert lib.dsa_sparse_attn(ref(batch), ref(attn), 0x10000, 2048, 0x10000, need - 1, None) == B.DSA_ERR_WORKSPACE
    assert lib.dsa_sparse_attn(ref(batch), ref(attn), None, 2048, 0x10000, need, None) == B.DSA_ERR_NULL
    fneed = lib.dsa_forward_workspace_bytes(ref(batch), ref(idx), ref(attn), 2048)
    assert lib.dsa_forward(ref(batch), ref(idx), ref(attn), 2048, None, 0x10000, fneed - 1, None) == B.DSA_ERR_WORKSPACE
    kv_mx = B.dsa_attn_args.from_buffer_copy(attn)
    kv_mx.kv.dtype = B.DSA_E4M3
    kv_mx.kv.scale_kind = B.DSA_SCALE_E8M0
    kv_mx.kv.group = 32
    assert lib.dsa_sparse_attn(ref(batch), ref(kv_mx), 0x10000, 16, 0x10000, need, None) == B.DSA_ERR_NULL


def test_pool_strides_are_validated_before_any_launch():
    """Strides in elements, 0 meaning dense: negative strides, rows narrower than the
    width, 16-byte misaligned BF16 rows or blocks, scale rows narrower than their
    groups and misaligned E8M0 index-key scale rows are refused with DSA_ERR_SHAPE."""
    lib = B.lib()
    ref = C.byref
    wl = make_workload(2, batch=2, lens=[100, 50])
    batch, idx, attn = _fake_structs(wl)

    def attn_status(**kv):
        a2 = B.dsa_attn_args.from_buffer_copy(attn)
        for k, v in kv.items():
            setattr(a2.kv, k, v)
        return lib.dsa_sparse_attn(ref(batch), ref(a2), 0x10000, 2048, None, 0, None)

    for bad in (dict(row_stride=-1), dict(block_stride=-64), dict(row_stride=575), dict(row_stride=577),
                dict(block_stride=64 * 576 + 4), dict(row_stride=1 << 41)):
        assert attn_status(**bad) == B.DSA_ERR_SHAPE, bad
    # a valid padded layout passes validation and reaches the workspace check
    assert attn_status(row_stride=584, block_stride=64 * 584 + 128) == B.DSA_ERR_WORKSPACE
    wl6 = make_workload(6, batch=2, lens=[100, 50])
    batch6, idx6, _ = _fake_structs(wl6)

    def idx_status(**kv):
        i2 = B.dsa_indexer_args.from_buffer_copy(idx6)
        i2.q_scale, i2.k.scales, i2.k.scale_kind, i2.k.group = 0x10000, 0x20000, B.DSA_SCALE_E8M0, 32
        for k, v in kv.items():
            setattr(i2.k, k, v)
        return lib.dsa_indexer_scores(ref(batch6), ref(i2), None, 128, None)

    assert idx_status(scale_row_stride=3) == B.DSA_ERR_SHAPE      # fewer than the 4 groups
    assert idx_status(scale_row_stride=6) == B.DSA_ERR_SHAPE      # a row's 4 bytes not 4-byte aligned
    assert idx_status(scale_row_stride=8, scale_block_stride=520) == B.DSA_ERR_NULL  # valid; scores NULL


def test_indexer_query_alignment_is_validated_before_any_launch():
    """BF16 and E4M3 indexer queries arrive in 16-byte pieces, head weights and
    query scales in 4-byte ones: misaligned pointers are refused with DSA_ERR_SHAPE."""
    lib = B.lib()
    ref = C.byref
    for cfg in (2, 5, 6):
        wl = make_workload(cfg, batch=2, lens=[100, 50])
        batch, idx, _ = _fake_structs(wl)

        def status(**kv):
            i2 = B.dsa_indexer_args.from_buffer_copy(idx)
            if cfg != 2:
                i2.q_scale, i2.k.scales = 0x30000, 0x20000
                i2.k.scale_kind, i2.k.group = ((B.DSA_SCALE_F32, 128) if cfg == 5 else (B.DSA_SCALE_E8M0, 32))
            for k, v in kv.items():
                setattr(i2, k, v)
            return lib.dsa_indexer_scores(ref(batch), ref(i2), None, 128, None)

        assert status() == B.DSA_ERR_NULL, cfg  # valid: the NULL scores are what remains
        assert status(q=0x10008) == B.DSA_ERR_SHAPE, cfg
        assert status(head_w=0x10002) == B.DSA_ERR_SHAPE, cfg
        if cfg != 2:
            assert status(q_scale=0x30002) == B.DSA_ERR_SHAPE, cfg


def test_noalloc_forward_refuses_batches_beyond_its_scratch_before_any_launch():
    """dsa_forward_noalloc checks the batch's workspace against its fixed per-GPU
    array on the host: a 4096-row prefill needs more and is refused without any
    HIP call (this runs without a GPU)."""
    lib = B.lib()
    assert lib.dsa_forward_noalloc_max_bytes() == 32 << 20
    wl = make_workload(2, batch=1, n_q=4096, lens=[4096], top_k=2048)
    batch, idx, attn = _fake_structs(wl)
    ref = C.byref
    assert lib.dsa_forward_workspace_bytes(ref(batch), ref(idx), ref(attn), 2048) > (32 << 20)
    assert lib.dsa_forward_noalloc(ref(batch), ref(idx), ref(attn), 2048, None, None) == B.DSA_ERR_WORKSPACE
    assert lib.dsa_forward_noalloc(None, ref(idx), ref(attn), 2048, None, None) == B.DSA_ERR_NULL


def test_workspace_sizes_follow_the_split_rule():
    lib = B.lib()
    for cfg, kw in ((2, {}), (4, dict(lens=[5000] * 8)), (5, dict(batch=64, lens=100))):
        wl = make_workload(cfg, **kw) if cfg != 5 else make_workload(2, batch=64, lens=100)
        batch, idx, attn = _fake_structs(wl)
        rows = wl.rows
        n = lib.dsa_sparse_attn_workspace_bytes(C.byref(batch), C.byref(attn), 2048)
        splits = n // (rows * 128 * (2 * 512 + 4))   # bf16 partials + fp32 LSEs
        assert n == rows * splits * 128 * (2 * 512 + 4)
        # two head halves per row, then the index list is split until ~256 workgroups
        assert 1 < splits <= 32 and 2 * rows * splits >= 256
        f = lib.dsa_forward_workspace_bytes(C.byref(batch), C.byref(idx), C.byref(attn), 2048)
        ld = (wl.max_seq_len + 63) // 64 * 64
        assert f >= 4 * rows * ld + 4 * rows * 2048 + n
    # enough rows: no splits, no partials
    wl = make_workload(2, batch=128, lens=70)
    batch, idx, attn = _fake_structs(wl)
    assert lib.dsa_sparse_attn_workspace_bytes(C.byref(batch), C.byref(attn), 2048) == 0
    assert lib.dsa_topk_workspace_bytes(C.byref(batch), 2048) == 0


def test_prolog_validation_errors_are_returned_before_any_launch():
    lib = B.lib()
    fake = 0x10000
    ok = dict(rows=32, d_x=7168, n_heads=64, head_dim=128, x=fake, w_q=fake, w_h=fake, k=fake, k_gain=fake,
              eps=1e-6, q_dtype=B.DSA_E4M3, q_out=fake, q_scale_out=fake, head_w_out=fake, k_out=fake)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.dsa_indexer_prolog(C.byref(B.dsa_prolog_args(**a)), None)

    assert lib.dsa_indexer_prolog(None, None) == B.DSA_ERR_NULL
    assert call(rows=0) == B.DSA_OK                       # nothing to do, nothing launched
    for bad in (dict(rows=-1), dict(rows=65535 * 64 + 1), dict(d_x=0), dict(d_x=7168 + 64), dict(d_x=7168 + 128), dict(head_dim=48), dict(head_dim=288),
                dict(n_heads=0), dict(eps=-1.0), dict(eps=float("nan")), dict(eps=float("inf")),
                dict(x=fake + 8), dict(w_q=fake + 2), dict(q_out=fake + 4), dict(head_w_out=fake + 2),
                dict(k_out=fake + 1)):
        assert call(**bad) == B.DSA_ERR_SHAPE, bad
    for bad in (dict(q_dtype=B.DSA_F32), dict(q_dtype=7)):
        assert call(**bad) == B.DSA_ERR_UNSUPPORTED, bad
    for name in ("x", "w_q", "w_h", "k", "k_gain", "q_out", "q_scale_out", "head_w_out", "k_out"):
        assert call(**{name: None}) == B.DSA_ERR_NULL, name
