"""bench.py's host-side contract (CPU only): the one-GPU scope and the
algorithmic counts that its roofline divides by."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_counts_of_the_decode_workload():
    """Decode B32 x 8k: the attention stage moves 1152 B per selected position plus q,
    out and the indices per row (84.67 MB) and computes 2*128*(576+512) flops per
    selected position; the indexer reads each sequence's index keys once."""
    import bench
    from sparse_attention_lightningindexer_amd.inputs import make_workload
    wl = make_workload(2)
    a = bench.algorithmic(wl)
    sel = 32 * 2048
    assert a["attention"][0] == sel * 1152 + 32 * (128 * 576 * 2 + 128 * 512 * 2 + 2048 * 4) == 84672512
    assert a["attention"][1] == 2 * sel * 128 * (576 + 512)
    assert a["indexer"][0] == 32 * 8192 * 256 + 32 * (64 * 128 * 2 + 64 * 4)
    assert a["topk"][0] == 32 * 2048 * 4


def test_prolog_bytes_count_every_operand_once():
    import bench
    nb = bench.prolog_bytes(32, 7168, 64, 128, mx=False)
    assert nb == 2 * (8192 + 64) * 7168 + 2 * 32 * 7168 + 2 * 32 * 128 + 4 * 128 + 32 * 8192 * 2 + 4 * 32 * 64 + 2 * 32 * 128
    assert bench.prolog_bytes(32, 7168, 64, 128, mx=True) == nb - 32 * 8192 + 32 * 256
