"""dsa_forward_noalloc (the entry point that allocates nothing and works in the
library's per-GPU scratch array) gives the same bytes as dsa_forward with a
caller workspace, on two calls in a row, the second with a smaller batch."""
import sys

import numpy as np
import pytest
import torch

from sparse_attention_lightningindexer_amd import binding as B
from sparse_attention_lightningindexer_amd.inputs import make_workload

pytestmark = pytest.mark.gpu


def _both(wl):
    ref = B.DeviceInputs(wl)
    idx_ref = torch.empty((wl.rows, wl.top_k), dtype=torch.int32, device="cuda")
    B.dsa_forward(ref, indices_out=idx_ref)
    got = B.DeviceInputs(wl)
    got.out.fill_(7)
    got.lse.fill_(7)
    idx = torch.full((wl.rows, wl.top_k), -7, dtype=torch.int32, device="cuda")
    B.dsa_forward_noalloc(got, indices_out=idx)
    torch.cuda.synchronize()
    return (ref.out, ref.lse, idx_ref), (got.out, got.lse, idx)


def test_noalloc_forward_matches_the_workspace_forward_on_two_calls():
    print("[no_alloc] decode B32 x 8k, then a smaller batch", file=sys.stderr, flush=True)
    big = make_workload(2, poison=True)
    small = make_workload(2, batch=4, lens=[3000, 700, 2049, 64], poison=True)
    assert B.dsa_forward_workspace_bytes(B.DeviceInputs(small)) < B.dsa_forward_workspace_bytes(B.DeviceInputs(big))
    assert B.dsa_forward_workspace_bytes(B.DeviceInputs(big)) <= int(B.lib().dsa_forward_noalloc_max_bytes())
    for wl in (big, small):
        (o0, l0, i0), (o1, l1, i1) = _both(wl)
        assert torch.equal(i0, i1), "indices differ"
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)), "outputs differ"
        assert np.array_equal(l0.cpu().numpy().view(np.uint32), l1.cpu().numpy().view(np.uint32)), "lse differs"
    # without indices_out, same output bytes
    dev = B.DeviceInputs(small)
    B.dsa_forward_noalloc(dev, indices_out=None)
    torch.cuda.synchronize()
    assert torch.equal(dev.out.view(torch.int16), o0.view(torch.int16))


def test_noalloc_forward_rejects_a_batch_beyond_its_scratch():
    wl = make_workload(2, batch=1, n_q=3000, lens=[3000], top_k=2048)  # 36 MB of scores
    dev = B.DeviceInputs(wl)
    assert B.dsa_forward_workspace_bytes(dev) > int(B.lib().dsa_forward_noalloc_max_bytes())
    with pytest.raises(B.DsaError, match="WORKSPACE"):
        B.dsa_forward_noalloc(dev)
