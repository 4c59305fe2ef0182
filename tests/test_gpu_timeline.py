"""The timeline build (libmpgemm_timeline.so, include/mpgemm_timeline.h)
computes what the product computes, and its per-workgroup records are
well-formed.

The timeline build is the product source with stamps added: thread 0 of
each workgroup of the pipelined kernel writes clock values into LDS and
copies them out after its last store.  Its results must be bitwise those of
the product library on the same inputs (the stamps touch no operand, sum or
output), and every record must hold a start, one publish per K tile (up to
41) in order, the end of the K loop and the end of the epilogue, on a
clock that never runs backwards, with the launch's K-tile count and a valid
XCD id.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_amd as mp
from dense_mixed_precision_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [(2048, 2048, 2048), (1000, 800, 617), (256, 256, 256), (640, 384, 8192)])
def test_timeline_build_matches_the_product_and_records_are_ordered(M, N, K):
    print(f"timeline case {M}x{N}x{K}", flush=True)
    dev = torch.device("cuda:0")
    A, B, _ = make_inputs(M, N, K, "uniform", seed=77)
    Ad, Bd = A.to(dev), B.to(dev)
    C1 = torch.empty((M, N), dtype=torch.float32, device=dev)
    C2 = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    cfg = mp.mpgemm_f16f32_query(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N, C1.data_ptr(), N, 1.0, 0.0)
    assert cfg["kind_name"] == "pipe"
    stream = torch.cuda.current_stream().cuda_stream
    assert mp.mpgemm_f16f32(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N, C1.data_ptr(), N, 1.0, 0.0, stream) == 0
    lib = mp.load_timeline()
    assert lib.mpgemm_timeline_clear() == 0
    assert lib.mpgemm_f16f32(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N, C2.data_ptr(), N, 1.0, 0.0, stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)

    nwg = int(cfg["grid"])
    rec = np.zeros((nwg + 1, mp.TIMELINE_SLOTS), dtype=np.uint64)
    assert lib.mpgemm_timeline_read(rec.ctypes.data, rec.size) == 0
    assert not rec[nwg].any()          # nothing past the launch's workgroups
    r = rec[:nwg].astype(np.int64)
    num_k = -(-(K - K % 8) // cfg["bk"])
    assert (r[:, 43] == num_k).all()
    nrec = min(num_k, 41)
    stamps = np.concatenate([r[:, 1:2], r[:, 2:2 + nrec], r[:, 44:46]], axis=1)
    assert (np.diff(stamps, axis=1) >= 0).all()
    assert (r[:, 2 + nrec:43] == 0).all()
    assert (r[:, 46] > r[:, 0]).all()
    assert ((r[:, 47] >> 32) < 8).all()
    # every XCD ran some of the workgroups when there are enough of them
    if nwg >= 64:
        assert len(set(((r[:, 47] >> 32) & 0xF).tolist())) == 8
