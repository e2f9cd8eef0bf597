"""Ragged batches replayed from a captured graph.

A batch of short sequences is a chain of small launches per sequence, so a caller that serves the
same shapes repeatedly captures the batch calls once (HIP graph capture through
torch.cuda.CUDAGraph) and replays them.  Nothing in the index or attention path issues a memset, a
copy or an allocation, and every counter, status word and claim the kernels use is cleared by a
kernel of the same call, so a replay recomputes everything from its inputs.
"""
import numpy as np
import pytest
import torch

import gen
import dynamic_block_sparse_flexprefill_amd as fpa
from tests import parity as P

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _batch(lens, seed, Hq=6, Hkv=2):
    cs = [gen.CONFIGS["tiny"].with_(S=S, Hq=Hq, Hkv=Hkv) for S in lens]
    Ls = [gen.make(c, seed=seed + k) for k, c in enumerate(cs)]
    pack = lambda name: torch.cat([P.dev_bf16(getattr(L, name), "cuda").reshape(-1) for L in Ls])
    return cs[0], pack("q"), pack("k"), pack("v")


def _same_index(a, b):
    nnz, njob = a.nnz, int(a.job_ptr[-1].item())
    assert nnz == b.nnz and njob == int(b.job_ptr[-1].item())
    for f, n in (("row_ptr", None), ("col_idx", nnz), ("job_ptr", None), ("job_blk", njob), ("job_mask", njob),
                 ("job_order", None), ("pattern", None), ("jsd", None), ("status", None)):
        x, y = getattr(a, f), getattr(b, f)
        n = x.numel() if n is None else n
        assert torch.equal(x[:n], y[:n]), f


def test_batch_graph_replay_matches_eager():
    """Index and attention of a five-sequence batch (with a run of equal lengths) captured in one
    graph and replayed three times, with eager calls on other inputs (and their own workspace) and synchronisations
    between the replays; every replay equals the eager result bit for bit."""
    lens = [1024, 1024, 384, 2048, 256]     # the first two run as one call
    say(f"graph replay of a ragged batch, S = {lens}")
    c, Q, K, V = _batch(lens, seed=31)
    c2, Q2, K2, V2 = _batch(lens, seed=57)
    longest = fpa.shape_of(max(lens), c.b, c.Hq, c.Hkv)
    run = lambda q, k, v, ws: (lambda ix: (ix, fpa.attn_batch(q, k, v, lens, ix, ws=ws)))(
        fpa.index_batch(q, k, lens, c.b, c.Hq, c.Hkv, c.gamma, c.tau, ws=ws))
    ws_eager = fpa.Workspace(longest, "cuda", lens)
    idx_e, O_e = run(Q, K, V, ws_eager)
    torch.cuda.synchronize()
    ws_graph = fpa.Workspace(longest, "cuda", lens)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                       # warm-up off the default stream
        for _ in range(2):
            run(Q, K, V, ws_graph)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        idx_g, O_g = run(Q, K, V, ws_graph)
    for rep in range(3):
        other_idx, other_O = run(Q2, K2, V2, ws_eager)  # eager work between the replays
        torch.cuda.synchronize()
        O_g.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}: comparing")
        assert torch.equal(O_g.view(torch.int16), O_e.view(torch.int16))
        for a, b in zip(idx_g, idx_e):
            _same_index(a, b)
        assert all(int(ix.status.item()) == 0 for ix in other_idx)
