"""Memory Parallel on one GPU ([README] Overall Design > Inference Pipeline:
the routing keys are sharded over GPUs, each scores its shard locally and a
global reduce follows; [MSA-arXiv26] 核心方法 > Memory Parallel 推理).  The
store is split into contiguous document shards; each shard is scored and
selected on its own (the calls one GPU of G would make, at that GPU's shape)
and msa_topk_merge reduces the shards' lists.  The merged top-k equals the
unsharded one bit for bit, every shard's scores equal the unsharded scores of
its documents, and msa_topk_merge equals the oracle's merge."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.helpers import dev

pytestmark = pytest.mark.gpu

import sparse_attention_long_msa_amd as M  # noqa: E402  (a missing library fails loudly)


@pytest.mark.parametrize("G,B,k_in,k", [(1, 3, 16, 16), (3, 5, 16, 16), (8, 32, 16, 16), (8, 2, 64, 64),
                                        (64, 4, 64, 64), (5, 7, 4, 1), (2, 1, 3, 5)])
def test_topk_merge_matches_oracle(G, B, k_in, k):
    r = np.random.default_rng(G * 100 + k_in)
    vals = np.round(r.normal(size=(G, B, k_in)), 1).astype(np.float32)   # exact ties, also across shards
    vals[r.random(size=vals.shape) < 0.05] = -np.inf
    ids = np.stack([np.stack([r.permutation(4 * k_in)[:k_in] for _ in range(B)]) for _ in range(G)]).astype(np.int32)
    ids[r.random(size=ids.shape) < 0.1] = -1                          # empty slots
    vals[r.random(size=vals.shape) < 0.05] = np.nan                   # excluded documents
    off = np.cumsum(np.concatenate([[0], r.integers(4 * k_in, 8 * k_in, size=G - 1)])).astype(np.int64)
    gi, gv = M.msa_topk_merge(torch.from_numpy(vals).to(dev()), torch.from_numpy(ids).to(dev()),
                              torch.from_numpy(off).to(dev()), k)
    wi, wv = O.topk_merge(vals, ids, off, k)
    np.testing.assert_array_equal(gi.cpu().numpy(), wi)
    np.testing.assert_array_equal(gv.cpu().numpy().astype(np.float64), wv)   # NaN where the oracle has NaN


def _aligned_cuts(chunk_off, G):
    """G contiguous document shards whose first chunks sit on 16-chunk group
    boundaries, so each shard is a slice of the tiled store."""
    D = len(chunk_off) - 1
    ok = np.flatnonzero(chunk_off[:-1] % 16 == 0)
    cuts = [0]
    for g in range(1, G):
        c = int(ok[np.searchsorted(ok, g * D // G)])
        assert c > cuts[-1]
        cuts.append(c)
    return np.array(cuts + [D], dtype=np.int64)


@pytest.mark.parametrize("name,G", [("cfg4", 8), ("cfg3", 4), ("cfg5", 8), ("cfg2", 3)])
def test_sharded_routing_equals_unsharded(name, G):
    from synth import configs
    from tests.preset_run import GpuLayer, HostLayer
    p = getattr(configs, name)()
    gl = GpuLayer(p, 0, HostLayer(p, 0))
    kr = gl.store[synth.T_KR]
    co = p.chunk_off
    D, k, B = p.n_docs, p.k, p.B
    lay = M.MSA_LAYOUT_TILED
    score0 = M.msa_route_score(gl.qr, kr, gl.cd, D, layout=lay)
    ids0, vals0 = M.msa_topk(score0, k)
    cuts = _aligned_cuts(co, G)
    vals = torch.full((G, B, k), float("nan"), dtype=torch.float32, device=dev())
    ids = torch.full((G, B, k), -1, dtype=torch.int32, device=dev())
    for g in range(G):
        lo, hi = int(cuts[g]), int(cuts[g + 1])
        c0, c1 = int(co[lo]), int(co[hi])
        nc = c1 - c0
        shard = kr[c0:c0 + M.padded_chunks(nc, lay)]
        co_g = torch.from_numpy(co[lo:hi + 1] - c0).to(dev())
        cd_g = M.msa_chunk_doc_map(co_g, nc)
        score_g = M.msa_route_score(gl.qr, shard, cd_g, hi - lo, layout=lay)
        assert torch.equal(score_g, score0[:, lo:hi]), f"shard {g}: scores differ"
        kk = min(k, hi - lo)
        i_g, v_g = M.msa_topk(score_g, kk)
        ids[g, :, :kk], vals[g, :, :kk] = i_g, v_g
    mi, mv = M.msa_topk_merge(vals, ids, torch.from_numpy(cuts[:-1]).to(dev()), k)
    assert torch.equal(mi, ids0)
    assert torch.equal(mv, vals0)
    del gl
    torch.cuda.empty_cache()
