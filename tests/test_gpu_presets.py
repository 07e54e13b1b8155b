"""End-to-end parity per workload preset (pool -> route -> top-k -> gather ->
attention).  The tiny preset is compared in full; the 1M-token preset with the
oracle's full ranking of one layer; the 10M-token, 100M-token and batched
decode presets at their full per-layer size with the oracle on sampled
documents (every selected document, every needle and random others) plus the
attention of sampled queries on the selection the GPU made."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import configs
from tests.helpers import ATOL_ATTN, BAND, RTOL_SCORE, check_ids, check_scores

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

import sparse_attention_long_msa_amd as M  # noqa: E402  (a missing library fails loudly)
from tests.preset_run import GpuLayer, HostLayer  # noqa: E402


def _log(*a):
    print("[preset]", *a, flush=True)


def _check_sampled(p, host, g, n_random=200, seed=0):
    """Sampled routing parity: oracle scores of the sampled documents equal
    the GPU's; no sampled document outside the GPU selection beats it by
    more than the tie band; the GPU's values equal the oracle's scores of the
    selected documents."""
    rtol = RTOL_SCORE[host.dt]
    rng = np.random.default_rng(seed)
    docs = set(rng.choice(p.n_docs, size=min(n_random, p.n_docs), replace=False).tolist())
    docs |= set(int(x) for x in g["ids"].ravel()) | set(host.owner)
    docs = np.array(sorted(docs))
    ref = host.doc_scores(docs)                            # [B, n]
    got = g["doc_score"][:, docs]
    scale = np.abs(ref).max(axis=1, keepdims=True)
    err = (np.abs(got - ref) / scale).max()
    _log(f"{p.name} layer {host.l}: {len(docs)} sampled docs, normwise score err {err:.3g}")
    assert err <= rtol
    for b in range(p.B):
        sel = [int(x) for x in g["ids"][b]]
        col = {int(d): j for j, d in enumerate(docs)}
        sel_ref = np.array([ref[b, col[d]] for d in sel])
        np.testing.assert_allclose(g["vals"][b], sel_ref, rtol=rtol, atol=rtol * scale[b, 0])
        worst_sel = sel_ref.min()
        others = [ref[b, j] for j, d in enumerate(docs) if int(d) not in set(sel)]
        if others:
            assert max(others) <= worst_sel + BAND, f"query {b}: a sampled document beats the selection"
        for r in range(p.k - 1):
            assert sel_ref[r] >= sel_ref[r + 1] - BAND
    return docs


def _needle_recall(p, host, g):
    hits = [int(nd) in set(g["ids"][b].tolist()) for nd, b in host.owner.items()]
    return float(np.mean(hits))


def test_preset_tiny_full():
    p = configs.cfg1()
    host = HostLayer(p, 0)
    g = GpuLayer(p, 0, host).run()
    # full oracle of the layer from the raw tokens
    stores = {}
    for tid in (synth.T_KR, synth.T_K, synth.T_V):
        stores[tid] = np.concatenate([host.store(tid, doc) for doc in range(p.n_docs)])
    ref = O.layer(host.qr, stores[synth.T_KR], p.chunk_off, stores[synth.T_K], stores[synth.T_V], p.k, host.q,
                  *[np.stack([host.local(b)[i] for b in range(p.B)]) for i in (0, 1)],
                  q_pos_offset=p.qpo, base=p.rope_base, ids_override=g["ids"])
    err = check_scores(g["doc_score"], ref["doc_score"], RTOL_SCORE["f32"], p.k)
    exact = check_ids(g["ids"], ref["doc_score"], p.k)
    e = np.abs(g["out"] - ref["out"]).max()
    _log(f"cfg1: score err {err:.3g}, ids exact-branch {exact}, attention max-abs {e:.3g}")
    assert e <= ATOL_ATTN["f32"]
    assert g["ids"][0, 0] == host.needles[0]          # the planted needle ranks first


def test_preset_1m_full_ranking():
    p = configs.cfg2()
    host = HostLayer(p, 0)
    g = GpuLayer(p, 0, host).run()
    _log("cfg2: GPU layer done; oracle ranking of all 2048 documents")
    ref = host.doc_scores(np.arange(p.n_docs))
    err = check_scores(g["doc_score"], ref, RTOL_SCORE["bf16"], p.k)
    exact = check_ids(g["ids"], ref, p.k)
    out_ref = host.attention(0, g["ids"][0])
    e = np.abs(g["out"][0] - out_ref).max()
    _log(f"cfg2: score err {err:.3g}, ids exact-branch {exact}, attention max-abs {e:.3g}, "
         f"needle recall {_needle_recall(p, host, g)}")
    assert e <= ATOL_ATTN["bf16"]


@pytest.mark.parametrize("name,tier", [("cfg3", "hbm"), ("cfg4", "hbm"), ("cfg4", "host"), ("cfg5", "hbm")])
def test_preset_full_size_sampled(name, tier):
    p = configs.PRESETS[name]()
    layer = 17 if name == "cfg4" else 5
    host = HostLayer(p, layer)
    # HBM tier: the selected rows are read in place, with top-k and the
    # context index in one call (the path bench.py times); host tier: the
    # selected rows are gathered over the host link
    mode = M.MSA_SRC_HOST_MAPPED if tier == "host" else M.MSA_SRC_DEVICE
    g = GpuLayer(p, layer, host, src_mode=mode, indexed=tier == "hbm").run()
    _log(f"{name}: GPU layer {layer} done (ctx_len {g['ctx_len'][:4].tolist()}...)")
    _check_sampled(p, host, g, n_random=120 if name == "cfg5" else 200)
    for b in ([0, 13, 31] if p.B > 1 else [0]):
        out_ref = host.attention(b, g["ids"][b])
        e = np.abs(g["out"][b] - out_ref).max()
        _log(f"{name}: query {b} attention max-abs {e:.3g}")
        assert e <= ATOL_ATTN["bf16"]
    _log(f"{name}: needle recall {_needle_recall(p, host, g)}")
    assert _needle_recall(p, host, g) >= 0.75
