"""The block-by-block oracle scoring that the full-size GPU parity tests use
(every document of a layer, pooled a block of documents at a time) equals the
per-document oracle scoring on small memories: token-level with ragged
lengths and a block boundary inside the memory, and pooled-level.  Raw rows
come from the host copy of the generator here (no GPU)."""
import numpy as np
import pytest

import synth
from synth import configs
from tests.preset_run import HostLayer, _STORE_CACHE


def _host_rows(host):
    p = host.p

    def gen(r0, r1):
        return synth.normal(p.seed, synth.stream_id(host.l, synth.T_KR), r0 * p.H * p.d, (r1 - r0) * p.H * p.d,
                            bf16=p.bf16).reshape(r1 - r0, p.H, p.d)
    return gen


def _small(pooled, B):
    lens = synth.lognormal_lengths(40_000, 600.0, 1.0, 64, 8192, seed=77) if not pooled else \
        synth.uniform_lengths(300, 512)
    return configs.Preset("small", 4242, True, 2, lens, 64, 8, 128, 32, B, 1 if B > 1 else 16, 64, 4,
                          B if B > 1 else 2, needle_per_query=B > 1, pooled_level=pooled, query_seed=4243)


@pytest.mark.parametrize("pooled,B", [(False, 1), (False, 3), (True, 1)])
def test_block_scores_equal_per_document_scores(pooled, B):
    p = _small(pooled, B)
    host = HostLayer(p, 1)
    _STORE_CACHE.clear()
    # block sizes that cut the memory into several blocks (and documents
    # into several scoring blocks)
    store = host.routing_store(gen_rows=_host_rows(host), blk_rows=5000 if not pooled else 700)
    got = host.all_doc_scores(store, blk_docs=7)
    docs = np.arange(p.n_docs)
    ref = host.doc_scores(docs)
    # the stores are bit-equal; the scores differ only by the BLAS summation order
    per_doc = np.concatenate([host.store(synth.T_KR, doc) for doc in docs])
    np.testing.assert_array_equal(store, per_doc)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)
    # the needles are in their query's top k
    for nd, b in host.owner.items():
        assert nd in np.argsort(-got[b])[: p.k]
    _STORE_CACHE.clear()
