"""MI355X-native MSA (Memory Sparse Attention) routing + sparse-attention path.

Thin Python binding over the C-ABI library ``libmsa.so`` (``include/msa.h``):
argument marshalling only; every step runs in the library's HIP kernels.
PyTorch provides device memory and streams.  Importing fails loudly if the
library has not been built (``python sparse_attention_long_msa_amd/build.py``).
"""
from ._binding import (  # noqa: F401
    MSA_BF16,
    MSA_F32,
    MSA_LAYOUT_ROWS,
    MSA_LAYOUT_TILED,
    MSA_SRC_DEVICE,
    MSA_SRC_HOST_MAPPED,
    MSA_SRC_HOST_MEMCPY,
    MsaError,
    lib,
    lib_path,
    msa_abi_version,
    msa_chunk_doc_map,
    msa_chunk_offsets,
    msa_chunk_scores,
    msa_segment_max,
    msa_context_append,
    msa_context_index,
    msa_encode,
    msa_exclude_docs,
    msa_gather_kv,
    msa_pool_backward,
    msa_pool_encode,
    msa_route_argmax,
    msa_route_argmax_workspace,
    msa_route_loss,
    msa_route_score_backward,
    msa_route_score,
    msa_rope_table,
    msa_rope_table_rows,
    msa_route_score_workspace,
    msa_sparse_attn,
    msa_sparse_attn_backward,
    msa_sparse_attn_backward_workspace,
    msa_sparse_attn_indexed,
    msa_sparse_attn_indexed_noalloc,
    MSA_NOALLOC_SCRATCH_BYTES,
    msa_sparse_attn_workspace,
    msa_topk,
    msa_topk_context_index,
    msa_tile_routing_keys,
    msa_topk_workspace,
    msa_stream_read,
    padded_chunks,
)
from .pipeline import LayerRunner, StepGraph  # noqa: F401
