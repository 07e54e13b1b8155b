"""ctypes binding of the device copy of the generator (synth_device.hip)."""
from __future__ import annotations

import ctypes
import os

import torch

from . import stream_id

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa_synth.so")
_h = None


def _lib():
    global _h
    if _h is None:
        if not os.path.exists(_LIB):
            raise ImportError(f"{_LIB} is not built: run `python sparse_attention_long_msa_amd/build.py`")
        _h = ctypes.CDLL(_LIB)
        _h.msa_synth_fill.restype = ctypes.c_int
        _h.msa_synth_fill.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return _h


def fill(out: torch.Tensor, seed: int, layer: int, tensor_id: int, start: int = 0, scale_pow2: int = 0,
         stream=None) -> torch.Tensor:
    """out.view(-1)[i] = generator value start + i of stream (layer, tensor_id)."""
    return fill_stream(out, seed, stream_id(layer, tensor_id), start, scale_pow2, stream)


def fill_stream(out: torch.Tensor, seed: int, stream_no: int, start: int = 0, scale_pow2: int = 0,
                stream=None) -> torch.Tensor:
    """out.view(-1)[i] = generator value start + i of the numbered stream."""
    assert out.is_cuda and out.is_contiguous()
    assert out.dtype in (torch.float32, torch.bfloat16)
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream.cuda_stream
    rc = _lib().msa_synth_fill(int(out.dtype == torch.bfloat16), seed, stream_no, start, out.numel(), scale_pow2,
                               out.data_ptr(), s)
    if rc != 0:
        raise RuntimeError(f"msa_synth_fill failed ({rc})")
    return out
