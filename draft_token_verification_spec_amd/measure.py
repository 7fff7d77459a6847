"""Binding of libsvbench.so, the measurement aids of ``bench.py`` (not part
of the verification library): a read-bandwidth probe with the access pattern
of the verification's statistics kernel.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsvbench.so")
_lib = None


def lib_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m draft_token_verification_spec_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.svb_read_probe_sink_words.restype = ctypes.c_size_t
        lib.svb_read_probe_sink_words.argtypes = [ctypes.c_size_t]
        lib.svb_read_probe.restype = ctypes.c_int
        lib.svb_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                       ctypes.c_size_t]
        _lib = lib
    return _lib


def read_probe_sink_words(nbytes: int) -> int:
    return int(_load().svb_read_probe_sink_words(nbytes))


def read_probe(data: torch.Tensor, *, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Read ``data`` (contiguous device tensor, 16-byte aligned, a multiple of
    16 bytes) on the current stream; returns the sink (one XOR word per wave,
    as int32)."""
    if not data.is_cuda or not data.is_contiguous():
        raise ValueError("data must be a contiguous device tensor")
    nbytes = data.numel() * data.element_size()
    words = read_probe_sink_words(nbytes)
    if sink is None or sink.numel() < words:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=data.device)
    st = _load().svb_read_probe(ctypes.c_void_p(torch.cuda.current_stream(data.device).cuda_stream),
                                ctypes.c_void_p(data.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                sink.numel())
    if st != 0:
        raise RuntimeError(f"svb_read_probe failed (status {st})")
    return sink
