"""Python binding of libspecverify.so: batched draft-token verification and
the online acceptance estimator on AMD MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libspecverify.so``; torch supplies device memory and the current
stream.  There is no CPU fallback: if the library is not built, or a tensor is
not on a HIP device, the calls raise.

The functions carry the names of the C entry points in
``include/specverify.h`` and return the output tensors they allocate.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "SV_MAX_K",
    "SV_MAX_V",
    "SV_MAX_B",
    "SV_F32",
    "SV_BF16",
    "lib_path",
    "sv_workspace_size",
    "sv_status_string",
    "sv_spec_verify",
    "sv_filtered_workspace_size",
    "sv_spec_verify_filtered",
    "sv_av_score",
    "sv_av_fit_step",
    "sv_av_budget",
    "sv_av_calib_accumulate",
    "sv_av_calib_metrics",
    "sv_tts_grad",
    "sv_workspace_status",
    "sv_spec_verify_static",
    "SV_STATIC_SCRATCH_BYTES",
    "Workspace",
]

SV_MAX_K = 16
SV_MAX_V = 1 << 21
SV_MAX_B = 1 << 18
SV_BUDGET_MAX_ITEMS = 4096
SV_CALIB_AUC_BINS = 4096
SV_CALIB_WORDS = 33 + 2 * SV_CALIB_AUC_BINS
SV_F32, SV_BF16 = 0, 1
SV_STATIC_SCRATCH_BYTES = 8 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libspecverify.so")
_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_f = ctypes.c_float

_SIGNATURES = {
    "sv_workspace_size": (_sz, [_i, _i, _i, _i]),
    "sv_filtered_workspace_size": (_sz, [_i, _i, _i, _i]),
    "sv_spec_verify_filtered": (_i, [_p, _i, _i, _i, _i,
                                     _p, _p, _i64, _p, _p, _i64,
                                     _p, _p, _p, _p, _p, _p, _p, _p,
                                     _p, _p, _p, _p, _p, _p,
                                     _p, _sz]),
    "sv_spec_verify": (_i, [_p, _i, _i, _i, _i,
                            _p, _p, _i64, _p, _p, _i64,
                            _p, _p, _p, _p, _p, _p,
                            _p, _p, _p, _p, _p,
                            _p, _p, _p,
                            _p, _sz]),
    "sv_av_score": (_i, [_p, _i, _i, _i, _i, _p, _p, _i64, _p, _p, _p, _f, _p, _p, _p, _p, _sz]),
    "sv_av_fit_step": (_i, [_p, _i, _i, _p, _p, _p, _p, _f, _f, _f, _i]),
    "sv_status_string": (ctypes.c_char_p, [_i]),
    "sv_av_budget": (_i, [_p, _i, _i, _p, _p, _p, _p, _p, _p]),
    "sv_av_calib_accumulate": (_i, [_p, _i, _i, _p, _p, _p]),
    "sv_av_calib_metrics": (_i, [_p, _p, _p, _i]),
    "sv_tts_grad": (_i, [_p, _i, _i, _i, _i, _p, _p, _i64, _p, _p, _i64, _p, _p, _i64, _p, _p, _p, _f, _p, _p,
                         _p, _sz]),
    "sv_workspace_status": (_i, [_p, _p, _sz, _p, _i]),
    "sv_spec_verify_static": (_i, [_p, _i, _i, _i, _i,
                                   _p, _p, _i64, _p, _p, _i64,
                                   _p, _p, _p, _p, _p, _p,
                                   _p, _p, _p, _p, _p,
                                   _p, _p, _p]),
}


def lib_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is not built; run `python -m draft_token_verification_spec_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def sv_status_string(status: int) -> str:
    return _load().sv_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise RuntimeError(f"{what}: {sv_status_string(status)} (status {status})")


def sv_workspace_size(B: int, V: int, max_k: int, dtype: int) -> int:
    return int(_load().sv_workspace_size(B, V, max_k, dtype))


def sv_av_budget(score: torch.Tensor, num_draft: torch.Tensor, draft_cost_ms: torch.Tensor,
                 verify_cost_ms: torch.Tensor, *, out: Optional[dict] = None) -> dict:
    """The global draft budget of a batch; see ``sv_av_budget``.  ``score``
    float32 [B, max_k]; ``num_draft`` int32 [B]; both cost tables float32
    with at least B*max_k + 1 entries.  Returns ``num_kept`` int32 [B] and
    ``budget`` int32 [1], on the device (no host synchronisation)."""
    if score.dim() != 2:
        raise ValueError("score must be [B, max_k]")
    B, max_k = score.shape
    dev = score.device
    _dev(score, "score", torch.float32)
    _dev(num_draft, "num_draft", torch.int32, B)
    for name, t in (("draft_cost_ms", draft_cost_ms), ("verify_cost_ms", verify_cost_ms)):
        _dev(t, name, torch.float32)
        if t.numel() < B * max_k + 1:
            raise ValueError(f"{name} needs at least B*max_k + 1 = {B * max_k + 1} entries")
    o = {} if out is None else out
    _need(o, "num_kept", (B,), torch.int32, dev)
    _need(o, "budget", (1,), torch.int32, dev)
    _dev(o["num_kept"], "num_kept", torch.int32, B)
    _dev(o["budget"], "budget", torch.int32, 1)
    st = _load().sv_av_budget(_stream(dev), B, max_k, _ptr(score), _ptr(num_draft), _ptr(draft_cost_ms),
                              _ptr(verify_cost_ms), _ptr(o["num_kept"]), _ptr(o["budget"]))
    _check(st, "sv_av_budget")
    return o


def sv_av_calib_accumulate(score: torch.Tensor, labels: torch.Tensor, accum: torch.Tensor) -> None:
    """Add the labelled (score, label) items of one step to the calibration
    accumulator (float64 [SV_CALIB_WORDS], zero-filled before a stream's
    first step); see ``sv_av_calib_accumulate``."""
    if score.dim() != 2:
        raise ValueError("score must be [B, max_k]")
    B, max_k = score.shape
    dev = score.device
    _dev(score, "score", torch.float32)
    _dev(labels, "labels", torch.int8, B * max_k)
    _dev(accum, "accum", torch.float64, SV_CALIB_WORDS)
    _check(_load().sv_av_calib_accumulate(_stream(dev), B, max_k, _ptr(score), _ptr(labels), _ptr(accum)),
           "sv_av_calib_accumulate")


def sv_av_calib_metrics(accum: torch.Tensor, reset: bool = False, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """AUC, log-loss and ECE of the accumulated stream as a float64 [3]
    device tensor (no host synchronisation); ``reset`` zero-fills the
    accumulator afterwards."""
    dev = accum.device
    _dev(accum, "accum", torch.float64, SV_CALIB_WORDS)
    if out is None:
        out = torch.empty(3, dtype=torch.float64, device=dev)
    _dev(out, "out", torch.float64, 3)
    _check(_load().sv_av_calib_metrics(_stream(dev), _ptr(accum), _ptr(out), int(bool(reset))),
           "sv_av_calib_metrics")
    return out


def sv_tts_grad(draft_logits: torch.Tensor, draft_row_start: torch.Tensor, target_logits: torch.Tensor,
                target_row_start: torch.Tensor, num_draft: torch.Tensor, temperature: torch.Tensor,
                weights: torch.Tensor, max_k: int, lam: float = 0.0, *, prev_logits: Optional[torch.Tensor] = None,
                prev_row_start: Optional[torch.Tensor] = None, verify_workspace: Optional[Workspace] = None,
                out: Optional[dict] = None) -> dict:
    """Distillation gradient and loss over the canvas; see ``sv_tts_grad``.
    ``verify_workspace``: the Workspace of the sv_spec_verify call just made
    on the same rows, whose row statistics are then reused.  Returns ``grad``
    [B*max_k, V] (the logits' dtype) and ``loss`` float32 [B, max_k]."""
    dtype = _logits(target_logits, "target_logits")
    V = target_logits.shape[1]
    B = num_draft.numel()
    dev = target_logits.device
    if _logits(draft_logits, "draft_logits") != dtype or draft_logits.shape[1] != V:
        raise ValueError("draft_logits and target_logits must share dtype and V")
    _dev(draft_row_start, "draft_row_start", torch.int64, B)
    _dev(target_row_start, "target_row_start", torch.int64, B)
    _dev(num_draft, "num_draft", torch.int32)
    _dev(temperature, "temperature", torch.float32, B)
    _dev(weights, "weights", torch.float32, max_k)
    if prev_logits is not None:
        if _logits(prev_logits, "prev_logits") != dtype or prev_logits.shape[1] != V:
            raise ValueError("prev_logits must share dtype and V with the draft rows")
        _dev(prev_row_start, "prev_row_start", torch.int64, B)
    o = {} if out is None else out
    _need(o, "grad", (B * max_k, V), target_logits.dtype, dev)
    _need(o, "loss", (B, max_k), torch.float32, dev)
    _dev(o["grad"], "grad", target_logits.dtype, B * max_k * V)
    _dev(o["loss"], "loss", torch.float32, B * max_k)
    ws = None
    if verify_workspace is not None:
        ws = verify_workspace.get(dev, sv_workspace_size(B, V, max_k, dtype))
    st = _load().sv_tts_grad(
        _stream(dev), B, V, max_k, dtype, _ptr(draft_logits), _ptr(draft_row_start), draft_logits.stride(0),
        _ptr(target_logits), _ptr(target_row_start), target_logits.stride(0),
        _ptr(prev_logits), _ptr(prev_row_start), prev_logits.stride(0) if prev_logits is not None else V,
        _ptr(num_draft), _ptr(temperature), _ptr(weights), float(lam), _ptr(o["grad"]), _ptr(o["loss"]),
        _ptr(ws), ws.numel() if ws is not None else 0)
    _check(st, "sv_tts_grad")
    return o


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _dev(t: torch.Tensor, name: str, dtype: Optional[torch.dtype] = None, numel: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a HIP device (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} needs at least {numel} elements (got {t.numel()})")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _logits(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D [rows, V] tensor with unit stride along V")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a HIP device (got {t.device})")
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"{name} must be bfloat16 or float32 (got {t.dtype})")


def _need(o: dict, key: str, shape, dtype, dev):
    """Allocate output ``key`` unless the caller supplied it."""
    if key not in o:
        o[key] = torch.empty(shape, dtype=dtype, device=dev)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class Workspace:
    """Device workspace for sv_spec_verify / sv_av_score, zero-filled once.

    The kernels leave its counter arena at zero and write nothing else there,
    so one workspace serves any sequence of calls of any shapes on one stream.
    ``get`` replaces it by a larger zero-filled one when a call needs more.
    """

    def __init__(self):
        self._buf: dict = {}

    def peek(self, device: torch.device) -> Optional[torch.Tensor]:
        """The buffer held for ``device``, or None."""
        return self._buf.get((device.type, device.index))

    def get(self, device: torch.device, nbytes: int) -> torch.Tensor:
        key = (device.type, device.index)
        buf = self._buf.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._buf[key] = buf
        return buf


_default_ws = Workspace()


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def _verify_args(draft_logits, draft_row_start, target_logits, target_row_start, num_draft, draft_tokens,
                 temperature, u_accept, u_residual, u_bonus, max_k, av_params, want_feature, want_probs,
                 want_labels, out):
    """Check the verification's inputs, allocate missing outputs; returns
    (B, V, dtype, device, outputs, the arguments of the C call between the
    stream and the workspace)."""
    dtype = _logits(target_logits, "target_logits")
    V = target_logits.shape[1]
    B = num_draft.numel()
    dev = target_logits.device
    if max_k > 0:
        if _logits(draft_logits, "draft_logits") != dtype or draft_logits.shape[1] != V:
            raise ValueError("draft_logits and target_logits must share dtype and V")
    _dev(draft_row_start, "draft_row_start", torch.int64, B)
    _dev(target_row_start, "target_row_start", torch.int64, B)
    _dev(num_draft, "num_draft", torch.int32)
    _dev(draft_tokens, "draft_tokens", torch.int32, B * max_k)
    _dev(temperature, "temperature", torch.float32, B)
    _dev(u_accept, "u_accept", torch.float32, B * max_k)
    _dev(u_residual, "u_residual", torch.float32, B)
    _dev(u_bonus, "u_bonus", torch.float32, B)
    if av_params is not None:
        _dev(av_params, "av_params", torch.float32, max_k + 1)

    o = {} if out is None else out
    _need(o, "accept_len", (B), torch.int32, dev)
    _need(o, "out_tokens", (B, max_k + 1), torch.int32, dev)
    if want_labels:
        _need(o, "labels", (B, max_k), torch.int8, dev)
    if want_probs:
        _need(o, "p_draft", (B, max_k), torch.float32, dev)
        _need(o, "p_target", (B, max_k), torch.float32, dev)
    if want_feature:
        _need(o, "av_feature", (B, max_k), torch.float32, dev)
        if av_params is not None:
            _need(o, "av_score", (B, max_k), torch.float32, dev)
    for key, dt, n in (("accept_len", torch.int32, B), ("out_tokens", torch.int32, B * (max_k + 1)),
                       ("labels", torch.int8, B * max_k), ("p_draft", torch.float32, B * max_k),
                       ("p_target", torch.float32, B * max_k), ("av_feature", torch.float32, B * max_k),
                       ("av_score", torch.float32, B * max_k)):
        if key in o:
            _dev(o[key], key, dt, n)
    args = [B, V, max_k, dtype,
            _ptr(draft_logits) if max_k > 0 else None, _ptr(draft_row_start),
            draft_logits.stride(0) if max_k > 0 else V,
            _ptr(target_logits), _ptr(target_row_start), target_logits.stride(0),
            _ptr(num_draft), _ptr(draft_tokens), _ptr(temperature), _ptr(u_accept), _ptr(u_residual),
            _ptr(u_bonus), _ptr(o["accept_len"]), _ptr(o["out_tokens"]), _ptr(o.get("labels")),
            _ptr(o.get("p_draft")), _ptr(o.get("p_target")), _ptr(av_params), _ptr(o.get("av_feature")),
            _ptr(o.get("av_score"))]
    return B, V, dtype, dev, o, args


def sv_spec_verify(draft_logits: torch.Tensor, draft_row_start: torch.Tensor,
                   target_logits: torch.Tensor, target_row_start: torch.Tensor,
                   num_draft: torch.Tensor, draft_tokens: torch.Tensor, temperature: torch.Tensor,
                   u_accept: torch.Tensor, u_residual: torch.Tensor, u_bonus: torch.Tensor,
                   max_k: int, *, av_params: Optional[torch.Tensor] = None, want_feature: bool = False,
                   want_probs: bool = True, want_labels: bool = True, workspace: Optional[Workspace] = None,
                   out: Optional[dict] = None) -> dict:
    """Verify one step of B requests; see ``sv_spec_verify`` in specverify.h.

    ``draft_logits`` [rows, V] and ``target_logits`` [rows, V] (bf16 or fp32,
    same dtype); ``*_row_start`` int64 [B]; ``num_draft`` int32 [B];
    ``draft_tokens`` int32 [B, max_k]; ``temperature`` float32 [B];
    ``u_accept`` float32 [B, max_k]; ``u_residual``/``u_bonus`` float32 [B].
    Returns a dict with accept_len, out_tokens, and when requested labels,
    p_draft, p_target, av_feature, av_score.
    """
    B, V, dtype, dev, o, args = _verify_args(draft_logits, draft_row_start, target_logits, target_row_start,
                                             num_draft, draft_tokens, temperature, u_accept, u_residual, u_bonus,
                                             max_k, av_params, want_feature, want_probs, want_labels, out)
    nbytes = sv_workspace_size(B, V, max_k, dtype)
    if nbytes == 0 and B > 0:
        _check(-2, "sv_spec_verify")
    ws = (workspace or _default_ws).get(dev, nbytes)
    _check(_load().sv_spec_verify(_stream(dev), *args, _ptr(ws), ws.numel()), "sv_spec_verify")
    return o


def sv_spec_verify_static(draft_logits: torch.Tensor, draft_row_start: torch.Tensor,
                          target_logits: torch.Tensor, target_row_start: torch.Tensor,
                          num_draft: torch.Tensor, draft_tokens: torch.Tensor, temperature: torch.Tensor,
                          u_accept: torch.Tensor, u_residual: torch.Tensor, u_bonus: torch.Tensor,
                          max_k: int, *, av_params: Optional[torch.Tensor] = None, want_feature: bool = False,
                          want_probs: bool = True, want_labels: bool = True, out: Optional[dict] = None) -> dict:
    """``sv_spec_verify`` on the library's static scratch instead of a
    workspace; see ``sv_spec_verify_static``.  With every output supplied in
    ``out`` nothing is allocated; otherwise the missing outputs are."""
    _, _, _, dev, o, args = _verify_args(draft_logits, draft_row_start, target_logits, target_row_start,
                                         num_draft, draft_tokens, temperature, u_accept, u_residual, u_bonus,
                                         max_k, av_params, want_feature, want_probs, want_labels, out)
    _check(_load().sv_spec_verify_static(_stream(dev), *args), "sv_spec_verify_static")
    return o


def sv_filtered_workspace_size(B: int, V: int, max_k: int, dtype: int) -> int:
    return int(_load().sv_filtered_workspace_size(B, V, max_k, dtype))


def sv_spec_verify_filtered(draft_logits: torch.Tensor, draft_row_start: torch.Tensor,
                            target_logits: torch.Tensor, target_row_start: torch.Tensor,
                            num_draft: torch.Tensor, draft_tokens: torch.Tensor, temperature: torch.Tensor,
                            top_k: torch.Tensor, top_p: torch.Tensor, u_accept: torch.Tensor,
                            u_residual: torch.Tensor, u_bonus: torch.Tensor, max_k: int, *,
                            want_probs: bool = True, want_labels: bool = True, want_kept: bool = True,
                            workspace: Optional[Workspace] = None, out: Optional[dict] = None) -> dict:
    """Verify one step on top-k / top-p filtered rows; see
    ``sv_spec_verify_filtered``.  Arguments as for ``sv_spec_verify`` plus
    ``top_k`` int32 [B] and ``top_p`` float32 [B]; returns accept_len,
    out_tokens and, when requested, labels, p_draft, p_target and ``kept``
    int32 [B, 2*max_k + 1]."""
    dtype = _logits(target_logits, "target_logits")
    V = target_logits.shape[1]
    B = num_draft.numel()
    dev = target_logits.device
    if max_k > 0:
        if _logits(draft_logits, "draft_logits") != dtype or draft_logits.shape[1] != V:
            raise ValueError("draft_logits and target_logits must share dtype and V")
    _dev(draft_row_start, "draft_row_start", torch.int64, B)
    _dev(target_row_start, "target_row_start", torch.int64, B)
    _dev(num_draft, "num_draft", torch.int32)
    _dev(draft_tokens, "draft_tokens", torch.int32, B * max_k)
    _dev(temperature, "temperature", torch.float32, B)
    _dev(top_k, "top_k", torch.int32, B)
    _dev(top_p, "top_p", torch.float32, B)
    _dev(u_accept, "u_accept", torch.float32, B * max_k)
    _dev(u_residual, "u_residual", torch.float32, B)
    _dev(u_bonus, "u_bonus", torch.float32, B)
    o = {} if out is None else out
    _need(o, "accept_len", (B), torch.int32, dev)
    _need(o, "out_tokens", (B, max_k + 1), torch.int32, dev)
    if want_labels:
        _need(o, "labels", (B, max_k), torch.int8, dev)
    if want_probs:
        _need(o, "p_draft", (B, max_k), torch.float32, dev)
        _need(o, "p_target", (B, max_k), torch.float32, dev)
    if want_kept:
        _need(o, "kept", (B, 2 * max_k + 1), torch.int32, dev)
    for key, dt, n in (("accept_len", torch.int32, B), ("out_tokens", torch.int32, B * (max_k + 1)),
                       ("labels", torch.int8, B * max_k), ("p_draft", torch.float32, B * max_k),
                       ("p_target", torch.float32, B * max_k), ("kept", torch.int32, B * (2 * max_k + 1))):
        if key in o:
            _dev(o[key], key, dt, n)
    nbytes = sv_filtered_workspace_size(B, V, max_k, dtype)
    if nbytes == 0 and B > 0:
        _check(-2, "sv_spec_verify_filtered")
    ws = (workspace or _default_ws).get(dev, nbytes)
    st = _load().sv_spec_verify_filtered(
        _stream(dev), B, V, max_k, dtype,
        _ptr(draft_logits) if max_k > 0 else None, _ptr(draft_row_start),
        draft_logits.stride(0) if max_k > 0 else V,
        _ptr(target_logits), _ptr(target_row_start), target_logits.stride(0),
        _ptr(num_draft), _ptr(draft_tokens), _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(u_accept),
        _ptr(u_residual), _ptr(u_bonus), _ptr(o["accept_len"]), _ptr(o["out_tokens"]), _ptr(o.get("labels")),
        _ptr(o.get("p_draft")), _ptr(o.get("p_target")), _ptr(o.get("kept")), _ptr(ws), ws.numel())
    _check(st, "sv_spec_verify_filtered")
    return o


def sv_av_score(draft_logits: torch.Tensor, draft_row_start: torch.Tensor, num_draft: torch.Tensor,
                temperature: torch.Tensor, params: torch.Tensor, max_k: int, prune_threshold: float = 0.0,
                *, want_kept: bool = True, workspace: Optional[Workspace] = None,
                out: Optional[dict] = None) -> dict:
    """Estimator feature, score and kept count; see ``sv_av_score``."""
    dtype = _logits(draft_logits, "draft_logits")
    V = draft_logits.shape[1]
    B = num_draft.numel()
    dev = draft_logits.device
    _dev(draft_row_start, "draft_row_start", torch.int64, B)
    _dev(num_draft, "num_draft", torch.int32)
    _dev(temperature, "temperature", torch.float32, B)
    _dev(params, "params", torch.float32, max_k + 1)
    o = {} if out is None else out
    _need(o, "feature", (B, max_k), torch.float32, dev)
    _need(o, "score", (B, max_k), torch.float32, dev)
    if want_kept:
        _need(o, "num_kept", (B), torch.int32, dev)
    for key, dt, n in (("feature", torch.float32, B * max_k), ("score", torch.float32, B * max_k),
                       ("num_kept", torch.int32, B)):
        if key in o:
            _dev(o[key], key, dt, n)
    nbytes = sv_workspace_size(B, V, max_k, dtype)
    if nbytes == 0 and B > 0:
        _check(-2, "sv_av_score")
    ws = (workspace or _default_ws).get(dev, nbytes)
    st = _load().sv_av_score(_stream(dev), B, V, max_k, dtype, _ptr(draft_logits), _ptr(draft_row_start),
                             draft_logits.stride(0), _ptr(num_draft), _ptr(temperature), _ptr(params),
                             float(prune_threshold), _ptr(o["feature"]), _ptr(o["score"]),
                             _ptr(o.get("num_kept")), _ptr(ws), ws.numel())
    _check(st, "sv_av_score")
    return o


def sv_av_fit_step(feature: torch.Tensor, labels: torch.Tensor, params: torch.Tensor, accum: torch.Tensor,
                   damping_c: float = 10.0, ridge: float = 1e-6, do_update: bool = False,
                   max_step: float = 1.0) -> None:
    """One refit step, in place on ``params`` (float32 [max_k+1]) and
    ``accum`` (float64 [max_k, 6]); see ``sv_av_fit_step``."""
    if feature.dim() != 2:
        raise ValueError("feature must be [B, max_k]")
    B, max_k = feature.shape
    dev = feature.device
    _dev(feature, "feature", torch.float32)
    _dev(labels, "labels", torch.int8, B * max_k)
    _dev(params, "params", torch.float32, max_k + 1)
    _dev(accum, "accum", torch.float64, 6 * max_k)
    st = _load().sv_av_fit_step(_stream(dev), B, max_k, _ptr(feature), _ptr(labels), _ptr(params),
                                _ptr(accum), float(damping_c), float(ridge), float(max_step), int(bool(do_update)))
    _check(st, "sv_av_fit_step")


def sv_workspace_status(workspace: Optional[Workspace], device=None, clear: bool = True,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The status word of ``workspace`` on ``device`` (default: the current
    device) as an int32 [1] device tensor, 0 when every call on it completed
    normally; ``clear`` zeroes the word afterwards.  ``workspace`` None: the
    static scratch of ``sv_spec_verify_static``.  See ``sv_workspace_status``.
    A workspace never used on the device has status 0."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    if out is None:
        out = torch.empty(1, dtype=torch.int32, device=dev)
    _dev(out, "out", torch.int32, 1)
    if workspace is None:
        with torch.cuda.device(dev):
            _check(_load().sv_workspace_status(_stream(dev), None, 0, _ptr(out), int(bool(clear))),
                   "sv_workspace_status")
        return out
    ws = workspace.peek(dev)
    if ws is None:
        out.zero_()
        return out
    _check(_load().sv_workspace_status(_stream(dev), _ptr(ws), ws.numel(), _ptr(out), int(bool(clear))),
           "sv_workspace_status")
    return out
