"""Sorting-free decode-step sampling for AMD Instinct MI355X (gfx950).

Python binding of libdss.so: torch tensors in, device pointers and the
current HIP stream out to the C ABI.  Every step of every op runs in the
library's HIP kernels; this module only marshals arguments and allocates the
output tensors.  Names follow the FlashInfer sampling API the pages list
(charlestar explainer, "当前 FlashInfer API 应怎样选择").

Tensors: ``probs`` / ``logits`` are float32 [rows, vocab] on a GPU.  Per
output parameters (``top_k``, ``top_p``, ``min_p``) are Python scalars or
1-D tensors (int32 / float32) with one entry per output.  ``seed`` and
``offset`` are Python ints (one stream per output index) or int64 tensors
with one value per output, read as unsigned 64-bit.
"""

import ctypes

import torch

from . import _lib
from ._lib import (DSS_FLAG_FROM_ZERO, DSS_FLAG_ORDER_JOINT, DSS_FLAG_SINGLE_PIVOT,  # noqa: F401
                   DSS_FLAG_STREAMING,
                   DssError, OP_IDS)

__all__ = [
    "sampling_from_probs", "top_k_sampling_from_probs", "top_p_sampling_from_probs",
    "min_p_sampling_from_probs", "top_k_top_p_sampling_from_probs",
    "top_k_renorm_probs", "top_p_renorm_probs", "top_k_mask_logits",
    "softmax", "top_k_top_p_sampling_from_logits", "top_k", "chain_speculative_sampling",
    "workspace_status", "reset_workspace",
    "DssError", "DSS_FLAG_FROM_ZERO", "DSS_FLAG_STREAMING", "DSS_FLAG_ORDER_JOINT",
    "DSS_FLAG_SINGLE_PIVOT",
]

_U64_MASK = (1 << 64) - 1
_workspaces = {}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(device, nbytes):
    """Zero-filled scratch kept per (device, stream); the kernels leave it
    zeroed.  Calls on different streams may run concurrently and so get
    different buffers.  A buffer is allocated while its stream is current, so
    the caching allocator hands its memory back only to work ordered after
    the kernels that used it when it grows."""
    if nbytes == 0:
        return None, 0
    key = (device, _stream(device))
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.device(device):
            buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    return buf.data_ptr(), buf.numel()


def workspace_status(device=None):
    """Resident control blocks of this stream's cached workspace whose row
    barrier was given up (dss_workspace_status): a list of slot numbers,
    empty when the workspace is clean.  Waits for the stream."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    buf = _workspaces.get((device, _stream(device)))
    if buf is None:
        return []
    flags = (ctypes.c_uint8 * 256)()
    with torch.cuda.device(device):
        n = _lib.load().dss_workspace_status(buf.data_ptr(), buf.numel(), flags, _stream(device))
    if n < 0:
        _lib.check(n, "workspace_status")
    return [i for i in range(256) if flags[i]]


def reset_workspace(device=None):
    """Zero this stream's cached workspace again (after a resident wait gave
    up: see workspace_status).  Enqueued on the current stream."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    buf = _workspaces.get((device, _stream(device)))
    if buf is not None:
        buf.zero_()


def _check_rows(x, name):
    if not (isinstance(x, torch.Tensor) and x.is_cuda and x.dtype == torch.float32
            and x.dim() == 2 and x.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous float32 [rows, vocab] GPU tensor")


def _param(v, dtype, n, device, name):
    """(device pointer or None, scalar) for a per-output parameter."""
    if isinstance(v, torch.Tensor):
        if v.dtype != dtype or v.device != device or v.numel() != n or not v.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dtype} tensor with {n} entries "
                             f"on {device}")
        return v, (0 if dtype == torch.int32 else 0.0)
    return None, (int(v) if dtype == torch.int32 else float(v))


def _rng(v, n, device, name):
    if isinstance(v, torch.Tensor):
        if v.dtype not in (torch.int64, torch.uint64) or v.device != device \
                or v.numel() != n or not v.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 64-bit integer tensor with {n} "
                             f"entries on {device}")
        return v, 0
    return None, int(v) & _U64_MASK


def _sample(fn_name, probs, params, indices, seed, offset, return_valid, return_rounds,
            flags):
    _check_rows(probs, "probs")
    device = probs.device
    rows, vocab = probs.shape
    if indices is not None:
        if indices.dtype != torch.int32 or indices.device != device or indices.dim() != 1:
            raise ValueError("indices must be a 1-D int32 tensor on the probs device")
        indices = indices.contiguous()
        n = indices.numel()
    else:
        n = rows
    if seed is None:
        seed = int(torch.randint(0, 2**62, (1,)).item())
    seed_arr, seed_val = _rng(seed, n, device, "seed")
    off_arr, off_val = _rng(offset, n, device, "offset")
    samples = torch.empty(n, dtype=torch.int32, device=device)
    valid = torch.empty(n, dtype=torch.uint8, device=device) if return_valid else None
    rounds = torch.empty(n, dtype=torch.int32, device=device) if return_rounds else None
    lib = _lib.load()
    ws, ws_bytes = _workspace(device, lib.dss_workspace_size(
        OP_IDS[fn_name], rows, vocab, n, flags))
    args = [probs.data_ptr(), rows, vocab, _ptr(indices), n, _ptr(seed_arr), seed_val,
            _ptr(off_arr), off_val]
    keep = []
    for value, dtype, name, *count in params:   # count: entries of an array (default n)
        arr, scalar = _param(value, dtype, count[0] if count else n, device, name)
        keep.append(arr)
        args += [_ptr(arr), scalar]
    args += [samples.data_ptr(), _ptr(valid), _ptr(rounds), flags, ws, ws_bytes,
             _stream(device)]
    with torch.cuda.device(device):
        _lib.check(getattr(lib, "dss_" + fn_name)(*args), fn_name)
    out = [samples]
    if return_valid:
        out.append(valid)
    if return_rounds:
        out.append(rounds)
    return out[0] if len(out) == 1 else tuple(out)


def sampling_from_probs(probs, *, indices=None, seed=None, offset=0, return_valid=False,
                        return_rounds=False, flags=0):
    """Inverse-transform sampling of one token per output."""
    return _sample("sampling_from_probs", probs, [], indices, seed, offset, return_valid,
                   return_rounds, flags)


def top_k_sampling_from_probs(probs, top_k, *, indices=None, seed=None, offset=0,
                              return_valid=False, return_rounds=False, flags=0):
    return _sample("top_k_sampling_from_probs", probs, [(top_k, torch.int32, "top_k")],
                   indices, seed, offset, return_valid, return_rounds, flags)


def top_p_sampling_from_probs(probs, top_p, *, indices=None, seed=None, offset=0,
                              return_valid=False, return_rounds=False, flags=0):
    return _sample("top_p_sampling_from_probs", probs, [(top_p, torch.float32, "top_p")],
                   indices, seed, offset, return_valid, return_rounds, flags)


def min_p_sampling_from_probs(probs, min_p, *, indices=None, seed=None, offset=0,
                              return_valid=False, return_rounds=False, flags=0):
    return _sample("min_p_sampling_from_probs", probs, [(min_p, torch.float32, "min_p")],
                   indices, seed, offset, return_valid, return_rounds, flags)


def top_k_top_p_sampling_from_probs(probs, top_k, top_p, *, indices=None, seed=None,
                                    offset=0, filter_apply_order="top_k_first",
                                    return_valid=False, return_rounds=False, flags=0):
    if filter_apply_order == "joint":
        flags |= DSS_FLAG_ORDER_JOINT
    elif filter_apply_order != "top_k_first":
        raise ValueError("filter_apply_order must be 'top_k_first' or 'joint'")
    return _sample("top_k_top_p_sampling_from_probs", probs,
                   [(top_k, torch.int32, "top_k"), (top_p, torch.float32, "top_p")],
                   indices, seed, offset, return_valid, return_rounds, flags)


def _renorm(fn_name, x, value, dtype, name, out, return_status, flags):
    _check_rows(x, "input")
    device = x.device
    rows, vocab = x.shape
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_rows(out, "out")
        if out.shape != x.shape or out.device != device:
            raise ValueError("out must match the input's shape and device")
    status = torch.empty(rows, dtype=torch.uint8, device=device) if return_status else None
    arr, scalar = _param(value, dtype, rows, device, name)
    lib = _lib.load()
    ws, ws_bytes = _workspace(device, lib.dss_workspace_size(OP_IDS[fn_name], rows, vocab,
                                                             rows, flags))
    with torch.cuda.device(device):
        _lib.check(getattr(lib, "dss_" + fn_name)(
            x.data_ptr(), out.data_ptr(), rows, vocab, _ptr(arr), scalar,
            _ptr(status), flags, ws, ws_bytes, _stream(device)), fn_name)
    return (out, status) if return_status else out


def top_k_renorm_probs(probs, top_k, *, out=None, return_status=False, flags=0):
    """Keep the top-k probabilities of each row (ties kept) and renormalise."""
    return _renorm("top_k_renorm_probs", probs, top_k, torch.int32, "top_k", out,
                   return_status, flags)


def top_p_renorm_probs(probs, top_p, *, out=None, return_status=False, flags=0):
    """Keep each row's top-p nucleus (ties kept) and renormalise."""
    return _renorm("top_p_renorm_probs", probs, top_p, torch.float32, "top_p", out,
                   return_status, flags)


def softmax(logits, temperature=1.0, *, out=None, return_status=False, flags=0):
    """Probabilities exp(z / T) / sum exp(z / T) per row (temperature: scalar
    or one value per row); invalid rows come out NaN with status 1."""
    return _renorm("softmax", logits, temperature, torch.float32, "temperature", out,
                   return_status, flags)


def top_k_top_p_sampling_from_logits(logits, top_k, top_p, temperature=1.0, *, indices=None,
                                     seed=None, offset=0, filter_apply_order="top_k_first",
                                     return_valid=False, return_rounds=False, flags=0):
    """softmax(logits / temperature) per row, then top_k_top_p_sampling_from_probs;
    the temperature is per row (scalar or `rows` values), k and p per output."""
    if filter_apply_order == "joint":
        flags |= DSS_FLAG_ORDER_JOINT
    elif filter_apply_order != "top_k_first":
        raise ValueError("filter_apply_order must be 'top_k_first' or 'joint'")
    rows = logits.shape[0] if isinstance(logits, torch.Tensor) and logits.dim() == 2 else 0
    return _sample("top_k_top_p_sampling_from_logits", logits,
                   [(top_k, torch.int32, "top_k"), (top_p, torch.float32, "top_p"),
                    (temperature, torch.float32, "temperature", rows)],
                   indices, seed, offset, return_valid, return_rounds, flags)


def top_k(x, k, *, return_status=False, flags=0):
    """The k largest entries of every row: (values, indices), each [rows, k],
    values descending, equal values by ascending index."""
    _check_rows(x, "input")
    device = x.device
    rows, vocab = x.shape
    values = torch.empty(rows, k, dtype=torch.float32, device=device)
    indices = torch.empty(rows, k, dtype=torch.int32, device=device)
    status = torch.empty(rows, dtype=torch.uint8, device=device) if return_status else None
    lib = _lib.load()
    ws, ws_bytes = _workspace(device, lib.dss_workspace_size(OP_IDS["top_k"], rows, vocab,
                                                             rows, flags))
    with torch.cuda.device(device):
        _lib.check(lib.dss_top_k(x.data_ptr(), rows, vocab, int(k), values.data_ptr(),
                                 indices.data_ptr(), _ptr(status), flags, ws, ws_bytes,
                                 _stream(device)), "top_k")
    return (values, indices, status) if return_status else (values, indices)


def chain_speculative_sampling(draft_probs, draft_token_ids, target_probs, *, seed=None,
                               offset=0, return_valid=False, flags=0):
    """Verify a chain of draft tokens per row against the target model.

    draft_probs [rows, n, vocab] float32, draft_token_ids [rows, n] int32,
    target_probs [rows, n + 1, vocab] float32.  Returns (tokens [rows, n + 1]
    int32: the accepted drafts, then the residual or bonus token, then -1;
    accepted [rows] int32) and, with return_valid, valid [rows] uint8."""
    def _chk(t, name, dtype, dims):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype
                and t.dim() == dims and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {dtype} {dims}-D GPU tensor")
    _chk(target_probs, "target_probs", torch.float32, 3)
    _chk(draft_probs, "draft_probs", torch.float32, 3)
    _chk(draft_token_ids, "draft_token_ids", torch.int32, 2)
    rows, n1, vocab = target_probs.shape
    n = n1 - 1
    device = target_probs.device
    if tuple(draft_probs.shape) != (rows, n, vocab) or tuple(draft_token_ids.shape) != (rows, n) \
            or draft_probs.device != device or draft_token_ids.device != device:
        raise ValueError("draft_probs [rows, n, vocab] and draft_token_ids [rows, n] must "
                         "match target_probs [rows, n + 1, vocab] on one device")
    if seed is None:
        seed = int(torch.randint(0, 2**62, (1,)).item())
    seed_arr, seed_val = _rng(seed, rows, device, "seed")
    off_arr, off_val = _rng(offset, rows, device, "offset")
    tokens = torch.empty(rows, n + 1, dtype=torch.int32, device=device)
    accepted = torch.empty(rows, dtype=torch.int32, device=device)
    valid = torch.empty(rows, dtype=torch.uint8, device=device) if return_valid else None
    lib = _lib.load()
    ws, ws_bytes = _workspace(device, lib.dss_workspace_size(
        OP_IDS["chain_speculative_sampling"], rows, vocab, n, flags))
    with torch.cuda.device(device):
        _lib.check(lib.dss_chain_speculative_sampling(
            draft_probs.data_ptr(), draft_token_ids.data_ptr(), target_probs.data_ptr(), rows, n,
            vocab, _ptr(seed_arr), seed_val, _ptr(off_arr), off_val, tokens.data_ptr(),
            accepted.data_ptr(), _ptr(valid), flags, ws, ws_bytes, _stream(device)),
            "chain_speculative_sampling")
    return (tokens, accepted, valid) if return_valid else (tokens, accepted)


def top_k_mask_logits(logits, top_k, *, out=None, return_status=False, flags=0):
    """Keep the top-k logits of each row (ties kept), set the rest to -inf."""
    return _renorm("top_k_mask_logits", logits, top_k, torch.int32, "top_k", out,
                   return_status, flags)
