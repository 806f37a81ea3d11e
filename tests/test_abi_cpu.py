"""C-ABI contract checks that need no GPU.

libdss.so must load, export every function include/dss.h declares, and reject
bad arguments with the documented status before making any HIP call (so
these run on a machine without a GPU).  No compute call is made here.
"""

import ctypes
import os
import re

import pytest

from decode_step_sampling_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dss.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "dss_hooks.h")]

NULL = None
FAKE = 0x1000          # never dereferenced: validation fails before any use


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*|int32_t)\s+(dss_\w+)\s*\(",
                                 text, re.M)))


def header_macro(name):
    m = re.search(rf"#define\s+{name}\s+\(?\s*(-?\w+)", open(HEADER).read())
    return int(m.group(1).rstrip("uU"), 0)


def test_library_exports_every_declared_function():
    lib = _lib.load()
    names = declared_functions()
    assert len(names) == 22
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_header_constants_match_binding():
    for name in ("DSS_OK", "DSS_ERR_INVALID_ARG", "DSS_ERR_WORKSPACE", "DSS_ERR_UNSUPPORTED",
                 "DSS_ERR_HIP", "DSS_ERR_DEVICE", "DSS_FLAG_ORDER_JOINT", "DSS_FLAG_FROM_ZERO",
                 "DSS_FLAG_STREAMING", "DSS_FLAG_SINGLE_PIVOT"):
        assert header_macro(name) == getattr(_lib, name), name
    assert eval(re.search(r"#define\s+DSS_MAX_VOCAB\s+\((.*)\)", open(HEADER).read())
                .group(1)) == _lib.DSS_MAX_VOCAB
    for op, i in _lib.OP_IDS.items():
        assert header_macro({
            "sampling_from_probs": "DSS_OP_SAMPLING",
            "top_k_sampling_from_probs": "DSS_OP_TOP_K_SAMPLING",
            "top_p_sampling_from_probs": "DSS_OP_TOP_P_SAMPLING",
            "min_p_sampling_from_probs": "DSS_OP_MIN_P_SAMPLING",
            "top_k_top_p_sampling_from_probs": "DSS_OP_TOP_K_TOP_P",
            "top_k_renorm_probs": "DSS_OP_TOP_K_RENORM",
            "top_p_renorm_probs": "DSS_OP_TOP_P_RENORM",
            "top_k_mask_logits": "DSS_OP_TOP_K_MASK_LOGITS",
            "top_k_top_p_sampling_from_logits": "DSS_OP_TOP_K_TOP_P_FROM_LOGITS",
            "softmax": "DSS_OP_SOFTMAX",
            "top_k": "DSS_OP_TOP_K_SELECT",
            "chain_speculative_sampling": "DSS_OP_CHAIN_SPECULATIVE"}[op]) == i


def _plain(lib, probs=FAKE, rows=1, vocab=8, indices=NULL, n=1, samples=FAKE, flags=0,
           ws=NULL, ws_bytes=0):
    return lib.dss_sampling_from_probs(probs, rows, vocab, indices, n, NULL, 1, NULL, 0,
                                       samples, NULL, NULL, flags, ws, ws_bytes, NULL)


def _topk_topp(lib, flags=0, rows=1, vocab=8, n=1):
    return lib.dss_top_k_top_p_sampling_from_probs(FAKE, rows, vocab, NULL, n, NULL, 1, NULL, 0,
                                                   NULL, 5, NULL, 0.9, FAKE, NULL, NULL, flags,
                                                   NULL, 0, NULL)


def test_sampling_validation_before_any_hip_call():
    lib = _lib.load()
    assert _plain(lib, probs=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert _plain(lib, samples=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert _plain(lib, rows=-1) == _lib.DSS_ERR_INVALID_ARG
    assert _plain(lib, vocab=0) == _lib.DSS_ERR_INVALID_ARG
    assert _plain(lib, vocab=-5) == _lib.DSS_ERR_INVALID_ARG
    assert _plain(lib, n=-1, indices=FAKE) == _lib.DSS_ERR_INVALID_ARG
    assert _plain(lib, rows=2, n=3) == _lib.DSS_ERR_INVALID_ARG      # n != rows, no indices
    assert _plain(lib, vocab=_lib.DSS_MAX_VOCAB + 1) == _lib.DSS_ERR_UNSUPPORTED
    assert _plain(lib, flags=0x100) == _lib.DSS_ERR_INVALID_ARG
    # the joint order belongs to the combined filter only; there it is
    # validated and sized like top-k-first
    assert _plain(lib, flags=_lib.DSS_FLAG_ORDER_JOINT) == _lib.DSS_ERR_UNSUPPORTED
    assert _topk_topp(lib, flags=_lib.DSS_FLAG_ORDER_JOINT, vocab=0) == _lib.DSS_ERR_INVALID_ARG
    assert _topk_topp(lib, flags=_lib.DSS_FLAG_ORDER_JOINT, vocab=4096) == _lib.DSS_ERR_WORKSPACE
    assert _topk_topp(lib, vocab=4096) == _lib.DSS_ERR_WORKSPACE
    # empty batches are a successful no-op and touch nothing
    assert _plain(lib, probs=NULL, samples=NULL, rows=0, n=0) == _lib.DSS_OK
    assert _plain(lib, probs=NULL, samples=NULL, rows=3, n=0, indices=FAKE) == _lib.DSS_OK
    assert _topk_topp(lib, rows=0, n=0) == _lib.DSS_OK


def test_renorm_and_mask_validation():
    lib = _lib.load()
    for fn, param in ((lib.dss_top_k_renorm_probs, 3), (lib.dss_top_p_renorm_probs, 0.5),
                      (lib.dss_top_k_mask_logits, 3), (lib.dss_softmax, 1.0)):
        assert fn(NULL, FAKE, 1, 8, NULL, param, NULL, 0, NULL, 0, NULL) == _lib.DSS_ERR_INVALID_ARG
        assert fn(FAKE, NULL, 1, 8, NULL, param, NULL, 0, NULL, 0, NULL) == _lib.DSS_ERR_INVALID_ARG
        assert fn(FAKE, FAKE, -1, 8, NULL, param, NULL, 0, NULL, 0, NULL) == _lib.DSS_ERR_INVALID_ARG
        assert fn(FAKE, FAKE, 1, 0, NULL, param, NULL, 0, NULL, 0, NULL) == _lib.DSS_ERR_INVALID_ARG
        assert fn(FAKE, FAKE, 1, _lib.DSS_MAX_VOCAB + 1, NULL, param, NULL, 0, NULL, 0,
                  NULL) == _lib.DSS_ERR_UNSUPPORTED
        assert fn(FAKE, FAKE, 1, 8, NULL, param, NULL, 0x80, NULL, 0, NULL) == \
            _lib.DSS_ERR_INVALID_ARG
        assert fn(NULL, NULL, 0, 8, NULL, param, NULL, 0, NULL, 0, NULL) == _lib.DSS_OK


def test_workspace_size_and_strings():
    lib = _lib.load()
    for op in range(10):
        for rows, vocab, n in ((1, 8, 1), (64, 151936, 64), (512, 256000, 512), (0, 1, 0)):
            size = lib.dss_workspace_size(op, rows, vocab, n, 0)
            assert size >= 0
            # the streaming engine needs none; the logits path still holds its
            # probabilities, past the fixed region that other calls keep at zero
            probs_bytes = ((rows * vocab * 4 + 255) // 256) * 256 if op == 8 and n > 0 else 0
            fixed = FIXED_REGION_BYTES if op == 8 and n > 0 else 0
            assert lib.dss_workspace_size(op, rows, vocab, n, _lib.DSS_FLAG_STREAMING) == \
                probs_bytes + fixed
    for code in (0, -1, -2, -3, -4, -5):
        assert _lib.strerror(code) not in ("", "unknown status")
    assert _lib.strerror(7) == "unknown status"
    assert lib.dss_version() >= 100
    # the timing hook takes both event handles or neither; no HIP call is made
    assert lib.dss_set_timing_events(ctypes.c_void_p(16), None) == _lib.DSS_ERR_INVALID_ARG
    assert lib.dss_set_timing_events(None, None) == _lib.DSS_OK
    # the streaming-read reference checks its arguments before touching HIP
    out = ctypes.c_void_p(16)
    assert lib.dss_stream_read_reference(None, 4, out, None) == _lib.DSS_ERR_INVALID_ARG
    assert lib.dss_stream_read_reference(ctypes.c_void_p(16), 6, out, None) == _lib.DSS_ERR_INVALID_ARG
    assert lib.dss_stream_read_reference(ctypes.c_void_p(18), 8, out, None) == _lib.DSS_ERR_INVALID_ARG
    assert lib.dss_stream_read_reference(ctypes.c_void_p(16), 8, None, None) == _lib.DSS_ERR_INVALID_ARG
    # workspace state: argument checks and workspaces too small to hold the
    # resident slots need no HIP call
    flags = (ctypes.c_uint8 * 256)()
    assert lib.dss_workspace_status(None, 64, flags, None) == _lib.DSS_ERR_INVALID_ARG
    assert lib.dss_workspace_status(None, 0, flags, None) == 0
    assert lib.dss_workspace_status(ctypes.c_void_p(16), 4096, None, None) == 0
    assert lib.dss_set_spin_limit(2**64 - 1) == _lib.DSS_OK   # restores the default
    # forced foreign hand-offs: 0 or 1 only
    for bad in (2, -1):
        assert lib.dss_set_handoff_test(bad) == _lib.DSS_ERR_INVALID_ARG
    assert lib.dss_set_handoff_test(0) == _lib.DSS_OK
    # forced split slices: powers of two up to 16, or 0; the workspace follows
    for bad in (3, 32, -1):
        assert lib.dss_set_split_slices(bad) == _lib.DSS_ERR_INVALID_ARG
    auto = lib.dss_workspace_size(4, 1, 151936, 1, 0)
    assert lib.dss_set_split_slices(4) == _lib.DSS_OK
    try:
        assert lib.dss_workspace_size(4, 1, 151936, 1, 0) < auto    # W=16 by default
    finally:
        assert lib.dss_set_split_slices(0) == _lib.DSS_OK
    assert lib.dss_workspace_size(4, 1, 151936, 1, 0) == auto


def test_noalloc_entry_point_validation():
    """Host checks of the allocation-free call, before any HIP call: the
    same argument checks as the workspace call, and shapes whose scratch
    would exceed the library's 64 MiB static array are refused."""
    lib = _lib.load()
    fn = lib.dss_top_k_top_p_sampling_from_probs_noalloc

    def call(probs=FAKE, rows=4, vocab=1000, n=4, indices=NULL, samples=FAKE, flags=0):
        return fn(probs, rows, vocab, indices, n, NULL, 1, NULL, 0, NULL, 5, NULL, 0.9, samples,
                  NULL, NULL, flags, NULL)
    assert call(probs=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert call(samples=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert call(rows=3) == _lib.DSS_ERR_INVALID_ARG            # n != rows without indices
    assert call(flags=0x100) == _lib.DSS_ERR_INVALID_ARG
    assert call(vocab=_lib.DSS_MAX_VOCAB + 1) == _lib.DSS_ERR_UNSUPPORTED
    assert call(probs=NULL, samples=NULL, rows=0, n=0) == _lib.DSS_OK
    assert call(rows=4096, vocab=151936, n=4096) == _lib.DSS_ERR_WORKSPACE


# control words (16 KiB), 256 resident slots of 67,840 bytes, 256 key lists of
# 8192 words: the region every call leaves at zero or owns
FIXED_REGION_BYTES = 16384 + 256 * 67840 + 256 * 8192 * 4


@pytest.mark.parametrize("flags", [0, _lib.DSS_FLAG_STREAMING, _lib.DSS_FLAG_FROM_ZERO,
                                   _lib.DSS_FLAG_ORDER_JOINT])
@pytest.mark.parametrize("rows,vocab,n", [(64, 151936, 64), (3, 50257, 5), (2, 1000, 2),
                                          (1, 7, 1), (256, 128256, 512)])
def test_logits_probabilities_never_overlap_the_fixed_region(flags, rows, vocab, n):
    """The from-logits call places its probabilities at the end of its
    workspace (size - the probabilities' bytes); that offset must lie past the
    control words and resident slots for every shape and flag."""
    lib = _lib.load()
    size = lib.dss_workspace_size(8, rows, vocab, n, flags)
    probs_bytes = ((rows * vocab * 4 + 255) // 256) * 256
    assert size - probs_bytes >= FIXED_REGION_BYTES
    # and the sampling call on those probabilities fits the engine part
    assert size - probs_bytes >= lib.dss_workspace_size(4, rows, vocab, n, flags)


def test_top_k_selection_validation():
    lib = _lib.load()

    def call(x=FAKE, rows=1, vocab=8, k=3, values=FAKE, indices=FAKE, flags=0, ws=NULL,
             ws_bytes=0):
        return lib.dss_top_k(x, rows, vocab, k, values, indices, NULL, flags, ws, ws_bytes, NULL)
    assert call(x=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert call(values=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert call(indices=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert call(k=0) == _lib.DSS_ERR_INVALID_ARG
    assert call(k=9) == _lib.DSS_ERR_INVALID_ARG               # k > vocab
    assert call(rows=-1) == _lib.DSS_ERR_INVALID_ARG
    assert call(flags=0x100) == _lib.DSS_ERR_INVALID_ARG
    assert call(vocab=10000, k=4097) == _lib.DSS_ERR_UNSUPPORTED
    assert call(x=NULL, values=NULL, indices=NULL, rows=0) == _lib.DSS_OK
    # B=64, V=151936: the split engine (k <= 2048) needs its hand-off area;
    # the one-work-group path (k above 2048, or STREAMING) needs none
    need = lib.dss_workspace_size(10, 64, 151936, 64, 0)
    assert need > 0
    assert lib.dss_workspace_size(10, 64, 151936, 64, _lib.DSS_FLAG_STREAMING) == 0
    assert call(rows=64, vocab=151936, k=50) == _lib.DSS_ERR_WORKSPACE
    assert call(rows=64, vocab=151936, k=50, ws=FAKE, ws_bytes=need - 1) == _lib.DSS_ERR_WORKSPACE
    for kw in (dict(k=3000), dict(k=50, flags=_lib.DSS_FLAG_STREAMING),
               dict(k=50, ws=FAKE, ws_bytes=need)):
        assert call(rows=64, vocab=151936, **kw) != _lib.DSS_ERR_WORKSPACE, kw


def test_logits_sampling_validation():
    lib = _lib.load()

    def call(logits=FAKE, rows=1, vocab=8, indices=NULL, n=1, samples=FAKE, flags=0, ws=NULL,
             ws_bytes=0):
        return lib.dss_top_k_top_p_sampling_from_logits(
            logits, rows, vocab, indices, n, NULL, 1, NULL, 0, NULL, 5, NULL, 0.9, NULL, 1.0,
            samples, NULL, NULL, flags, ws, ws_bytes, NULL)
    assert call(logits=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert call(samples=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert call(vocab=0) == _lib.DSS_ERR_INVALID_ARG
    assert call(rows=2, n=3) == _lib.DSS_ERR_INVALID_ARG
    assert call(flags=0x100) == _lib.DSS_ERR_INVALID_ARG
    assert call(vocab=_lib.DSS_MAX_VOCAB + 1) == _lib.DSS_ERR_UNSUPPORTED
    assert call() == _lib.DSS_ERR_WORKSPACE                        # probabilities need room
    need = lib.dss_workspace_size(8, 1, 8, 1, 0)
    assert need >= 32
    assert call(ws=FAKE, ws_bytes=need - 1) == _lib.DSS_ERR_WORKSPACE
    assert call(logits=NULL, samples=NULL, rows=0, n=0) == _lib.DSS_OK


def test_binding_refuses_cpu_tensors():
    import torch
    import decode_step_sampling_amd as dss
    with pytest.raises(ValueError):
        dss.sampling_from_probs(torch.ones(2, 8))
    with pytest.raises(ValueError):
        dss.top_p_renorm_probs(torch.ones(2, 8), 0.5)


def test_chain_speculative_validation():
    lib = _lib.load()

    def call(q=FAKE, ids=FAKE, p=FAKE, rows=1, n=2, vocab=8, tokens=FAKE, acc=FAKE, flags=0,
             ws=NULL, ws_bytes=0):
        return lib.dss_chain_speculative_sampling(q, ids, p, rows, n, vocab, NULL, 1, NULL, 0,
                                                  tokens, acc, NULL, flags, ws, ws_bytes, NULL)
    assert call(p=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert call(tokens=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert call(acc=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert call(q=NULL) == _lib.DSS_ERR_INVALID_ARG          # drafts need their rows
    assert call(ids=NULL) == _lib.DSS_ERR_INVALID_ARG
    assert call(n=-1) == _lib.DSS_ERR_INVALID_ARG
    assert call(vocab=0) == _lib.DSS_ERR_INVALID_ARG
    assert call(flags=0x100) == _lib.DSS_ERR_INVALID_ARG
    assert call(n=65) == _lib.DSS_ERR_UNSUPPORTED             # more drafts than one wave
    assert call(vocab=6) == _lib.DSS_ERR_UNSUPPORTED          # rows not in 16-byte vectors
    assert call(p=ctypes.c_void_p(20)) == _lib.DSS_ERR_UNSUPPORTED
    assert call(rows=0, p=NULL, tokens=NULL, acc=NULL) == _lib.DSS_OK
    # B=64, V=151936: W > 1, so the hand-off needs its workspace
    need = lib.dss_workspace_size(11, 64, 151936, 4, 0)
    assert need > 0
    assert call(rows=64, n=4, vocab=151936) == _lib.DSS_ERR_WORKSPACE
    assert call(rows=64, n=4, vocab=151936, ws=FAKE, ws_bytes=need - 1) == _lib.DSS_ERR_WORKSPACE
    assert call(rows=64, n=4, vocab=151936, ws=FAKE, ws_bytes=need) != _lib.DSS_ERR_WORKSPACE
    # n = 0 needs no draft arrays
    assert call(q=NULL, ids=NULL, n=0, rows=64, vocab=151936, ws=FAKE,
                ws_bytes=need) != _lib.DSS_ERR_INVALID_ARG


def test_workspace_covers_the_pair_search_plans():
    """Top-k then top-p with a scalar k may run the resident pair search,
    whose plans reach vocabularies the other resident plans do not (up to
    sixteen slices of 64 values per thread): the workspace size must cover
    its fixed region there, and a call whose buffer is smaller than the plan
    it would launch is refused before any HIP call."""
    lib = _lib.load()
    for vocab in (528384, 985600, 2**20 - 4):
        size = lib.dss_workspace_size(4, 2, vocab, 2, 0)
        assert size >= FIXED_REGION_BYTES, (vocab, size)
        r = lib.dss_top_k_top_p_sampling_from_probs(FAKE, 2, vocab, NULL, 2, NULL, 1, NULL, 0,
                                                    NULL, 1000, NULL, 0.9, FAKE, NULL, NULL, 0,
                                                    FAKE, size - 1, NULL)
        assert r == _lib.DSS_ERR_WORKSPACE, (vocab, r)
        # no workspace at all (a size query of 0 once left callers passing none)
        r = lib.dss_top_k_top_p_sampling_from_probs(FAKE, 2, vocab, NULL, 2, NULL, 1, NULL, 0,
                                                    NULL, 1000, NULL, 0.9, FAKE, NULL, NULL, 0,
                                                    NULL, 0, NULL)
        assert r == _lib.DSS_ERR_WORKSPACE, (vocab, r)


def test_queried_workspace_always_suffices():
    """A sampling call given exactly dss_workspace_size bytes is never refused
    for its workspace, whatever engine and plan it would take (the call then
    stops at the device check on a machine without a GPU)."""
    import itertools
    lib = _lib.load()

    def call(op, rows, vocab, n, k, karr, flags, ws, wsb):
        head = (FAKE, rows, vocab, FAKE if n != rows else NULL, n, NULL, 1, NULL, 0)
        tail = (FAKE, NULL, NULL, flags, ws, wsb, NULL)
        if op == 0:
            return lib.dss_sampling_from_probs(*head, *tail)
        if op == 1:
            return lib.dss_top_k_sampling_from_probs(*head, karr, k, *tail)
        if op == 2:
            return lib.dss_top_p_sampling_from_probs(*head, NULL, 0.9, *tail)
        if op == 3:
            return lib.dss_min_p_sampling_from_probs(*head, NULL, 0.1, *tail)
        return lib.dss_top_k_top_p_sampling_from_probs(*head, karr, k, NULL, 0.9, *tail)

    shapes = itertools.product((1, 2, 4, 64, 300, 512),
                               (1024, 32000, 50257, 151936, 256000, 528384, 2**20 - 4, 2**20))
    for rows, vocab in shapes:
        for op in range(5):
            ks = ((50, NULL), (1000, NULL), (3000, NULL), (9000, NULL), (0, FAKE)) if op in (1, 4) \
                else ((50, NULL),)
            for n, (k, karr), flags in itertools.product((rows, 2 * rows), ks,
                                                         (0, _lib.DSS_FLAG_STREAMING)):
                need = lib.dss_workspace_size(op, rows, vocab, n, flags)
                r = call(op, rows, vocab, n, k, karr, flags, FAKE if need else NULL, need)
                assert r != _lib.DSS_ERR_WORKSPACE, (op, rows, vocab, n, k, karr is not NULL, flags)
