"""C ABI checks that need no GPU: the library loads, exports every entry
point include/la.h declares, and validates arguments before any HIP call."""
import ctypes as C
import os
import re

import pytest

import lasynth
import lookahead_decoding_la_amd as la

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "la.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared() == sorted(la.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = la.lib()
    for name in declared():
        assert hasattr(lib, name), name


def _cfg(**kw):
    return la.make_config(lasynth.get_config("tiny", **kw), 256)


def test_workspace_bytes_validates():
    lib = la.lib()
    assert lib.la_workspace_bytes(C.byref(_cfg())) > 0
    assert lib.la_workspace_bytes(None) == 0
    for bad in [dict(N=1), dict(N=33), dict(W=-1), dict(n_kv_heads=3),
                dict(head_dim=31), dict(W=100, G=100)]:
        assert lib.la_workspace_bytes(C.byref(_cfg(**bad))) == 0, bad
    bf = la.make_config(lasynth.get_config("7b"), 1024)
    n = lib.la_workspace_bytes(C.byref(bf))
    # repacked weights + KV cache dominate: > 13.2 GB of weights alone
    assert n > 13_000_000_000


def test_create_rejects_bad_config_without_gpu():
    lib = la.lib()
    h = C.c_void_p()
    ptrs = (C.c_void_p * 400)(*([1] * 400))
    c = _cfg(N=1)
    assert lib.la_create(C.byref(c), ptrs, C.c_void_p(1), 1 << 20, None, C.byref(h)) == la.LA_ERR_INVALID_ARG
    assert not h.value
    c = la.make_config(lasynth.get_config("7b", dtype="bf16", d_model=4008), 1024)
    assert lib.la_create(C.byref(c), ptrs, C.c_void_p(1), 1 << 20, None, C.byref(h)) == la.LA_ERR_UNSUPPORTED
    # bf16 attention addresses a head's V^T rows with 32-bit offsets: max_ctx <= 2^24
    c = la.make_config(lasynth.get_config("7b", dtype="bf16"), (1 << 24) + 1)
    assert lib.la_create(C.byref(c), ptrs, C.c_void_p(1), 1 << 20, None, C.byref(h)) == la.LA_ERR_UNSUPPORTED
    c = _cfg()
    assert lib.la_create(C.byref(c), ptrs, C.c_void_p(1), 16, None, C.byref(h)) == la.LA_ERR_OUT_OF_CAPACITY
    assert lib.la_create(C.byref(c), None, C.c_void_p(1), 1 << 30, None, C.byref(h)) == la.LA_ERR_INVALID_ARG
    assert lib.la_create(C.byref(c), ptrs, C.c_void_p(1), 1 << 30, None, None) == la.LA_ERR_INVALID_ARG


def test_calls_on_null_context():
    lib = la.lib()
    r = la.LaStepResult()
    assert lib.la_step(None, C.byref(r)) == la.LA_ERR_INVALID_ARG
    assert lib.la_destroy(None) == la.LA_OK
    assert lib.la_step_rows(None) == 0
    assert lib.la_status_string(la.LA_ERR_STATE) == b"invalid state"
    toks = (C.c_int32 * 4)(1, 2, 3, 4)
    assert lib.la_seed_pool(None, toks, 4) == la.LA_ERR_INVALID_ARG
    us = C.c_float()
    assert lib.la_profile_kernel(None, 3, 8, C.byref(us)) == la.LA_ERR_INVALID_ARG
    assert lib.la_step_submit(None) == la.LA_ERR_INVALID_ARG
    assert lib.la_step_collect(None, C.byref(r)) == la.LA_ERR_INVALID_ARG


def test_attention_argument_checks_without_gpu():
    lib = la.lib()
    one = C.c_void_p(1)
    # head_dim other than 128 is unsupported; bad stride is invalid
    assert lib.la_attention(one, one, one, one, 32, 32, 64, 16, 256, 15, 5, 15, one, 1 << 30, None) == la.LA_ERR_UNSUPPORTED
    assert lib.la_attention(one, one, one, one, 32, 32, 128, 16, 100, 15, 5, 15, one, 1 << 30, None) == la.LA_ERR_INVALID_ARG
    assert lib.la_attention(one, one, one, one, 32, 32, 128, 200, 256, 15, 5, 15, one, 1 << 30, None) == la.LA_ERR_INVALID_ARG
    assert lib.la_attention(one, one, one, one, 32, 32, 128, 16, 256, 15, 5, 15, one, 8, None) == la.LA_ERR_OUT_OF_CAPACITY
    assert lib.la_attention(one, one, one, one, 32, 32, 128, 16, (1 << 24) + 64, 15, 5, 15, one, 1 << 30,
                            None) == la.LA_ERR_UNSUPPORTED
    assert lib.la_attention_workspace_bytes(32, 128, 1152, 15, 5, 15) > 0


def test_sampling_and_batch_argument_checks_without_gpu():
    lib = la.lib()
    one = C.c_void_p(1)
    toks = (C.c_int32 * 4)(1, 2, 3, 4)
    first = C.c_int32()
    assert lib.la_set_sampling(None, 0, 0.8, 0, 1.0, 1) == la.LA_ERR_INVALID_ARG
    assert lib.la_prefill_seq(None, 0, toks, 4, None, C.byref(first)) == la.LA_ERR_INVALID_ARG
    assert lib.la_seed_pool_seq(None, 0, toks, 4) == la.LA_ERR_INVALID_ARG
    assert lib.la_debug_pool_insert_seq(None, 0, 1, toks) == la.LA_ERR_INVALID_ARG
    # la_sample validates before touching the device
    assert lib.la_sample(None, 1, 16, 1.0, 0, 1.0, 0, one, one, None) == la.LA_ERR_INVALID_ARG
    assert lib.la_sample(one, 1, 16, 0.0, 0, 1.0, 0, one, one, None) == la.LA_ERR_INVALID_ARG
    assert lib.la_sample(one, 1, 16, 1.0, -1, 1.0, 0, one, one, None) == la.LA_ERR_INVALID_ARG
    assert lib.la_sample(one, 1, 16, 1.0, 0, 0.0, 0, one, one, None) == la.LA_ERR_INVALID_ARG
    assert lib.la_sample(one, 1, 16, 1.0, 0, 1.5, 0, one, one, None) == la.LA_ERR_INVALID_ARG
    assert lib.la_sample(one, 1, 32769, 1.0, 0, 1.0, 0, one, one, None) == la.LA_ERR_UNSUPPORTED
    assert lib.la_sample(one, 0, 16, 1.0, 0, 1.0, 0, one, one, None) == la.LA_OK


def test_batch_config_limits():
    import lasynth
    cfg = lasynth.get_config("7b")                      # 121 rows per sequence
    assert la.workspace_bytes(cfg, 1024, batch=2) > la.workspace_bytes(cfg, 1024, batch=1)
    assert la.workspace_bytes(cfg, 1024, batch=3) == 0  # 363 rows > 256
    assert la.workspace_bytes(cfg, 1024, batch=0) == la.workspace_bytes(cfg, 1024, batch=1)
    assert la.workspace_bytes(cfg, 1024, batch=-1) == 0


def _attn_splits(lib, H, W, N, G, ctx):
    """Split count the bf16 attention launch provides, read back from its workspace size."""
    T = 1 + (W + G) * (N - 1)
    rows16 = (T + 15) // 16 * 16
    nbytes = lib.la_attention_workspace_bytes(H, 128, ctx, W, N, G)
    for s in range(1, 17):
        rows = H * s * rows16
        al = lambda x: (x + 255) // 256 * 256
        if al(rows * 128 * 4) + al(rows * 8) == nbytes:
            return s
    raise AssertionError(nbytes)


def test_attention_split_counts_without_gpu():
    # Splits per (head, row group) for the longest context: about three 64-key chunks each
    # (one or two up to 16 rows, at most 8), capped near one wave per SIMD (1024 waves) up
    # to 128 rows and near 512 workgroups above; measured choices for the step shapes.
    lib = la.lib()
    assert _attn_splits(lib, 32, 15, 5, 15, 1152) == 4   # 7B step: 4 row groups x 2 waves
    assert _attn_splits(lib, 40, 10, 5, 10, 1280) == 4   # 13B step: 3 row groups x 2 waves
    assert _attn_splits(lib, 64, 7, 5, 7, 2240) == 4     # 34B step: one 64-row group x 4 waves
    assert _attn_splits(lib, 32, 0, 5, 0, 4096) == 8     # one-token decode: up to 8
    assert _attn_splits(lib, 32, 15, 5, 15, 256) == 2    # short context: ~3 chunks per split
    assert _attn_splits(lib, 32, 25, 5, 25, 4096) == 16  # > 128 rows: 512-workgroup cap, max 16
