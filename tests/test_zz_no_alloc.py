"""la_attention_noalloc (the kernel-level attention for callers that cannot
allocate) against la_attention with a caller workspace, through the C ABI:
calls in a row, each smaller than the one before, all with split-KV
partials in the library's scratch array (the split kernel, and the
one-row kernel with its merge); the results must be
bit-identical (the same kernels in the same order).  A call needing more
than the array holds is refused before any launch."""
import ctypes as C

import pytest
import torch

import lookahead_decoding_la_amd as la

pytestmark = pytest.mark.gpu


def _inputs(H, Hkv, prefix, W, N, G, seed):
    T = 1 + (W + G) * (N - 1)
    ctx = ((prefix + T + 63) // 64) * 64
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn((T, H, 128), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((Hkv, ctx, 128), generator=g, device="cuda").to(torch.bfloat16)
    vt = torch.randn((Hkv, 128, ctx), generator=g, device="cuda").to(torch.bfloat16)
    return T, ctx, q, k, vt


# (heads, KV heads, committed prefix, W, N, G): all use split-KV partials
# (cache rows above the per-tile kernel's 2048 keys; one row: 8 key
# splits), each call a smaller problem than the one before
CASES = [(32, 32, 2100, 15, 5, 15), (32, 32, 2100, 0, 2, 0), (8, 2, 2100, 3, 3, 3)]


def test_noalloc_attention_equals_workspace_attention():
    lib = la.lib()
    for i, (H, Hkv, prefix, W, N, G) in enumerate(CASES):
        T, ctx, q, k, vt = _inputs(H, Hkv, prefix, W, N, G, seed=100 + i)
        need = int(lib.la_attention_workspace_bytes(H, 128, ctx, W, N, G))
        assert 0 < need <= la.LA_ATTENTION_NOALLOC_SCRATCH_BYTES
        ref = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        got = torch.full((T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        la.attention(q, k, vt, ref, H, Hkv, prefix, W, N, G)
        la.attention_noalloc(q, k, vt, got, H, Hkv, prefix, W, N, G)
        torch.cuda.synchronize()
        assert not torch.isnan(ref.float()).any()
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), (H, prefix, T)


def test_noalloc_attention_refuses_more_than_its_scratch():
    lib = la.lib()
    H, W, N, G, ctx = 256, 15, 5, 15, 2048
    assert lib.la_attention_workspace_bytes(H, 128, ctx, W, N, G) > la.LA_ATTENTION_NOALLOC_SCRATCH_BYTES
    p = C.c_void_p(1)  # never dereferenced: refused before any HIP call
    st = lib.la_attention_noalloc(p, p, p, p, H, H, 128, 0, ctx, W, N, G, None)
    assert st == la.LA_ERR_OUT_OF_CAPACITY
