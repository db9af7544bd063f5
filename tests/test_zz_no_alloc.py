"""engram_gated_residual_noalloc, the gated residual for callers that cannot
allocate, against engram_gated_residual through the C ABI.

Bar: the streams of two calls in a row (the second with fewer tokens, planned to
another kernel) equal engram_gated_residual's bit for bit -- the same kernels run
in the same order, only the scratch lives elsewhere -- and a call whose scratch
would not fit the library's array is refused before anything runs.
"""
import ctypes
import gc

import pytest
import torch

from engram_harness import DEV, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def eng():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import hashed_gram_memory_tid2eid_amd as e
    return e


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _call(eng, fn, L, rows, wkv, x, keep, T, *extra):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p
    args = [L.handle, P(rows.data_ptr()), rows.shape[1], wkv.handle, 4,
            P(keep.data_ptr()) if keep is not None else None, P(x.data_ptr())]
    return fn(*args, *extra, T, stream)


def test_noalloc_equals_gated_residual_on_two_calls(eng):
    # prefill geometry: 2 heads x 3 orders of 512 elements (k_pad 3,072) -> 4,096
    L = eng.engram_layout_create(vocab_size=8, compressed_vocab=4, pad_token_id=7, heads_per_order=2,
                                 rows=[100_000] * 3, row_dim=512, table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                 row_pitch_bytes=512)
    K, N, Tmax = L.info.k_pad, 4096, 1536
    g = torch.Generator(device=DEV)
    g.manual_seed(2026)
    rows = torch.randn((Tmax, K), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    x0 = torch.randn((Tmax, 4, N), generator=g, device=DEV).to(torch.bfloat16)
    keep = (torch.rand(Tmax, generator=g, device=DEV) > 0.1).to(torch.uint8)
    wkv = eng.engram_wkv_create(L, w, Tmax)
    v = torch.empty((Tmax, N), dtype=torch.float32, device=DEV)
    plans = []
    # first call: 1,536 tokens (the packed kernel); second: 256 (split-K, 4 slices)
    for T in (1536, 256):
        plans.append(wkv.plan(T))
        x_ref = x0[:T].clone()
        x_na = x0[:T].clone()
        assert _call(eng, eng._lib.engram_gated_residual, L, rows, wkv, x_ref, keep, T,
                     ctypes.c_void_p(v.data_ptr())) == 0
        assert _call(eng, eng._lib.engram_gated_residual_noalloc, L, rows, wkv, x_na, keep, T) == 0
        torch.cuda.synchronize()
        assert eng.engram_get_error() == 0
        assert torch.equal(x_ref.view(torch.int16), x_na.view(torch.int16)), T
        assert not torch.equal(x_na.view(torch.int16), x0[:T].view(torch.int16))
    assert [p[0] for p in plans] == ["packed", "splitk"], plans
    # past the array: 2,049 tokens x 4,096 floats of v (8 MiB floats hold 2,048)
    big = eng.engram_wkv_create(L, w, 4096)
    rows2 = torch.zeros((2049, K), dtype=torch.bfloat16, device=DEV)
    x2 = torch.zeros((2049, 4, N), dtype=torch.bfloat16, device=DEV)
    rc = _call(eng, eng._lib.engram_gated_residual_noalloc, L, rows2, big, x2, None, 2049)
    assert rc == eng.ENGRAM_E_SCRATCH
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    assert not x2.view(torch.int16).any()
    log(f"no-alloc gated residual: plans {plans} bit-identical to engram_gated_residual; "
        f"2,049 tokens refused ({eng.engram_strerror(rc)})")
    del rows, w, x0, v, wkv, big, rows2, x2
    _free()
