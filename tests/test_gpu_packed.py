"""The projection from the weight in matrix-core fragment order
(engram_pack_weight + engram_project_packed), through the C ABI.

Bars: the packed bytes sit where the header's index formula puts them (checked
element by element on the host); v is bit-identical to engram_project (16 x 16 x 32
matrix-core products against its 32 x 32 x 16 ones: the matrix core sums each
output's bf16 products in the same k order under both shapes), and within the fp32
accumulation bound of torch's fp32 matmul of the same operands; the runtime
picks the packed kernel for many-token calls and its streams match the oracle
(the prefill and full-scale parity tests in test_gpu_parity.py run through it).
"""
import gc

import numpy as np
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


def _layout(eng, cols, D):
    return eng.engram_layout_create(vocab_size=8, compressed_vocab=4, pad_token_id=7,
                                    heads_per_order=cols // 3, rows=[100_000] * 3, row_dim=D,
                                    table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                    row_pitch_bytes=(D + 15) // 16 * 16)


def _operands(L, M, N, seed):
    K = L.info.k_pad
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    A = torch.randn((M, K), generator=g, device=DEV).to(torch.bfloat16)
    B = (torch.randn((N, K), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    return A, B


def test_packed_bytes_follow_the_index_formula(eng):
    """Every element of a ragged weight (hidden 72: five column tiles of 16, the last
    one part padding; w_ld past k_pad) lands at the documented bf16 index, the padding
    rows of the last tile are zero, and the buffer past the last tile (sized for
    hidden rounded up to 32 rows) is left as it was."""
    L = _layout(eng, 3, 64)
    K = L.info.k_pad  # 192
    N, ld = 72, K + 8
    w = torch.arange(N * ld, dtype=torch.int32, device=DEV).remainder(30011).to(torch.int16)
    w = w.view(N, ld).view(torch.bfloat16)
    packed = torch.full((eng.engram_packed_weight_bytes(L, N),), 0xAB, dtype=torch.uint8, device=DEV)
    eng.engram_pack_weight(L, w, packed)
    torch.cuda.synchronize()
    got = packed.view(torch.int16).cpu().numpy()
    wh = w.view(torch.int16).cpu().numpy()
    n16 = (N + 15) // 16
    assert got.size == (N + 31) // 32 * 32 * K
    o = np.arange(n16 * 16)[:, None]
    k = np.arange(K)[None, :]
    idx = (((o // 16) * (K // 32) + k // 32) * 64 + o % 16 + 16 * ((k % 32) // 8)) * 8 + k % 8
    # the formula is a permutation of [0, n16 * 16 * K)
    assert np.array_equal(np.sort(idx.ravel()), np.arange(n16 * 16 * K))
    expect = np.full(got.size, np.uint16(0xABAB).view(np.int16), np.int16)
    expect[:n16 * 16 * K] = 0
    expect[idx[:N].ravel()] = wh[:, :K].ravel()
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("M,N,cols,D", [(1, 8, 3, 64), (77, 200, 3, 100), (300, 512, 6, 128),
                                        (1000, 264, 3, 192), (4097, 4096, 3, 512),
                                        (513, 300, 6, 1000), (256, 256, 3, 64),
                                        (300, 264, 6, 2048), (700, 520, 6, 2200), (255, 40, 3, 4097)])
def test_packed_projection_equals_unpacked(eng, M, N, cols, D):
    """Ragged M and N (row and column tile tails, a 264-wide weight whose last
    256-column block holds one 32-column tile) and K from 192 to 6,144 (128 x 256
    tiles; 12,288, the largest k_pad they take), and 13,248 and 12,352 (256 x 256 tiles,
    k_pad past 12,288)."""
    L = _layout(eng, cols, D)
    K = L.info.k_pad
    A, B = _operands(L, M, N, seed=M * 1000 + N)
    packed = torch.empty(eng.engram_packed_weight_bytes(L, N), dtype=torch.uint8, device=DEV)
    eng.engram_pack_weight(L, B, packed)
    v0 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    v1 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    eng.engram_project(L, A, B, v0)
    eng.engram_project_packed(L, A, packed, N, v1)
    ref = A.float() @ B.float().T
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    assert torch.equal(v0.view(torch.int32), v1.view(torch.int32))
    bound = 2 * K * 2.0 ** -24 * (A.float().abs() @ B.float().abs().T) + 1e-6
    assert ((v1 - ref).abs() <= bound).all()
    del A, B, packed, v0, v1, ref
    _free()


def test_packed_projection_prefill_shape_and_row_stride(eng):
    """The prefill workload's projection (16,384 tokens, k_pad 3,072 -> 4,096) with a
    row stride past k_pad, and a second call on fewer tokens into the same v:
    bit-identical to engram_project, rows past T untouched."""
    L = _layout(eng, 6, 512)
    K = L.info.k_pad
    M, N = 16384, 4096
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    A = torch.randn((M, K + 64), generator=g, device=DEV).to(torch.bfloat16)
    B = (torch.randn((N, K), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    packed = torch.empty(eng.engram_packed_weight_bytes(L, N), dtype=torch.uint8, device=DEV)
    eng.engram_pack_weight(L, B, packed)
    v0 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    v1 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    eng.engram_project(L, A, B, v0)
    eng.engram_project_packed(L, A, packed, N, v1)
    torch.cuda.synchronize()
    assert torch.equal(v0.view(torch.int32), v1.view(torch.int32))
    v1[5000:].fill_(-7.0)
    eng.engram_project_packed(L, A, packed, N, v1, T=5000)
    torch.cuda.synchronize()
    assert torch.equal(v0[:5000].view(torch.int32), v1[:5000].view(torch.int32))
    assert bool((v1[5000:] == -7.0).all())
    log(f"packed projection {M}x{N}x{K}: bit-identical to the unpacked kernel")
    del A, B, packed, v0, v1
    _free()


def test_runtime_picks_packed_for_many_tokens(eng):
    """The library's weight handle (behind the runtime) packs the weight when its
    calls can be large and plans the packed kernel exactly for calls of at least
    64 x 256 x 256 outputs."""
    import engram_inputs as ei
    cfg = ei.get_config("tiny")
    tid2eid = torch.from_numpy(ei.make_tid2eid(cfg.vocab, cfg.vc)).to(DEV)
    tables = ei.make_tables(cfg, DEV)
    weight = ei.make_weight(cfg, DEV)
    kw = dict(vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
              heads_per_order=cfg.heads, rows=[cfg.rows] * 3, row_dim=cfg.row_dim,
              table_dtype=cfg.table_dtype, row_pitch_bytes=cfg.row_pitch_bytes, tid2eid=tid2eid,
              tables=tables.data, scales=tables.scale, weight=weight, hidden=cfg.hidden)
    T_small = cfg.n_seqs * cfg.seq_len
    small = eng.Engram(max_tokens=T_small, **kw)
    assert all(small.projection_kind(0, t) in ("plain", "splitk") for t in (1, T_small // 2, T_small))
    big_T = 64 * 256 * 256 // cfg.hidden  # 16,384 tokens at hidden 256
    big = eng.Engram(max_tokens=big_T, **kw)
    assert big.projection_kind(0, big_T) == "packed"
    assert big.projection_kind(0, big_T - 1) != "packed"
    # the same rows through both kinds
    rows = big.rows
    rows.copy_(torch.randn(rows.shape, device=DEV).to(torch.bfloat16))
    big.project(0, rows, big_T)
    v_packed = big.v.clone()
    eng.engram_project(big.layout, rows, big.weight, big.v, T=big_T)
    torch.cuda.synchronize()
    assert torch.equal(v_packed.view(torch.int32), big.v.view(torch.int32))
    del small, big, rows, v_packed
    _free()


@pytest.mark.parametrize("shape", ["prefill", "decode", "between", "full"])
def test_gated_residual_runs_the_planned_kernel(eng, shape):
    """engram_gated_residual, called straight through ctypes with a weight handle,
    leaves the v and streams of the single kernel its plan names, bit for bit:
    the packed projection at the prefill shape (16,384 x 3,072 -> 4,096) and the
    full shape (65,536 x 19,584 -> 4,096), split-K at the decode shape (256 tokens),
    the plain kernel in between (3,000 x 3,072 -> 1,024); then engram_gate_add (or
    the slice sum) with a keep mask."""
    import ctypes
    M, cols, D, N, kind = {"prefill": (16384, 6, 512, 4096, "packed"),
                           "decode": (256, 6, 512, 4096, "splitk"),
                           "between": (3000, 6, 512, 1024, "plain"),
                           "full": (65536, 3, 6500, 4096, "packed")}[shape]
    L = _layout(eng, cols, D)
    K = L.info.k_pad
    A, B = _operands(L, M, N, seed=5)
    g = torch.Generator(device=DEV)
    g.manual_seed(6)
    x0 = torch.randn((M, 4, N), generator=g, device=DEV).to(torch.bfloat16)
    keep = (torch.rand(M, generator=g, device=DEV) > 0.1).to(torch.uint8)
    wkv = eng.engram_wkv_create(L, B, M)
    plan = wkv.plan(M)
    assert plan[0] == kind, plan
    v1 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    x1 = x0.clone()
    stream = torch.cuda.current_stream().cuda_stream
    rc = eng._lib.engram_gated_residual(L.handle, ctypes.c_void_p(A.data_ptr()), K, wkv.handle, 4,
                                        ctypes.c_void_p(keep.data_ptr()), ctypes.c_void_p(x1.data_ptr()),
                                        ctypes.c_void_p(v1.data_ptr()), M, ctypes.c_void_p(stream))
    assert rc == 0
    v2 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    x2 = x0.clone()
    if kind == "packed":
        packed = torch.empty(eng.engram_packed_weight_bytes(L, N), dtype=torch.uint8, device=DEV)
        eng.engram_pack_weight(L, B, packed)
        eng.engram_project_packed(L, A, packed, N, v2)
        eng.engram_gate_add(L, v2, x2, keep=keep)
    elif kind == "splitk":
        parts = torch.empty(plan[1] * M * N, dtype=torch.float32, device=DEV)
        eng.engram_project_splitk(L, A, B, parts, plan[1])
        eng.engram_gate_add_partials(L, parts, plan[1], x2, keep=keep, v=v2)
    else:
        eng.engram_project(L, A, B, v2)
        eng.engram_gate_add(L, v2, x2, keep=keep)
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    assert torch.equal(v1.view(torch.int32), v2.view(torch.int32))
    assert torch.equal(x1.view(torch.int16), x2.view(torch.int16))
    dropped = keep == 0
    assert torch.equal(x1[dropped].view(torch.int16), x0[dropped].view(torch.int16))
    assert not torch.equal(x1[~dropped].view(torch.int16), x0[~dropped].view(torch.int16))
    # the two halves give the same again
    v3 = torch.empty_like(v1)
    x3 = x0.clone()
    eng.engram_wkv_project(L, A, wkv, v3)
    eng.engram_wkv_gate_add(L, wkv, v3, x3, keep=keep)
    torch.cuda.synchronize()
    assert torch.equal(v1.view(torch.int32), v3.view(torch.int32))
    assert torch.equal(x1.view(torch.int16), x3.view(torch.int16))
    log(f"gated_residual {shape}: {kind} plan {plan}, bit-identical to the single kernels")
    del A, B, v1, v2, v3, x0, x1, x2, x3, wkv
    _free()


def test_packed_projection_random_shapes(eng):
    """48 seeded random shapes (tokens 1..2,000, hidden a multiple of 8 up to 1,200;
    1 or 2 heads with rows of 1..1,100 elements, and every fourth case 2 heads with rows
    of 2,100..3,000, so k_pad past 12,288 and both tile heights): bit-identical to
    engram_project each time."""
    import numpy as np
    rng = np.random.default_rng(20261202)
    for case in range(48):
        M = int(rng.integers(1, 2001))
        N = 8 * int(rng.integers(1, 151))
        if case % 4 == 0:  # k_pad past 12,288: the 256-row tiles
            cols, D = 6, int(rng.integers(2100, 3001))
        else:
            cols, D = 3 * int(rng.integers(1, 3)), int(rng.integers(1, 1101))
        L = _layout(eng, cols, D)
        A, B = _operands(L, M, N, seed=case)
        packed = torch.empty(eng.engram_packed_weight_bytes(L, N), dtype=torch.uint8, device=DEV)
        eng.engram_pack_weight(L, B, packed)
        v0 = torch.empty((M, N), dtype=torch.float32, device=DEV)
        v1 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        eng.engram_project(L, A, B, v0)
        eng.engram_project_packed(L, A, packed, N, v1)
        torch.cuda.synchronize()
        assert torch.equal(v0.view(torch.int32), v1.view(torch.int32)), (case, M, N, cols, D, L.info.k_pad)
        del A, B, packed, v0, v1
    assert eng.engram_get_error() == 0
    _free()
