"""GPU parity of the fused gather + dequant + projection (engram_gather_project).

Bars: the fused v equals the two-call path (engram_gather_dequant then
engram_project) bit for bit -- both accumulate the same bf16 products in the same
order on the matrix cores -- and matches the oracle's fp64 projection of the
oracle's dequantised rows within the fp32-accumulation bound.  Shapes cover
ragged token counts and hidden sizes (tile tails), row dims that leave segment
padding, several heads per order, and NaN bytes in the row padding.
"""
import gc

import numpy as np
import pytest
import torch

import engram_inputs as ei
import oracle
from engram_harness import (DEV, Site, assert_streams_close, assert_v_close, bf16_bits_np, log)

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


def _random_fp8_tables(rows, pitch, D, seed):
    """Random e4m3fn bytes (no NaN codes inside the row) with NaN bytes in the row
    padding [D, pitch), and positive non-power-of-two scales."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    tabs, scales = [], []
    for _ in range(3):
        t = torch.randint(0, 256, (rows, pitch), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
        t[t == 0x7F] = 0x7E
        t[t == 0xFF] = 0xFE
        if pitch > D:
            t[:, D:] = 0xFF
        tabs.append(t.reshape(-1))
        scales.append(torch.exp(torch.randn(rows, generator=g, device=DEV) * 0.5 - 6.0))
    return tabs, scales


@pytest.mark.parametrize("M,N,H,D,pitch", [
    (1, 8, 1, 64, 64),
    (77, 200, 1, 100, 128),
    (300, 512, 2, 128, 128),
    (1000, 264, 1, 192, 256),
    (513, 256, 8, 256, 256),
    (4097, 4096, 1, 512, 512),
    (600, 512, 1, 6500, 6528),
])
def test_fused_equals_split_bitwise(eng, M, N, H, D, pitch):
    rows = 50_000
    L = eng.engram_layout_create(vocab_size=8, compressed_vocab=4, pad_token_id=7, heads_per_order=H,
                                 rows=[rows] * 3, row_dim=D, table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                 row_pitch_bytes=pitch)
    info = L.info
    tabs, scales = _random_fp8_tables(rows, pitch, D, seed=M * 7 + N)
    g = torch.Generator(device=DEV)
    g.manual_seed(M + 13 * N)
    rid = torch.randint(0, rows, (M, 3, H), generator=g, device=DEV, dtype=torch.int32)
    w = (torch.randn((N, info.k_pad), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
    e16 = torch.empty((M, info.k_pad), dtype=torch.bfloat16, device=DEV)
    v_split = torch.empty((M, N), dtype=torch.float32, device=DEV)
    v_fused = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    eng.engram_gather_dequant(L, tabs, scales, rid, e16)
    eng.engram_project(L, e16, w, v_split)
    eng.engram_gather_project(L, tabs, scales, rid, w, v_fused)
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    assert torch.equal(v_split.view(torch.int32), v_fused.view(torch.int32)), \
        f"fused differs from split on {int((v_split != v_fused).sum())} outputs"
    # and both against torch's fp32 product of the same bf16 operands
    ref = e16.float() @ w.float().T
    bound = 2 * info.k_pad * 2.0 ** -24 * (e16.float().abs() @ w.float().abs().T) + 1e-30
    assert ((v_fused - ref).abs() <= bound).all()
    del tabs, scales
    _free()


def test_fused_tiny_against_oracle(eng):
    """Whole tiny workload through Engram(path="fused"): ids exact, v within the
    fp32 bound of the oracle's fp64 projection, streams within 2e-2."""
    cfg = ei.get_config("tiny")
    batch = ei.make_batch(cfg)
    T = batch.T
    site = Site(cfg, max_tokens=T)
    fused = eng.Engram(vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
                       heads_per_order=cfg.heads, rows=[cfg.rows] * 3, row_dim=cfg.row_dim,
                       table_dtype=cfg.table_dtype, row_pitch_bytes=cfg.row_pitch_bytes,
                       tid2eid=site.tid2eid, tables=site.tables.data, scales=site.tables.scale,
                       weight=site.weight, hidden=cfg.hidden, max_tokens=T, path="fused")
    assert fused.rows is None
    db = site.device_batch(batch)
    streams = ei.make_streams(cfg, T, DEV)
    x0 = bf16_bits_np(streams)
    fused.forward(db["tokens"], db["cu_seqlens"], streams)
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    e_ref, r_ref = site.oracle_hash(batch)
    assert np.array_equal(fused.row_ids[:T].cpu().numpy(), r_ref)
    _, b16 = site.oracle_dequant(r_ref)
    E = b16.reshape(T, -1)
    W = site.weight_bits()
    v_ref = oracle.project(E, W)
    assert_v_close(fused.v[:T].cpu().numpy(), v_ref, E, W, "fused tiny v")
    y_ref, _ = oracle.gate_add(x0, v_ref)
    worst = assert_streams_close(bf16_bits_np(streams), y_ref, "fused tiny streams")
    log(f"fused tiny: streams within tolerance on all {T} tokens (worst {worst:.2e})")
    _free()


def test_fused_bad_row_ids_latch_and_contribute_zero(eng):
    cfg = ei.get_config("tiny")
    site = Site(cfg, max_tokens=64)
    L = site.site.layout
    H = cfg.heads
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    rid = torch.randint(0, cfg.rows, (64, 3, H), generator=g, device=DEV, dtype=torch.int32)
    rid[3, 1, 0] = cfg.rows
    rid[40, 2, 1] = -1
    e16 = torch.empty((64, site.info.k_pad), dtype=torch.bfloat16, device=DEV)
    v_split = torch.empty((64, cfg.hidden), dtype=torch.float32, device=DEV)
    v_fused = torch.empty_like(v_split)
    assert eng.engram_get_error() == 0
    eng.engram_gather_dequant(L, site.tables.data, site.tables.scale, rid, e16)
    assert eng.engram_get_error() == eng.ENGRAM_E_ROW_RANGE
    eng.engram_project(L, e16, site.site.weight, v_split)
    eng.engram_gather_project(L, site.tables.data, site.tables.scale, rid, site.site.weight, v_fused)
    assert eng.engram_get_error() == eng.ENGRAM_E_ROW_RANGE
    torch.cuda.synchronize()
    assert torch.equal(v_split.view(torch.int32), v_fused.view(torch.int32))
    _free()


def test_fused_refuses_bf16_tables(eng):
    cfg = ei.get_config("tiny")
    L = eng.engram_layout_create(vocab_size=cfg.vocab, compressed_vocab=cfg.vc,
                                 pad_token_id=cfg.pad_token_id, heads_per_order=cfg.heads,
                                 rows=[cfg.rows] * 3, row_dim=cfg.row_dim,
                                 table_dtype=eng.ENGRAM_DTYPE_BF16, row_pitch_bytes=2 * cfg.row_dim)
    t = [torch.zeros(cfg.rows * 2 * cfg.row_dim, dtype=torch.uint8, device=DEV)] * 3
    s = [torch.ones(cfg.rows, dtype=torch.float32, device=DEV)] * 3
    rid = torch.zeros((4, 3, cfg.heads), dtype=torch.int32, device=DEV)
    w = torch.zeros((cfg.hidden, L.info.k_pad), dtype=torch.bfloat16, device=DEV)
    v = torch.empty((4, cfg.hidden), dtype=torch.float32, device=DEV)
    with pytest.raises(eng.EngramError) as ex:
        eng.engram_gather_project(L, t, s, rid, w, v)
    assert ex.value.status == eng.ENGRAM_E_UNSUPPORTED


@pytest.mark.parametrize("split", ["order", "site"])
def test_fused_second_site_equals_split(eng, split):
    """Two sites sharing one hash pass: the fused kernel reads site 1's columns of
    the shared row-id array (and, with one table per site, every segment from that
    site's table) exactly like the two-call path."""
    H, D, rows, T, N = 2, 128, 60_000, 700, 512
    per_site = split == "site"
    L = eng.engram_layout_create(
        vocab_size=8, compressed_vocab=4, pad_token_id=7, heads_per_order=H,
        rows=[rows, 0, 0] if per_site else [rows] * 3, row_dim=D,
        table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN, row_pitch_bytes=D, hash_floor=1000, num_sites=2,
        table_split=eng.ENGRAM_TABLE_PER_SITE if per_site else eng.ENGRAM_TABLES_PER_ORDER)
    info = L.info
    tabs, scales = _random_fp8_tables(rows, D, D, seed=77)
    if per_site:
        tabs, scales = tabs[:1], scales[:1]
    g = torch.Generator(device=DEV)
    g.manual_seed(78)
    rid = torch.empty((T, 2, 3, H), dtype=torch.int32, device=DEV)
    for s in range(2):
        for n in range(3):
            for h in range(H):
                lo = int(info.site_offsets[s][n][h])
                p = int(info.site_primes[s][n][h])
                rid[:, s, n, h] = torch.randint(lo, lo + p, (T,), generator=g, device=DEV, dtype=torch.int32)
    w = (torch.randn((N, info.k_pad), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
    e16 = torch.empty((T, info.k_pad), dtype=torch.bfloat16, device=DEV)
    v_split = torch.empty((T, N), dtype=torch.float32, device=DEV)
    v_fused = torch.empty_like(v_split)
    for s in range(2):
        eng.engram_gather_dequant(L, tabs, scales, rid, e16, site=s)
        eng.engram_project(L, e16, w, v_split)
        eng.engram_gather_project(L, tabs, scales, rid, w, v_fused, site=s)
        torch.cuda.synchronize()
        assert eng.engram_get_error() == 0
        assert torch.equal(v_split.view(torch.int32), v_fused.view(torch.int32)), f"site {s}"
    _free()


def _random_e8m0_tables(rows, pitch, D, seed, n_tables=3):
    """Random e4m3fn bytes (no NaN codes) with NaN bytes in the row padding, and
    (1, 32) e8m0 block scales: mostly exponents near 2^-7, some rows at the
    smallest codes (0 = 2^-127, 1 = 2^-126) and some up to 2^3."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    tabs, scales = [], []
    for _ in range(n_tables):
        t = torch.randint(0, 256, (rows, pitch), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
        t[t == 0x7F] = 0x7E
        t[t == 0xFF] = 0xFE
        if pitch > D:
            t[:, D:] = 0xFF
        tabs.append(t.reshape(-1))
        s = torch.randint(110, 131, (rows, D // 32), generator=g, device=DEV, dtype=torch.int32)
        s[::97] = 0
        s[1::89] = 1
        scales.append(s.to(torch.uint8).reshape(-1))
    return tabs, scales


@pytest.mark.parametrize("M,N,H,D,pitch", [
    (1, 8, 1, 32, 64),
    (77, 200, 1, 96, 128),
    (300, 512, 2, 128, 128),
    (700, 512, 8, 256, 256),
    (4097, 1024, 8, 256, 256),
])
def test_fused_block_scales_equal_split_bitwise(eng, M, N, H, D, pitch):
    """(1, 32) e8m0 block-scaled tables: the fused kernel picks each 32-element
    block's exponent from the row's scale bytes and equals gather + projection bit
    for bit (rows of up to 256 elements, the released layout's width)."""
    rows = 40_000
    L = eng.engram_layout_create(vocab_size=8, compressed_vocab=4, pad_token_id=7, heads_per_order=H,
                                 rows=[rows] * 3, row_dim=D, table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                 row_pitch_bytes=pitch, scale_layout=eng.ENGRAM_SCALE_BLOCK32_E8M0)
    info = L.info
    tabs, scales = _random_e8m0_tables(rows, pitch, D, seed=M * 11 + D)
    g = torch.Generator(device=DEV)
    g.manual_seed(M + 17 * N)
    rid = torch.randint(0, rows, (M, 3, H), generator=g, device=DEV, dtype=torch.int32)
    w = (torch.randn((N, info.k_pad), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
    e16 = torch.empty((M, info.k_pad), dtype=torch.bfloat16, device=DEV)
    v_split = torch.empty((M, N), dtype=torch.float32, device=DEV)
    v_fused = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    eng.engram_gather_dequant(L, tabs, scales, rid, e16)
    eng.engram_project(L, e16, w, v_split)
    eng.engram_gather_project(L, tabs, scales, rid, w, v_fused)
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    assert torch.equal(v_split.view(torch.int32), v_fused.view(torch.int32)), \
        f"fused differs from split on {int((v_split != v_fused).sum())} outputs"
    del tabs, scales
    _free()


def test_fused_released_layout_two_sites_equals_split(eng):
    """The v41_small workload (two sites sharing one hash pass, one table per site,
    3 x 8 heads of 256 elements, e8m0 block scales) through Engram(path="fused") and
    the split path on the same inputs: every stream bit for bit."""
    cfg = ei.get_config("v41_small")
    batch = ei.make_batch(cfg)
    T = batch.T
    tid = torch.from_numpy(ei.make_tid2eid(cfg.vocab, cfg.vc)).to(DEV)
    tables = [ei.make_tables(cfg, DEV, site=s) for s in range(cfg.n_sites)]
    weights = [ei.make_weight(cfg, DEV, site=s) for s in range(cfg.n_sites)]
    outs = {}
    for path in ("split", "fused"):
        e = eng.Engram(vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
                       heads_per_order=cfg.heads, rows=[cfg.rows], row_dim=cfg.row_dim,
                       table_dtype=cfg.table_dtype, row_pitch_bytes=cfg.row_pitch_bytes, tid2eid=tid,
                       tables=[t.data for t in tables], scales=[t.scale for t in tables], weight=weights,
                       hidden=cfg.hidden, hc_mult=cfg.hc_mult, max_tokens=T, hash_floor=cfg.hash_floor,
                       num_sites=cfg.n_sites, table_split=cfg.table_split, scale_block=cfg.scale_block,
                       path=path)
        streams = [ei.make_streams(cfg, T, DEV, step=s) for s in range(cfg.n_sites)]
        e.forward(torch.from_numpy(batch.tokens).to(DEV), torch.from_numpy(batch.cu_seqlens).to(DEV),
                  streams)
        torch.cuda.synchronize()
        assert eng.engram_get_error() == 0
        outs[path] = [bf16_bits_np(x) for x in streams]
        del e
    for s in range(cfg.n_sites):
        assert np.array_equal(outs["split"][s], outs["fused"][s]), f"site {s}"
    log(f"v41_small: fused and split paths give the same streams on all {T} tokens of both sites")
    del tables, weights
    _free()
