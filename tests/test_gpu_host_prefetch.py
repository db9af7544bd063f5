"""Host-resident tables and the prefetch stream.

Bars: a gather that reads its tables from pinned host memory (a grid-stride
launch on a few workgroups) writes the oracle's fp32 and bf16 rows exactly on
every token, and the same bytes as the HBM gather; a pipeline that hashes and
gathers call i+1 on a prefetch stream while call i projects and gates on the main
stream leaves every call's streams bit for bit equal to the sequential forward,
and within the tolerance of the oracle on a seeded 1,024-token sample of each
call (its rows exact on every token).
"""
import gc

import numpy as np
import pytest
import torch

import engram_inputs as ei
import oracle
from engram_harness import (DEV, Site, assert_streams_close, bf16_bits_np, log,
                            oracle_dequant, oracle_gate_add, oracle_project, sample_tokens)

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


def _pinned_copy(t):
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def _d(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("name", ["prefill", "v41_small"])
def test_host_resident_tables_equal_device_tables(eng, name):
    cfg = ei.get_config(name)
    batch = ei.make_batch(cfg)
    T = batch.T
    tid = _d(ei.make_tid2eid(cfg.vocab, cfg.vc))
    tabs = ei.make_tables(cfg, DEV)
    L = eng.engram_layout_create(
        vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
        heads_per_order=cfg.heads, rows=[cfg.rows] * 3, row_dim=cfg.row_dim,
        table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN, row_pitch_bytes=cfg.row_pitch_bytes,
        hash_floor=cfg.hash_floor, num_sites=cfg.n_sites,
        table_split=eng.ENGRAM_TABLE_PER_SITE if cfg.table_split == "site" else eng.ENGRAM_TABLES_PER_ORDER,
        scale_layout=eng.ENGRAM_SCALE_BLOCK32_E8M0 if cfg.scale_block else eng.ENGRAM_SCALE_ROW_F32)
    info = L.info
    eids = torch.empty(T, dtype=torch.int32, device=DEV)
    rid = torch.empty((T, cfg.n_sites, 3, cfg.heads), dtype=torch.int32, device=DEV)
    eng.engram_compress_hash(L, tid, _d(batch.tokens), _d(batch.cu_seqlens), eids, rid)
    h_data = [_pinned_copy(t) for t in tabs.data]
    h_scale = [_pinned_copy(s) for s in tabs.scale]
    torch.cuda.synchronize()
    # the oracle's rows of site 0 on every token: its own row ids, the input tables' bytes
    per_site = cfg.table_split == "site"
    if per_site:
        ols = oracle.site_layouts(cfg.n_sites, cfg.heads, cfg.hash_floor, True)
    else:
        ols = [oracle.fit_layout([cfg.rows] * 3, cfg.heads)]
    _, r_ref = oracle.compress_hash(ols[0], vocab=cfg.vocab, vc=cfg.vc, pad_token_id=cfg.pad_token_id,
                                    tid2eid=ei.make_tid2eid(cfg.vocab, cfg.vc), tokens=batch.tokens,
                                    cu_seqlens=batch.cu_seqlens)
    H, D = cfg.heads, cfg.row_dim
    raw = np.zeros((T, 3 * H, D), np.uint8)
    sc = np.zeros((T, 3 * H, D // 32), np.uint8) if cfg.scale_block else np.zeros((T, 3 * H), np.float32)
    for n in range(3):
        tab = 0 if per_site else n
        for h in range(H):
            ii = torch.from_numpy(r_ref[:, n, h].astype(np.int64)).to(DEV)
            raw[:, n * H + h] = tabs.row_view(tab).index_select(0, ii)[:, :D].cpu().numpy()
            sc[:, n * H + h] = tabs.scale[tab].index_select(0, ii).cpu().numpy()
    f_ref, b_ref = oracle_dequant(raw.reshape(-1, D), sc.reshape(T * 3 * H, -1).squeeze(-1)
                                  if not cfg.scale_block else sc.reshape(-1, D // 32),
                                  block32=bool(cfg.scale_block))
    f_ref, b_ref = f_ref.reshape(T, 3 * H, D), b_ref.reshape(T, 3 * H, D)
    for dtype in (torch.float32, torch.bfloat16):
        a = torch.empty((T, info.k_pad), dtype=dtype, device=DEV)
        b = torch.full((T, info.k_pad), 7, dtype=dtype, device=DEV)
        eng.engram_gather_dequant(L, tabs.data, tabs.scale, rid, a, site=0)
        eng.engram_gather_dequant(L, h_data, h_scale, rid, b, site=0)
        torch.cuda.synchronize()
        assert eng.engram_get_error() == 0
        got = b.view(T, 3 * H, info.seg_pitch)[:, :, :D]
        if dtype == torch.float32:
            assert np.array_equal(got.cpu().numpy().view(np.uint32), f_ref.view(np.uint32)), name
        else:
            assert np.array_equal(bf16_bits_np(got), b_ref), name
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{name} {dtype}"
    log(f"{name}: host-resident gather equals the oracle's rows and the HBM gather on all {T} tokens")
    del tabs, h_data, h_scale
    _free()


@pytest.mark.parametrize("host", [False, True])
def test_prefetch_pipeline_equals_sequential(eng, host):
    cfg = ei.get_config("prefill")
    calls = [ei.make_batch(ei.get_config("prefill", seed=100 + i)) for i in range(4)]
    T = calls[0].T
    ref = Site(cfg, max_tokens=T)
    tables = ref.tables
    if host:
        tabs = [_pinned_copy(t) for t in tables.data]
        scs = [_pinned_copy(s) for s in tables.scale]
    else:
        tabs, scs = tables.data, tables.scale
    pipe = eng.Engram(vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
                      heads_per_order=cfg.heads, rows=[cfg.rows] * 3, row_dim=cfg.row_dim,
                      table_dtype=cfg.table_dtype, row_pitch_bytes=cfg.row_pitch_bytes,
                      tid2eid=ref.tid2eid, tables=tabs, scales=scs, weight=ref.weight,
                      hidden=cfg.hidden, max_tokens=T, prefetch_slots=2)
    # sequential reference
    expect = []
    for i, b in enumerate(calls):
        x = ei.make_streams(cfg, T, DEV, step=i)
        ref.site.forward(_d(b.tokens), _d(b.cu_seqlens), x)
        expect.append(bf16_bits_np(x))
    torch.cuda.synchronize()
    # pipelined: the prefetch of call i+1 is enqueued before call i's projection
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    xs = [ei.make_streams(cfg, T, DEV, step=i) for i in range(len(calls))]
    inputs = [(_d(b.tokens), _d(b.cu_seqlens)) for b in calls]
    torch.cuda.synchronize()
    pre = pipe.prefetch(*inputs[0], stream=side)
    for i in range(len(calls)):
        nxt = pipe.prefetch(*inputs[i + 1], stream=side) if i + 1 < len(calls) else None
        pipe.apply(pre, 0, xs[i], stream=main)
        pre = nxt
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    for i in range(len(calls)):
        assert np.array_equal(bf16_bits_np(xs[i]), expect[i]), f"call {i}"
    # against the oracle: the first and the last call, rows on every token, v and the
    # pipelined streams on a seeded 1,024-token sample
    W = ref.weight_bits()
    for i in (0, len(calls) - 1):
        b = calls[i]
        _, r_ref = ref.oracle_hash(b)
        _, b16 = ref.oracle_dequant(r_ref)
        slot = i % 2
        got = bf16_bits_np(pipe.pre_rows[slot][0][:T].view(T, 3 * cfg.heads, ref.info.seg_pitch))
        if i == len(calls) - 1:  # the last call's rows are still in its ring slot
            assert np.array_equal(got[:, :, :cfg.row_dim], b16), f"call {i} rows"
        idx = sample_tokens(b, 1024, seed=7 + i)
        E = b16[idx].reshape(len(idx), -1)
        v_ref = oracle_project(E, W)
        x0 = bf16_bits_np(ei.make_streams(cfg, T, DEV, step=i)[torch.from_numpy(idx).to(DEV)])
        y_ref, _ = oracle_gate_add(x0, v_ref)
        worst = assert_streams_close(bf16_bits_np(xs[i])[idx], y_ref, f"pipelined call {i}")
        log(f"prefetch pipeline call {i}: {len(idx)} sampled streams within tolerance of the oracle "
            f"(worst {worst:.2e})")
    log(f"prefetch pipeline ({'host' if host else 'HBM'} tables): {len(calls)} calls equal sequential")
    del ref, pipe, tabs, scs
    _free()


def test_fused_path_refuses_host_tables(eng):
    """The fused gather + projection streams rows by direct-to-LDS loads from HBM
    tables; given tables in host memory it refuses instead of guessing."""
    cfg = ei.get_config("tiny")
    site = Site(cfg, max_tokens=64)
    h_data = [_pinned_copy(t) for t in site.tables.data]
    h_scale = [_pinned_copy(s) for s in site.tables.scale]
    rid = torch.zeros((64, 3, cfg.heads), dtype=torch.int32, device=DEV)
    v = torch.empty((64, cfg.hidden), dtype=torch.float32, device=DEV)
    with pytest.raises(eng.EngramError) as ex:
        eng.engram_gather_project(site.site.layout, h_data, h_scale, rid, site.site.weight, v)
    assert ex.value.status == eng.ENGRAM_E_UNSUPPORTED
    _free()


def test_prefetch_refuses_to_overwrite_an_unapplied_slot(eng):
    """With two slots, a third prefetch before the first call is applied would
    overwrite rows an apply still has to read: it raises instead.  Applying the
    first call frees its slot; applying a site twice raises too."""
    cfg = ei.get_config("tiny")
    batch = ei.make_batch(cfg)
    ref = Site(cfg, max_tokens=batch.T)
    pipe = eng.Engram(vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
                      heads_per_order=cfg.heads, rows=[cfg.rows] * 3, row_dim=cfg.row_dim,
                      table_dtype=cfg.table_dtype, row_pitch_bytes=cfg.row_pitch_bytes,
                      tid2eid=ref.tid2eid, tables=ref.tables.data, scales=ref.tables.scale,
                      weight=ref.weight, hidden=cfg.hidden, max_tokens=batch.T, prefetch_slots=2)
    tok, cu = _d(batch.tokens), _d(batch.cu_seqlens)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    p0 = pipe.prefetch(tok, cu, stream=side)
    p1 = pipe.prefetch(tok, cu, stream=side)
    with pytest.raises(RuntimeError):
        pipe.prefetch(tok, cu, stream=side)
    x = ei.make_streams(cfg, batch.T, DEV)
    pipe.apply(p0, 0, x)
    with pytest.raises(RuntimeError):
        pipe.apply(p0, 0, x)
    p2 = pipe.prefetch(tok, cu, stream=side)  # slot 0 is free again
    pipe.apply(p1, 0, x)
    pipe.apply(p2, 0, x)
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    del ref, pipe
    _free()
