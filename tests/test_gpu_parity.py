"""GPU parity of the HIP path against the oracle, through the C ABI.

Bars: compressed ids and row ids bit-exact; dequantised rows bit-exact in fp32
and in bf16; projection within the fp32-accumulation bound; final bf16 streams
within 2e-2 relative error (1e-3 absolute floor); keep = 0 streams bit for bit.

Coverage (the oracle runs on host-thread token shards, see engram_harness):
  tiny, prefill (with and without image spans), decode (both shapes, all 64 steps):
      every output of every token;
  long prefill: integers and fp32 / bf16 rows on every token, v and streams on a
      seeded 4,096-token sample;
  full FP8 and full BF16: integers on every token, rows, v and streams on a seeded
      1,024-token sample.
Samples always include the first three and the last token of each sequence.  The
large workloads run in the launch configuration the benchmark uses, and the fused
and look-ahead paths are compared with the oracle on the same tokens.
"""
import gc

import numpy as np
import pytest
import torch

import engram_inputs as ei
import oracle
from engram_harness import (DEV, Site, assert_streams_close, assert_v_close, bf16_bits_np,
                            bits_to_f64, log, oracle_gate_add, oracle_project, sample_tokens)

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


def _no_device_error(eng, what):
    st = eng.engram_get_error()
    assert st == 0, f"{what}: device status {st} ({eng.engram_strerror(st)})"


# ---------------------------------------------------------------------------
# dequant of every e4m3fn code
# ---------------------------------------------------------------------------

def test_fp8_every_code_and_scale(eng):
    log("fp8 codes: start")
    R, D = 1024, 256
    L = eng.engram_layout_create(vocab_size=8, compressed_vocab=4, pad_token_id=7, heads_per_order=1,
                                 rows=[R] * 3, row_dim=D, table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                 row_pitch_bytes=D)
    rng = np.random.default_rng(99)
    codes = ((np.arange(D)[None, :] + np.arange(R)[:, None] * 7) % 256).astype(np.uint8)
    k = (np.arange(R) % 41) - 20
    scales = np.where(np.arange(R) % 2 == 0, 2.0 ** k, rng.random(R) * 3 + 1e-3).astype(np.float32)
    tabs = [torch.from_numpy(np.roll(codes, n, axis=0).copy()).to(DEV) for n in range(3)]
    scs = [torch.from_numpy(np.roll(scales, n).copy()).to(DEV) for n in range(3)]
    T = 700
    rid = rng.integers(0, R, size=(T, 3, 1)).astype(np.int32)
    rid_d = torch.from_numpy(rid).to(DEV)
    out32 = torch.full((T, L.info.k_pad), 7.0, dtype=torch.float32, device=DEV)
    out16 = torch.full((T, L.info.k_pad), 7.0, dtype=torch.bfloat16, device=DEV)
    eng.engram_gather_dequant(L, tabs, scs, rid_d, out32)
    eng.engram_gather_dequant(L, tabs, scs, rid_d, out16)
    torch.cuda.synchronize()
    _no_device_error(eng, "gather")
    g32 = out32.cpu().numpy().reshape(T, 3, L.info.seg_pitch)
    g16 = bf16_bits_np(out16).reshape(T, 3, L.info.seg_pitch)
    for n in range(3):
        raw = np.roll(codes, n, axis=0)[rid[:, n, 0]]
        sc = np.roll(scales, n)[rid[:, n, 0]]
        nan = (raw == 0x7F) | (raw == 0xFF)
        f32, b16 = oracle.dequant_rows(np.where(nan, 0, raw).astype(np.uint8), sc)
        got32, got16 = g32[:, n, :D], g16[:, n, :D]
        assert np.all(np.isnan(got32[nan]))
        assert np.array_equal(got32[~nan].view(np.uint32), f32[~nan].view(np.uint32))
        assert np.array_equal(got16[~nan], b16[~nan])
    log("fp8 codes: ok")


# ---------------------------------------------------------------------------
# tiny: every output
# ---------------------------------------------------------------------------

def _check_rows(site, row_ids_ref, T, rows_dev, f32_dev=None):
    f32_ref, b16_ref = site.oracle_dequant(row_ids_ref)
    D = site.cfg.row_dim
    got = bf16_bits_np(site.unpad(rows_dev, T))
    assert np.array_equal(got[:, :, :D], b16_ref), "bf16 rows differ"
    assert not got[:, :, D:].any(), "segment padding not zero"
    if f32_dev is not None:
        g32 = f32_dev[:T].view(T, -1, site.info.seg_pitch).cpu().numpy()
        assert np.array_equal(g32[:, :, :D].view(np.uint32), f32_ref.view(np.uint32)), "fp32 rows differ"
        assert not g32[:, :, D:].any()
    return b16_ref


def test_tiny_end_to_end(eng):
    cfg = ei.get_config("tiny")
    site = Site(cfg, max_tokens=cfg.tokens_per_call)
    batch = ei.make_batch(cfg)
    T = batch.T
    db = site.device_batch(batch)
    streams = ei.make_streams(cfg, T, DEV)
    x0 = bf16_bits_np(streams)
    site.site.forward(db["tokens"], db["cu_seqlens"], streams, seq_start=db["seq_start"])
    torch.cuda.synchronize()
    _no_device_error(eng, "tiny forward")
    e_ref, r_ref = site.oracle_hash(batch)
    assert np.array_equal(site.site.eids[:T].cpu().numpy(), e_ref)
    assert np.array_equal(site.site.row_ids[:T].cpu().numpy(), r_ref)
    out32 = torch.empty((T, site.info.k_pad), dtype=torch.float32, device=DEV)
    eng.engram_gather_dequant(site.site.layout, site.tables.data, site.tables.scale, site.site.row_ids,
                              out32, T=T)
    torch.cuda.synchronize()
    b16_ref = _check_rows(site, r_ref, T, site.site.rows, out32)
    E = b16_ref.reshape(T, -1)
    W = site.weight_bits()
    v_ref = oracle_project(E, W)
    assert_v_close(site.site.v[:T].cpu().numpy(), v_ref, E, W, "tiny v")
    y_ref, _ = oracle_gate_add(x0, v_ref)
    worst = assert_streams_close(bf16_bits_np(streams), y_ref, "tiny streams")
    log(f"tiny: worst stream rel err {worst:.2e}")


def test_tiny_pow2_off_scales_fp32_exact(eng):
    """Scales amax/448 (not powers of two): fp32 rows are the single IEEE product,
    bf16 rows its round-to-nearest-even."""
    cfg = ei.get_config("tiny")
    site = Site(cfg, max_tokens=cfg.tokens_per_call, scale_mode="amax")
    batch = ei.make_batch(cfg)
    T = batch.T
    db = site.device_batch(batch)
    eng.engram_compress_hash(site.site.layout, site.tid2eid, db["tokens"], db["cu_seqlens"],
                             site.site.eids, site.site.row_ids)
    out32 = torch.empty((T, site.info.k_pad), dtype=torch.float32, device=DEV)
    eng.engram_gather_dequant(site.site.layout, site.tables.data, site.tables.scale, site.site.row_ids,
                              out32, T=T)
    eng.engram_gather_dequant(site.site.layout, site.tables.data, site.tables.scale, site.site.row_ids,
                              site.site.rows, T=T)
    torch.cuda.synchronize()
    _no_device_error(eng, "amax gather")
    _, r_ref = site.oracle_hash(batch)
    _check_rows(site, r_ref, T, site.site.rows, out32)


def test_gather_padded_leading_dimension(eng):
    """A gathered-row buffer wider than k_pad (rows not back to back) takes the
    per-lane store path; it must hold exactly what the packed layout holds."""
    cfg = ei.get_config("tiny")
    site = Site(cfg, max_tokens=cfg.tokens_per_call)
    batch = ei.make_batch(cfg)
    T = batch.T
    db = site.device_batch(batch)
    eng.engram_compress_hash(site.site.layout, site.tid2eid, db["tokens"], db["cu_seqlens"],
                             site.site.eids, site.site.row_ids)
    kp = site.info.k_pad
    wide = torch.full((T, kp + 72), 5.0, dtype=torch.bfloat16, device=DEV)
    eng.engram_gather_dequant(site.site.layout, site.tables.data, site.tables.scale, site.site.row_ids,
                              wide, T=T)
    eng.engram_gather_dequant(site.site.layout, site.tables.data, site.tables.scale, site.site.row_ids,
                              site.site.rows, T=T)
    torch.cuda.synchronize()
    _no_device_error(eng, "padded gather")
    assert torch.equal(wide[:, :kp].view(torch.int16), site.site.rows[:T].view(torch.int16))
    assert (wide[:, kp:].float() == 5.0).all()  # columns past k_pad untouched


def _ragged_batch(cfg, seed):
    rng = np.random.default_rng(seed)
    lens = np.array([0, 1, 2, 3, 100, 5, 0, 64, 63, 65, 888, 4], dtype=np.int32)
    S = len(lens)
    cu = np.zeros(S + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    tokens = ei.zipf_tokens(rng, T)
    seq_start = np.array([1, 0, 1, 0, 0, 1, 0, 0, 1, 0, 0, 1], np.uint8)
    slots = np.array([3, 0, 7, 1, 2, -1, 9, 4, 5, 6, 8, 10], np.int32)
    seq_start[slots < 0] = 1
    dead = ei.make_dead_spans(T, seed, n_spans=12, max_len=9)
    return ei.Batch(tokens=tokens, cu_seqlens=cu, seq_start=seq_start, slots=slots, dead=dead)


def test_tiny_ragged_store_and_dead(eng):
    """Ragged sequences (empty, 1..3 tokens, across wave and block edges), mixed
    starts and continuations through the store, image-span dead positions."""
    cfg = ei.get_config("tiny")
    batch = _ragged_batch(cfg, 5)
    T = batch.T
    site = Site(cfg, max_tokens=T)
    num_slots = 12
    store0 = np.random.default_rng(6).integers(0, cfg.vc, size=(num_slots, 3)).astype(np.int32)
    store_d = site.site.make_store(num_slots, ids=torch.from_numpy(store0).to(DEV))
    db = site.device_batch(batch)
    streams = ei.make_streams(cfg, T, DEV, step=3)
    x0 = bf16_bits_np(streams)
    site.site.forward(db["tokens"], db["cu_seqlens"], streams, seq_start=db["seq_start"],
                      slots=db["slots"], store=store_d, dead=db["dead"], keep=db["keep"])
    torch.cuda.synchronize()
    _no_device_error(eng, "ragged forward")
    store_ref = store0.copy()
    e_ref, r_ref = site.oracle_hash(batch, store_ref)
    assert np.array_equal(site.site.eids[:T].cpu().numpy(), e_ref)
    assert np.array_equal(site.site.row_ids[:T].cpu().numpy(), r_ref)
    assert np.array_equal(store_d.ids().cpu().numpy(), store_ref)
    b16_ref = _check_rows(site, r_ref, T, site.site.rows)
    E = b16_ref.reshape(T, -1)
    v_ref = oracle_project(E, site.weight_bits())
    keep = (batch.dead == 0).astype(np.uint8)
    y_ref, _ = oracle_gate_add(x0, v_ref, keep)
    y = bf16_bits_np(streams)
    assert np.array_equal(y[keep == 0], x0[keep == 0]), "dead tokens' streams changed"
    assert_streams_close(y, y_ref, "ragged streams")


def test_decode_equals_prefill_at_five_splits(eng):
    """The pages' equivalence check on the device: prompt then one-token steps
    through the store give the prefill's row ids exactly, with an image span that
    lies in the prompt for some splits and in the steps for others."""
    cfg = ei.get_config("tiny")
    site = Site(cfg, max_tokens=256)
    L = site.site.layout
    rng = np.random.default_rng(17)
    T = 48
    tokens = ei.zipf_tokens(rng, T)
    dead = np.zeros(T, np.uint8)
    dead[12:16] = 1
    full = ei.Batch(tokens=tokens, cu_seqlens=np.array([0, T], np.int32), seq_start=None, dead=dead)
    e_ref, r_ref = site.oracle_hash(full)
    db = site.device_batch(full)
    eids = torch.empty(T, dtype=torch.int32, device=DEV)
    rows = torch.empty((T, 3, cfg.heads), dtype=torch.int32, device=DEV)
    eng.engram_compress_hash(L, site.tid2eid, db["tokens"], db["cu_seqlens"], eids, rows, dead=db["dead"])
    torch.cuda.synchronize()
    assert np.array_equal(rows.cpu().numpy(), r_ref)
    others = torch.tensor([[1, 2, 3], [4, 5, 6], [0, 0, 0], [7, 8, 9]], dtype=torch.int32, device=DEV)
    for split in (0, 1, 3, 13, 40):
        store = site.site.make_store(4, ids=others)
        slots = torch.tensor([2], dtype=torch.int32, device=DEV)
        got_e, got_r = [], []
        pieces = [(0, split, 1)] + [(t, t + 1, 0) for t in range(split, T)]
        for a, b, start in pieces:
            n = b - a
            tk = db["tokens"][a:b].contiguous()
            dd = db["dead"][a:b].contiguous()
            cu = torch.tensor([0, n], dtype=torch.int32, device=DEV)
            ss = torch.tensor([start], dtype=torch.uint8, device=DEV)
            e = torch.empty(max(n, 1), dtype=torch.int32, device=DEV)
            r = torch.empty((max(n, 1), 3, cfg.heads), dtype=torch.int32, device=DEV)
            eng.engram_compress_hash(L, site.tid2eid, tk, cu, e, r, seq_start=ss, slots=slots,
                                     store=store, dead=dd)
            got_e.append(e[:n].cpu().numpy())
            got_r.append(r[:n].cpu().numpy())
        torch.cuda.synchronize()
        _no_device_error(eng, f"split {split}")
        assert np.array_equal(np.concatenate(got_e), e_ref), split
        assert np.array_equal(np.concatenate(got_r), r_ref), split
        # only slot 2 was used; the other slots keep their ids
        assert torch.equal(store.ids()[[0, 1, 3]], others[[0, 1, 3]])


def _decode_run(eng, name, steps):
    cfg = ei.get_config(name)
    worst = 0.0
    site = Site(cfg, max_tokens=cfg.n_seqs)
    store0 = ei.make_store_init(cfg)
    store_d = site.site.make_store(cfg.n_seqs, ids=torch.from_numpy(store0).to(DEV))
    store_ref = store0.copy()
    W = site.weight_bits()
    for k, batch in enumerate(ei.make_decode_steps(cfg, steps)):
        db = site.device_batch(batch)
        streams = ei.make_streams(cfg, batch.T, DEV, step=k)
        x0 = bf16_bits_np(streams)
        site.site.forward(db["tokens"], db["cu_seqlens"], streams, seq_start=db["seq_start"],
                          slots=db["slots"], store=store_d)
        torch.cuda.synchronize()
        _no_device_error(eng, f"{name} step {k}")
        e_ref, r_ref = site.oracle_hash(batch, store_ref)
        assert np.array_equal(site.site.eids[:batch.T].cpu().numpy(), e_ref), k
        assert np.array_equal(site.site.row_ids[:batch.T].cpu().numpy(), r_ref), k
        assert np.array_equal(store_d.ids().cpu().numpy(), store_ref), k
        # every token of every step: rows exact, v within the fp32 bound, streams
        b16 = _check_rows(site, r_ref, batch.T, site.site.rows)
        E = b16.reshape(batch.T, -1)
        v_ref = oracle_project(E, W)
        assert_v_close(site.site.v[:batch.T].cpu().numpy(), v_ref, E, W, f"{name} step {k} v")
        y_ref, _ = oracle_gate_add(x0, v_ref)
        worst = max(worst, assert_streams_close(bf16_bits_np(streams), y_ref, f"{name} step {k}"))
    log(f"{name}: {steps} steps x {cfg.n_seqs} tokens, every output checked against the oracle "
        f"(worst stream rel err {worst:.2e}; projection {site.site.projection_plan(0, cfg.n_seqs)})")


def test_decode_tiny_64_steps(eng):
    _decode_run(eng, "decode_tiny", 64)


def test_decode_prefill_shapes_64_steps(eng):
    _decode_run(eng, "decode", 64)
    _free()


# ---------------------------------------------------------------------------
# large workloads: every integer, sampled floats
# ---------------------------------------------------------------------------

def _large_run(eng, name, f32_sample, stream_sample, tables=None):
    cfg = ei.get_config(name)
    batch = ei.make_batch(cfg)
    T = batch.T
    site = Site(cfg, max_tokens=T, tables=tables)
    db = site.device_batch(batch)
    streams = ei.make_streams(cfg, T, DEV)
    log(f"{name}: forward over {T} tokens, {batch.S} sequences")
    idx = sample_tokens(batch, stream_sample, seed=cfg.seed)
    idx_d = torch.from_numpy(idx).to(DEV)
    x0 = bf16_bits_np(streams[idx_d])
    site.site.forward(db["tokens"], db["cu_seqlens"], streams, seq_start=db["seq_start"])
    torch.cuda.synchronize()
    _no_device_error(eng, f"{name} forward")
    e_ref, r_ref = site.oracle_hash(batch)
    assert np.array_equal(site.site.eids[:T].cpu().numpy(), e_ref)
    assert np.array_equal(site.site.row_ids[:T].cpu().numpy(), r_ref)
    log(f"{name}: eids and row ids exact on all tokens")
    fidx = sample_tokens(batch, f32_sample, seed=cfg.seed + 1)
    fidx_d = torch.from_numpy(fidx).to(DEV)
    rid_s = site.site.row_ids[fidx_d].contiguous()
    out32 = torch.empty((len(fidx), site.info.k_pad), dtype=torch.float32, device=DEV)
    eng.engram_gather_dequant(site.site.layout, site.tables.data, site.tables.scale, rid_s, out32)
    torch.cuda.synchronize()
    f32_ref, b16_ref = site.oracle_dequant(r_ref[fidx])
    D = cfg.row_dim
    g32 = out32.view(len(fidx), -1, site.info.seg_pitch).cpu().numpy()
    assert np.array_equal(g32[:, :, :D].view(np.uint32), f32_ref.view(np.uint32))
    g16 = bf16_bits_np(site.unpad(site.site.rows, T)[fidx_d])
    assert np.array_equal(g16[:, :, :D], b16_ref)
    assert not g16[:, :, D:].any()
    log(f"{name}: fp32 / bf16 rows exact on {len(fidx)} sampled tokens")
    if np.array_equal(idx, fidx):
        b16_s = b16_ref
    else:
        _, b16_s = site.oracle_dequant(r_ref[idx])
    E = b16_s.reshape(len(idx), -1)
    del b16_ref, f32_ref, g32, g16
    W = site.weight_bits()
    v_ref = oracle_project(E, W)
    v_rel = assert_v_close(site.site.v[idx_d].cpu().numpy(), v_ref, E, W, f"{name} v")
    y_ref, _ = oracle_gate_add(x0, v_ref)
    worst = assert_streams_close(bf16_bits_np(streams[idx_d]), y_ref, f"{name} streams")
    log(f"{name}: v and streams against the oracle on {len(idx)} of {T} tokens "
        f"(v within the fp32 bound, worst rel {v_rel:.1e}; streams worst {worst:.2e}; "
        f"projection {site.site.projection_plan(0, T)})")
    if cfg.table_dtype == "fp8":
        # the fused gather + projection at the same size: v equal bit for bit on every token
        v_f = torch.empty((T, cfg.hidden), dtype=torch.float32, device=DEV)
        eng.engram_gather_project(site.site.layout, site.tables.data, site.tables.scale,
                                  site.site.row_ids, site.site.weight, v_f, T=T)
        torch.cuda.synchronize()
        _no_device_error(eng, f"{name} fused")
        assert torch.equal(v_f.view(torch.int32), site.site.v[:T].view(torch.int32))
        assert_v_close(v_f[idx_d].cpu().numpy(), v_ref, E, W, f"{name} fused v")
        log(f"{name}: fused gather+projection equals the split path on all {T} tokens, and the "
            f"oracle on {len(idx)}")
        del v_f
        # the look-ahead order the benchmark times (next call's hash, projection, next
        # call's gather, gate), on the same tables: streams equal the sequential pass above
        # bit for bit, for the call gathered ahead and for the one gathered in between
        la = eng.Engram(
            vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
            heads_per_order=cfg.heads, rows=[cfg.rows] * 3, row_dim=cfg.row_dim,
            table_dtype=cfg.table_dtype, row_pitch_bytes=cfg.row_pitch_bytes,
            tid2eid=site.tid2eid, tables=site.tables.data, scales=site.tables.scale,
            weight=site.weight, hidden=cfg.hidden, hc_mult=cfg.hc_mult, max_tokens=T, lookahead=True)
        la.gather_ahead(db["tokens"], db["cu_seqlens"], seq_start=db["seq_start"])
        for nxt in (True, False):
            x = ei.make_streams(cfg, T, DEV)
            kw = dict(next_tokens=db["tokens"], next_cu_seqlens=db["cu_seqlens"],
                      next_seq_start=db["seq_start"]) if nxt else {}
            la.run_ahead(x, **kw)
            torch.cuda.synchronize()
            _no_device_error(eng, f"{name} look-ahead")
            assert torch.equal(x.view(torch.int16), streams.view(torch.int16))
            assert_streams_close(bf16_bits_np(x[idx_d]), y_ref, f"{name} look-ahead streams")
            del x
        log(f"{name}: look-ahead order equals the sequential pass on all {T} tokens "
            f"({la.projection_kind(0, T)} projection)")
        del la
    return site


def test_prefill_parity(eng):
    _large_run(eng, "prefill", f32_sample=None, stream_sample=None)
    _free()


def test_prefill_with_image_spans(eng):
    """The prefill workload with image spans (runs of dead positions, up to 64 long):
    compressed ids and row ids exact on every token, the streams of dead tokens
    untouched bit for bit, and the rows, v and streams of every token (including
    the three positions after each span, whose lookback the span blocks) against
    the oracle."""
    cfg = ei.get_config("prefill")
    b0 = ei.make_batch(cfg)
    T = b0.T
    dead = ei.make_dead_spans(T, 21, n_spans=48, max_len=64)
    batch = ei.Batch(tokens=b0.tokens, cu_seqlens=b0.cu_seqlens, seq_start=b0.seq_start,
                     slots=b0.slots, dead=dead)
    site = Site(cfg, max_tokens=T)
    db = site.device_batch(batch)
    streams = ei.make_streams(cfg, T, DEV)
    x_all = bf16_bits_np(streams)
    site.site.forward(db["tokens"], db["cu_seqlens"], streams, seq_start=db["seq_start"],
                      dead=db["dead"], keep=db["keep"])
    torch.cuda.synchronize()
    _no_device_error(eng, "prefill with image spans")
    e_ref, r_ref = site.oracle_hash(batch)
    assert np.array_equal(site.site.eids[:T].cpu().numpy(), e_ref)
    assert np.array_equal(site.site.row_ids[:T].cpu().numpy(), r_ref)
    y = bf16_bits_np(streams)
    keep = (dead == 0).astype(np.uint8)
    assert np.array_equal(y[keep == 0], x_all[keep == 0]), "a dead token's streams changed"
    after = [p for p in range(1, T) if dead[p - 1] and not dead[p]]
    _check_rows(site, r_ref, T, site.site.rows)
    _, b16 = site.oracle_dequant(r_ref)
    E = b16.reshape(T, -1)
    W = site.weight_bits()
    v_ref = oracle_project(E, W)
    assert_v_close(site.site.v[:T].cpu().numpy(), v_ref, E, W, "prefill with image spans v")
    y_ref, _ = oracle_gate_add(x_all, v_ref, keep=keep)
    worst = assert_streams_close(y, y_ref, "prefill with image spans")
    log(f"prefill with {int(dead.sum())} dead positions in {len(after)} spans: ids exact, dead streams "
        f"untouched, rows, v and streams of all {T} tokens against the oracle (worst {worst:.2e})")
    del site
    _free()


def test_long_prefill_parity(eng):
    _large_run(eng, "long", f32_sample=None, stream_sample=4096)
    _free()


@pytest.mark.timeout(900)
def test_full_scale_fp8_parity(eng):
    _large_run(eng, "full", f32_sample=1024, stream_sample=1024)
    _free()


@pytest.mark.timeout(900)
def test_full_scale_bf16_parity(eng):
    _large_run(eng, "full_bf16", f32_sample=1024, stream_sample=1024)
    _free()


# ---------------------------------------------------------------------------
# errors, determinism, projection shapes
# ---------------------------------------------------------------------------

def test_device_errors_are_reported(eng):
    cfg = ei.get_config("tiny")
    site = Site(cfg, max_tokens=64)
    L = site.site.layout
    e = torch.empty(64, dtype=torch.int32, device=DEV)
    r = torch.empty((64, 3, cfg.heads), dtype=torch.int32, device=DEV)
    cu = torch.tensor([0, 8], dtype=torch.int32, device=DEV)
    assert eng.engram_get_error() == 0
    bad_tok = torch.tensor([1, 2, 3, cfg.vocab, 5, 6, 7, 8], dtype=torch.int32, device=DEV)
    eng.engram_compress_hash(L, site.tid2eid, bad_tok, cu, e, r)
    assert eng.engram_get_error() == eng.ENGRAM_E_TOKEN_RANGE
    assert eng.engram_get_error() == 0  # cleared
    tok = torch.arange(8, dtype=torch.int32, device=DEV)
    eng.engram_compress_hash(L, site.tid2eid, tok, torch.tensor([0, 7], dtype=torch.int32, device=DEV), e, r)
    assert eng.engram_get_error() == eng.ENGRAM_E_SEQLENS
    eng.engram_compress_hash(L, site.tid2eid, tok, torch.tensor([2, 8], dtype=torch.int32, device=DEV), e, r)
    assert eng.engram_get_error() == eng.ENGRAM_E_SEQLENS
    ss0 = torch.zeros(1, dtype=torch.uint8, device=DEV)
    eng.engram_compress_hash(L, site.tid2eid, tok, cu, e, r, seq_start=ss0)
    assert eng.engram_get_error() == eng.ENGRAM_E_NEED_STORE
    store = site.site.make_store(4)
    eng.engram_compress_hash(L, site.tid2eid, tok, cu, e, r, seq_start=ss0,
                             slots=torch.tensor([4], dtype=torch.int32, device=DEV), store=store)
    assert eng.engram_get_error() == eng.ENGRAM_E_SLOT_RANGE
    bad_rows = torch.zeros((8, 3, cfg.heads), dtype=torch.int32, device=DEV)
    bad_rows[3, 1, 0] = cfg.rows
    bad_rows[4, 2, 1] = -1
    out = torch.full((8, site.info.k_pad), 3.0, dtype=torch.bfloat16, device=DEV)
    eng.engram_gather_dequant(L, site.tables.data, site.tables.scale, bad_rows, out)
    assert eng.engram_get_error() == eng.ENGRAM_E_ROW_RANGE
    seg = out.view(8, 3 * cfg.heads, site.info.seg_pitch)
    assert (seg[3, 1 * cfg.heads + 0].float() == 0).all() and (seg[4, 2 * cfg.heads + 1].float() == 0).all()
    bad_map = site.tid2eid.clone()
    bad_map[5] = cfg.vc
    with pytest.raises(eng.EngramError) as ex:
        eng.engram_tid2eid_check(L, bad_map)
    assert ex.value.status == eng.ENGRAM_E_MAP_RANGE
    assert eng.engram_tid2eid_check(L, site.tid2eid) == site.pad_eid
    assert eng.engram_get_error() == 0


def test_repeat_runs_are_bitwise_identical(eng):
    cfg = ei.get_config("prefill")
    batch = ei.make_batch(cfg)
    site = Site(cfg, max_tokens=batch.T)
    db = site.device_batch(batch)
    outs = []
    for _ in range(2):
        streams = ei.make_streams(cfg, batch.T, DEV)
        site.site.forward(db["tokens"], db["cu_seqlens"], streams, seq_start=db["seq_start"])
        torch.cuda.synchronize()
        outs.append((site.site.row_ids.clone(), site.site.rows.clone(), site.site.v.clone(), streams))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                           b.view(torch.uint8) if b.dtype != torch.int32 else b)
    del outs, site
    _free()


@pytest.mark.parametrize("M,N,cols,D", [(1, 8, 3, 64), (77, 200, 3, 100), (300, 512, 6, 128),
                                        (1000, 264, 3, 192), (4097, 4096, 3, 512)])
def test_projection_ragged_shapes_vs_torch_fp32(eng, M, N, cols, D):
    """The MFMA projection on ragged M and N (tile tails) against torch's fp32
    matmul of the same bf16 operands."""
    H = cols // 3
    L = eng.engram_layout_create(vocab_size=8, compressed_vocab=4, pad_token_id=7, heads_per_order=H,
                                 rows=[100_000] * 3, row_dim=D, table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                 row_pitch_bytes=(D + 15) // 16 * 16)
    K = L.info.k_pad
    g = torch.Generator(device=DEV)
    g.manual_seed(M * 1000 + N)
    A = torch.randn((M, K), generator=g, device=DEV).to(torch.bfloat16)
    B = (torch.randn((N, K), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
    v = torch.empty((M, N), dtype=torch.float32, device=DEV)
    eng.engram_project(L, A, B, v)
    ref = A.float() @ B.float().T
    torch.cuda.synchronize()
    # both results carry an fp32 accumulation error of at most K u sum|a b|
    bound = 2 * K * 2.0 ** -24 * (A.float().abs() @ B.float().abs().T) + 1e-6
    assert ((v - ref).abs() <= bound).all()
