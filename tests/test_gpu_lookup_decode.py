"""engram_lookup_decode: a decode step's compress, hash and gather in one launch.

Bars: bit for bit what engram_compress_hash (each token its own sequence) followed by
engram_gather_dequant write -- compressed ids, row ids, the store and the bf16 rows --
and, through Engram.decode_step, the same v and streams as Engram.forward; against
the oracle: ids, row ids and the store exact and the rows exact on every token of
every step, v within the fp32 bound and the streams within 2e-2 on every token of
the first and last steps.  Covered: 64 steps at the tiny shapes and 16 at the
prefill shapes (256 slots), tokens without a slot (they start their sequence) and
dead tokens among them, slots in any order, and device errors.
"""
import gc

import numpy as np
import pytest
import torch

import engram_inputs as ei
from engram_harness import (DEV, Site, assert_streams_close, assert_v_close, bf16_bits_np, log,
                            oracle_gate_add, oracle_project)

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


def _d(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("name,steps", [("decode_tiny", 64), ("decode", 16)])
def test_decode_step_equals_forward_and_the_oracle(eng, name, steps):
    cfg = ei.get_config(name)
    S = cfg.n_seqs
    a = Site(cfg, max_tokens=S)
    b = Site(cfg, max_tokens=S, tables=a.tables)
    assert b.site.decode_lookup_supported
    store0 = ei.make_store_init(cfg)
    st_a = a.site.make_store(S, ids=_d(store0))
    st_b = b.site.make_store(S, ids=_d(store0))
    store_ref = store0.copy()
    W = a.weight_bits()
    for k, batch in enumerate(ei.make_decode_steps(cfg, steps)):
        db = a.device_batch(batch)
        xa = ei.make_streams(cfg, S, DEV, step=k)
        xb = xa.clone()
        x0 = bf16_bits_np(xa)
        a.site.forward(db["tokens"], db["cu_seqlens"], xa, seq_start=db["seq_start"], slots=db["slots"],
                       store=st_a)
        b.site.decode_step(db["tokens"], xb, slots=db["slots"], store=st_b)
        torch.cuda.synchronize()
        assert eng.engram_get_error() == 0
        assert torch.equal(a.site.eids[:S], b.site.eids[:S]), k
        assert torch.equal(a.site.row_ids[:S], b.site.row_ids[:S]), k
        assert torch.equal(st_a.ids(), st_b.ids()), k
        assert torch.equal(a.site.rows[:S].view(torch.int16), b.site.rows[:S].view(torch.int16)), k
        assert torch.equal(a.site.v[:S].view(torch.int32), b.site.v[:S].view(torch.int32)), k
        assert torch.equal(xa.view(torch.int16), xb.view(torch.int16)), k
        e_ref, r_ref = b.oracle_hash(batch, store_ref)
        assert np.array_equal(b.site.eids[:S].cpu().numpy(), e_ref), k
        assert np.array_equal(b.site.row_ids[:S].cpu().numpy(), r_ref), k
        assert np.array_equal(st_b.ids().cpu().numpy(), store_ref), k
        _, b16 = b.oracle_dequant(r_ref)
        got = bf16_bits_np(b.unpad(b.site.rows, S))
        assert np.array_equal(got[:, :, :cfg.row_dim], b16), k
        assert not got[:, :, cfg.row_dim:].any(), k
        if k in (0, steps - 1):
            E = b16.reshape(S, -1)
            v_ref = oracle_project(E, W)
            assert_v_close(b.site.v[:S].cpu().numpy(), v_ref, E, W, f"{name} step {k} v")
            y_ref, _ = oracle_gate_add(x0, v_ref)
            assert_streams_close(bf16_bits_np(xb), y_ref, f"{name} step {k} streams")
    log(f"{name}: {steps} decode steps through the one-launch lookup equal forward bit for bit; ids, "
        f"row ids, store and rows equal the oracle on every step, v and streams on the first and last")
    del a, b
    _free()


def test_starts_dead_tokens_and_slot_order(eng):
    """Tokens without a slot start their sequence; dead tokens hash an all-PAD window and
    leave the PAD tail; slots come in any order and the store has more of them than
    the call has tokens.  Equal to engram_compress_hash (cu_seqlens 0..T, seq_start 1
    for tokens without a slot) + engram_gather_dequant, and to the oracle."""
    cfg = ei.get_config("decode_tiny")
    T, num_slots = 200, 300
    site = Site(cfg, max_tokens=T)
    L = site.site.layout
    rng = np.random.default_rng(31)
    tokens = ei.zipf_tokens(rng, T).astype(np.int32)
    slots = rng.permutation(num_slots)[:T].astype(np.int32)
    slots[rng.random(T) < 0.2] = -1
    dead = (rng.random(T) < 0.15).astype(np.uint8)
    store0 = rng.integers(0, cfg.vc, size=(num_slots, 3)).astype(np.int32)
    cu = np.arange(T + 1, dtype=np.int32)
    seq_start = (slots < 0).astype(np.uint8)
    batch = ei.Batch(tokens=tokens, cu_seqlens=cu, seq_start=seq_start, slots=slots, dead=dead)
    # the one-launch lookup
    st1 = site.site.make_store(num_slots, ids=_d(store0))
    e1 = torch.empty(T, dtype=torch.int32, device=DEV)
    r1 = torch.empty((T, 3, cfg.heads), dtype=torch.int32, device=DEV)
    rows1 = torch.full((T, site.info.k_pad + 8), 7, dtype=torch.bfloat16, device=DEV)
    eng.engram_lookup_decode(L, site.tid2eid, _d(tokens), e1, r1, site.tables.data, site.tables.scale,
                             rows1, slots=_d(slots), store=st1, dead=_d(dead))
    # the two kernels it stands for
    st2 = site.site.make_store(num_slots, ids=_d(store0))
    e2 = torch.empty_like(e1)
    r2 = torch.empty_like(r1)
    rows2 = torch.full_like(rows1, 7)
    eng.engram_compress_hash(L, site.tid2eid, _d(tokens), _d(cu), e2, r2, seq_start=_d(seq_start),
                             slots=_d(slots), store=st2, dead=_d(dead))
    eng.engram_gather_dequant(L, site.tables.data, site.tables.scale, r2, rows2, T=T)
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    assert torch.equal(e1, e2) and torch.equal(r1, r2) and torch.equal(st1.ids(), st2.ids())
    assert torch.equal(rows1.view(torch.int16), rows2.view(torch.int16))  # incl. the untouched columns
    store_ref = store0.copy()
    e_ref, r_ref = site.oracle_hash(batch, store_ref)
    assert np.array_equal(e1.cpu().numpy(), e_ref)
    assert np.array_equal(r1.cpu().numpy(), r_ref)
    assert np.array_equal(st1.ids().cpu().numpy(), store_ref)
    _, b16 = site.oracle_dequant(r_ref)
    got = bf16_bits_np(rows1[:, :site.info.k_pad].contiguous()).reshape(T, 3 * cfg.heads, -1)
    assert np.array_equal(got[:, :, :cfg.row_dim], b16)
    log(f"lookup_decode: {T} tokens ({int((slots < 0).sum())} without a slot, {int(dead.sum())} dead) "
        f"equal compress_hash + gather_dequant and the oracle")
    del site
    _free()


def test_lookup_decode_device_errors(eng):
    """A token outside the vocabulary latches ENGRAM_E_TOKEN_RANGE and a slot past the
    store ENGRAM_E_SLOT_RANGE, as engram_compress_hash does; the outputs of the other
    tokens still equal the two-kernel path's."""
    cfg = ei.get_config("decode_tiny")
    T = 64
    site = Site(cfg, max_tokens=T)
    L = site.site.layout
    rng = np.random.default_rng(5)
    tokens = ei.zipf_tokens(rng, T).astype(np.int32)
    for bad_tok, bad_slot, expect in ((True, False, eng.ENGRAM_E_TOKEN_RANGE),
                                      (False, True, eng.ENGRAM_E_SLOT_RANGE)):
        tk = tokens.copy()
        slots = np.arange(T, dtype=np.int32)
        if bad_tok:
            tk[9] = cfg.vocab
        if bad_slot:
            slots[9] = T + 5
        st = site.site.make_store(T, ids=_d(ei.make_store_init(cfg, T)))
        e = torch.empty(T, dtype=torch.int32, device=DEV)
        r = torch.empty((T, 3, cfg.heads), dtype=torch.int32, device=DEV)
        rows = torch.empty((T, site.info.k_pad), dtype=torch.bfloat16, device=DEV)
        eng.engram_lookup_decode(L, site.tid2eid, _d(tk), e, r, site.tables.data, site.tables.scale,
                                 rows, slots=_d(slots), store=st)
        torch.cuda.synchronize()
        assert eng.engram_get_error() == expect
        assert eng.engram_get_error() == 0  # read and cleared
        keep = np.arange(T) != 9
        st2 = site.site.make_store(T, ids=_d(ei.make_store_init(cfg, T)))
        e2, r2 = torch.empty_like(e), torch.empty_like(r)
        rows2 = torch.empty_like(rows)
        cu = np.arange(T + 1, dtype=np.int32)
        ss = np.zeros(T, np.uint8)
        eng.engram_compress_hash(L, site.tid2eid, _d(tk), _d(cu), e2, r2, seq_start=_d(ss),
                                 slots=_d(np.where(slots < T, slots, -1).astype(np.int32)), store=st2)
        eng.engram_gather_dequant(L, site.tables.data, site.tables.scale, r2, rows2, T=T)
        torch.cuda.synchronize()
        eng.engram_get_error()
        k = torch.from_numpy(keep).to(DEV)
        assert torch.equal(e[k], e2[k]) and torch.equal(r[k], r2[k])
        assert torch.equal(rows[k].view(torch.int16), rows2[k].view(torch.int16))
    del site
    _free()
