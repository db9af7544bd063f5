"""Seeded random layouts end to end against the oracle.

Each case draws a layout the named workloads do not cover -- 1 to 3 heads per order,
row widths from 1 to 520 elements (most not a multiple of 16 or 64), vocabularies
and compressed vocabularies of any size, a random PAD token, tables of 64 to 60,000
rows, e4m3fn tables with power-of-two or amax/448 row scales or bf16 tables, hidden
sizes that are any multiple of 8 up to 1,032, and a forced or chosen split of the
projection -- and a ragged call through the store: empty and one-token sequences,
starts and continuations, sequences without a slot, image-span dead positions.

Bars: compressed ids, row ids and the store bit-exact on every token; the bf16 rows
bit-exact with zero segment padding; v within the fp32 accumulation bound of the
oracle's fp64 projection; the streams within 2e-2 of the oracle, and bit for bit
unchanged for dead tokens.
"""
import gc

import numpy as np
import pytest
import torch

import engram_inputs as ei
from engram_harness import (DEV, Site, assert_streams_close, assert_v_close, bf16_bits_np, log,
                            oracle_gate_add, oracle_project)

pytestmark = pytest.mark.gpu

CASES = 40


@pytest.fixture(scope="module")
def eng():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import hashed_gram_memory_tid2eid_amd as e
    return e


def _case(k: int):
    rng = np.random.default_rng(np.random.SeedSequence([20261203, k]))
    heads = int(rng.integers(1, 4))
    row_dim = int(rng.integers(1, 521))
    table_dtype = "bf16" if k % 4 == 3 else "fp8"
    scale_mode = "amax" if k % 4 == 1 else "pow2"
    vc = int(rng.integers(2, 65537))
    vocab = int(rng.integers(vc, vc + 200_000))
    pad = int(rng.integers(0, vocab))
    rows = int(rng.integers(64, 60_001))
    hidden = 8 * int(rng.integers(1, 130))
    splits = int(rng.choice([0, 0, 1, 2]))
    k_pad = 3 * heads * (-(-row_dim // 64) * 64)
    if splits == 2 and k_pad % 128:
        splits = 1  # a forced split must divide k_pad into whole 64-wide steps
    cfg = ei.EngramConfig(f"random{k}", 1000 + k, 1, 1, "zipf" if k % 2 else "uniform", rows, heads,
                          row_dim, hidden, table_dtype=table_dtype, vocab=vocab, vc=vc, pad_token_id=pad)
    # a ragged call: 1..14 sequences of 0..120 tokens, some continuing from the store
    S = int(rng.integers(1, 15))
    lens = rng.integers(0, 121, size=S).astype(np.int32)
    lens[rng.random(S) < 0.2] = 0
    lens[rng.random(S) < 0.2] = 1
    cu = np.zeros(S + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    tokens = (ei.zipf_tokens(rng, T, vocab) if k % 2 else ei.uniform_tokens(rng, T, vocab)).astype(np.int32)
    num_slots = S + 3
    slots = rng.permutation(num_slots)[:S].astype(np.int32)
    slots[rng.random(S) < 0.15] = -1
    seq_start = (rng.random(S) < 0.4).astype(np.uint8)
    seq_start[slots < 0] = 1
    dead = ei.make_dead_spans(T, 1000 + k, n_spans=int(rng.integers(0, 6)), max_len=7)
    store0 = rng.integers(0, vc, size=(num_slots, 3)).astype(np.int32)
    batch = ei.Batch(tokens=tokens, cu_seqlens=cu, seq_start=seq_start, slots=slots, dead=dead)
    return cfg, scale_mode, splits, batch, store0


@pytest.mark.parametrize("k", range(CASES))
def test_random_layout_end_to_end(eng, k):
    cfg, scale_mode, splits, batch, store0 = _case(k)
    T = batch.T
    log(f"case {k}: H={cfg.heads} D={cfg.row_dim} {cfg.table_dtype}/{scale_mode} vocab={cfg.vocab} "
        f"vc={cfg.vc} pad={cfg.pad_token_id} rows={cfg.rows} hidden={cfg.hidden} splits={splits} "
        f"T={T} S={batch.S}")
    site = Site(cfg, max_tokens=max(T, 1), scale_mode=scale_mode, proj_splits=splits)
    store_d = site.site.make_store(store0.shape[0], ids=torch.from_numpy(store0).to(DEV))
    db = site.device_batch(batch)
    streams = ei.make_streams(cfg, T, DEV, step=k)
    x0 = bf16_bits_np(streams)
    site.site.forward(db["tokens"], db["cu_seqlens"], streams, seq_start=db["seq_start"],
                      slots=db["slots"], store=store_d, dead=db["dead"], keep=db["keep"])
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    store_ref = store0.copy()
    e_ref, r_ref = site.oracle_hash(batch, store_ref)
    assert np.array_equal(store_d.ids().cpu().numpy(), store_ref), "store"
    if T == 0:
        log(f"case {k}: no tokens; the store equals the oracle's")
        return
    assert np.array_equal(site.site.eids[:T].cpu().numpy(), e_ref), "compressed ids"
    assert np.array_equal(site.site.row_ids[:T].cpu().numpy(), r_ref), "row ids"
    _, b16 = site.oracle_dequant(r_ref)
    got = bf16_bits_np(site.unpad(site.site.rows, T))
    D = cfg.row_dim
    assert np.array_equal(got[:, :, :D], b16), "rows"
    assert not got[:, :, D:].any(), "segment padding"
    E = b16.reshape(T, -1)
    W = site.weight_bits()
    v_ref = oracle_project(E, W)
    assert_v_close(site.site.v[:T].cpu().numpy(), v_ref, E, W, f"case {k} v")
    keep = (batch.dead == 0).astype(np.uint8)
    y_ref, _ = oracle_gate_add(x0, v_ref, keep)
    y = bf16_bits_np(streams)
    assert np.array_equal(y[keep == 0], x0[keep == 0]), "dead tokens' streams changed"
    worst = assert_streams_close(y, y_ref, f"case {k} streams")
    log(f"case {k}: every output equals the oracle ({site.site.projection_plan(0, T)}, streams worst "
        f"{worst:.1e})")
    del site, store_d, streams
    gc.collect()
    torch.cuda.empty_cache()
