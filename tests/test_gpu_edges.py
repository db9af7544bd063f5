"""Edge cases on the device: calls with no tokens, sequences with no tokens, and a
gather of more than 2^31 16-element output chunks (one kernel launch indexes fewer,
so the library splits such a call by tokens).

Bars: a call with no tokens returns OK and leaves every output byte as it was;
empty sequences update the slot store exactly as the oracle's store does; the split
gather equals the oracle's dequant (bf16 bits, exact) on sampled tokens at both ends
and on both sides of the launch boundary.
"""
import gc

import numpy as np
import pytest
import torch

import engram_inputs as ei
import oracle
from engram_harness import DEV, Site, log

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


def test_calls_without_tokens_leave_outputs_untouched(eng):
    cfg = ei.get_config("tiny")
    site = Site(cfg, max_tokens=64)
    L = site.site.layout
    info = site.info
    w = site.site.weight
    eids = torch.full((64,), -7, dtype=torch.int32, device=DEV)
    rid = torch.full((64, 3, cfg.heads), -7, dtype=torch.int32, device=DEV)
    rows = torch.full((64, info.k_pad), 3.0, dtype=torch.bfloat16, device=DEV)
    v = torch.full((64, cfg.hidden), 5.0, dtype=torch.float32, device=DEV)
    partials = torch.full((4 * 64 * cfg.hidden,), 9.0, dtype=torch.float32, device=DEV)
    streams = torch.full((64, 4, cfg.hidden), 1.5, dtype=torch.bfloat16, device=DEV)
    before = [t.clone() for t in (eids, rid, rows, v, partials, streams)]
    tok = torch.empty(0, dtype=torch.int32, device=DEV)
    cu = torch.zeros(1, dtype=torch.int32, device=DEV)
    assert eng.engram_get_error() == 0
    eng.engram_compress_hash(L, site.tid2eid, tok, cu, eids, rid)
    eng.engram_gather_dequant(L, site.tables.data, site.tables.scale, rid, rows, T=0)
    eng.engram_project(L, rows, w, v, T=0)
    eng.engram_gather_project(L, site.tables.data, site.tables.scale, rid, w, v, T=0)
    eng.engram_project_splitk(L, rows, w, partials, 4, T=0)
    eng.engram_gate_add(L, v, streams, T=0)
    eng.engram_gate_add_partials(L, partials, 4, streams, T=0)
    wkv = eng.engram_wkv_create(L, w, 64)
    eng.engram_gated_residual(L, rows, wkv, streams, v, T=0)
    eng.engram_wkv_project(L, rows, wkv, v, T=0)
    eng.engram_wkv_gate_add(L, wkv, v, streams, T=0)
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    for a, b in zip(before, (eids, rid, rows, v, partials, streams)):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    _free()


def test_empty_sequences_update_the_store_like_the_oracle(eng):
    """A call whose sequences hold no tokens: a sequence that starts here resets its
    slot to the pad id, one that continues leaves its slot as it was; mixed with
    non-empty sequences in a second call."""
    cfg = ei.get_config("tiny")
    site = Site(cfg, max_tokens=64)
    L = site.site.layout
    rng = np.random.default_rng(77)
    num_slots = 10
    store0 = rng.integers(0, cfg.vc, size=(num_slots, 3)).astype(np.int32)
    e = torch.empty(64, dtype=torch.int32, device=DEV)
    r = torch.empty((64, 3, cfg.heads), dtype=torch.int32, device=DEV)
    calls = [
        ei.Batch(tokens=np.zeros(0, np.int32), cu_seqlens=np.zeros(4, np.int32),
                 seq_start=np.array([1, 0, 1], np.uint8), slots=np.array([2, 5, 7], np.int32)),
        ei.Batch(tokens=ei.zipf_tokens(rng, 9), cu_seqlens=np.array([0, 0, 4, 4, 9, 9], np.int32),
                 seq_start=np.array([1, 0, 1, 0, 0], np.uint8), slots=np.array([0, 2, 3, 5, 8], np.int32)),
    ]
    store = site.site.make_store(num_slots, ids=torch.from_numpy(store0).to(DEV))
    ref = store0.copy()
    after = []
    for b in calls:
        db = site.device_batch(b)
        eng.engram_compress_hash(L, site.tid2eid, db["tokens"], db["cu_seqlens"], e, r,
                                 seq_start=db["seq_start"], slots=db["slots"], store=store)
        torch.cuda.synchronize()
        assert eng.engram_get_error() == 0
        e_ref, r_ref = site.oracle_hash(b, ref)
        assert np.array_equal(store.ids().cpu().numpy(), ref)
        if b.T:
            assert np.array_equal(e[:b.T].cpu().numpy(), e_ref)
            assert np.array_equal(r[:b.T].cpu().numpy(), r_ref)
        after.append(ref.copy())
    # the first call reset slots 2 and 7 and left slot 5 (and the unused ones) alone
    first = after[0]
    assert (first[[2, 7]] == site.pad_eid).all()
    keep = [i for i in range(num_slots) if i not in (2, 7)]
    assert np.array_equal(first[keep], store0[keep])
    _free()


def test_gather_split_past_2_31_chunks(eng):
    """3 orders x 8 heads of 256-element rows: 384 chunks per token, so one launch
    takes at most 5,592,404 tokens; 3,000 more force a second launch.  The output is
    68.8 GB of bf16."""
    H, D, rows = 8, 256, 4096
    L = eng.engram_layout_create(vocab_size=8, compressed_vocab=4, pad_token_id=7, heads_per_order=H,
                                 rows=[rows] * 3, row_dim=D, table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                 row_pitch_bytes=D)
    info = L.info
    cols = 3 * H
    chunks_per_token = cols * (info.seg_pitch // 16)
    per_launch = (1 << 31) // chunks_per_token - 1
    T = per_launch + 3000
    assert T * chunks_per_token >= (1 << 31)
    g = torch.Generator(device=DEV)
    g.manual_seed(2024)
    tabs, scales = [], []
    for _ in range(3):
        t = torch.randint(0, 256, (rows, D), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
        t[t == 0x7F] = 0x7E
        t[t == 0xFF] = 0xFE
        tabs.append(t.reshape(-1))
        scales.append(torch.exp(torch.randn(rows, generator=g, device=DEV) * 0.5 - 6.0))
    prime = torch.tensor([info.site_primes[0][n][h] for n in range(3) for h in range(H)], device=DEV)
    off = torch.tensor([info.site_offsets[0][n][h] for n in range(3) for h in range(H)], device=DEV)
    rid = torch.empty((T, cols), dtype=torch.int32, device=DEV)
    step = 1 << 22
    for t0 in range(0, T, step):
        n = min(step, T - t0)
        x = torch.randint(0, 1 << 30, (n, cols), generator=g, device=DEV, dtype=torch.int64)
        rid[t0:t0 + n] = (x % prime + off).to(torch.int32)
        del x
    out = torch.empty((T, info.k_pad), dtype=torch.bfloat16, device=DEV)
    log(f"split gather: T={T:,} tokens, {T * chunks_per_token:,} chunks, "
        f"{out.numel() * 2 / 1e9:.1f} GB out, {per_launch:,} tokens per launch")
    eng.engram_gather_dequant(L, tabs, scales, rid, out)
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    edge = [0, 1, 2, per_launch - 2, per_launch - 1, per_launch, per_launch + 1, T - 2, T - 1]
    rng = np.random.default_rng(5)
    sample = np.unique(np.concatenate([edge, rng.integers(0, T, size=64)])).astype(np.int64)
    idx = torch.from_numpy(sample).to(DEV)
    rs = rid.index_select(0, idx).cpu().numpy()  # [n][cols]
    got = out.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
    n_s = len(sample)
    raw = np.zeros((n_s, cols, D), np.uint8)
    sc = np.zeros((n_s, cols), np.float32)
    for c in range(cols):
        o = c // H
        ridx = torch.from_numpy(rs[:, c].astype(np.int64)).to(DEV)
        raw[:, c] = tabs[o].view(rows, D).index_select(0, ridx).cpu().numpy()
        sc[:, c] = scales[o].index_select(0, ridx).cpu().numpy()
    _, b16 = oracle.dequant_rows(raw.reshape(-1, D), sc.reshape(-1))
    assert np.array_equal(got.reshape(n_s, cols, D), b16.reshape(n_s, cols, D))
    log(f"split gather: {n_s} sampled tokens (both launch edges) equal the oracle")
    del out, rid, tabs, scales
    _free()


@pytest.mark.parametrize("S", [255, 3000])
def test_many_short_sequences_against_the_oracle(eng, S):
    """Sequences of 0..4 tokens with a slot store, mixed starts and dead spans, over
    several workgroups (the store update runs as its own kernel after the hash)."""
    cfg = ei.get_config("tiny")
    rng = np.random.default_rng(91 + S)
    lens = rng.integers(0, 5, size=S).astype(np.int32)
    cu = np.zeros(S + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    num_slots = S + 500
    site = Site(cfg, max_tokens=T)
    L = site.site.layout
    batch = ei.Batch(tokens=ei.zipf_tokens(rng, T), cu_seqlens=cu,
                     seq_start=(rng.random(S) < 0.5).astype(np.uint8),
                     slots=rng.permutation(num_slots)[:S].astype(np.int32),
                     dead=ei.make_dead_spans(T, 11, n_spans=T // 50, max_len=3))
    store0 = rng.integers(0, cfg.vc, size=(num_slots, 3)).astype(np.int32)
    store = site.site.make_store(num_slots, ids=torch.from_numpy(store0).to(DEV))
    e = torch.empty(T, dtype=torch.int32, device=DEV)
    r = torch.empty((T, 3, cfg.heads), dtype=torch.int32, device=DEV)
    db = site.device_batch(batch)
    eng.engram_compress_hash(L, site.tid2eid, db["tokens"], db["cu_seqlens"], e, r,
                             seq_start=db["seq_start"], slots=db["slots"], store=store, dead=db["dead"])
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    ref = store0.copy()
    e_ref, r_ref = site.oracle_hash(batch, ref)
    assert np.array_equal(e.cpu().numpy(), e_ref)
    assert np.array_equal(r.cpu().numpy(), r_ref)
    assert np.array_equal(store.ids().cpu().numpy(), ref)
    log(f"{S} sequences, {T} tokens: ids, row ids and store equal the oracle")
    _free()
