"""The look-ahead order (Engram.gather_ahead / run_ahead): the next call's hash and
gather placed between this call's projection and gate, on one stream.

Bar: every output (streams, and v of the last call) equals sequential
Engram.forward calls bit for bit -- the same kernels run on the same inputs, only
in another order -- for one site with the plain, packed and split-K projections
(with a dead span in one call), for two sites with per-site row buffers, and for
decode steps that continue their stored history (the store equal too).
"""
import gc

import pytest
import torch

import engram_inputs as ei
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


def _calls(cfg, n, T):
    """n calls of the workload's batch shape with different tokens (rotations of its
    token stream), the second with a dead span and the matching keep mask."""
    b = ei.make_batch(cfg)
    tok = torch.from_numpy(b.tokens).to(DEV)
    cu = torch.from_numpy(b.cu_seqlens).to(DEV)
    calls = []
    for k in range(n):
        dead = keep = None
        if k == 1:
            dead = torch.zeros(T, dtype=torch.uint8, device=DEV)
            dead[T // 3: T // 3 + 17] = 1
            keep = 1 - dead
        calls.append(dict(tokens=torch.roll(tok, 37 * k).contiguous(), cu=cu, dead=dead, keep=keep))
    return calls


def _engram(eng, cfg, T, lookahead, **kw):
    NS = cfg.n_sites
    tables = [ei.make_tables(cfg, DEV, site=s) for s in range(NS)]
    weights = [ei.make_weight(cfg, DEV, site=s) for s in range(NS)]
    one = NS == 1
    return eng.Engram(vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
                      heads_per_order=cfg.heads,
                      rows=[cfg.rows] if cfg.table_split == "site" else [cfg.rows] * 3,
                      row_dim=cfg.row_dim, table_dtype=cfg.table_dtype,
                      row_pitch_bytes=cfg.row_pitch_bytes,
                      tid2eid=torch.from_numpy(ei.make_tid2eid(cfg.vocab, cfg.vc)).to(DEV),
                      tables=tables[0].data if one else [t.data for t in tables],
                      scales=tables[0].scale if one else [t.scale for t in tables],
                      weight=weights[0] if one else weights, hidden=cfg.hidden,
                      max_tokens=T, num_sites=NS, table_split=cfg.table_split,
                      scale_block=cfg.scale_block, hash_floor=cfg.hash_floor, lookahead=lookahead, **kw)


def _streams(cfg, T, n):
    NS = cfg.n_sites
    out = []
    for k in range(n):
        per = [ei.make_streams(cfg, T, DEV, step=10 * k + s) for s in range(NS)]
        out.append(per[0] if NS == 1 else per)
    return out


def _run_both(eng, cfg, n=3, **kw):
    T = ei.make_batch(cfg).T
    calls = _calls(cfg, n, T)
    seq_site = _engram(eng, cfg, T, False, **kw)
    seq_out = _streams(cfg, T, n)
    for c, x in zip(calls, seq_out):
        seq_site.forward(c["tokens"], c["cu"], x, dead=c["dead"], keep=c["keep"])
    torch.cuda.synchronize()
    v_seq = seq_site.v.clone()
    kind = seq_site.projection_kind(0, T)
    del seq_site
    _free()
    la_site = _engram(eng, cfg, T, True, **kw)
    la_out = _streams(cfg, T, n)
    la_site.gather_ahead(calls[0]["tokens"], calls[0]["cu"], dead=calls[0]["dead"])
    for k in range(n):
        nxt = calls[k + 1] if k + 1 < n else None
        la_site.run_ahead(la_out[k], keep=calls[k]["keep"],
                          next_tokens=None if nxt is None else nxt["tokens"],
                          next_cu_seqlens=None if nxt is None else nxt["cu"],
                          next_dead=None if nxt is None else nxt["dead"])
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    assert la_site.pending_T is None
    for a, b in zip(seq_out, la_out):
        for x, y in zip(a if isinstance(a, list) else [a], b if isinstance(b, list) else [b]):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.equal(v_seq.view(torch.int32), la_site.v.view(torch.int32))
    del la_site
    _free()
    return kind


@pytest.mark.parametrize("name,proj_splits,expect", [("tiny", 1, "plain"), ("tiny", 4, "splitk"),
                                                      ("prefill", 0, "packed")])
def test_lookahead_equals_sequential_one_site(eng, name, proj_splits, expect):
    cfg = ei.get_config(name)
    kind = _run_both(eng, cfg, proj_splits=proj_splits)
    assert kind == expect
    log(f"look-ahead order, {name} ({kind} projection): bit-identical to sequential calls")


def test_lookahead_equals_sequential_two_sites(eng):
    cfg = ei.get_config("v41_small")
    kind = _run_both(eng, cfg)
    log(f"look-ahead order, v41_small (two sites, {kind} projection): bit-identical")


def test_lookahead_needs_a_gathered_call(eng):
    cfg = ei.get_config("tiny")
    T = ei.make_batch(cfg).T
    site = _engram(eng, cfg, T, True)
    x = ei.make_streams(cfg, T, DEV)
    with pytest.raises(RuntimeError):
        site.run_ahead(x)
    plain = _engram(eng, cfg, T, False)
    c = _calls(cfg, 1, T)[0]
    with pytest.raises(ValueError):
        plain.gather_ahead(c["tokens"], c["cu"])
    # a waiting call's rows are not overwritten by a plain forward
    site.gather_ahead(c["tokens"], c["cu"])
    with pytest.raises(RuntimeError):
        site.forward(c["tokens"], c["cu"], x)
    with pytest.raises(RuntimeError):
        site.gather_ahead(c["tokens"], c["cu"])
    site.run_ahead(x)
    site.forward(c["tokens"], c["cu"], x)
    del site, plain
    _free()


def test_lookahead_decode_steps_with_store(eng):
    """Decode steps (256 slots, one new token each, continuing their stored
    history) in the look-ahead order: every step's streams and the store after the
    last step equal sequential forward calls bit for bit (the split-K projection)."""
    cfg = ei.get_config("decode")
    steps = ei.make_decode_steps(cfg, 6)
    T = steps[0].T
    dev_steps = [dict(tokens=torch.from_numpy(b.tokens).to(DEV), cu=torch.from_numpy(b.cu_seqlens).to(DEV),
                      ss=torch.from_numpy(b.seq_start).to(DEV), sl=torch.from_numpy(b.slots).to(DEV))
                 for b in steps]
    store0 = torch.from_numpy(ei.make_store_init(cfg)).to(DEV)
    seq_site = _engram(eng, cfg, T, False)
    store_seq = seq_site.make_store(cfg.n_seqs, ids=store0)
    seq_out = [ei.make_streams(cfg, T, DEV, step=k) for k in range(len(steps))]
    for c, x in zip(dev_steps, seq_out):
        seq_site.forward(c["tokens"], c["cu"], x, seq_start=c["ss"], slots=c["sl"], store=store_seq)
    torch.cuda.synchronize()
    kind = seq_site.projection_kind(0, T)
    ids_seq = store_seq.ids()
    del seq_site, store_seq
    _free()
    la_site = _engram(eng, cfg, T, True)
    store_la = la_site.make_store(cfg.n_seqs, ids=store0)
    la_out = [ei.make_streams(cfg, T, DEV, step=k) for k in range(len(steps))]
    c0 = dev_steps[0]
    la_site.gather_ahead(c0["tokens"], c0["cu"], seq_start=c0["ss"], slots=c0["sl"], store=store_la)
    for k in range(len(steps)):
        nxt = dev_steps[k + 1] if k + 1 < len(steps) else None
        if nxt is None:
            la_site.run_ahead(la_out[k])
        else:
            la_site.run_ahead(la_out[k], next_tokens=nxt["tokens"], next_cu_seqlens=nxt["cu"],
                              next_seq_start=nxt["ss"], next_slots=nxt["sl"], next_store=store_la)
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    for x, y in zip(seq_out, la_out):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.equal(ids_seq, store_la.ids())
    assert kind == "splitk"
    log(f"look-ahead order, {len(steps)} decode steps with the store ({kind} projection): bit-identical")
    del la_site
    _free()
