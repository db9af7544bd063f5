"""Production decode on the device: speculative rollback of the slot store and a
decode step captured in a HIP graph.

Rollback bar: after a verify call over draft tokens and engram_store_rollback to
keep_len tokens per sequence, the store equals what the oracle's store holds
after running only the kept tokens, and the next step's row ids equal the
oracle's (integers, exact).

Graph bar: every replay of a captured decode step (compress_hash with the store,
gather, projection, gate) equals an eager run of the same step bit for bit, with
eager work and synchronisations between replays.
"""
import gc

import numpy as np
import pytest
import torch

import engram_inputs as ei
from engram_harness import DEV, Site, bf16_bits_np, log

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


def _truncate(batch: ei.Batch, keep: np.ndarray) -> ei.Batch:
    """The first keep[s] tokens of every sequence of the batch."""
    cu = batch.cu_seqlens
    parts = [np.arange(cu[s], cu[s] + keep[s]) for s in range(len(keep))]
    idx = np.concatenate(parts).astype(np.int64) if parts else np.zeros(0, np.int64)
    ncu = np.zeros(len(keep) + 1, np.int32)
    ncu[1:] = np.cumsum(keep)
    return ei.Batch(tokens=batch.tokens[idx], cu_seqlens=ncu, seq_start=batch.seq_start,
                    slots=batch.slots, dead=None if batch.dead is None else batch.dead[idx])


def test_speculative_rollback_matches_truncated_oracle(eng):
    cfg = ei.get_config("tiny")
    site = Site(cfg, max_tokens=512)
    L = site.site.layout
    rng = np.random.default_rng(31)
    S, num_slots, draft = 24, 40, 5
    slots = rng.permutation(num_slots)[:S].astype(np.int32)
    store0 = rng.integers(0, cfg.vc, size=(num_slots, 3)).astype(np.int32)
    # prompt: ragged lengths, some sequences start here, some continue the store
    plen = rng.integers(0, 12, size=S).astype(np.int32)
    pcu = np.zeros(S + 1, np.int32)
    pcu[1:] = np.cumsum(plen)
    prompt = ei.Batch(tokens=ei.zipf_tokens(rng, int(pcu[-1])), cu_seqlens=pcu,
                      seq_start=(rng.random(S) < 0.5).astype(np.uint8), slots=slots,
                      dead=ei.make_dead_spans(int(pcu[-1]), 3, n_spans=4, max_len=3))
    # verify call: draft + 1 tokens per sequence, continuing; dead positions too
    vcu = (np.arange(S + 1) * (draft + 1)).astype(np.int32)
    Tv = int(vcu[-1])
    vdead = ei.make_dead_spans(Tv, 4, n_spans=6, max_len=2)
    verify = ei.Batch(tokens=ei.zipf_tokens(rng, Tv), cu_seqlens=vcu, seq_start=np.zeros(S, np.uint8),
                      slots=slots, dead=vdead)
    keep = rng.integers(0, draft + 2, size=S).astype(np.int32)
    keep[:6] = [0, 1, 2, 3, draft, draft + 1]
    # one more step after the rollback
    nxt = ei.Batch(tokens=ei.zipf_tokens(rng, S), cu_seqlens=np.arange(S + 1, dtype=np.int32),
                   seq_start=np.zeros(S, np.uint8), slots=slots, dead=None)

    store = site.site.make_store(num_slots, ids=_d(store0))
    e = torch.empty(512, dtype=torch.int32, device=DEV)
    r = torch.empty((512, 3, cfg.heads), dtype=torch.int32, device=DEV)

    def run(b):
        db = site.device_batch(b)
        eng.engram_compress_hash(L, site.tid2eid, db["tokens"], db["cu_seqlens"], e, r,
                                 seq_start=db["seq_start"], slots=db["slots"], store=store,
                                 dead=db["dead"])
        return db

    run(prompt)
    slots_d = _d(slots)
    snap = torch.empty((S, 3), dtype=torch.int32, device=DEV)
    eng.engram_store_read(store, slots_d, snap)
    dbv = run(verify)
    eng.engram_store_rollback(L, site.tid2eid, store, slots_d, dbv["cu_seqlens"], e[:Tv], _d(keep),
                              snapshot=snap, seq_start=dbv["seq_start"], dead=dbv["dead"])
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    got_store = store.ids().cpu().numpy()

    ref = store0.copy()
    site.oracle_hash(prompt, ref)
    site.oracle_hash(_truncate(verify, keep), ref)
    assert np.array_equal(got_store, ref), "rolled-back store differs from the oracle's"
    run(nxt)
    torch.cuda.synchronize()
    _, r_ref = site.oracle_hash(nxt, ref)
    assert np.array_equal(r[:S].cpu().numpy(), r_ref)
    assert np.array_equal(store.ids().cpu().numpy(), ref)
    log(f"rollback: {S} sequences, keep {keep.tolist()}")

    # keep_len beyond the call's length: latched, that slot untouched
    before = store.ids()
    bad = _d(np.full(S, draft + 2, np.int32))
    eng.engram_store_rollback(L, site.tid2eid, store, slots_d, dbv["cu_seqlens"], e[:Tv], bad,
                              snapshot=snap, seq_start=dbv["seq_start"], dead=dbv["dead"])
    assert eng.engram_get_error() == eng.ENGRAM_E_SEQLENS
    assert torch.equal(store.ids(), before)
    _free()


def test_store_handle_checks_ids_and_layout(eng):
    """The store is bound to its layout: writes of ids outside [0, V_c) are refused
    on the device (row untouched, ENGRAM_E_ID_RANGE latched), slots outside the
    store latch ENGRAM_E_SLOT_RANGE, reset returns slots to the pad id, and a
    layout with another compressed vocabulary cannot use it (ENGRAM_E_ARG)."""
    cfg = ei.get_config("tiny")
    site = Site(cfg, max_tokens=64)
    pad = site.pad_eid
    st = site.site.make_store(8)
    assert np.array_equal(st.ids().cpu().numpy(), np.full((8, 3), pad, np.int32))
    rng = np.random.default_rng(5)
    ids = rng.integers(0, cfg.vc, size=(8, 3)).astype(np.int32)
    st.load(_d(ids))
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    assert np.array_equal(st.ids().cpu().numpy(), ids)
    bad = np.array([[1, 2, 3], [4, cfg.vc, 5], [-1, 0, 0]], np.int32)
    eng.engram_store_write(st, _d(np.array([0, 1, 2], np.int32)), _d(bad))
    assert eng.engram_get_error() == eng.ENGRAM_E_ID_RANGE
    want = ids.copy()
    want[0] = [1, 2, 3]
    assert np.array_equal(st.ids().cpu().numpy(), want)
    eng.engram_store_write(st, _d(np.array([8], np.int32)), _d(np.zeros((1, 3), np.int32)))
    assert eng.engram_get_error() == eng.ENGRAM_E_SLOT_RANGE
    eng.engram_store_reset(st, _d(np.array([3, 5], np.int32)))
    want[[3, 5]] = pad
    assert np.array_equal(st.ids().cpu().numpy(), want)
    assert eng.engram_get_error() == 0
    # another layout (other compressed vocabulary): its calls refuse this store
    other = eng.engram_layout_create(vocab_size=cfg.vocab, compressed_vocab=cfg.vc // 2,
                                     pad_token_id=cfg.pad_token_id, heads_per_order=cfg.heads,
                                     rows=[cfg.rows] * 3, row_dim=cfg.row_dim,
                                     table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                     row_pitch_bytes=cfg.row_pitch_bytes)
    e = torch.empty(4, dtype=torch.int32, device=DEV)
    r = torch.empty((4, 3, cfg.heads), dtype=torch.int32, device=DEV)
    tok = _d(np.array([1, 2, 3, 4], np.int32))
    with pytest.raises(eng.EngramError) as ex:
        eng.engram_compress_hash(other, site.tid2eid, tok, _d(np.array([0, 4], np.int32)), e, r,
                                 slots=_d(np.array([0], np.int32)), store=st,
                                 seq_start=_d(np.zeros(1, np.uint8)))
    assert ex.value.status == eng.ENGRAM_E_ARG
    _free()


def test_decode_step_graph_replays_equal_eager(eng):
    cfg = ei.get_config("decode_tiny")
    S = cfg.n_seqs
    steps = ei.make_decode_steps(cfg, 9)
    site = Site(cfg, max_tokens=S)
    b0 = steps[0]
    tok = _d(b0.tokens)
    cu = _d(b0.cu_seqlens)
    ss = _d(b0.seq_start)
    sl = _d(b0.slots)
    init = _d(ei.make_store_init(cfg))
    store_g = site.site.make_store(S, ids=init)
    store_e = site.site.make_store(S, ids=init)
    streams_g = torch.zeros((S, cfg.hc_mult, cfg.hidden), dtype=torch.bfloat16, device=DEV)

    def step(streams, store):
        site.site.forward(tok, cu, streams, seq_start=ss, slots=sl, store=store)

    # warm up eagerly on a scratch store (kernel attributes are set on first use)
    scratch = site.site.make_store(S, ids=init)
    step(streams_g.clone(), scratch)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            step(streams_g, store_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capture does not run the work: the graph's state is still the initial one
    assert torch.equal(store_g.ids(), store_e.ids())
    for k, b in enumerate(steps[1:]):
        tok.copy_(_d(b.tokens))
        x = ei.make_streams(cfg, S, DEV, step=k)
        streams_g.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        rows_g, v_g, y_g, st_g = (site.site.row_ids.clone(), site.site.v.clone(), streams_g.clone(),
                                  store_g.ids())
        streams_e = x.clone()
        step(streams_e, store_e)
        torch.cuda.synchronize()
        assert eng.engram_get_error() == 0
        assert torch.equal(rows_g, site.site.row_ids), k
        assert torch.equal(st_g, store_e.ids()), k
        assert torch.equal(v_g.view(torch.int32), site.site.v.view(torch.int32)), k
        assert np.array_equal(bf16_bits_np(y_g), bf16_bits_np(streams_e)), k
    log(f"graph: {len(steps) - 1} replays equal eager")
    del g
    _free()


@pytest.mark.parametrize("M,N,H,D,splits", [(256, 4096, 2, 512, 8), (256, 4096, 2, 512, 4),
                                            (77, 264, 1, 128, 2), (512, 256, 2, 128, 2),
                                            (1, 8, 1, 256, 4)])
def test_projection_splitk_and_partial_gate(eng, M, N, H, D, splits):
    """Split-K projection against torch's fp32 product of the same bf16 operands
    (fp32 accumulation bound), and the gate over the partial slices against the
    plain gate given the summed v (bit for bit)."""
    L = eng.engram_layout_create(vocab_size=8, compressed_vocab=4, pad_token_id=7, heads_per_order=H,
                                 rows=[100_000] * 3, row_dim=D, table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                 row_pitch_bytes=D)
    K = L.info.k_pad
    g = torch.Generator(device=DEV)
    g.manual_seed(M * 31 + N + splits)
    A = torch.randn((M, K), generator=g, device=DEV).to(torch.bfloat16)
    B = (torch.randn((N, K), generator=g, device=DEV) * 0.05).to(torch.bfloat16)
    parts = torch.full((splits * M * N,), float("nan"), dtype=torch.float32, device=DEV)
    eng.engram_project_splitk(L, A, B, parts, splits)
    x = torch.randn((M, 4, N), generator=g, device=DEV).to(torch.bfloat16)
    y = x.clone()
    v = torch.empty((M, N), dtype=torch.float32, device=DEV)
    keep = (torch.rand(M, generator=g, device=DEV) > 0.2).to(torch.uint8)
    eng.engram_gate_add_partials(L, parts, splits, y, keep=keep, v=v)
    ref = A.float() @ B.float().T
    torch.cuda.synchronize()
    bound = 2 * K * 2.0 ** -24 * (A.float().abs() @ B.float().abs().T) + 1e-6
    assert ((v - ref).abs() <= bound).all()
    # the slices sum to v in slice order
    p = parts.view(splits, M, N)
    acc = p[0].clone()
    for s in range(1, splits):
        acc += p[s]
    assert torch.equal(acc.view(torch.int32), v.view(torch.int32))
    y2 = x.clone()
    eng.engram_gate_add(L, v, y2, keep=keep)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    dead = keep == 0
    assert torch.equal(y[dead].view(torch.int16), x[dead].view(torch.int16))
