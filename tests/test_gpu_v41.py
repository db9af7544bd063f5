"""GPU parity of the released V4.1 layout: two Engram sites sharing one hash
pass, 3 orders x 8 heads, row dim 256, one table per site, (1, 32) e8m0 block
scales.

Bars (as for the single-site path): compressed ids and every site's row ids
bit-exact on every token; dequantised rows bit-exact in fp32 and bf16; the
projection within the fp32-accumulation bound; streams within 2e-2 relative
error.  v41_small is checked on every token's rows; v41 (the released sizes,
2 x 98 GB of e4m3fn) on every integer and on seeded token samples.
"""
import gc

import numpy as np
import pytest
import torch

import engram_inputs as ei
import oracle
from engram_harness import (DEV, assert_streams_close, assert_v_close, bf16_bits_np, log, oracle_dequant,
                            oracle_gate_add, oracle_project, sample_tokens)

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


def test_e8m0_every_code_and_exponent(eng):
    """Every finite e4m3fn code against a spread of e8m0 exponents (including the
    subnormal 2^-127 and the largest finite ones), fp32 and bf16 outputs."""
    D = 256
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    exps = np.array([0, 1, 2, 60, 100, 119, 120, 121, 127, 128, 150, 200, 240, 253, 254], np.uint8)
    rows = len(exps) * 2
    tab = np.zeros((rows, D), np.uint8)
    sc = np.zeros((rows, D // 32), np.uint8)
    for i, e in enumerate(exps):
        tab[2 * i] = codes[np.arange(D) % len(codes)]
        tab[2 * i + 1] = codes[(np.arange(D) + D) % len(codes)]
        sc[2 * i] = e
        sc[2 * i + 1] = np.roll(exps, i)[: D // 32]
    L = eng.engram_layout_create(vocab_size=8, compressed_vocab=4, pad_token_id=7, heads_per_order=1,
                                 rows=[rows, 0, 0], row_dim=D, table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                 row_pitch_bytes=D, hash_floor=2, num_sites=1,
                                 table_split=eng.ENGRAM_TABLE_PER_SITE,
                                 scale_layout=eng.ENGRAM_SCALE_BLOCK32_E8M0)
    t_d, s_d = _d(tab.reshape(-1)), _d(sc.reshape(-1))
    # token i reads row i in all three columns
    rid = torch.arange(rows, dtype=torch.int32, device=DEV)[:, None].repeat(1, 3).contiguous()
    out32 = torch.empty((rows, L.info.k_pad), dtype=torch.float32, device=DEV)
    out16 = torch.empty((rows, L.info.k_pad), dtype=torch.bfloat16, device=DEV)
    eng.engram_gather_dequant(L, [t_d], [s_d], rid, out32)
    eng.engram_gather_dequant(L, [t_d], [s_d], rid, out16)
    torch.cuda.synchronize()
    assert eng.engram_get_error() == 0
    f_ref, b_ref = oracle.dequant_rows_block32(tab, sc)
    g32 = out32.view(rows, 3, L.info.seg_pitch).cpu().numpy()[:, :, :D]
    g16 = bf16_bits_np(out16).reshape(rows, 3, L.info.seg_pitch)[:, :, :D]
    for c in range(3):
        assert np.array_equal(g32[:, c].view(np.uint32), f_ref.view(np.uint32))
        assert np.array_equal(g16[:, c], b_ref)


class Sites:
    """The two sites of a released-layout workload on the device, plus the
    oracle's per-site layouts."""

    def __init__(self, eng, cfg, max_tokens):
        self.cfg = cfg
        self.tid2eid_h = ei.make_tid2eid(cfg.vocab, cfg.vc)
        self.tid2eid = _d(self.tid2eid_h)
        self.tables = [ei.make_tables(cfg, DEV, site=s) for s in range(cfg.n_sites)]
        self.weights = [ei.make_weight(cfg, DEV, site=s) for s in range(cfg.n_sites)]
        self.eng = eng.Engram(
            vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
            heads_per_order=cfg.heads, rows=[cfg.rows], row_dim=cfg.row_dim,
            table_dtype=cfg.table_dtype, row_pitch_bytes=cfg.row_pitch_bytes, tid2eid=self.tid2eid,
            tables=[t.data for t in self.tables], scales=[t.scale for t in self.tables],
            weight=self.weights, hidden=cfg.hidden, hc_mult=cfg.hc_mult, max_tokens=max_tokens,
            hash_floor=cfg.hash_floor, num_sites=cfg.n_sites, table_split=cfg.table_split,
            scale_block=cfg.scale_block)
        self.olayouts = oracle.site_layouts(cfg.n_sites, cfg.heads, cfg.hash_floor,
                                            cfg.table_split == "site")
        torch.cuda.synchronize()

    def oracle_hash(self, batch, store=None):
        cfg = self.cfg
        e_ref, rows = None, []
        for s, ol in enumerate(self.olayouts):
            st = store if s == 0 else (None if store is None else store.copy())
            e, r = oracle.compress_hash(ol, vocab=cfg.vocab, vc=cfg.vc, pad_token_id=cfg.pad_token_id,
                                        tid2eid=self.tid2eid_h, tokens=batch.tokens,
                                        cu_seqlens=batch.cu_seqlens, seq_start=batch.seq_start,
                                        slots=batch.slots, store=st, dead=batch.dead)
            if e_ref is None:
                e_ref = e
            assert np.array_equal(e, e_ref)
            rows.append(r)
        return e_ref, np.stack(rows, axis=1)  # [T][site][3][H]

    def oracle_rows(self, site, row_ids):
        """bf16 / f32 dequantised rows [n][3H][D] of one site from the device
        tables (torch indexing), through the oracle."""
        cfg = self.cfg
        tab, sc = self.tables[site].data[0], self.tables[site].scale[0]
        n = row_ids.shape[0]
        idx = torch.from_numpy(row_ids.reshape(-1).astype(np.int64)).to(DEV)
        raw = tab.index_select(0, idx)[:, :cfg.row_dim].cpu().numpy()
        s8 = sc.index_select(0, idx).cpu().numpy()
        f32, b16 = oracle_dequant(raw, s8, block32=True)
        return f32.reshape(n, -1, cfg.row_dim), b16.reshape(n, -1, cfg.row_dim)


def _run(eng, name, f32_sample, stream_sample):
    cfg = ei.get_config(name)
    batch = ei.make_batch(cfg)
    T = batch.T
    st = Sites(eng, cfg, T)
    info = st.eng.info
    log(f"{name}: {cfg.n_sites} sites, site rows {[info.site_rows(s) for s in range(cfg.n_sites)]}, "
        f"T={T}, k_pad={info.k_pad}")
    assert [info.site_rows(s) for s in range(cfg.n_sites)] == [
        int(ol.offsets[2, -1] + ol.primes[2, -1]) for ol in st.olayouts]
    tok, cu = _d(batch.tokens), _d(batch.cu_seqlens)
    streams = [ei.make_streams(cfg, T, DEV, step=s) for s in range(cfg.n_sites)]
    idx = sample_tokens(batch, stream_sample, seed=cfg.seed)
    idx_d = torch.from_numpy(idx).to(DEV)
    x0 = [bf16_bits_np(x[idx_d]) for x in streams]
    # hash once, then per site: gather (kept for the row check), project, gate
    st.eng.hash(tok, cu)
    e_ref, r_ref = st.oracle_hash(batch)
    torch.cuda.synchronize()
    assert np.array_equal(st.eng.eids[:T].cpu().numpy(), e_ref)
    assert np.array_equal(st.eng.row_ids[:T].cpu().numpy(), r_ref)
    log(f"{name}: eids and both sites' row ids exact on all {T} tokens")
    fidx = np.arange(T) if f32_sample is None else sample_tokens(batch, f32_sample, seed=cfg.seed + 1)
    fidx_d = torch.from_numpy(fidx).to(DEV)
    D = cfg.row_dim
    for s in range(cfg.n_sites):
        st.eng.site_forward(s, streams[s], T)
        torch.cuda.synchronize()
        assert eng.engram_get_error() == 0
        rows16 = st.eng.rows[:T].view(T, 3 * cfg.heads, info.seg_pitch)
        out32 = torch.empty((len(fidx), info.k_pad), dtype=torch.float32, device=DEV)
        rid_s = st.eng.row_ids[fidx_d].contiguous()
        eng.engram_gather_dequant(st.eng.layout, st.eng.site_tables[s], st.eng.site_scales[s], rid_s,
                                  out32, site=s)
        f_ref, b_ref = st.oracle_rows(s, r_ref[fidx, s])
        g32 = out32.view(len(fidx), -1, info.seg_pitch).cpu().numpy()[:, :, :D]
        assert np.array_equal(g32.view(np.uint32), f_ref.view(np.uint32))
        g16 = bf16_bits_np(rows16[fidx_d])
        assert np.array_equal(g16[:, :, :D], b_ref)
        assert not g16[:, :, D:].any()
        log(f"{name} site {s}: fp32 / bf16 rows exact on {len(fidx)} tokens")
        _, b16s = st.oracle_rows(s, r_ref[idx, s])
        E = np.zeros((len(idx), 3 * cfg.heads, D), np.uint16)
        E[:] = b16s
        E = E.reshape(len(idx), -1)
        W = bf16_bits_np(st.weights[s])
        v_ref = oracle_project(E, W)
        assert_v_close(st.eng.v[idx_d].cpu().numpy(), v_ref, E, W, f"{name} site {s} v")
        y_ref, _ = oracle_gate_add(x0[s], v_ref)
        worst = assert_streams_close(bf16_bits_np(streams[s][idx_d]), y_ref, f"{name} site {s} streams")
        log(f"{name} site {s}: streams within tolerance on {len(idx)} tokens (worst {worst:.2e})")
    del st, streams
    _free()


def test_v41_small_two_sites(eng):
    _run(eng, "v41_small", f32_sample=None, stream_sample=None)


@pytest.mark.timeout(900)
def test_v41_released_sizes(eng):
    _run(eng, "v41", f32_sample=1024, stream_sample=1024)


def test_two_sites_per_order_tables_against_oracle(eng):
    """Two sites sharing one hash pass with three tables per order each: every
    site's row ids exact against the oracle's per-site layouts, and each site's
    gather reads its own tables (fp32 rows exact)."""
    cfg = ei.get_config("tiny")
    batch = ei.make_batch(cfg)
    T = batch.T
    floor_ = 1000
    L = eng.engram_layout_create(vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
                                 heads_per_order=cfg.heads, rows=[cfg.rows] * 3, row_dim=cfg.row_dim,
                                 table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                 row_pitch_bytes=cfg.row_pitch_bytes, hash_floor=floor_, num_sites=2)
    tid_h = ei.make_tid2eid(cfg.vocab, cfg.vc)
    tid = _d(tid_h)
    eids = torch.empty(T, dtype=torch.int32, device=DEV)
    rid = torch.empty((T, 2, 3, cfg.heads), dtype=torch.int32, device=DEV)
    eng.engram_compress_hash(L, tid, _d(batch.tokens), _d(batch.cu_seqlens), eids, rid)
    ols = oracle.site_layouts(2, cfg.heads, floor_, False)
    refs = []
    for ol in ols:
        _, r = oracle.compress_hash(ol, vocab=cfg.vocab, vc=cfg.vc, pad_token_id=cfg.pad_token_id,
                                    tid2eid=tid_h, tokens=batch.tokens, cu_seqlens=batch.cu_seqlens)
        refs.append(r)
    torch.cuda.synchronize()
    assert np.array_equal(rid.cpu().numpy(), np.stack(refs, axis=1))
    tabs = [ei.make_tables(cfg, DEV, site=s) for s in range(2)]
    out = torch.empty((T, L.info.k_pad), dtype=torch.float32, device=DEV)
    D = cfg.row_dim
    for s in range(2):
        eng.engram_gather_dequant(L, tabs[s].data, tabs[s].scale, rid, out, site=s)
        torch.cuda.synchronize()
        raw = np.zeros((T, 3 * cfg.heads, D), np.uint8)
        sc = np.zeros((T, 3 * cfg.heads), np.float32)
        for n in range(3):
            for h in range(cfg.heads):
                idx = torch.from_numpy(refs[s][:, n, h].astype(np.int64)).to(DEV)
                raw[:, n * cfg.heads + h] = tabs[s].row_view(n).index_select(0, idx).cpu().numpy()
                sc[:, n * cfg.heads + h] = tabs[s].scale[n].index_select(0, idx).cpu().numpy()
        f_ref, _ = oracle.dequant_rows(raw.reshape(-1, D), sc.reshape(-1))
        got = out.view(T, -1, L.info.seg_pitch).cpu().numpy()[:, :, :D]
        assert np.array_equal(got.reshape(-1, D).view(np.uint32), f_ref.view(np.uint32)), f"site {s}"
    assert eng.engram_get_error() == 0
    _free()
