"""Host-side checks of the C ABI that need no GPU: the library loads and exports
every symbol include/engram.h declares; the host layout (bucket primes, floor
fit, row-count guard, segment geometry) matches the oracle; argument errors."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import engram_inputs as ei
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

eng = pytest.importorskip("hashed_gram_memory_tid2eid_amd")


def declared_functions():
    with open(os.path.join(ROOT, "include", "engram.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(engram_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 14, names
    lib = ctypes.CDLL(eng.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", eng.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(engram_\w+)", out))
    assert set(names) <= exported


def test_status_codes_have_messages():
    for name, code in eng.STATUS.items():
        msg = eng.engram_strerror(code)
        assert msg and msg != "unknown status", name
    assert eng.engram_strerror(12345) == "unknown status"


def _layout(cfg, **kw):
    args = dict(vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
                heads_per_order=cfg.heads, rows=[cfg.rows] * 3, row_dim=cfg.row_dim,
                table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN if cfg.table_dtype == "fp8" else eng.ENGRAM_DTYPE_BF16,
                row_pitch_bytes=cfg.row_pitch_bytes)
    args.update(kw)
    return eng.engram_layout_create(**args)


@pytest.mark.parametrize("name", ["tiny", "prefill", "decode", "long", "full", "full_bf16"])
def test_layout_matches_oracle(name):
    cfg = ei.get_config(name)
    L = _layout(cfg)
    ref = oracle.fit_layout([cfg.rows] * 3, cfg.heads)
    info = L.info
    assert info.hash_floor == ref.floor
    assert np.array_equal(np.array(info.primes, dtype=np.uint64), ref.primes)
    assert np.array_equal(np.array(info.offsets, dtype=np.uint64), ref.offsets)
    assert list(info.prime_sum) == [int(s) for s in ref.primes.sum(axis=1)]
    assert info.seg_pitch % 64 == 0 and cfg.row_dim <= info.seg_pitch < cfg.row_dim + 64
    assert info.k_pad == 3 * cfg.heads * info.seg_pitch


def test_layout_given_floor_pages_case(golden):
    cfg = ei.get_config("tiny")
    L = _layout(cfg, rows=[1024] * 3, hash_floor=64)
    assert sum(sum(p) for p in L.info.primes) == golden["prime_sum_floor64"]["value"]
    ref = oracle.layout_at_floor([1024] * 3, 2, 64)
    assert np.array_equal(np.array(L.info.primes, dtype=np.uint64), ref.primes)


def test_layout_real_model_floor_heads8():
    """Per-order tables at the released floor 16,000,000 with 8 heads: the prime
    sums of the three orders add up to the page's first-layer row count."""
    cfg = ei.get_config("tiny")
    L = _layout(cfg, heads_per_order=8, rows=[130_000_000] * 3, hash_floor=16_000_000)
    assert sum(L.info.prime_sum) == 384_006_168
    ref = oracle.layout_at_floor([130_000_000] * 3, 8, 16_000_000)
    assert np.array_equal(np.array(L.info.primes, dtype=np.uint64), ref.primes)


def test_layout_errors():
    cfg = ei.get_config("tiny")
    ref = oracle.layout_at_floor([1024] * 3, 2, 64)
    need = [int(s) for s in ref.primes.sum(axis=1)]
    with pytest.raises(eng.EngramError) as e:
        _layout(cfg, rows=[need[0], need[1] - 1, need[2]], hash_floor=64)
    assert e.value.status == eng.ENGRAM_E_LAYOUT_ROWS
    _layout(cfg, rows=need, hash_floor=64)
    with pytest.raises(eng.EngramError) as e:
        _layout(cfg, compressed_vocab=65537)
    assert e.value.status == eng.ENGRAM_E_VC_RANGE
    with pytest.raises(eng.EngramError) as e:
        _layout(cfg, row_pitch_bytes=120)
    assert e.value.status == eng.ENGRAM_E_ALIGN
    with pytest.raises(eng.EngramError) as e:
        _layout(cfg, row_pitch_bytes=136)  # not a multiple of 16
    assert e.value.status == eng.ENGRAM_E_ALIGN
    with pytest.raises(eng.EngramError) as e:
        _layout(cfg, heads_per_order=9)
    assert e.value.status == eng.ENGRAM_E_ARG
    with pytest.raises(eng.EngramError) as e:
        _layout(cfg, max_ngram=3)
    assert e.value.status == eng.ENGRAM_E_ARG
    with pytest.raises(eng.EngramError) as e:
        _layout(cfg, pad_token_id=cfg.vocab)
    assert e.value.status == eng.ENGRAM_E_ARG
    with pytest.raises(eng.EngramError) as e:
        _layout(cfg, rows=[1, 1, 1])
    assert e.value.status == eng.ENGRAM_E_NOFIT
    # bf16 tables need twice the pitch
    with pytest.raises(eng.EngramError) as e:
        _layout(cfg, table_dtype=eng.ENGRAM_DTYPE_BF16, row_pitch_bytes=128)
    assert e.value.status == eng.ENGRAM_E_ALIGN


def test_gather_host_argument_errors_need_no_device():
    """Errors the host sees are returned before any launch."""
    cfg = ei.get_config("tiny")
    L = _layout(cfg)
    lib = eng._lib
    P = ctypes.c_void_p
    three = (P * 3)(None, None, None)
    rc = lib.engram_gather_dequant(L.handle, three, three, None, 0, 4, 99, None, L.info.k_pad, None)
    assert rc == eng.ENGRAM_E_ARG
    # a site the layout does not have
    rc = lib.engram_gather_dequant(L.handle, three, three, None, 1, 4, eng.ENGRAM_DTYPE_BF16, None,
                                   L.info.k_pad, None)
    assert rc == eng.ENGRAM_E_ARG
    rc = lib.engram_project(L.handle, None, L.info.k_pad, None, L.info.k_pad, 0, None, 4, None)
    assert rc == eng.ENGRAM_E_ARG
    rc = lib.engram_gate_add(L.handle, None, 256, 3, None, None, 4, None)
    assert rc == eng.ENGRAM_E_UNSUPPORTED
    rc = lib.engram_gate_add(L.handle, None, 250, 4, None, None, 4, None)
    assert rc == eng.ENGRAM_E_ALIGN
    rc = lib.engram_compress_hash(L.handle, P(16), P(16), 5, P(16), 0, None, None, None, 0, None,
                                  P(16), P(16), None)
    assert rc == eng.ENGRAM_E_ARG
    # empty calls are no-ops
    assert lib.engram_compress_hash(L.handle, P(16), None, 0, None, 0, None, None, None, 0, None,
                                    None, None, None) == 0


def test_gather_project_host_errors_need_no_device():
    """The fused gather+projection refuses what it cannot read, before any launch."""
    cfg = ei.get_config("tiny")
    lib = eng._lib
    P = ctypes.c_void_p
    some = (P * 3)(P(256), P(256), P(256))
    # bf16 tables: the fused kernel dequantises e4m3fn only
    L16 = _layout(cfg, table_dtype=eng.ENGRAM_DTYPE_BF16, row_pitch_bytes=2 * cfg.row_dim)
    rc = lib.engram_gather_project(L16.handle, some, some, P(256), 0, 4, P(256), L16.info.k_pad,
                                   cfg.hidden, P(256), None)
    assert rc == eng.ENGRAM_E_UNSUPPORTED
    # a row pitch shorter than the 64-aligned segment would read past the row
    Lshort = _layout(cfg, row_dim=100, row_pitch_bytes=112)
    assert Lshort.info.seg_pitch == 128
    rc = lib.engram_gather_project(Lshort.handle, some, some, P(256), 0, 4, P(256), Lshort.info.k_pad,
                                   cfg.hidden, P(256), None)
    assert rc == eng.ENGRAM_E_ALIGN
    L = _layout(cfg)
    # weight leading dimension below k_pad
    rc = lib.engram_gather_project(L.handle, some, some, P(256), 0, 4, P(256), L.info.k_pad - 8,
                                   cfg.hidden, P(256), None)
    assert rc == eng.ENGRAM_E_ALIGN
    # missing scales
    rc = lib.engram_gather_project(L.handle, some, None, P(256), 0, 4, P(256), L.info.k_pad,
                                   cfg.hidden, P(256), None)
    assert rc == eng.ENGRAM_E_ARG
    # e8m0 block scales: rows of at most 256 elements (a thread keeps a row's 8 exponent
    # bytes in registers), and for 256-element rows 8-byte aligned scale arrays
    Lwide = _layout(cfg, row_dim=320, row_pitch_bytes=384, scale_layout=eng.ENGRAM_SCALE_BLOCK32_E8M0)
    rc = lib.engram_gather_project(Lwide.handle, some, some, P(256), 0, 4, P(256), Lwide.info.k_pad,
                                   cfg.hidden, P(256), None)
    assert rc == eng.ENGRAM_E_UNSUPPORTED
    L256 = _layout(cfg, row_dim=256, row_pitch_bytes=256, scale_layout=eng.ENGRAM_SCALE_BLOCK32_E8M0)
    odd = (P * 3)(P(260), P(260), P(260))
    rc = lib.engram_gather_project(L256.handle, some, odd, P(256), 0, 4, P(256), L256.info.k_pad,
                                   cfg.hidden, P(256), None)
    assert rc == eng.ENGRAM_E_ALIGN
    # empty call is a no-op
    assert lib.engram_gather_project(L.handle, some, some, None, 0, 0, None, L.info.k_pad,
                                     cfg.hidden, None, None) == 0


def test_store_rollback_host_errors_need_no_device():
    cfg = ei.get_config("tiny")
    L = _layout(cfg)
    lib = eng._lib
    P = ctypes.c_void_p
    # empty call is a no-op
    assert lib.engram_store_rollback(L.handle, None, None, None, 0, None, 0, None, None, None,
                                     None, None, None) == 0
    # missing store / slots / keep_len
    rc = lib.engram_store_rollback(L.handle, P(256), None, P(256), 2, P(256), 4, P(256), None, None,
                                   None, P(256), None)
    assert rc == eng.ENGRAM_E_ARG
    rc = lib.engram_store_rollback(L.handle, P(256), P(256), None, 2, P(256), 4, P(256), None, None,
                                   None, P(256), None)
    assert rc == eng.ENGRAM_E_ARG
    rc = lib.engram_store_rollback(L.handle, P(256), P(256), P(256), 2, P(256), 4, P(256), None, None,
                                   None, None, None)
    assert rc == eng.ENGRAM_E_ARG


def test_store_and_wkv_handles_host_errors_need_no_device():
    """The store and weight handles refuse bad arguments before touching a device:
    a store needs a layout, at least one slot and a pad id inside [0, V_c); a weight
    handle needs a weight with a leading dimension of at least k_pad (a multiple of
    8), 16-byte alignment, a positive size, and a forced split count that divides
    k_pad into steps of 64.  Calls with no handle are refused too."""
    cfg = ei.get_config("tiny")
    L = _layout(cfg)
    lib = eng._lib
    P = ctypes.c_void_p
    K = L.info.k_pad
    out = P()
    assert lib.engram_store_create(None, 0, 4, None, ctypes.byref(out)) == eng.ENGRAM_E_ARG
    assert lib.engram_store_create(L.handle, 0, 0, None, ctypes.byref(out)) == eng.ENGRAM_E_ARG
    assert lib.engram_store_create(L.handle, -1, 4, None, ctypes.byref(out)) == eng.ENGRAM_E_ARG
    assert lib.engram_store_create(L.handle, cfg.vc, 4, None, ctypes.byref(out)) == eng.ENGRAM_E_ARG
    assert lib.engram_store_create(L.handle, 0, 4, None, None) == eng.ENGRAM_E_ARG
    for fn in (lib.engram_store_reset,):
        assert fn(None, None, 0, None) == eng.ENGRAM_E_ARG
    assert lib.engram_store_write(None, None, 0, P(256), None) == eng.ENGRAM_E_ARG
    assert lib.engram_store_read(None, None, 0, P(256), None) == eng.ENGRAM_E_ARG
    n, pad = ctypes.c_int32(), ctypes.c_int32()
    assert lib.engram_store_query(None, ctypes.byref(n), ctypes.byref(pad)) == eng.ENGRAM_E_ARG
    ok = P(256)
    wc = lib.engram_wkv_create
    assert wc(L.handle, None, K, cfg.hidden, 64, 0, None, ctypes.byref(out)) == eng.ENGRAM_E_ARG
    assert wc(L.handle, ok, K, 0, 64, 0, None, ctypes.byref(out)) == eng.ENGRAM_E_ARG
    assert wc(L.handle, ok, K, cfg.hidden, 0, 0, None, ctypes.byref(out)) == eng.ENGRAM_E_ARG
    assert wc(L.handle, ok, K, cfg.hidden, 64, -1, None, ctypes.byref(out)) == eng.ENGRAM_E_ARG
    assert wc(L.handle, ok, K - 8, cfg.hidden, 64, 0, None, ctypes.byref(out)) == eng.ENGRAM_E_ALIGN
    assert wc(L.handle, P(264), K, cfg.hidden, 64, 0, None, ctypes.byref(out)) == eng.ENGRAM_E_ALIGN
    # k_pad 768 = 64 x 12: 4 splits divide it, 5 do not
    assert wc(L.handle, ok, K, cfg.hidden, 64, 5, None, ctypes.byref(out)) == eng.ENGRAM_E_ALIGN
    plan = eng.engram_proj_plan()
    assert lib.engram_wkv_plan(None, 4, ctypes.byref(plan)) == eng.ENGRAM_E_ARG
    assert lib.engram_wkv_project(L.handle, ok, K, None, ok, 4, None) == eng.ENGRAM_E_ARG
    assert lib.engram_wkv_gate_add(L.handle, None, ok, 4, None, ok, 4, None) == eng.ENGRAM_E_ARG
    assert lib.engram_gated_residual(L.handle, ok, K, None, 4, None, ok, ok, 4, None) == eng.ENGRAM_E_ARG
    assert lib.engram_gated_residual_noalloc(L.handle, ok, K, None, 4, None, ok, 4, None) == eng.ENGRAM_E_ARG


def test_lookup_decode_host_errors_need_no_device():
    """engram_lookup_decode checks the layout it supports (one site, e4m3fn tables
    with fp32 row scales), its pointers, the store and the rows' leading dimension on
    the host, and returns before any launch."""
    cfg = ei.get_config("tiny")
    L = _layout(cfg)
    lib = eng._lib
    P = ctypes.c_void_p
    K = L.info.k_pad
    ok = P(256)
    three = (P * 3)(ok, ok, ok)
    f = lib.engram_lookup_decode

    def call(layout, T=4, tid=ok, tok=ok, slots=None, store=None, rows=ok, ld=K, tables=three,
             scales=three):
        return f(layout, tid, tok, T, slots, store, None, ok, ok, tables, scales, rows, ld, None)
    assert call(L.handle, T=0) == 0
    assert call(L.handle, T=-1) == eng.ENGRAM_E_ARG
    assert call(L.handle, tid=None) == eng.ENGRAM_E_ARG
    assert call(L.handle, tok=None) == eng.ENGRAM_E_ARG
    assert call(L.handle, rows=None) == eng.ENGRAM_E_ARG
    assert call(L.handle, scales=None) == eng.ENGRAM_E_ARG
    assert call(L.handle, ld=K - 8) == eng.ENGRAM_E_ALIGN
    assert call(L.handle, ld=K + 4) == eng.ENGRAM_E_ALIGN
    assert call(L.handle, rows=P(264)) == eng.ENGRAM_E_ALIGN
    assert call(L.handle, tables=(P * 3)(P(8), ok, ok)) == eng.ENGRAM_E_ALIGN
    assert call(L.handle, slots=ok) == eng.ENGRAM_E_NEED_STORE
    assert call(None) == eng.ENGRAM_E_ARG
    # layouts it does not take: bf16 tables, (1, 32) block scales, two sites
    bf = _layout(cfg, table_dtype=eng.ENGRAM_DTYPE_BF16, row_pitch_bytes=2 * cfg.row_pitch_bytes)
    assert call(bf.handle) == eng.ENGRAM_E_UNSUPPORTED
    blk = _layout(cfg, scale_layout=eng.ENGRAM_SCALE_BLOCK32_E8M0)
    assert call(blk.handle) == eng.ENGRAM_E_UNSUPPORTED
    two = _layout(cfg, num_sites=2, rows=[cfg.rows * 2] * 3)
    assert call(two.handle) == eng.ENGRAM_E_UNSUPPORTED


def test_projection_and_gate_host_errors_need_no_device():
    """The projection, split-K and gate calls check sizes, leading dimensions and
    alignment on the host and return before any launch."""
    cfg = ei.get_config("tiny")
    L = _layout(cfg)
    lib = eng._lib
    P = ctypes.c_void_p
    K = L.info.k_pad
    ok = P(256)
    # leading dimensions below k_pad or not a multiple of 8 elements
    assert lib.engram_project(L.handle, ok, K - 8, ok, K, cfg.hidden, ok, 4, None) == eng.ENGRAM_E_ALIGN
    assert lib.engram_project(L.handle, ok, K, ok, K + 4, cfg.hidden, ok, 4, None) == eng.ENGRAM_E_ALIGN
    # operands not 16-byte aligned
    assert lib.engram_project(L.handle, P(264), K, ok, K, cfg.hidden, ok, 4, None) == eng.ENGRAM_E_ALIGN
    # negative token count, no hidden
    assert lib.engram_project(L.handle, ok, K, ok, K, cfg.hidden, ok, -1, None) == eng.ENGRAM_E_ARG
    assert lib.engram_project(L.handle, ok, K, ok, K, 0, ok, 4, None) == eng.ENGRAM_E_ARG
    # split-K: at least one split, and k_pad a multiple of 64 x splits (768 = 64 x 12)
    assert lib.engram_project_splitk(L.handle, ok, K, ok, K, cfg.hidden, ok, 0, 4, None) == eng.ENGRAM_E_ARG
    assert lib.engram_project_splitk(L.handle, ok, K, ok, K, cfg.hidden, ok, 5, 4, None) == eng.ENGRAM_E_ALIGN
    assert lib.engram_project_splitk(L.handle, ok, K, ok, K, cfg.hidden, ok, 4, 0, None) == 0
    # the gate: hc_mult 4 only, hidden a multiple of 8 up to 8,192, 16-byte aligned rows
    assert lib.engram_gate_add_partials(L.handle, ok, 2, cfg.hidden, 2, None, ok, None, 4,
                                        None) == eng.ENGRAM_E_UNSUPPORTED
    assert lib.engram_gate_add_partials(L.handle, ok, 2, 8200, 4, None, ok, None, 4,
                                        None) == eng.ENGRAM_E_UNSUPPORTED
    assert lib.engram_gate_add_partials(L.handle, ok, 0, cfg.hidden, 4, None, ok, None, 4,
                                        None) == eng.ENGRAM_E_ARG
    assert lib.engram_gate_add_partials(L.handle, ok, 2, cfg.hidden, 4, None, ok, P(260), 4,
                                        None) == eng.ENGRAM_E_ALIGN
    assert lib.engram_gate_add(L.handle, P(260), cfg.hidden, 4, None, ok, 4, None) == eng.ENGRAM_E_ALIGN
    assert lib.engram_gate_add(L.handle, None, cfg.hidden, 4, None, ok, 4, None) == eng.ENGRAM_E_ARG


def test_packed_projection_host_errors_need_no_device():
    """The packed-weight size, the pack and the packed projection check their
    arguments on the host and return before any launch."""
    cfg = ei.get_config("tiny")
    L = _layout(cfg)
    lib = eng._lib
    P = ctypes.c_void_p
    K = L.info.k_pad
    ok = P(256)
    # size: ceil(hidden / 32) * 32 rows of k_pad bf16
    assert eng.engram_packed_weight_bytes(L, 256) == 256 * K * 2
    assert eng.engram_packed_weight_bytes(L, 264) == 288 * K * 2
    assert eng.engram_packed_weight_bytes(L, 1) == 32 * K * 2
    n = ctypes.c_int64(0)
    assert lib.engram_packed_weight_bytes(L.handle, 0, ctypes.byref(n)) == eng.ENGRAM_E_ARG
    assert lib.engram_packed_weight_bytes(L.handle, 8, None) == eng.ENGRAM_E_ARG
    # pack: leading dimension >= k_pad and a multiple of 8, 16-byte aligned pointers
    assert lib.engram_pack_weight(L.handle, ok, K - 8, cfg.hidden, ok, None) == eng.ENGRAM_E_ALIGN
    assert lib.engram_pack_weight(L.handle, ok, K + 4, cfg.hidden, ok, None) == eng.ENGRAM_E_ALIGN
    assert lib.engram_pack_weight(L.handle, P(264), K, cfg.hidden, ok, None) == eng.ENGRAM_E_ALIGN
    assert lib.engram_pack_weight(L.handle, ok, K, cfg.hidden, P(8), None) == eng.ENGRAM_E_ALIGN
    assert lib.engram_pack_weight(L.handle, ok, K, 0, ok, None) == eng.ENGRAM_E_ARG
    assert lib.engram_pack_weight(L.handle, None, K, cfg.hidden, ok, None) == eng.ENGRAM_E_ARG
    # packed projection
    assert lib.engram_project_packed(L.handle, ok, K - 8, ok, cfg.hidden, ok, 4, None) == eng.ENGRAM_E_ALIGN
    assert lib.engram_project_packed(L.handle, P(264), K, ok, cfg.hidden, ok, 4, None) == eng.ENGRAM_E_ALIGN
    assert lib.engram_project_packed(L.handle, ok, K, ok, cfg.hidden, P(258), 4, None) == eng.ENGRAM_E_ALIGN
    assert lib.engram_project_packed(L.handle, ok, K, ok, cfg.hidden, ok, -1, None) == eng.ENGRAM_E_ARG
    assert lib.engram_project_packed(L.handle, ok, K, ok, 0, ok, 4, None) == eng.ENGRAM_E_ARG
    assert lib.engram_project_packed(L.handle, None, K, ok, cfg.hidden, ok, 4, None) == eng.ENGRAM_E_ARG
    # 256 rows of this leading dimension do not fit 32-bit byte offsets
    assert lib.engram_project_packed(L.handle, ok, 1 << 22, ok, cfg.hidden, ok, 4,
                                     None) == eng.ENGRAM_E_UNSUPPORTED
    # no tokens: nothing to do
    assert lib.engram_project_packed(L.handle, ok, K, ok, cfg.hidden, ok, 0, None) == 0


def test_multi_site_layout_matches_oracle_and_pages(golden):
    """Two sites, 8 heads, floor 16,000,000, one table per site: the product's
    primes and offsets equal the oracle's, and each site's table size is the
    row count the pages print."""
    g = golden["engram_num_embeddings"]
    floor_, H = g["args"]["floor"], g["heads_reading"]
    rows = max(g["value"])
    args = dict(vocab_size=129280, compressed_vocab=65536, pad_token_id=129279, heads_per_order=H,
                rows=[rows, 0, 0], row_dim=256, table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                row_pitch_bytes=256, hash_floor=floor_, num_sites=2,
                table_split=eng.ENGRAM_TABLE_PER_SITE, scale_layout=eng.ENGRAM_SCALE_BLOCK32_E8M0)
    L = eng.engram_layout_create(**args)
    info = L.info
    assert info.num_sites == 2 and info.k_pad == 24 * 256
    assert [info.site_rows(s) for s in range(2)] == g["value"]
    ref = oracle.site_layouts(2, H, floor_, True)
    for s in range(2):
        assert np.array_equal(np.array(info.site_primes[s], dtype=np.uint64), ref[s].primes)
        assert np.array_equal(np.array(info.site_offsets[s], dtype=np.uint64), ref[s].offsets)
    # one row short of the second site's buckets
    with pytest.raises(eng.EngramError) as e:
        eng.engram_layout_create(**{**args, "rows": [rows - 1, 0, 0]})
    assert e.value.status == eng.ENGRAM_E_LAYOUT_ROWS
    # block scales need D % 32 == 0
    with pytest.raises(eng.EngramError) as e:
        eng.engram_layout_create(**{**args, "row_dim": 250})
    assert e.value.status == eng.ENGRAM_E_ALIGN
    # per-order tables, three sites: offsets restart per order, as the oracle's
    L3 = eng.engram_layout_create(vocab_size=129280, compressed_vocab=65536, pad_token_id=129279,
                                  heads_per_order=2, rows=[10_000] * 3, row_dim=128,
                                  table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN, row_pitch_bytes=128,
                                  hash_floor=64, num_sites=3)
    ref3 = oracle.site_layouts(3, 2, 64, False)
    for s in range(3):
        assert np.array_equal(np.array(L3.info.site_primes[s], dtype=np.uint64), ref3[s].primes)
        assert np.array_equal(np.array(L3.info.site_offsets[s], dtype=np.uint64), ref3[s].offsets)
    with pytest.raises(eng.EngramError) as e:
        eng.engram_layout_create(**{**args, "num_sites": 5})
    assert e.value.status == eng.ENGRAM_E_ARG


def test_multi_site_fit_is_largest_floor():
    """With no floor given, the fitted floor is the largest at which every site's
    buckets fit, and one floor above it does not fit (oracle draw)."""
    rows = 50_000
    L = eng.engram_layout_create(vocab_size=16, compressed_vocab=8, pad_token_id=15, heads_per_order=2,
                                 rows=[rows, 0, 0], row_dim=64, table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                 row_pitch_bytes=64, num_sites=2, table_split=eng.ENGRAM_TABLE_PER_SITE)
    f = L.info.hash_floor

    def fits(fl):
        return all(int(l.primes.sum()) <= rows for l in oracle.site_layouts(2, 2, fl, True))
    assert fits(f) and not fits(f + 1)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for more it exits with a message, before it
    touches a device."""
    import subprocess
    import sys
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert out.returncode == 2 and "one GPU" in out.stderr


def test_projection_plan():
    """The library's choice of projection kernel for a call (engram_projection_plan,
    host logic, no device): the packed kernel once a packed weight exists and the call
    has 64 x 256 x 256 outputs or more; below that, split-K with the largest of 2, 4, 8
    splits that keeps at most one workgroup of 128 x 128 tiles per CU, four k-steps of
    64 per split and k_pad a multiple of 64 x splits; else the plain kernel."""
    def lay(k_cols, D):
        return eng.engram_layout_create(vocab_size=8, compressed_vocab=4, pad_token_id=7,
                                        heads_per_order=k_cols // 3, rows=[100_000] * 3, row_dim=D,
                                        table_dtype=eng.ENGRAM_DTYPE_FP8_E4M3FN,
                                        row_pitch_bytes=(D + 15) // 16 * 16)
    full = lay(3, 6500)        # k_pad 19,584
    pre = lay(6, 512)          # k_pad 3,072
    tiny = lay(6, 128)         # k_pad 768
    odd = lay(3, 100)          # k_pad 384 = 64 x 6: 2 splits divide it, 4 do not
    plan = eng.engram_projection_plan
    # many tokens: the packed kernel when a packed weight exists, else the plain one
    assert plan(full, 4096, 65536, packed=True) == ("packed", 1)
    assert plan(full, 4096, 65536, packed=False) == ("plain", 1)
    assert plan(pre, 4096, 16384, packed=True) == ("packed", 1)
    assert plan(pre, 4096, 1024, packed=True) == ("packed", 1)   # 1,024 x 4,096 = 64 x 256 x 256
    # decode: 256 tokens x 4,096 outputs = 64 tiles -> 4 splits (8 would need 512 CUs)
    assert plan(pre, 4096, 256, packed=True) == ("splitk", 4)
    # tiny: 512 x 256 = 8 tiles; 4 splits would leave 192 k per split (< 4 steps)
    assert plan(tiny, 256, 512, packed=False) == ("splitk", 2)
    # k_pad 384: 2 splits leave 192 k (< 4 steps), so none
    assert plan(odd, 256, 64, packed=False) == ("plain", 1)
    # a single token: 32 tiles of 128 columns -> 8 splits when k_pad allows (3,072 =
    # 64 x 48); 19,584 = 64 x 306 allows only 2
    assert plan(pre, 4096, 1, packed=True) == ("splitk", 8)
    assert plan(full, 4096, 1, packed=True) == ("splitk", 2)
    # a forced split count applies below the packed size
    assert plan(pre, 4096, 256, packed=True, splits=2) == ("splitk", 2)
    assert plan(pre, 4096, 256, packed=True, splits=1) == ("plain", 1)
    assert plan(pre, 4096, 16384, packed=True, splits=2) == ("packed", 1)


def test_bench_traffic_is_keyed_to_the_kernel_source(tmp_path):
    """bench.py reports counter-measured traffic only while the kernel's code (its source
    without comments) hashes to the value recorded with the counters; an edited kernel
    gives null."""
    import importlib.util
    import shutil
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    full = ei.get_config("full")
    proj = ("gemm_bf16_nt_packed_{tag}_counters.txt", "gemm_packed.hip")
    gate = ("gate_add_{tag}_traffic.txt", "gate.hip")
    assert 1000.0 < bench.measured_mfma_ceiling() < bench.BF16_PEAK_TFLOPS  # the probe's best rate
    assert bench.measured_traffic(full) > bench.algorithmic_per_token(full)["gather_bytes"] * 65536
    assert bench.measured_traffic(full, *proj) > 0
    assert bench.measured_traffic(full, *gate) > bench.algorithmic_per_token(full)["gate_bytes"] * 65536
    assert bench.measured_traffic(ei.get_config("tiny")) is None  # no counters for it
    # the same files under another root, with one comment added to each kernel source
    shutil.copytree(os.path.join(ROOT, "profiles"), tmp_path / "profiles")
    kdir = tmp_path / "hashed_gram_memory_tid2eid_amd" / "csrc" / "kernels"
    kdir.mkdir(parents=True)
    for name in ("gather.hip", "gemm_packed.hip", "gate.hip"):
        src = open(os.path.join(ROOT, "hashed_gram_memory_tid2eid_amd", "csrc", "kernels", name)).read()
        (kdir / name).write_text(src)
    bench.ROOT = str(tmp_path)
    measured = lambda: [bench.measured_traffic(full), bench.measured_traffic(full, *proj),
                        bench.measured_traffic(full, *gate)]
    assert None not in measured()
    # a comment edit leaves the kernel as it was measured; a code edit does not
    for name in ("gather.hip", "gemm_packed.hip", "gate.hip"):
        (kdir / name).write_text((kdir / name).read_text() + "// edited\n/* edited */\n")
    assert None not in measured()
    for name in ("gather.hip", "gemm_packed.hip", "gate.hip"):
        (kdir / name).write_text((kdir / name).read_text() + "static int edited;\n")
    assert measured() == [None, None, None]


def test_readme_c_example_compiles_against_the_header(tmp_path):
    """The C example of the README compiles as C11 against include/engram.h (the ABI
    is plain C), and every engram_* function it calls is one the library exports."""
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or the ROCm headers are not available")
    text = open(os.path.join(ROOT, "README.md")).read()
    m = re.search(r"```c\n(.*?)```", text, re.S)
    assert m, "the README holds a C example"
    src = tmp_path / "example.c"
    src.write_text(m.group(1))
    obj = tmp_path / "example.o"
    out = subprocess.run([gcc, "-std=c11", "-c", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                          "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src),
                          "-o", str(obj)], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    nm = subprocess.run(["nm", str(obj)], capture_output=True, text=True, check=True).stdout
    called = {ln.split()[-1] for ln in nm.splitlines() if ln.strip().startswith("U engram_")}
    assert called and called <= set(declared_functions())


def test_loaded_library_is_built_from_the_tree():
    """The loaded library records the hash of the sources it was built from, and it
    equals the hash of csrc/ and include/ as they stand (the build step rebuilds a
    library whose hash differs, so no stale binary is loaded)."""
    import runpy
    bl = runpy.run_path(os.path.join(ROOT, "hashed_gram_memory_tid2eid_amd", "build_lib.py"))
    sha = bl["source_hash"]()
    assert eng.engram_build_id() == bl["BUILD_ID_PREFIX"] + sha
    assert bl["built_hash"](eng.LIB_PATH) == sha
    assert bl["built_hash"](os.path.join(ROOT, "README.md")) is None


def test_build_identity_does_not_depend_on_where_the_tree_sits(tmp_path):
    """A copy of the sources and the build script in another directory hashes to the
    same identity, so a tree moved or copied elsewhere keeps its built library
    instead of rebuilding it; a changed source byte changes the identity."""
    import runpy
    import shutil
    pkg = os.path.join(ROOT, "hashed_gram_memory_tid2eid_amd")
    here = runpy.run_path(os.path.join(pkg, "build_lib.py"))["source_hash"]()
    dst = tmp_path / "elsewhere"
    shutil.copytree(os.path.join(pkg, "csrc"), dst / "hashed_gram_memory_tid2eid_amd" / "csrc")
    shutil.copytree(os.path.join(ROOT, "include"), dst / "include")
    shutil.copy(os.path.join(pkg, "build_lib.py"), dst / "hashed_gram_memory_tid2eid_amd" / "build_lib.py")
    script = str(dst / "hashed_gram_memory_tid2eid_amd" / "build_lib.py")
    assert runpy.run_path(script)["source_hash"]() == here
    with open(dst / "include" / "engram.h", "a") as f:
        f.write("\n")
    assert runpy.run_path(script)["source_hash"]() != here


def test_bench_cpu_baseline_leg_runs_pinned_on_host_tensors():
    """bench.py's oracle leg on CPU copies of small workloads (one site and the
    two-site released structure): it reports a positive rate on one core with the
    host CPU model, and gives the calling thread its CPU mask back afterwards."""
    import importlib.util
    import torch
    spec = importlib.util.spec_from_file_location("bench_cpu_leg", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    mask = os.sched_getaffinity(0)
    for name in ("tiny", "v41_small"):
        cfg = ei.get_config(name)
        batch = ei.make_batch(cfg)
        tabs = [ei.make_tables(cfg, "cpu", site=s) for s in range(cfg.n_sites)]
        ws = [ei.make_weight(cfg, "cpu", site=s) for s in range(cfg.n_sites)]
        xs = [ei.make_streams(cfg, batch.T, "cpu", step=s).view(torch.int16).numpy().view(np.uint16)
              for s in range(cfg.n_sites)]
        r = bench.cpu_baseline(cfg, batch, tabs, ws, xs, 0.5)
        assert r["value"] > 0 and r["cores"] == 1 and r["kind"] == "oracle"
        assert r["cpu_model"] and "pinned to host core" in r["sample"]
        assert os.sched_getaffinity(0) == mask
