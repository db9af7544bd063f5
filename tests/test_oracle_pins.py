"""Pins of the oracle against what the pages and the mathematics fix.

Each test ties an oracle function to something other than itself: a number
printed on the pages (tests/golden/pages_values.json), a library routine, an
exact rational computation, a sieve, or a brute-force enumeration written in a
different formulation.  No GPU is needed.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import engram_inputs as ei


# ---------------------------------------------------------------------------
# helpers that are independent of the oracle
# ---------------------------------------------------------------------------

def sieve(limit: int) -> np.ndarray:
    """Eratosthenes: boolean primality of 0..limit."""
    is_p = np.ones(limit + 1, dtype=bool)
    is_p[:2] = False
    for i in range(2, int(limit ** 0.5) + 1):
        if is_p[i]:
            is_p[i * i::i] = False
    return is_p


def draw_by_sieve(is_p, n_layers, max_ngram, heads, floor_):
    """The bucket draw stated set-wise: for every (layer, order), the `heads` smallest
    primes >= floor that no earlier (layer, order) took."""
    primes = np.flatnonzero(is_p[floor_:]) + floor_
    taken = set()
    out = []
    for _layer in range(n_layers):
        for _order in range(2, max_ngram + 1):
            got = [int(p) for p in primes if int(p) not in taken][:heads]
            taken.update(got)
            out.append(got)
    return np.asarray(out, dtype=np.uint64).reshape(n_layers, max_ngram - 1, heads)


# ---------------------------------------------------------------------------
# layout
# ---------------------------------------------------------------------------

def test_prime_draw_pages_462(golden):
    g = golden["prime_sum_floor64"]
    a = g["args"]
    p = oracle.draw_primes(a["layers"], a["max_ngram"], a["heads"], a["floor"])
    assert int(p.sum()) == g["value"]


def test_prime_draw_pages_engram_num_embeddings(golden):
    g = golden["engram_num_embeddings"]
    a = g["args"]
    p = oracle.draw_primes(a["layers"], a["max_ngram"], g["heads_reading"], a["floor"])
    assert [int(x) for x in p.reshape(a["layers"], -1).sum(axis=1)] == g["value"]


def test_ngram_param_count_matches_pages(golden):
    rows = sum(golden["engram_num_embeddings"]["value"])
    params = rows * 256
    assert abs(params / 1e9 - golden["ngram_params_billion_2dp"]["value"]) < 0.005
    assert abs(params / 1e9 - golden["ngram_params_billion"]["value"]) < 0.05


@pytest.mark.parametrize("args", [(1, 4, 2, 64), (2, 4, 2, 64), (1, 4, 3, 2011), (2, 4, 8, 1000),
                                  (1, 4, 1, 5_039_971), (1, 4, 2, 524_231)])
def test_prime_draw_vs_sieve(args):
    layers, mx, heads, fl = args
    is_p = sieve(fl + 20_000)
    assert np.array_equal(oracle.draw_primes(*args), draw_by_sieve(is_p, layers, mx, heads, fl))


def test_prime_draw_vs_trial_division():
    """The draw as a walk: every bucket, in (layer, order, head) order, takes the
    next integer at or above the floor that trial division finds prime and no
    earlier bucket took."""
    def is_prime(n):
        return n >= 2 and all(n % d for d in range(2, math.isqrt(n) + 1))

    for layers, mx, heads, fl in [(1, 4, 2, 64), (2, 4, 3, 1), (3, 4, 2, 1000)]:
        taken, got, cur = set(), [], fl
        for _ in range(layers * (mx - 1) * heads):
            while not is_prime(cur) or cur in taken:
                cur += 1
            taken.add(cur)
            got.append(cur)
        assert [int(x) for x in oracle.draw_primes(layers, mx, heads, fl).reshape(-1)] == got


@pytest.mark.parametrize("name", ["tiny", "prefill", "long", "full"])
def test_fit_layout_is_the_largest_fitting_floor(name):
    cfg = ei.get_config(name)
    R, H = cfg.rows, cfg.heads
    L = oracle.fit_layout([R] * 3, H)
    is_p = sieve(R // H + 40_000)
    # the fitted draw is the sieve draw at that floor and every order fits
    assert np.array_equal(L.primes, draw_by_sieve(is_p, 1, 4, H, L.floor)[0])
    assert all(int(s) <= R for s in L.primes.sum(axis=1))
    # every larger floor up to R/H fails for some order (brute force)
    for f in range(L.floor + 1, R // H + 1):
        d = draw_by_sieve(is_p, 1, 4, H, f)[0]
        assert any(int(s) > R for s in d.sum(axis=1)), f
    # offsets are prefix sums inside each table; every bucket lies inside its table
    for n in range(3):
        acc = 0
        for h in range(H):
            assert int(L.offsets[n, h]) == acc
            acc += int(L.primes[n, h])
        assert acc <= R


def test_layout_guard_rejects_short_tables_allows_long(golden):
    # the pages' synthetic case: 1024 rows against a prime sum of 462 is fine
    L = oracle.layout_at_floor([1024, 1024, 1024], 2, 64)
    assert int(L.primes.sum()) == golden["prime_sum_floor64"]["value"]
    # one row short of an order's prime sum is rejected
    need = [int(s) for s in L.primes.sum(axis=1)]
    with pytest.raises(oracle.OracleError) as e:
        oracle.layout_at_floor([need[0], need[1], need[2] - 1], 2, 64)
    assert e.value.code == oracle.ORC_E_ROWS
    oracle.layout_at_floor(need, 2, 64)


def test_full_scale_split_and_footprints(golden):
    cfg = ei.get_config("full")
    total = 3 * cfg.rows
    assert total == golden["total_rows_3_tables"]["value"]
    L = oracle.fit_layout([cfg.rows] * 3, cfg.heads)
    assert int(L.primes.sum()) <= total
    gib = 2 ** 30
    fp8 = total * (cfg.row_dim + 4) / gib      # e4m3fn bytes + one fp32 scale per row
    bf16 = total * cfg.row_dim * 2 / gib
    assert abs(fp8 / golden["fp8_gib"]["value"] - 1) < 0.005
    assert abs(bf16 / golden["bf16_gib"]["value"] - 1) < 0.005


def test_tid2eid_total_and_onto(golden):
    m = ei.make_tid2eid()
    assert m.shape == (golden["vocab_size"]["value"],)
    assert m.min() >= 0 and m.max() < ei.VC
    assert np.bincount(m, minlength=ei.VC).min() >= 1


# ---------------------------------------------------------------------------
# windows, hash, decode store: brute force in a different formulation
# ---------------------------------------------------------------------------

def windows_bruteforce(tid2eid, pad, tokens, cu, seq_start, slots, store, dead):
    """Windows stated by blocking positions rather than by a carried tail.  For token
    t the lookback j reads position t-j unless a dead position lies in [t-j, t], or
    t-j precedes a sequence that starts here; positions before a continuing sequence
    come from the slot's stored ids (oldest first).  A dead token's window is all pad.
    Returns (windows [T][4], new store)."""
    T = len(tokens)
    e = [pad if (dead is not None and dead[t]) else int(tid2eid[tokens[t]]) for t in range(T)]
    new_store = None if store is None else store.copy()
    W = np.zeros((T, 4), dtype=np.int64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        starts = True if seq_start is None else bool(seq_start[s])
        slot = -1 if slots is None else int(slots[s])
        for t in range(a, b):
            if dead is not None and dead[t]:
                W[t] = pad
                continue
            W[t, 0] = e[t]
            for j in (1, 2, 3):
                q = t - j
                lo = max(q, a)
                blocked = dead is not None and any(dead[lo:t])
                if blocked:
                    W[t, j] = pad
                elif q >= a:
                    W[t, j] = e[q]
                elif starts:
                    W[t, j] = pad
                else:
                    W[t, j] = store[slot][3 - (a - q)]
        if slot >= 0:
            if b > a:
                new_store[slot] = [W[b - 1, 2], W[b - 1, 1], W[b - 1, 0]]
            elif starts:
                new_store[slot] = [pad, pad, pad]
    return W, new_store


def digits_layout(vc, heads=2):
    """A layout whose primes all exceed vc^4, so row - offset is the key itself."""
    fl = vc ** 4 + 1
    return oracle.layout_at_floor([10 ** 9] * 3, heads, fl)


# small world: vocab 5, compressed ids 0..4, pad token 4 -> pad id 4; real tokens
# use ids 0..3 so a pad in a window can only come from blocking
SMALL_VC = 5
SMALL_MAP = np.arange(5, dtype=np.int32)
SMALL_PAD = 4


def run_oracle_small(layout, tokens, cu, seq_start=None, slots=None, store=None, dead=None):
    st = None if store is None else np.ascontiguousarray(store.copy(), dtype=np.int32)
    eids, rows = oracle.compress_hash(layout, vocab=5, vc=SMALL_VC, pad_token_id=4,
                                      tid2eid=SMALL_MAP, tokens=tokens, cu_seqlens=cu,
                                      seq_start=seq_start, slots=slots, store=st, dead=dead)
    return eids, rows, st


def decode_digits(rows, layout, vc):
    """row - offset = key_n = sum_j w_j vc^j -> the window digits w_0..w_{n-1}."""
    T = rows.shape[0]
    out = np.zeros((T, 3, 4), dtype=np.int64) - 1
    for t in range(T):
        for n in range(3):
            keys = {int(rows[t, n, h]) - int(layout.offsets[n, h]) for h in range(layout.heads)}
            assert len(keys) == 1, "heads disagree on the key when no modulus applies"
            k = keys.pop()
            for j in range(n + 2):
                out[t, n, j] = k % vc
                k //= vc
            assert k == 0, "key exceeds vc^n"
    return out


def check_windows(layout, tokens, cu, seq_start=None, slots=None, store=None, dead=None):
    eids, rows, new_store = run_oracle_small(layout, tokens, cu, seq_start, slots, store, dead)
    W, bf_store = windows_bruteforce(SMALL_MAP, SMALL_PAD, tokens, cu, seq_start, slots, store,
                                     dead)
    d = decode_digits(rows, layout, SMALL_VC)
    for n in range(3):
        assert np.array_equal(d[:, n, : n + 2], W[:, : n + 2]), (tokens, dead, n)
    assert np.array_equal(eids, W[:, 0])
    if store is not None:
        assert np.array_equal(new_store, bf_store)


def test_windows_exhaustive_single_sequence():
    layout = digits_layout(SMALL_VC)
    for L in range(0, 6):
        cu = np.array([0, L], dtype=np.int32)
        for toks in itertools.product(range(4), repeat=L):
            tokens = np.array(toks, dtype=np.int32)
            for mask in range(2 ** L):
                dead = np.array([(mask >> i) & 1 for i in range(L)], dtype=np.uint8)
                check_windows(layout, tokens, cu, dead=dead if L else None)


def test_windows_random_multi_sequence_with_store():
    layout = digits_layout(SMALL_VC)
    rng = np.random.default_rng(1234)
    for _ in range(3000):
        S = int(rng.integers(1, 5))
        lens = rng.integers(0, 6, size=S)
        cu = np.zeros(S + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens)
        T = int(cu[-1])
        tokens = rng.integers(0, 4, size=T).astype(np.int32)
        dead = (rng.random(T) < 0.2).astype(np.uint8)
        seq_start = (rng.random(S) < 0.5).astype(np.uint8)
        num_slots = S + 2
        slots = rng.permutation(num_slots)[:S].astype(np.int32)
        store = rng.integers(0, 5, size=(num_slots, 3)).astype(np.int32)
        check_windows(layout, tokens, cu, seq_start, slots, store, dead)


def test_hash_modulus_and_range():
    """With small primes the row is offset + (key mod p), where key is read off a
    run whose primes exceed every key; rows stay inside their buckets."""
    big = digits_layout(SMALL_VC)
    rng = np.random.default_rng(7)
    tokens = rng.integers(0, 4, size=400).astype(np.int32)
    cu = np.array([0, 150, 150, 400], dtype=np.int32)
    dead = (rng.random(400) < 0.1).astype(np.uint8)
    _, rows_big, _ = run_oracle_small(big, tokens, cu, dead=dead)
    for fl in (2, 7, 31, 97):
        small = oracle.layout_at_floor([10 ** 6] * 3, 2, fl)
        _, rows, _ = run_oracle_small(small, tokens, cu, dead=dead)
        for n in range(3):
            for h in range(2):
                key = rows_big[:, n, 0].astype(np.int64) - int(big.offsets[n, 0])
                p, off = int(small.primes[n, h]), int(small.offsets[n, h])
                assert np.array_equal(rows[:, n, h].astype(np.int64) - off, key % p)
                assert rows[:, n, h].min() >= off and rows[:, n, h].max() < off + p


def test_row_ids_refuse_int32_overflow():
    vc = 65536
    tid2eid = np.array([vc - 1, 0], dtype=np.int32)
    L = oracle.layout_at_floor([2 ** 40] * 3, 1, 2 ** 33)
    with pytest.raises(oracle.OracleError):
        oracle.compress_hash(L, vocab=2, vc=vc, pad_token_id=1, tid2eid=tid2eid,
                             tokens=np.array([0, 0, 0, 0], dtype=np.int32),
                             cu_seqlens=np.array([0, 4], dtype=np.int32))


def test_hash_residue_at_full_compressed_vocab():
    """Residues of the exact 64-bit key at vc = 65536 match Python integers on the
    windows the brute-force enumerator produces."""
    vc = 65536
    rng = np.random.default_rng(3)
    tid2eid = rng.integers(0, vc, size=1000).astype(np.int32)
    tid2eid[:4] = [vc - 1, vc - 1, vc - 2, 0]
    tokens = np.concatenate([[0, 1, 0, 1, 2, 3], rng.integers(0, 1000, size=300)]).astype(np.int32)
    cu = np.array([0, 6, 306], dtype=np.int32)
    dead = np.zeros(306, dtype=np.uint8)
    dead[100:105] = 1
    L = oracle.fit_layout([5_040_000] * 3, 1)
    eids, rows = oracle.compress_hash(L, vocab=1000, vc=vc, pad_token_id=999, tid2eid=tid2eid,
                                      tokens=tokens, cu_seqlens=cu, dead=dead)
    W, _ = windows_bruteforce(tid2eid, int(tid2eid[999]), tokens, cu, None, None, None, dead)
    for t in range(306):
        for n in range(3):
            key = sum(int(W[t, j]) * vc ** j for j in range(n + 2))
            assert key < vc ** (n + 2) <= 2 ** 64
            p, off = int(L.primes[n, 0]), int(L.offsets[n, 0])
            assert int(rows[t, n, 0]) == off + key % p


@pytest.mark.parametrize("with_dead", [False, True])
def test_decode_store_equals_prefill_at_every_split(with_dead):
    """The pages' equivalence method: prompt-then-steps at every split point equals the
    one-call prefill, exactly (integers)."""
    cfg = ei.get_config("tiny")
    tid2eid = ei.make_tid2eid()
    L = oracle.fit_layout([cfg.rows] * 3, cfg.heads)
    rng = np.random.default_rng(11)
    T = 40
    tokens = ei.uniform_tokens(rng, T)
    dead = None
    if with_dead:
        dead = np.zeros(T, dtype=np.uint8)
        dead[10:14] = 1   # an image span inside the prompt for some splits, after it for others
        dead[25] = 1
    kw = dict(vocab=cfg.vocab, vc=cfg.vc, pad_token_id=cfg.pad_token_id, tid2eid=tid2eid)
    ref_e, ref_r = oracle.compress_hash(L, tokens=tokens, cu_seqlens=np.array([0, T], np.int32),
                                        dead=dead, **kw)
    for split in range(0, T + 1):
        store = np.full((3, 3), -7, dtype=np.int32)
        slots = np.array([1], dtype=np.int32)
        e1, r1 = oracle.compress_hash(L, tokens=tokens[:split],
                                      cu_seqlens=np.array([0, split], np.int32),
                                      seq_start=np.array([1], np.uint8), slots=slots, store=store,
                                      dead=None if dead is None else dead[:split], **kw)
        es, rs = [e1], [r1]
        for t in range(split, T):   # one token per decode step
            e, r = oracle.compress_hash(L, tokens=tokens[t:t + 1], cu_seqlens=np.array([0, 1], np.int32),
                                        seq_start=np.array([0], np.uint8), slots=slots, store=store,
                                        dead=None if dead is None else dead[t:t + 1], **kw)
            es.append(e)
            rs.append(r)
        assert np.array_equal(np.concatenate(es), ref_e)
        assert np.array_equal(np.concatenate(rs), ref_r)
        assert store[0, 0] == -7 and store[2, 0] == -7  # other slots untouched


def test_continuation_without_store_is_refused():
    L = oracle.layout_at_floor([1000] * 3, 1, 100)
    with pytest.raises(oracle.OracleError) as e:
        oracle.compress_hash(L, vocab=5, vc=5, pad_token_id=4, tid2eid=SMALL_MAP,
                             tokens=np.array([1, 2], np.int32), cu_seqlens=np.array([0, 2], np.int32),
                             seq_start=np.array([0], np.uint8))
    assert e.value.code == oracle.ORC_E_NEED_STORE


def test_token_out_of_range_is_refused():
    L = oracle.layout_at_floor([1000] * 3, 1, 100)
    with pytest.raises(oracle.OracleError) as e:
        oracle.compress_hash(L, vocab=5, vc=5, pad_token_id=4, tid2eid=SMALL_MAP,
                             tokens=np.array([1, 5], np.int32), cu_seqlens=np.array([0, 2], np.int32))
    assert e.value.code == oracle.ORC_E_TOKEN


# ---------------------------------------------------------------------------
# dequant
# ---------------------------------------------------------------------------

def test_e4m3fn_decode_all_bytes_vs_torch(golden):
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    mine = np.array([oracle.e4m3fn_decode(i) for i in range(256)], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.flatnonzero(nan).tolist() == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # incl. signed zero
    assert mine[~nan].max() == golden["e4m3fn_max"]["value"]


def test_dequant_pow2_scale_is_exact():
    """q * 2^k is the exact rational for every finite e4m3fn q and k in [-20, 20], and
    its bf16 rounding changes nothing."""
    codes = np.array([i for i in range(256) if i not in (0x7F, 0xFF)], dtype=np.uint8)
    for k in range(-20, 21):
        scale = np.float32(2.0 ** k)
        f32, b16 = oracle.dequant_rows(codes[None, :], np.array([scale]))
        for c, got, gb in zip(codes, f32[0], b16[0]):
            q = torch.tensor([int(c)], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()
            exact = Fraction(q) * Fraction(2) ** k
            assert Fraction(float(got)) == exact
            gf = np.array([int(gb) << 16], dtype=np.uint32).view(np.float32)[0]
            assert Fraction(float(gf)) == exact


def test_dequant_arbitrary_scale_is_one_fp32_multiply():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=(64, 96)).astype(np.uint8)
    codes[codes == 0x7F] = 0
    codes[codes == 0xFF] = 0
    scales = (rng.random(64) * 0.02 + 1e-4).astype(np.float32)
    f32, b16 = oracle.dequant_rows(codes, scales)
    q = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    ref = (q * scales[:, None]).astype(np.float32)   # numpy float32 multiply: one IEEE op
    assert np.array_equal(f32.view(np.uint32), ref.view(np.uint32))
    ref_b16 = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16, ref_b16)


def test_dequant_nan_byte_is_reported():
    with pytest.raises(oracle.OracleError) as e:
        oracle.dequant_rows(np.array([[1, 0x7F]], np.uint8), np.array([1.0], np.float32))
    assert e.value.code == oracle.ORC_E_NAN


def test_dequant_bf16_table_widens_exactly():
    rng = np.random.default_rng(9)
    x = torch.from_numpy(rng.standard_normal((8, 33)).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    f32, b16 = oracle.dequant_rows(bits, None, bf16_table=True)
    assert np.array_equal(f32, x.float().numpy())
    assert np.array_equal(b16, bits)


def nearest_bf16_exact(x: float) -> int:
    """Brute force: the bf16 bit pattern nearest to x (exact rationals), ties to even."""
    fx = Fraction(x)
    if x == 0:
        return 0x8000 if math.copysign(1, x) < 0 else 0
    sign = 0x8000 if x < 0 else 0
    ax = abs(fx)
    # candidates: all finite positive bf16 around |x|
    f = np.array([abs(x)], dtype=np.float32)  # close float guess for the neighborhood
    base = int(f.view(np.uint32)[0] >> 16)
    best = None
    for bits in range(max(0, base - 2), min(0x7F7F, base + 3) + 1):
        v = Fraction(float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]))
        d = abs(v - ax)
        key = (d, bits & 1)
        if best is None or key < best[0]:
            best = (key, bits)
    return sign | best[1]


def test_bf16_rne_vs_torch_and_exact():
    rng = np.random.default_rng(21)
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormal range
        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 3.3895314e38,
                  3.4e38, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135], dtype=np.float32),
    ])
    mine = np.array([oracle.bf16_rne(float(v)) for v in f], dtype=np.uint16)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    # doubles that are not floats: exact nearest by rational arithmetic
    d = rng.standard_normal(3000) * np.exp(rng.uniform(-30, 30, 3000))
    for v in d:
        assert oracle.bf16_rne(float(v)) == nearest_bf16_exact(float(v)), v


# ---------------------------------------------------------------------------
# projection and gate
# ---------------------------------------------------------------------------

def bf16_bits(a) -> np.ndarray:
    return torch.as_tensor(a, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def test_project_vs_numpy_matmul():
    rng = np.random.default_rng(2)
    E = bf16_bits(rng.standard_normal((7, 96)))
    W = bf16_bits(rng.standard_normal((40, 96)) * 0.02)
    v = oracle.project(E, W)
    ref = bits_to_f64(E) @ bits_to_f64(W).T
    np.testing.assert_allclose(v, ref, rtol=1e-13, atol=1e-13)
    # a transposed operand would not match on a non-square case
    assert v.shape == (7, 40)


def test_gate_keep_zero_and_zero_v_leave_streams_bitwise():
    rng = np.random.default_rng(4)
    x = bf16_bits(rng.standard_normal((6, 4, 32)))
    v = rng.standard_normal((6, 32))
    keep = np.array([0, 1, 0, 1, 1, 0], np.uint8)
    y, g = oracle.gate_add(x, v, keep)
    assert np.array_equal(y[keep == 0], x[keep == 0])
    assert np.all(g[keep == 0] == 0)
    y0, _ = oracle.gate_add(x, np.zeros((6, 32)))
    assert np.array_equal(y0, x)


def test_gate_identical_streams_give_identical_outputs():
    rng = np.random.default_rng(6)
    one = bf16_bits(rng.standard_normal((5, 1, 64)))
    x = np.repeat(one, 4, axis=1)
    y, g = oracle.gate_add(x, rng.standard_normal((5, 64)))
    for s in range(1, 4):
        assert np.array_equal(y[:, s], y[:, 0])
        assert np.array_equal(g[:, s], g[:, 0])


def test_gate_zero_stream_takes_half_of_v():
    rng = np.random.default_rng(8)
    x = np.zeros((3, 4, 16), np.uint16)
    vb = bf16_bits(rng.standard_normal((3, 16)))
    v = bits_to_f64(vb)
    y, g = oracle.gate_add(x, v)
    assert np.all(g == 0.5)
    half = bf16_bits(bits_to_f64(vb) * 0.5)   # exact: halving a bf16 stays a bf16
    for s in range(4):
        assert np.array_equal(y[:, s], half)


def test_gate_matches_expit_closed_form():
    from scipy.special import expit
    rng = np.random.default_rng(10)
    hidden = 64
    x = bf16_bits(rng.standard_normal((50, 4, hidden)))
    v = rng.standard_normal((50, hidden))
    y, g = oracle.gate_add(x, v)
    xf = bits_to_f64(x)
    z = np.einsum("tsh,th->ts", xf, v) / math.sqrt(hidden)
    np.testing.assert_allclose(g, expit(z), rtol=1e-13, atol=0)
    ref = xf + expit(z)[:, :, None] * v[:, None, :]
    got = bits_to_f64(y)
    # one bf16 rounding of the fp64 value: within half an ulp (2^-9 relative)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-300)


def test_gate_logit_hand_computed_values():
    """Values worked out by hand from z = <x_s, v> / sqrt(hidden) and
    g = 1 / (1 + e^-z).  hidden = 64, v = 0.5 everywhere:
      stream 0: x = +0.5 -> <x, v> = 16, z = 2,  g = 1 / (1 + 0.1353352832366127)
                = 0.8807970779778823; y = 0.5 + 0.5 g = 0.94039853898894 -> bf16
                (step 2^-8 in [0.5, 1)) 241/256 = 0.94140625
      stream 1: x = -0.5 -> z = -2, g = 0.11920292202211755; y = -0.5 + 0.5 g
                = -0.44039853898894 -> bf16 (step 2^-9) -225/512 = -0.439453125
      stream 2: x = 0    -> z = 0,  g = 0.5; y = 0.25
      stream 3: x = +1.0 -> z = 4,  g = 1 / (1 + 0.01831563888873418)
                = 0.9820137900379085; y = 1 + 0.5 g = 1.4910068950189543 -> bf16
                (step 2^-7 in [1, 2)) 191/128 = 1.4921875
    A sign slip (sigma(-z)) or a 1/hidden scale (z = 0.25 for stream 0) fails here."""
    hidden = 64
    xs = np.array([0.5, -0.5, 0.0, 1.0])
    x = bf16_bits(np.repeat(xs[None, :, None], hidden, axis=2))     # [1][4][64]
    v = np.full((1, hidden), 0.5)
    y, g = oracle.gate_add(x, v)
    g_hand = [0.8807970779778823, 0.11920292202211755, 0.5, 0.9820137900379085]
    np.testing.assert_allclose(g[0], g_hand, rtol=1e-15, atol=0)
    y_hand = [0.94140625, -0.439453125, 0.25, 1.4921875]
    for s in range(4):
        assert np.all(bits_to_f64(y[0, s]) == y_hand[s]), s
    # one-hot: v has 8.0 at element 3 only and x_s has 1.0 there -> <x, v> = 8,
    # z = 1, g = 1 / (1 + 0.36787944117144233) = 0.7310585786300049; element 3
    # becomes 1 + 8 g = 6.848468629040039 -> bf16 (step 2^-5 in [4, 8)) 219/32 =
    # 6.84375; every other element keeps x exactly (v is 0 there)
    rng = np.random.default_rng(12)
    xr = bits_to_f64(bf16_bits(rng.standard_normal((1, 4, hidden))))
    xr[:, :, 3] = 1.0
    xr[:, :, 2] = 0.0   # element 2 of x never meets a non-zero v
    vr = np.zeros((1, hidden))
    vr[0, 3] = 8.0
    y2, g2 = oracle.gate_add(bf16_bits(xr), vr)
    np.testing.assert_allclose(g2[0], [0.7310585786300049] * 4, rtol=1e-15, atol=0)
    got = bits_to_f64(y2)
    assert np.all(got[0, :, 3] == 6.84375)
    keep = np.ones(hidden, bool)
    keep[3] = False
    assert np.array_equal(got[0][:, keep], xr[0][:, keep])


# ---------------------------------------------------------------------------
# sites sharing one hash pass; (1, 32) e8m0 block scales
# ---------------------------------------------------------------------------

def test_site_layout_released_tables(golden):
    """One table per site: each site's last bucket ends at its table's row count,
    which the pages print (384,006,168 / 384,016,682)."""
    g = golden["engram_num_embeddings"]
    L = oracle.site_layouts(g["args"]["layers"], g["heads_reading"], g["args"]["floor"], True)
    ends = [int(l.offsets[2, -1] + l.primes[2, -1]) for l in L]
    assert ends == g["value"]
    for l in L:
        flat_p = l.primes.reshape(-1).astype(np.int64)
        flat_o = l.offsets.reshape(-1).astype(np.int64)
        assert flat_o[0] == 0
        assert np.array_equal(flat_o[1:], np.cumsum(flat_p)[:-1])  # buckets back to back
    # site 1 draws after site 0: every prime larger, none shared
    assert L[1].primes.min() > L[0].primes.max()


def test_site_layout_per_order_tables_restart_offsets():
    L = oracle.site_layouts(3, 2, 64, False)
    p = oracle.draw_primes(3, 4, 2, 64)
    for s, l in enumerate(L):
        assert np.array_equal(l.primes, p[s])
        assert (l.offsets[:, 0] == 0).all()
        assert np.array_equal(l.offsets[:, 1], l.primes[:, 0])
    # one site is the single-site layout at the same floor
    one = oracle.layout_at_floor([10_000] * 3, 2, 64)
    assert np.array_equal(L[0].primes, one.primes) and np.array_equal(L[0].offsets, one.offsets)


def test_e8m0_decode_closed_forms():
    assert oracle.e8m0_decode(127) == 1.0
    assert oracle.e8m0_decode(128) == 2.0
    assert oracle.e8m0_decode(120) == 2.0 ** -7
    assert oracle.e8m0_decode(254) == 2.0 ** 127
    assert oracle.e8m0_decode(0) == 2.0 ** -127
    assert math.isnan(oracle.e8m0_decode(255))


def test_dequant_block32_against_torch_float8():
    """fp32(e4m3fn(q) * e8m0(b)) and its bf16 rounding against torch's own
    float8_e4m3fn / float8_e8m0fnu conversions and an fp32 multiply, over every
    e4m3 code, with a different exponent in every 32-element block (including
    the subnormal 2^-127 scale and the largest ones)."""
    import torch
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    D = 256
    n = 12
    rng = np.random.default_rng(3)
    rows = rng.choice(codes, size=(n, D)).astype(np.uint8)
    rows[0, :len(codes)] = codes  # every finite code once
    scales = rng.integers(100, 140, size=(n, D // 32)).astype(np.uint8)
    scales[1] = [0, 1, 2, 127, 128, 200, 253, 254]
    scales[2] = [0] * (D // 32)
    rows[2] = codes[np.arange(D) % len(codes)]
    f32, b16 = oracle.dequant_rows_block32(rows, scales)
    q = torch.from_numpy(rows).view(torch.float8_e4m3fn).float()
    s = torch.from_numpy(scales).view(torch.float8_e8m0fnu).float()
    ref = q * s.repeat_interleave(32, dim=1)
    assert np.array_equal(f32.view(np.uint32), ref.numpy().view(np.uint32))
    ref16 = ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16, ref16)


def test_dequant_block32_uniform_blocks_equal_row_scale():
    """With the same exponent in every block, block dequant equals the per-row
    scale path at scale 2^(b-127)."""
    rng = np.random.default_rng(4)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    rows = rng.choice(codes, size=(6, 64)).astype(np.uint8)
    b = np.array([90, 110, 120, 127, 130, 160], dtype=np.uint8)
    f_blk, b_blk = oracle.dequant_rows_block32(rows, np.repeat(b[:, None], 2, axis=1))
    f_row, b_row = oracle.dequant_rows(rows, (2.0 ** (b.astype(np.float64) - 127)).astype(np.float32))
    assert np.array_equal(f_blk.view(np.uint32), f_row.view(np.uint32))
    assert np.array_equal(b_blk, b_row)
