"""Shared set-up for the GPU parity tests (not collected by pytest).

`Site` builds one Engram site of a workload on the GPU through the C ABI (via
the Python binding) from the seeded inputs in engram_inputs, and keeps the host
copies the oracle needs.  The oracle side of every comparison is computed here
from the oracle package and those inputs only; nothing the HIP path produced is
fed to the oracle except what the comparison itself reads (row ids are taken
from the oracle, table rows are read from the input tables with torch indexing).

The oracle is single-threaded C; `oracle_project`, `oracle_gate_add` and
`oracle_dequant` cut a comparison into token shards and run the unchanged oracle
call on each shard on host threads side by side (ctypes releases the GIL during
the call), so every token of a workload can be checked in seconds.  Each shard's
result is exactly what one call over all tokens gives: the oracle treats tokens
independently.
"""
from __future__ import annotations

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import engram_inputs as ei
import oracle

DEV = "cuda:0"

REL_TOL = 2e-2
ABS_FLOOR = 1e-3

# host threads for oracle shards: the CPUs this process may use, at most 16
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
_POOL = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        oracle.lib()  # load (and build, if needed) once, before any worker thread
        _POOL = ThreadPoolExecutor(ORACLE_THREADS, thread_name_prefix="oracle")
    return _POOL


def _shards(n: int, parts: int):
    step = max(1, -(-n // parts))
    return [(a, min(n, a + step)) for a in range(0, n, step)]


def oracle_project(E: np.ndarray, W: np.ndarray) -> np.ndarray:
    """oracle.project over token shards on host threads: fp64 [T][hidden]."""
    E = np.ascontiguousarray(E, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    out = np.empty((E.shape[0], W.shape[0]), np.float64)

    def run(ab):
        a, b = ab
        out[a:b] = oracle.project(E[a:b], W)
    list(_pool().map(run, _shards(E.shape[0], ORACLE_THREADS * 4)))
    return out


def oracle_gate_add(x: np.ndarray, v: np.ndarray, keep=None):
    """oracle.gate_add over token shards on host threads: (y bits, gates)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.float64)
    kp = None if keep is None else np.ascontiguousarray(keep, dtype=np.uint8)
    y = np.empty_like(x)
    g = np.empty(x.shape[:2], np.float64)

    def run(ab):
        a, b = ab
        y[a:b], g[a:b] = oracle.gate_add(x[a:b], v[a:b], None if kp is None else kp[a:b])
    list(_pool().map(run, _shards(x.shape[0], ORACLE_THREADS * 4)))
    return y, g


def oracle_dequant(raw: np.ndarray, sc, *, bf16_table: bool = False, block32: bool = False):
    """oracle.dequant_rows (or dequant_rows_block32) over row shards on host threads:
    (f32 [n][D], bf16 bits [n][D])."""
    raw = np.ascontiguousarray(raw)
    n, D = raw.shape
    f32 = np.empty((n, D), np.float32)
    b16 = np.empty((n, D), np.uint16)

    def run(ab):
        a, b = ab
        if block32:
            f32[a:b], b16[a:b] = oracle.dequant_rows_block32(raw[a:b], sc[a:b])
        else:
            f32[a:b], b16[a:b] = oracle.dequant_rows(raw[a:b], None if sc is None else sc[a:b],
                                                     bf16_table=bf16_table)
    list(_pool().map(run, _shards(n, ORACLE_THREADS * 4)))
    return f32, b16


def log(msg: str):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def bf16_bits_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


class Site:
    def __init__(self, cfg: ei.EngramConfig, max_tokens: int, scale_mode: str = "pow2",
                 tables: "ei.Tables | None" = None, proj_splits: int = 0):
        import hashed_gram_memory_tid2eid_amd as eng
        self.eng = eng
        self.cfg = cfg
        t0 = time.time()
        self.tid2eid_h = ei.make_tid2eid(cfg.vocab, cfg.vc)
        self.tid2eid = torch.from_numpy(self.tid2eid_h).to(DEV)
        self.tables = tables if tables is not None else ei.make_tables(cfg, DEV, scale_mode)
        self.weight = ei.make_weight(cfg, DEV)  # logical bf16 [hidden][K]
        self.site = eng.Engram(
            vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
            heads_per_order=cfg.heads, rows=[cfg.rows] * 3, row_dim=cfg.row_dim,
            table_dtype=cfg.table_dtype, row_pitch_bytes=cfg.row_pitch_bytes,
            tid2eid=self.tid2eid, tables=self.tables.data, scales=self.tables.scale,
            weight=self.weight, hidden=cfg.hidden, hc_mult=cfg.hc_mult, max_tokens=max_tokens,
            proj_splits=proj_splits)
        self.olayout = oracle.fit_layout([cfg.rows] * 3, cfg.heads)
        self.pad_eid = int(self.tid2eid_h[cfg.pad_token_id])
        torch.cuda.synchronize()
        log(f"site {cfg.name}: tables + weight ready in {time.time() - t0:.1f}s")

    @property
    def info(self):
        return self.site.layout.info

    # ---- oracle side ----------------------------------------------------------
    def oracle_hash(self, batch: ei.Batch, store: "np.ndarray | None" = None):
        cfg = self.cfg
        return oracle.compress_hash(
            self.olayout, vocab=cfg.vocab, vc=cfg.vc, pad_token_id=cfg.pad_token_id,
            tid2eid=self.tid2eid_h, tokens=batch.tokens, cu_seqlens=batch.cu_seqlens,
            seq_start=batch.seq_start, slots=batch.slots, store=store, dead=batch.dead)

    def fetch_rows(self, row_ids: np.ndarray):
        """Input-table bytes and scales of the given rows (torch indexing on the
        input tensors), shaped [n][3H][D] / [n][3H]."""
        n = row_ids.shape[0]
        H, D = self.cfg.heads, self.cfg.row_dim
        is_bf16 = self.cfg.table_dtype == "bf16"
        raw = np.zeros((n, 3 * H, D), dtype=np.uint16 if is_bf16 else np.uint8)
        sc = None if is_bf16 else np.zeros((n, 3 * H), dtype=np.float32)
        for o in range(3):
            view = self.tables.row_view(o)
            for h in range(H):
                idx = torch.from_numpy(row_ids[:, o, h].astype(np.int64)).to(DEV)
                r = view.index_select(0, idx)
                if is_bf16:
                    raw[:, o * H + h] = r.view(torch.int16).cpu().numpy().view(np.uint16)
                else:
                    raw[:, o * H + h] = r.cpu().numpy()
                    sc[:, o * H + h] = self.tables.scale[o].index_select(0, idx).cpu().numpy()
        return raw, sc

    def oracle_dequant(self, row_ids: np.ndarray):
        """(f32 [n][3H][D], bf16 bits [n][3H][D]) for the given row ids."""
        raw, sc = self.fetch_rows(row_ids)
        n, C, D = raw.shape
        f32, b16 = oracle_dequant(raw.reshape(n * C, D), None if sc is None else sc.reshape(-1),
                                  bf16_table=self.cfg.table_dtype == "bf16")
        return f32.reshape(n, C, D), b16.reshape(n, C, D)

    def weight_bits(self) -> np.ndarray:
        return bf16_bits_np(self.weight)

    # ---- product side ----------------------------------------------------------
    def device_batch(self, batch: ei.Batch):
        def d(a):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        return dict(tokens=d(batch.tokens), cu_seqlens=d(batch.cu_seqlens), seq_start=d(batch.seq_start),
                    slots=d(batch.slots), dead=d(batch.dead),
                    keep=None if batch.dead is None else d((batch.dead == 0).astype(np.uint8)))

    def unpad(self, rows_dev: torch.Tensor, T: int) -> torch.Tensor:
        """[T][k_pad] -> [T][3H][seg_pitch]"""
        info = self.info
        return rows_dev[:T].view(T, 3 * info.heads, info.seg_pitch)


def assert_streams_close(y: np.ndarray, y_ref: np.ndarray, what: str):
    """|y - y_ref| / max(|y_ref|, 1e-3) <= 2e-2 element-wise (bf16 bits in), checked
    in token chunks to bound host memory."""
    worst = 0.0
    for a0 in range(0, max(1, y.shape[0]), 1024):
        a = bits_to_f64(y[a0:a0 + 1024])
        b = bits_to_f64(y_ref[a0:a0 + 1024])
        assert np.all(np.isfinite(a)), f"{what}: non-finite output"
        err = np.abs(a - b) / np.maximum(np.abs(b), ABS_FLOOR)
        if err.size:
            worst = max(worst, float(err.max()))
    assert worst <= REL_TOL, f"{what}: max relative error {worst:.3e} > {REL_TOL}"
    return worst


def assert_v_close(v: np.ndarray, v_ref: np.ndarray, E_bits: np.ndarray, W_bits: np.ndarray, what: str):
    """fp32 accumulation of K products: |v - v_ref| <= K * 2^-24 * sum_k |E_k W_k| (+ tiny),
    checked in token chunks.  Returns the largest relative error."""
    K = E_bits.shape[1]
    Wa = np.abs(bits_to_f64(W_bits)).T
    ratio, rel = 0.0, 0.0
    for a0 in range(0, max(1, v.shape[0]), 2048):
        absdot = np.abs(bits_to_f64(E_bits[a0:a0 + 2048])) @ Wa
        bound = K * 2.0 ** -24 * absdot + 1e-30
        r = v_ref[a0:a0 + 2048]
        err = np.abs(v[a0:a0 + 2048].astype(np.float64) - r)
        if err.size:
            ratio = max(ratio, float((err / bound).max()))
            rel = max(rel, float((err / np.maximum(np.abs(r), 1e-6)).max()))
    assert ratio <= 1.0, f"{what}: projection error exceeds the fp32 bound ({ratio:.3f})"
    return rel


def sample_tokens(batch: ei.Batch, n, seed: int) -> np.ndarray:
    """Seeded sample of token positions that includes the first three tokens and the
    last token of every sequence; n None = every token."""
    T = batch.T
    if n is None:
        return np.arange(T, dtype=np.int64)
    must = set()
    cu = batch.cu_seqlens
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for t in range(a, min(a + 3, b)):
            must.add(t)
        if b > a:
            must.add(b - 1)
    rng = np.random.default_rng(seed)
    extra = rng.choice(T, size=min(T, max(0, n - len(must))), replace=False) if T else []
    return np.array(sorted(must | {int(x) for x in extra}), dtype=np.int64)
