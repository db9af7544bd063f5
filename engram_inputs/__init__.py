"""Seeded synthetic inputs for the Engram n-gram memory workloads.

This module serves the HIP path (benchmark, tests) and the oracle alike.  It
holds no step of the method: it only draws token ids, the tid2eid map, document
lengths, decode-store contents, tables, projection weights and residual
streams.  Its shapes and distributions follow the workloads below.

Workloads (tokens per call; tables per order; heads per order; row dim; hidden):
  tiny        1 x 512, uniform ids; 3 x 4,096 rows; H=2; D=128; hidden 256
  prefill     4 x 4,096, Zipf(1.1); 3 x 1,048,576; H=2; D=512; hidden 4,096
  decode      256 slots x 1 token x 64 steps, Zipf(1.1), rolling store of 3 ids
              per slot (uniform random init); prefill's tables and projection
  decode_tiny the same decode loop on tiny's tables and projection
  long        1 x 65,536 Zipf(1.1) split into Geometric(mean 2,048) documents;
              3 x 4,194,304; H=1; D=1,024; hidden 4,096
  full        8 x 8,192 Zipf(1.1); 3 x 5,040,000 (15.12M) rows; H=1; D=6,500
              FP8 e4m3fn plus an fp32 scale per row; hidden 4,096
  full_bf16   full with BF16 tables (no scale)
  v41         the released layout: 2 Engram sites sharing one hash pass, 3 orders
              x 8 heads, D=256, one table per site of 384,006,168 / 384,016,682
              rows (bucket floor 16,000,000), (1, 32) e8m0 block scales;
              8 x 8,192 Zipf(1.1) tokens; hidden 4,096
  v41_small   the same structure at bucket floor 20,000 (~0.49M rows per site);
              4 x 2,048 Zipf(1.1) tokens; hidden 1,024

Table rows are N(0,1) per element, quantised per row to e4m3fn with a
power-of-two fp32 scale 2^ceil(log2(amax/448)) ("amax" mode uses amax/448
itself, a scale that is not a power of two); with (1, 32) block scales each
32-element block gets its own exponent e = ceil(log2(amax_block/448)), stored
as the e8m0 byte e + 127.  W ~ N(0, 0.02) in bf16 with
logical shape [hidden][3*H*D].  Streams ~ N(0,1) in bf16, [T][hc][hidden].
Token ids: uniform, or truncated Zipf over ranks 1..vocab with P(k) ~ k^-s,
drawn by inverse CDF, token = rank - 1.  tid2eid is one random surjection of
the 129,280 token ids onto 65,536 compressed ids (seed 0) for every workload.
The pad token is 129,279 (the rarest Zipf rank).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

VOCAB = 129_280
VC = 65_536
PAD_TOKEN_ID = VOCAB - 1
E4M3_MAX = 448.0


@dataclass(frozen=True)
class EngramConfig:
    name: str
    seed: int
    n_seqs: int
    seq_len: int
    token_dist: str          # "uniform" | "zipf"
    rows: int                # rows per table (one table per order 2,3,4)
    heads: int               # hash heads per order
    row_dim: int             # D
    hidden: int
    hc_mult: int = 4
    table_dtype: str = "fp8"  # "fp8" | "bf16"
    docs_mean: int = 0       # > 0: the token stream is split into geometric documents
    decode_steps: int = 0    # > 0: decode workload (seq_len tokens per slot per step)
    vocab: int = VOCAB
    vc: int = VC
    pad_token_id: int = PAD_TOKEN_ID
    zipf_s: float = 1.1
    w_std: float = 0.02
    n_sites: int = 1          # Engram sites sharing one hash pass
    table_split: str = "order"  # "order": 3 tables per site; "site": 1 table per site
    scale_block: int = 0      # 0: fp32 scale per row; 32: e8m0 exponent per 32 elements
    hash_floor: int = 0       # 0: fit the largest floor the tables hold

    @property
    def tokens_per_call(self) -> int:
        return self.n_seqs * self.seq_len

    @property
    def K(self) -> int:
        """Logical width of the concatenated rows of one token: 3 orders x H heads x D."""
        return 3 * self.heads * self.row_dim

    @property
    def elt_bytes(self) -> int:
        return 1 if self.table_dtype == "fp8" else 2

    @property
    def row_pitch_bytes(self) -> int:
        """Storage pitch of a table row: the row padded to a whole number of 128-byte lines."""
        return -(-self.row_dim * self.elt_bytes // 128) * 128


CONFIGS = {
    "tiny": EngramConfig("tiny", 0, 1, 512, "uniform", 4096, 2, 128, 256),
    "prefill": EngramConfig("prefill", 1, 4, 4096, "zipf", 1_048_576, 2, 512, 4096),
    "decode": EngramConfig("decode", 2, 256, 1, "zipf", 1_048_576, 2, 512, 4096, decode_steps=64),
    "decode_tiny": EngramConfig("decode_tiny", 2, 256, 1, "zipf", 4096, 2, 128, 256,
                                decode_steps=64),
    "long": EngramConfig("long", 3, 1, 65_536, "zipf", 4_194_304, 1, 1024, 4096, docs_mean=2048),
    "full": EngramConfig("full", 4, 8, 8192, "zipf", 5_040_000, 1, 6500, 4096),
    "full_bf16": EngramConfig("full_bf16", 4, 8, 8192, "zipf", 5_040_000, 1, 6500, 4096,
                              table_dtype="bf16"),
    "v41": EngramConfig("v41", 5, 8, 8192, "zipf", 384_016_682, 8, 256, 4096, n_sites=2,
                        table_split="site", scale_block=32, hash_floor=16_000_000),
    "v41_small": EngramConfig("v41_small", 6, 4, 2048, "zipf", 500_000, 8, 256, 1024, n_sites=2,
                              table_split="site", scale_block=32, hash_floor=20_000),
}


def get_config(name: str, **overrides) -> EngramConfig:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


# Sub-stream indices of numpy.random.SeedSequence(seed).spawn(8).
_TOKENS, _DOCS, _STORE, _W, _STREAMS, _TABLES, _DEAD, _SPARE = range(8)


def _streams(seed: int):
    return np.random.SeedSequence(seed).spawn(8)


def _rng(seed: int, which: int) -> np.random.Generator:
    return np.random.default_rng(_streams(seed)[which])


def _torch_seed(seed: int, which: int, extra: int = 0) -> int:
    ss = np.random.SeedSequence([seed, which, extra])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFF_FFFF_FFFF_FFFF)


# ---------------------------------------------------------------------------
# token ids and the compression map
# ---------------------------------------------------------------------------

def make_tid2eid(vocab: int = VOCAB, vc: int = VC, seed: int = 0) -> np.ndarray:
    """A random surjection [0, vocab) -> [0, vc): a random permutation of the token
    ids dealt round-robin onto the compressed ids, so every compressed id is hit."""
    if vocab < vc:
        raise ValueError("a surjection needs vocab >= vc")
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x7D2E]))
    perm = rng.permutation(vocab)
    out = np.empty(vocab, dtype=np.int32)
    out[perm] = np.arange(vocab, dtype=np.int64) % vc
    return out


_zipf_cdf_cache: dict = {}


def _zipf_cdf(vocab: int, s: float) -> np.ndarray:
    key = (vocab, s)
    if key not in _zipf_cdf_cache:
        w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
        c = np.cumsum(w)
        _zipf_cdf_cache[key] = c / c[-1]
    return _zipf_cdf_cache[key]


def zipf_tokens(rng: np.random.Generator, n: int, vocab: int = VOCAB, s: float = 1.1) -> np.ndarray:
    cdf = _zipf_cdf(vocab, s)
    u = rng.random(n)
    rank0 = np.searchsorted(cdf, u, side="right")
    return np.minimum(rank0, vocab - 1).astype(np.int32)


def uniform_tokens(rng: np.random.Generator, n: int, vocab: int = VOCAB) -> np.ndarray:
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def geometric_doc_lengths(rng: np.random.Generator, total: int, mean: int) -> np.ndarray:
    """Document lengths ~ Geometric(1/mean) on {1, 2, ...}; the last one is cut so
    the lengths sum to ``total``."""
    lens = []
    acc = 0
    while acc < total:
        n = int(rng.geometric(1.0 / mean))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return np.asarray(lens, dtype=np.int32)


@dataclass
class Batch:
    """One call's worth of token-side inputs (host arrays)."""
    tokens: np.ndarray                    # int32 [T]
    cu_seqlens: np.ndarray                # int32 [S+1]
    seq_start: Optional[np.ndarray]       # uint8 [S] or None (= every sequence starts here)
    slots: Optional[np.ndarray] = None    # int32 [S] or None
    dead: Optional[np.ndarray] = None     # uint8 [T] or None

    @property
    def T(self) -> int:
        return int(self.tokens.shape[0])

    @property
    def S(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)


def _draw_tokens(cfg: EngramConfig, rng: np.random.Generator, n: int) -> np.ndarray:
    if cfg.token_dist == "uniform":
        return uniform_tokens(rng, n, cfg.vocab)
    if cfg.token_dist == "zipf":
        return zipf_tokens(rng, n, cfg.vocab, cfg.zipf_s)
    raise ValueError(cfg.token_dist)


def make_batch(cfg: EngramConfig) -> Batch:
    """The prefill-style batch of a workload (all sequences start here)."""
    if cfg.decode_steps:
        raise ValueError("decode workloads use make_decode_steps")
    T = cfg.tokens_per_call
    tokens = _draw_tokens(cfg, _rng(cfg.seed, _TOKENS), T)
    if cfg.docs_mean:
        lens = geometric_doc_lengths(_rng(cfg.seed, _DOCS), T, cfg.docs_mean)
    else:
        lens = np.full(cfg.n_seqs, cfg.seq_len, dtype=np.int32)
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    return Batch(tokens=tokens, cu_seqlens=cu, seq_start=np.ones(len(lens), dtype=np.uint8))


def make_decode_steps(cfg: EngramConfig, steps: Optional[int] = None) -> list:
    """``steps`` decode calls: each slot s in [0, n_seqs) gets seq_len new tokens per
    step and continues its stored history (seq_start = 0)."""
    n = cfg.decode_steps if steps is None else steps
    rng = _rng(cfg.seed, _TOKENS)
    out = []
    S, L = cfg.n_seqs, cfg.seq_len
    cu = (np.arange(S + 1, dtype=np.int32) * L).astype(np.int32)
    for _ in range(n):
        out.append(Batch(tokens=_draw_tokens(cfg, rng, S * L), cu_seqlens=cu.copy(),
                         seq_start=np.zeros(S, dtype=np.uint8),
                         slots=np.arange(S, dtype=np.int32)))
    return out


def make_store_init(cfg: EngramConfig, num_slots: Optional[int] = None) -> np.ndarray:
    """Initial rolling store: 3 compressed ids per slot, uniform over [0, vc)."""
    n = cfg.n_seqs if num_slots is None else num_slots
    rng = _rng(cfg.seed, _STORE)
    return rng.integers(0, cfg.vc, size=(n, 3), dtype=np.int64).astype(np.int32)


def make_dead_spans(T: int, seed: int, n_spans: int, max_len: int) -> np.ndarray:
    """Dead (image-span) mask: ``n_spans`` runs of 1..max_len positions."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, _DEAD]))
    dead = np.zeros(T, dtype=np.uint8)
    for _ in range(n_spans):
        if T == 0:
            break
        a = int(rng.integers(0, T))
        ln = int(rng.integers(1, max_len + 1))
        dead[a:a + ln] = 1
    return dead


# ---------------------------------------------------------------------------
# tables, projection weights, streams (torch; on whichever device is asked)
# ---------------------------------------------------------------------------

@dataclass
class Tables:
    """The tables of one site in storage layout: three per-order tables, or one
    table for the site (table_split "site").

    fp8:  data[n] uint8 [rows][pitch] (first D bytes of a row are e4m3fn codes, the
          rest zero), scale[n] float32 [rows], or uint8 [rows][D/32] e8m0 bytes
          with (1, 32) block scales.
    bf16: data[n] uint8 [rows][pitch] holding D little-endian bf16 values, scale None.
    """
    data: list
    scale: Optional[list]
    row_dim: int
    pitch: int
    dtype: str

    def row_view(self, n: int):
        """Logical [rows][D] view of table n (uint8 for fp8, bfloat16 for bf16)."""
        import torch
        d = self.data[n]
        if self.dtype == "fp8":
            return d[:, : self.row_dim]
        return d[:, : 2 * self.row_dim].view(torch.bfloat16)


def make_tables(cfg: EngramConfig, device, scale_mode: str = "pow2",
                rows_per_chunk: Optional[int] = None, site: int = 0) -> Tables:
    """The tables of one site (seeded per site and table)."""
    import torch
    D, R, pitch = cfg.row_dim, cfg.rows, cfg.row_pitch_bytes
    if rows_per_chunk is None:
        rows_per_chunk = max(1, min(R, (1 << 27) // max(D, 1)))
    n_tables = 1 if cfg.table_split == "site" else 3
    gen = torch.Generator(device=device)
    data, scales = [], []
    for n in range(n_tables):
        gen.manual_seed(_torch_seed(cfg.seed, _TABLES, 3 * site + n))
        buf = torch.empty((R, pitch), dtype=torch.uint8, device=device)
        elt = cfg.elt_bytes
        if pitch > D * elt:
            buf[:, D * elt:].zero_()
        sc = None
        if cfg.table_dtype == "fp8":
            sc = (torch.empty((R, D // 32), dtype=torch.uint8, device=device) if cfg.scale_block
                  else torch.empty(R, dtype=torch.float32, device=device))
        for r0 in range(0, R, rows_per_chunk):
            r1 = min(R, r0 + rows_per_chunk)
            x = torch.randn((r1 - r0, D), generator=gen, device=device, dtype=torch.float32)
            if cfg.table_dtype == "bf16":
                buf[r0:r1, : 2 * D].view(torch.bfloat16).copy_(x.to(torch.bfloat16))
                continue
            if cfg.scale_block:
                xb = x.view(r1 - r0, D // 32, 32)
                amax = xb.abs().amax(dim=2).clamp_min(1e-30)
                e = torch.ceil(torch.log2(amax / E4M3_MAX))
                e = torch.where(amax / torch.exp2(e) > E4M3_MAX, e + 1, e).clamp_(-127, 127)
                q = (xb / torch.exp2(e)[:, :, None]).clamp_(-E4M3_MAX, E4M3_MAX)
                buf[r0:r1, :D].copy_(q.reshape(r1 - r0, D).to(torch.float8_e4m3fn).view(torch.uint8))
                sc[r0:r1] = (e + 127).to(torch.uint8)
                del x, xb, q
                continue
            amax = x.abs().amax(dim=1).clamp_min(1e-30)
            if scale_mode == "pow2":
                s = torch.exp2(torch.ceil(torch.log2(amax / E4M3_MAX)))
                s = torch.where(amax / s > E4M3_MAX, s * 2, s)
            elif scale_mode == "amax":
                s = amax / E4M3_MAX
            else:
                raise ValueError(scale_mode)
            q = (x / s[:, None]).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
            buf[r0:r1, :D].copy_(q.view(torch.uint8))
            sc[r0:r1] = s
            del x, q
        data.append(buf)
        scales.append(sc)
    return Tables(data=data, scale=scales if cfg.table_dtype == "fp8" else None, row_dim=D,
                  pitch=pitch, dtype=cfg.table_dtype)


def make_weight(cfg: EngramConfig, device, site: int = 0):
    """Down-projection W of one site, bf16 [hidden][K] (logical, unpadded), N(0, w_std)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(cfg.seed, _W, site))
    w = torch.randn((cfg.hidden, cfg.K), generator=gen, device=device, dtype=torch.float32)
    return (w * cfg.w_std).to(torch.bfloat16)


def make_streams(cfg: EngramConfig, T: int, device, step: int = 0):
    """Residual streams, bf16 [T][hc][hidden], N(0,1); decode steps draw fresh ones."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(cfg.seed, _STREAMS, step))
    out = torch.empty((T, cfg.hc_mult, cfg.hidden), dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    chunk = 1 << 26
    for a in range(0, flat.numel(), chunk):
        b = min(flat.numel(), a + chunk)
        flat[a:b].copy_(torch.randn(b - a, generator=gen, device=device, dtype=torch.float32))
    return out
