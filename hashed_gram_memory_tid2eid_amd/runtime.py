"""One Engram site on one GPU: the C-ABI calls chained over preallocated
device buffers.

``Engram.forward`` = engram_compress_hash (every site in one pass) -> for each
site engram_gather_dequant -> engram_gated_residual (the projection kernel the
site's wkv handle plans for the call, then the gated add), on one stream, no
host synchronisation, no allocation (path "split", the default).  Path "fused"
(e4m3fn tables) replaces the gather and the projection by engram_gather_project,
which keeps the gathered rows on chip: no [T][k_pad] bf16 row buffer, at a lower
projection rate.

The order follows the pages' forward: one hash pass over the flattened batch
before the layers ([vLLM-V41] "vllm/models/deepseek_v41/nvidia/model",
DeepseekV4Model.forward), then each Engram site writes its gated memory into the
residual streams ahead of its layer ([NeMo-V41]
"nemo_automodel.components.models.deepseek_v41.model", the forward contract).
"""
from __future__ import annotations

from typing import Optional, Sequence

from . import (ENGRAM_DTYPE_BF16, ENGRAM_DTYPE_FP8_E4M3FN, ENGRAM_SCALE_BLOCK32_E8M0,
               ENGRAM_SCALE_ROW_F32, ENGRAM_TABLE_PER_SITE, ENGRAM_TABLES_PER_ORDER, Layout, Wkv,
               engram_compress_hash, engram_gate_add, engram_gated_residual, engram_gather_dequant,
               engram_gather_project, engram_layout_create, engram_lookup_decode, engram_tid2eid_check,
               engram_wkv_gate_add, engram_wkv_project)


def pad_weight(w, layout: Layout):
    """Storage layout of the wkv weight, done once at load time: the logical
    [hidden][3*H*D] bf16 matrix placed in [hidden][k_pad] with each (order, head)
    segment starting at a multiple of seg_pitch and zeros in the gaps (the
    gathered rows carry zeros there too)."""
    import torch
    info = layout.info
    hidden, K = w.shape
    cols = 3 * info.heads
    D, sp = info.row_dim, info.seg_pitch
    if K != cols * D:
        raise ValueError(f"weight has {K} columns, layout wants {cols} x {D}")
    out = torch.zeros((hidden, info.k_pad), dtype=torch.bfloat16, device=w.device)
    out.view(hidden, cols, sp)[:, :, :D].copy_(w.view(hidden, cols, D))
    return out


class Engram:
    """Device state of the Engram sites that share one hash pass: layout,
    compression map, each site's tables, scales and padded weight, and the
    per-call work buffers sized for ``max_tokens`` (rows and v are reused site
    after site).

    One site: ``tables`` / ``scales`` are the site's table list, ``weight`` its
    [hidden][3*H*D] matrix.  Several sites: one such list (and one weight) per
    site, in site order."""

    def __init__(self, *, vocab_size: int, compressed_vocab: int, pad_token_id: int,
                 heads_per_order: int, rows: Sequence[int], row_dim: int, table_dtype: str,
                 row_pitch_bytes: int, tid2eid, tables: Sequence, scales: Optional[Sequence],
                 weight, hidden: int, hc_mult: int = 4, max_tokens: int, hash_floor: int = 0,
                 path: str = "split", num_sites: int = 1, table_split: str = "order",
                 scale_block: int = 0, prefetch_slots: int = 0, proj_splits: int = 0,
                 lookahead: bool = False, stream=None):
        import torch
        if path not in ("split", "fused"):
            raise ValueError(f"unknown path {path!r}")
        if path == "fused" and (table_dtype != "fp8" or (scale_block and row_dim > 256)):
            raise ValueError("the fused path reads e4m3fn tables with a per-row fp32 scale, or "
                             "(1, 32) e8m0 block scales on rows of at most 256 elements")
        if table_split not in ("order", "site"):
            raise ValueError(f"unknown table split {table_split!r}")
        self.path = path
        dt = ENGRAM_DTYPE_FP8_E4M3FN if table_dtype == "fp8" else ENGRAM_DTYPE_BF16
        self.layout = engram_layout_create(
            vocab_size=vocab_size, compressed_vocab=compressed_vocab, pad_token_id=pad_token_id,
            heads_per_order=heads_per_order, rows=list(rows) + [0] * (3 - len(rows)),
            row_dim=row_dim, table_dtype=dt, row_pitch_bytes=row_pitch_bytes, hash_floor=hash_floor,
            num_sites=num_sites,
            table_split=ENGRAM_TABLE_PER_SITE if table_split == "site" else ENGRAM_TABLES_PER_ORDER,
            scale_layout=ENGRAM_SCALE_BLOCK32_E8M0 if scale_block == 32 else ENGRAM_SCALE_ROW_F32)
        info = self.layout.info
        dev = tid2eid.device
        self.num_sites = num_sites
        self.tid2eid = tid2eid
        self.pad_eid = engram_tid2eid_check(self.layout, tid2eid, stream)
        if num_sites == 1:
            tables, scales, weight = [tables], [scales], [weight]
        if len(tables) != num_sites or len(weight) != num_sites or (scales is not None and
                                                                      len(scales) != num_sites):
            raise ValueError("one table list, scale list and weight per site")
        self.site_tables = [list(t) for t in tables]
        self.site_scales = [None if sc is None else list(sc) for sc in
                            (scales if scales is not None else [None] * num_sites)]
        self.site_weights = [pad_weight(w, self.layout) if w.shape[1] != info.k_pad else w
                             for w in weight]
        self.hidden = hidden
        self.hc_mult = hc_mult
        self.max_tokens = max_tokens
        # the split path projects through a wkv handle per site: the library packs the
        # weight when calls can be large, keeps the split-K workspace when they can be
        # small, and picks the kernel per call (proj_splits 0 = its choice)
        self.site_wkv = ([Wkv(self.layout, w, max_tokens, splits=proj_splits, stream=stream)
                          for w in self.site_weights] if path == "split" else [None] * num_sites)
        self.eids = torch.empty(max_tokens, dtype=torch.int32, device=dev)
        rid_shape = ((max_tokens, 3, info.heads) if num_sites == 1
                     else (max_tokens, num_sites, 3, info.heads))
        self.row_ids = torch.empty(rid_shape, dtype=torch.int32, device=dev)
        self.rows = (torch.empty((max_tokens, info.k_pad), dtype=torch.bfloat16, device=dev)
                     if path == "split" else None)
        # look-ahead order (run_ahead): each site's rows wait in a buffer of their own
        # from one call to the next; one site can use the shared buffer
        if lookahead and path != "split":
            raise ValueError("the look-ahead order gathers rows, which the split path alone keeps")
        self.lookahead = lookahead
        self.site_rows = ([self.rows] + [torch.empty_like(self.rows) for _ in range(num_sites - 1)]
                          if lookahead else None)
        self.pending_T = None  # tokens of the call whose rows wait for run_ahead
        self.v = torch.empty((max_tokens, hidden), dtype=torch.float32, device=dev)
        # prefetch ring: slot -> per-site gathered rows, and the event after which the
        # slot's last reader (apply) is done with it
        if prefetch_slots and path != "split":
            raise ValueError("prefetching gathers rows, which the split path alone keeps")
        self.pre_rows = [[torch.empty((max_tokens, info.k_pad), dtype=torch.bfloat16, device=dev)
                          for _ in range(num_sites)] for _ in range(prefetch_slots)]
        self.pre_free = [None] * prefetch_slots
        self.pre_pending = [set() for _ in range(prefetch_slots)]  # sites not yet applied
        self._next_slot = 0

    def make_store(self, num_slots: int, ids=None, stream=None):
        """A rolling store (engram_store_create) for this layout: num_slots slots of pad
        ids, or loaded with ``ids`` (int32 [num_slots][3] on the device)."""
        from . import engram_store_create
        return engram_store_create(self.layout, self.pad_eid, num_slots, ids=ids, stream=stream)

    # single-site views
    @property
    def tables(self):
        return self.site_tables[0]

    @property
    def scales(self):
        return self.site_scales[0]

    @property
    def weight(self):
        return self.site_weights[0]

    @property
    def info(self):
        return self.layout.info

    def hash(self, tokens, cu_seqlens, *, seq_start=None, slots=None, store=None, dead=None,
             stream=None):
        """Compressed ids and every site's row ids of one call, in one pass."""
        engram_compress_hash(self.layout, self.tid2eid, tokens, cu_seqlens, self.eids,
                             self.row_ids, seq_start=seq_start, slots=slots, store=store,
                             dead=dead, stream=stream)

    def site_forward(self, site: int, streams, T: int, *, keep=None, stream=None):
        """Gather, project and gate of one site from the row ids of the last hash."""
        if self.path == "fused":
            engram_gather_project(self.layout, self.site_tables[site], self.site_scales[site],
                                  self.row_ids, self.site_weights[site], self.v, site=site, T=T,
                                  stream=stream)
            engram_gate_add(self.layout, self.v, streams, keep=keep, T=T, stream=stream)
            return streams
        engram_gather_dequant(self.layout, self.site_tables[site], self.site_scales[site],
                              self.row_ids, self.rows, site=site, T=T, stream=stream)
        return self.project_gate(site, self.rows, streams, T, keep=keep, stream=stream)

    def projection_plan(self, site: int, T: int):
        """(kernel, splits) of a T-token projection of `site`: kernel "packed" (256-row
        tiles from the packed weight), "splitk" (few tokens) or "plain", as the
        library's wkv handle plans it."""
        if self.site_wkv[site] is None:
            return "fused", 1
        return self.site_wkv[site].plan(T)

    def projection_kind(self, site: int, T: int) -> str:
        return self.projection_plan(site, T)[0]

    @property
    def proj_splits(self) -> int:
        """Split-K factor of a max_tokens call of site 0."""
        return self.projection_plan(0, self.max_tokens)[1]

    def project(self, site: int, rows, T: int, *, stream=None):
        """First half of engram_gated_residual: v (or, split-K, its partial slices in
        the handle's workspace) of `rows` for `site`."""
        engram_wkv_project(self.layout, rows, self.site_wkv[site], self.v, T=T, stream=stream)

    def gate(self, site: int, streams, T: int, *, keep=None, stream=None):
        """Second half of engram_gated_residual: the gated add of v (split-K: the slices
        summed into v first) into `streams`."""
        engram_wkv_gate_add(self.layout, self.site_wkv[site], self.v, streams, keep=keep, T=T,
                            stream=stream)

    def project_gate(self, site: int, rows, streams, T: int, *, keep=None, stream=None):
        """Projection and gated residual of `site` from gathered `rows`, one C call.
        There is no variant without rows: a site with no looked-up rows is a caller
        error."""
        engram_gated_residual(self.layout, rows, self.site_wkv[site], streams, self.v, keep=keep, T=T,
                              stream=stream)
        return streams

    def forward(self, tokens, cu_seqlens, streams, *, seq_start=None, slots=None, store=None,
                dead=None, keep=None, stream=None):
        """Adds the Engram memory of ``tokens`` into ``streams`` (bf16 [T][hc][hidden],
        in place; with several sites, one such tensor per site, in site order).  With a
        dead mask the caller passes ``keep`` (1 = keep the gate), the complement of
        ``dead``."""
        T = tokens.numel()
        if T > self.max_tokens:
            raise ValueError(f"{T} tokens > max_tokens {self.max_tokens}")
        if dead is not None and keep is None:
            raise ValueError("a dead mask needs the matching keep mask")
        if self.pending_T is not None:
            raise RuntimeError("a gathered call waits for run_ahead; forward would overwrite its rows")
        per_site = [streams] if self.num_sites == 1 else list(streams)
        if len(per_site) != self.num_sites or any(x.shape[0] != T for x in per_site):
            raise ValueError("streams must hold one row per token (one tensor per site)")
        self.hash(tokens, cu_seqlens, seq_start=seq_start, slots=slots, store=store, dead=dead,
                  stream=stream)
        for s in range(self.num_sites):
            self.site_forward(s, per_site[s], T, keep=keep, stream=stream)
        return streams

    @property
    def decode_lookup_supported(self) -> bool:
        """Whether decode_step runs its lookup as one launch (engram_lookup_decode):
        one site, e4m3fn tables with fp32 row scales."""
        return (self.num_sites == 1 and self.layout.desc.table_dtype == ENGRAM_DTYPE_FP8_E4M3FN
                and self.layout.info.scale_layout == ENGRAM_SCALE_ROW_F32 and self.path == "split")

    def decode_step(self, tokens, streams, *, slots=None, store=None, dead=None, keep=None,
                    stream=None):
        """One decode step: token t is sequence t, continuing from store slot slots[t]
        (-1, or no slots: it starts its sequence).  The lookup (compress, hash with the
        store, gather) is one launch, then the projection and gate as in forward.  The
        result equals forward with cu_seqlens 0..T and seq_start 0 where a slot is given."""
        T = tokens.numel()
        if not self.decode_lookup_supported:
            raise ValueError("decode_step needs one site with e4m3fn tables and fp32 row scales")
        if T > self.max_tokens:
            raise ValueError(f"{T} tokens > max_tokens {self.max_tokens}")
        if dead is not None and keep is None:
            raise ValueError("a dead mask needs the matching keep mask")
        if self.pending_T is not None:
            raise RuntimeError("a gathered call waits for run_ahead; decode_step would overwrite its rows")
        if streams.shape[0] != T:
            raise ValueError("streams must hold one row per token")
        engram_lookup_decode(self.layout, self.tid2eid, tokens, self.eids, self.row_ids,
                             self.site_tables[0], self.site_scales[0], self.rows, slots=slots,
                             store=store, dead=dead, stream=stream)
        return self.project_gate(0, self.rows, streams, T, keep=keep, stream=stream)

    # ---- look-ahead order: the next call's lookup between projection and gate -------
    def gather_ahead(self, tokens, cu_seqlens, *, seq_start=None, slots=None, store=None,
                     dead=None, stream=None):
        """Hash and every site's gather of a call, into the look-ahead buffers, with
        no projection: the first call of a look-ahead sequence."""
        self._check_lookahead(tokens)
        if self.pending_T is not None:
            raise RuntimeError("a gathered call already waits for run_ahead; its rows would be overwritten")
        self.hash(tokens, cu_seqlens, seq_start=seq_start, slots=slots, store=store, dead=dead,
                  stream=stream)
        T = tokens.numel()
        for s in range(self.num_sites):
            engram_gather_dequant(self.layout, self.site_tables[s], self.site_scales[s], self.row_ids,
                                  self.site_rows[s], site=s, T=T, stream=stream)
        self.pending_T = T

    def run_ahead(self, streams, *, keep=None, next_tokens=None, next_cu_seqlens=None,
                  next_seq_start=None, next_slots=None, next_store=None, next_dead=None,
                  stream=None):
        """Adds the Engram memory of the call gathered last into ``streams`` (as
        ``forward`` would have), and, when ``next_tokens`` is given, hashes and gathers
        the next call in between, on the same stream: the next call's hash, then per
        site the projection of this call, the gather of the next and the gate of this
        one.  A site's projection has read its rows before the next gather overwrites
        them, and the gate's stream writes drain while the next projection runs,
        instead of under the next gather.  The lookup depends on token ids (and the
        image mask) alone, so it can run a call ahead ([VeOmni#1370] "feat: support
        DeepSeek-V4.1-Flash in SeedOmni", n-gram memory lookup commit: the lookup is
        its own graph node ahead of the backbone).  Every call still runs each kernel
        once; outputs equal sequential ``forward`` calls bit for bit."""
        if self.pending_T is None:
            raise RuntimeError("no gathered call is waiting: call gather_ahead first")
        T = self.pending_T
        per_site = [streams] if self.num_sites == 1 else list(streams)
        if len(per_site) != self.num_sites or any(x.shape[0] != T for x in per_site):
            raise ValueError("streams must hold one row per token of the waiting call (one tensor per site)")
        T_next = None
        if next_tokens is not None:
            self._check_lookahead(next_tokens)
            T_next = next_tokens.numel()
            self.hash(next_tokens, next_cu_seqlens, seq_start=next_seq_start, slots=next_slots,
                      store=next_store, dead=next_dead, stream=stream)
        for s in range(self.num_sites):
            self.project(s, self.site_rows[s], T, stream=stream)
            if T_next is not None:
                engram_gather_dequant(self.layout, self.site_tables[s], self.site_scales[s],
                                      self.row_ids, self.site_rows[s], site=s, T=T_next, stream=stream)
            self.gate(s, per_site[s], T, keep=keep, stream=stream)
        self.pending_T = T_next
        return streams

    def _check_lookahead(self, tokens):
        if not self.lookahead:
            raise ValueError("construct with lookahead=True for the look-ahead order")
        if tokens.numel() > self.max_tokens:
            raise ValueError(f"{tokens.numel()} tokens > max_tokens {self.max_tokens}")

    # ---- prefetch: gather ahead on a stream of its own ------------------------------
    def prefetch(self, tokens, cu_seqlens, *, stream, seq_start=None, slots=None, store=None,
                 dead=None) -> "Prefetched":
        """Hash and every site's gather of one call, enqueued on ``stream`` (the
        prefetch stream) into the next slot of the ring; returns the handle that
        ``apply`` waits on.  The slot is reused only after the apply calls of the
        call that last filled it (their stream's work up to then) are done."""
        import torch
        if not self.pre_rows:
            raise ValueError("construct with prefetch_slots > 0 to prefetch")
        T = tokens.numel()
        if T > self.max_tokens:
            raise ValueError(f"{T} tokens > max_tokens {self.max_tokens}")
        slot = self._next_slot
        if self.pre_pending[slot]:
            raise RuntimeError(f"prefetch slot {slot} still holds a call whose sites "
                               f"{sorted(self.pre_pending[slot])} are not applied; apply it first "
                               f"or construct with more prefetch_slots")
        self._next_slot = (slot + 1) % len(self.pre_rows)
        if self.pre_free[slot] is not None:
            stream.wait_event(self.pre_free[slot])
        self.hash(tokens, cu_seqlens, seq_start=seq_start, slots=slots, store=store, dead=dead,
                  stream=stream)
        for s in range(self.num_sites):
            engram_gather_dequant(self.layout, self.site_tables[s], self.site_scales[s], self.row_ids,
                                  self.pre_rows[slot][s], site=s, T=T, stream=stream)
        ready = torch.cuda.Event()
        ready.record(stream)
        self.pre_free[slot] = None
        self.pre_pending[slot] = set(range(self.num_sites))
        return Prefetched(slot=slot, T=T, ready=ready)

    def apply(self, pre: "Prefetched", site: int, streams, *, keep=None, stream=None):
        """Projection and gate of one site of a prefetched call, on ``stream``
        (default: the current stream), after the prefetch has landed."""
        import torch
        if site not in self.pre_pending[pre.slot]:
            raise RuntimeError(f"site {site} of prefetch slot {pre.slot} is already applied "
                               f"(or the slot was refilled)")
        st = stream if stream is not None else torch.cuda.current_stream()
        st.wait_event(pre.ready)
        self.project_gate(site, self.pre_rows[pre.slot][site], streams, pre.T, keep=keep, stream=st)
        done = torch.cuda.Event()
        done.record(st)
        self.pre_free[pre.slot] = done  # the last site's apply is the slot's last reader
        self.pre_pending[pre.slot].discard(site)
        return streams


class Prefetched:
    """One prefetched call: its ring slot, token count and readiness event."""

    def __init__(self, slot: int, T: int, ready):
        self.slot, self.T, self.ready = slot, T, ready
