"""MI355X (gfx950) Engram n-gram memory hot path: Python binding of libengram.so.

The functions below carry the names of the C ABI in ``include/engram.h`` and do
argument marshalling only: torch tensors provide device memory and the HIP
stream; every step of the path runs in the library's kernels.  Importing this
package fails loudly if the library has not been built (there is no fallback).
Build it with ``python hashed_gram_memory_tid2eid_amd/build_lib.py``.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libengram.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "engram.h")

ENGRAM_DTYPE_FP8_E4M3FN = 1
ENGRAM_DTYPE_BF16 = 2
ENGRAM_DTYPE_F32 = 3
ENGRAM_MAX_HEADS = 8
ENGRAM_MAX_SITES = 4
ENGRAM_TABLES_PER_ORDER = 0
ENGRAM_TABLE_PER_SITE = 1
ENGRAM_SCALE_ROW_F32 = 0
ENGRAM_SCALE_BLOCK32_E8M0 = 32
_MAX_COLUMNS = ENGRAM_MAX_SITES * 3 * ENGRAM_MAX_HEADS


def _status_codes():
    codes = {}
    with open(HEADER_PATH) as f:
        for m in re.finditer(r"#define\s+(ENGRAM_(?:OK|E_\w+))\s+\(?(-?\d+)\)?", f.read()):
            codes[m.group(1)] = int(m.group(2))
    return codes


STATUS = _status_codes()
globals().update(STATUS)


class EngramError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: {engram_strerror(status)} (status {status})"
        if status == STATUS.get("ENGRAM_E_HIP"):
            msg += f" [{_lib.engram_last_hip_error().decode()}]"
        super().__init__(msg)
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python hashed_gram_memory_tid2eid_amd/build_lib.py`")

# torch ships its own HIP runtime (libamdhip64.so, soname libamdhip64.so.7).  The
# library must bind to that same runtime, or torch's streams and the library's
# launches live in two runtimes that know nothing of each other.  Loading torch
# first makes the dynamic loader resolve the library's libamdhip64.so.7 to the
# copy already in the process.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


if len(_hip_runtimes_mapped()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process "
                      f"({_hip_runtimes_mapped()}); import torch before anything that loads "
                      "/opt/rocm's libamdhip64")
_P = ctypes.c_void_p
_i32, _i64 = ctypes.c_int32, ctypes.c_int64


class engram_layout_desc(ctypes.Structure):
    _fields_ = [
        ("vocab_size", _i64), ("compressed_vocab", _i64), ("pad_token_id", _i64),
        ("max_ngram", _i32), ("heads_per_order", _i32), ("rows", _i64 * 3), ("hash_floor", _i64),
        ("row_dim", _i32), ("table_dtype", _i32), ("row_pitch_bytes", _i64),
        ("num_sites", _i32), ("table_split", _i32), ("scale_layout", _i32), ("reserved", _i32),
    ]


class engram_layout_info(ctypes.Structure):
    _fields_ = [
        ("hash_floor", _i64), ("heads_per_order", _i32), ("row_dim", _i32), ("rows", _i64 * 3),
        ("primes", _i64 * _MAX_COLUMNS), ("offsets", _i64 * _MAX_COLUMNS),
        ("prime_sum", _i64 * (3 * ENGRAM_MAX_SITES)), ("seg_pitch", _i64), ("k_pad", _i64),
        ("num_sites", _i32), ("table_split", _i32), ("scale_layout", _i32), ("reserved", _i32),
    ]


def _sig(name, args, res=ctypes.c_int):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_sig("engram_layout_create", [ctypes.POINTER(engram_layout_desc), ctypes.POINTER(_P)])
_sig("engram_layout_destroy", [_P], None)
_sig("engram_layout_query", [_P, ctypes.POINTER(engram_layout_info)])
_sig("engram_tid2eid_check", [_P, _P, ctypes.POINTER(_i32), _P])
_sig("engram_store_create", [_P, _i32, _i32, _P, ctypes.POINTER(_P)])
_sig("engram_store_destroy", [_P], None)
_sig("engram_store_query", [_P, ctypes.POINTER(_i32), ctypes.POINTER(_i32)])
_sig("engram_store_reset", [_P, _P, _i32, _P])
_sig("engram_store_write", [_P, _P, _i32, _P, _P])
_sig("engram_store_read", [_P, _P, _i32, _P, _P])
_sig("engram_store_rollback", [_P, _P, _P, _P, _i32, _P, _i32, _P, _P, _P, _P, _P, _P])
_sig("engram_compress_hash", [_P, _P, _P, _i32, _P, _i32, _P, _P, _P, _P, _P, _P, _P])
_sig("engram_gather_dequant", [_P, ctypes.POINTER(_P), ctypes.POINTER(_P), _P, _i32, _i32, _i32, _P, _i64, _P])
_sig("engram_lookup_decode", [_P, _P, _P, _i32, _P, _P, _P, _P, _P, ctypes.POINTER(_P), ctypes.POINTER(_P),
                              _P, _i64, _P])
_sig("engram_project", [_P, _P, _i64, _P, _i64, _i32, _P, _i32, _P])
_sig("engram_gather_project", [_P, ctypes.POINTER(_P), ctypes.POINTER(_P), _P, _i32, _i32, _P, _i64, _i32, _P, _P])
_sig("engram_gate_add", [_P, _P, _i32, _i32, _P, _P, _i32, _P])
_sig("engram_packed_weight_bytes", [_P, _i32, ctypes.POINTER(_i64)])
_sig("engram_pack_weight", [_P, _P, _i64, _i32, _P, _P])
_sig("engram_project_packed", [_P, _P, _i64, _P, _i32, _P, _i32, _P])
_sig("engram_project_splitk", [_P, _P, _i64, _P, _i64, _i32, _P, _i32, _i32, _P])
_sig("engram_gate_add_partials", [_P, _P, _i32, _i32, _i32, _P, _P, _P, _i32, _P])
_sig("engram_projection_plan", [_P, _i32, _i32, _i32, _i32, _P])
_sig("engram_wkv_create", [_P, _P, _i64, _i32, _i32, _i32, _P, ctypes.POINTER(_P)])
_sig("engram_wkv_destroy", [_P], None)
_sig("engram_wkv_plan", [_P, _i32, _P])
_sig("engram_wkv_project", [_P, _P, _i64, _P, _P, _i32, _P])
_sig("engram_wkv_gate_add", [_P, _P, _P, _i32, _P, _P, _i32, _P])
_sig("engram_gated_residual", [_P, _P, _i64, _P, _i32, _P, _P, _P, _i32, _P])
_sig("engram_gated_residual_noalloc", [_P, _P, _i64, _P, _i32, _P, _P, _i32, _P])
_sig("engram_strerror", [ctypes.c_int], ctypes.c_char_p)
_sig("engram_host_device_pointer", [_P, ctypes.POINTER(_P)])
_sig("engram_get_error", [_P])
_sig("engram_last_hip_error", [], ctypes.c_char_p)
_sig("engram_build_id", [], ctypes.c_char_p)


def engram_build_id() -> str:
    """'engram-src-sha256:<16 hex>' of the sources the loaded library was built from."""
    return _lib.engram_build_id().decode()


def engram_strerror(status: int) -> str:
    return _lib.engram_strerror(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise EngramError(status, where)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _need(cond: bool, what: str):
    if not cond:
        raise ValueError(what)


def _dev(t, dtype=None, name="tensor", host_ok=False):
    """Device pointer of a contiguous CUDA tensor (or None).  With host_ok, a pinned
    host tensor is accepted too and its device-side address is returned (tables
    kept in host memory are read by the kernels over the host link)."""
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.is_cuda:
        return t.data_ptr()
    if host_ok and t.is_pinned():
        dp = _P()
        _check(_lib.engram_host_device_pointer(_P(t.data_ptr()), ctypes.byref(dp)),
               f"{name}: device address of pinned host memory")
        return dp.value
    raise TypeError(f"{name} must be a device tensor" + (" or pinned host tensor" if host_ok else ""))


# ---------------------------------------------------------------------------
# layout
# ---------------------------------------------------------------------------

@dataclass
class LayoutInfo:
    hash_floor: int
    heads: int
    row_dim: int
    rows: tuple
    primes: list      # [3][H] of site 0
    offsets: list     # [3][H] of site 0
    prime_sum: tuple  # [3] of site 0
    seg_pitch: int
    k_pad: int
    num_sites: int = 1
    table_split: int = 0
    scale_layout: int = 0
    site_primes: list = None      # [site][3][H]
    site_offsets: list = None     # [site][3][H]
    site_prime_sum: list = None   # [site][3]

    @property
    def cols(self) -> int:
        return 3 * self.heads

    def site_rows(self, site: int) -> int:
        """Buckets of one site: the rows its table (one per site) must hold."""
        return int(sum(self.site_prime_sum[site]))


class Layout:
    """Owner of an ``engram_layout*`` handle."""

    def __init__(self, handle: int, desc: engram_layout_desc):
        self.handle = handle
        self.desc = desc
        self.info = engram_layout_query(self)

    # the destroy function is bound when the class is made: at interpreter exit the
    # module's globals may already be gone when the last Layout is collected
    def __del__(self, _destroy=_lib.engram_layout_destroy):
        h, self.handle = getattr(self, "handle", None), None
        if h:
            _destroy(h)

    @property
    def _as_parameter_(self):
        return self.handle


def engram_layout_create(*, vocab_size: int, compressed_vocab: int, pad_token_id: int,
                         heads_per_order: int, rows: Sequence[int], row_dim: int,
                         table_dtype: int, row_pitch_bytes: int, hash_floor: int = 0,
                         max_ngram: int = 4, num_sites: int = 1,
                         table_split: int = ENGRAM_TABLES_PER_ORDER,
                         scale_layout: int = ENGRAM_SCALE_ROW_F32) -> Layout:
    d = engram_layout_desc()
    d.vocab_size, d.compressed_vocab, d.pad_token_id = vocab_size, compressed_vocab, pad_token_id
    d.max_ngram, d.heads_per_order = max_ngram, heads_per_order
    for i in range(3):
        d.rows[i] = int(rows[i])
    d.hash_floor, d.row_dim, d.table_dtype, d.row_pitch_bytes = hash_floor, row_dim, table_dtype, row_pitch_bytes
    d.num_sites, d.table_split, d.scale_layout = num_sites, table_split, scale_layout
    h = _P()
    _check(_lib.engram_layout_create(ctypes.byref(d), ctypes.byref(h)), "engram_layout_create")
    return Layout(h.value, d)


def engram_layout_query(layout: Layout) -> LayoutInfo:
    info = engram_layout_info()
    _check(_lib.engram_layout_query(layout.handle, ctypes.byref(info)), "engram_layout_query")
    H = info.heads_per_order
    S = info.num_sites
    sp = [[[info.primes[(s * 3 + n) * H + h] for h in range(H)] for n in range(3)] for s in range(S)]
    so = [[[info.offsets[(s * 3 + n) * H + h] for h in range(H)] for n in range(3)] for s in range(S)]
    ss = [[info.prime_sum[s * 3 + n] for n in range(3)] for s in range(S)]
    return LayoutInfo(
        hash_floor=info.hash_floor, heads=H, row_dim=info.row_dim, rows=tuple(info.rows),
        primes=sp[0], offsets=so[0], prime_sum=tuple(ss[0]), seg_pitch=info.seg_pitch,
        k_pad=info.k_pad, num_sites=S, table_split=info.table_split,
        scale_layout=info.scale_layout, site_primes=sp, site_offsets=so, site_prime_sum=ss)


def engram_tid2eid_check(layout: Layout, tid2eid, stream=None) -> int:
    import torch
    pad = _i32()
    _need(tid2eid.numel() == layout.desc.vocab_size, "tid2eid must hold vocab_size entries")
    _check(_lib.engram_tid2eid_check(layout.handle, _dev(tid2eid, torch.int32, "tid2eid"),
                                     ctypes.byref(pad), _stream(stream)), "engram_tid2eid_check")
    return pad.value


# ---------------------------------------------------------------------------
# store
# ---------------------------------------------------------------------------

class Store:
    """Owner of an ``engram_store*`` handle: the slot-keyed rolling store of the last
    three compressed ids per sequence, library-owned device memory bound to the
    layout it was made for."""

    def __init__(self, layout: Layout, pad_eid: int, num_slots: int, stream=None):
        h = _P()
        _check(_lib.engram_store_create(layout.handle, int(pad_eid), int(num_slots), _stream(stream),
                                        ctypes.byref(h)), "engram_store_create")
        self.handle = h.value
        self.layout = layout  # keeps the layout alive while the store is
        self.num_slots = int(num_slots)
        self.pad_eid = int(pad_eid)

    def __del__(self, _destroy=_lib.engram_store_destroy):
        h, self.handle = getattr(self, "handle", None), None
        if h:
            _destroy(h)

    @property
    def _as_parameter_(self):
        return self.handle

    def ids(self, stream=None):
        """A device int32 [num_slots][3] copy of every slot (engram_store_read)."""
        import torch
        out = torch.empty((self.num_slots, 3), dtype=torch.int32, device="cuda")
        engram_store_read(self, None, out, stream=stream)
        return out

    def load(self, ids, stream=None):
        """Every slot <- ids (int32 [num_slots][3], device), by engram_store_write."""
        _need(ids.numel() == 3 * self.num_slots, "ids must be [num_slots][3]")
        engram_store_write(self, None, ids, stream=stream)
        return self


def engram_store_create(layout: Layout, pad_eid: int, num_slots: int, *, ids=None, stream=None) -> Store:
    """A store of num_slots slots, all pad ids; with ``ids`` (int32 [num_slots][3] on
    the device) the slots are then loaded with them."""
    st = Store(layout, pad_eid, num_slots, stream=stream)
    if ids is not None:
        st.load(ids, stream=stream)
    return st


def _slots_arg(slots):
    import torch
    if slots is None:
        return None, 0
    return _dev(slots, torch.int32, "slots"), slots.numel()


def engram_store_reset(store: Store, slots=None, stream=None):
    sp, n = _slots_arg(slots)
    _check(_lib.engram_store_reset(store.handle, sp, n, _stream(stream)), "engram_store_reset")


def engram_store_write(store: Store, slots, ids, stream=None):
    """store[slots[i]] <- ids[i]; slots None = every slot in order."""
    import torch
    sp, n = _slots_arg(slots)
    _need(ids.numel() >= 3 * (n if slots is not None else store.num_slots), "ids must be [n][3]")
    _check(_lib.engram_store_write(store.handle, sp, n, _dev(ids, torch.int32, "ids"), _stream(stream)),
           "engram_store_write")


def engram_store_read(store: Store, slots, ids, stream=None):
    """ids[i] <- store[slots[i]]; slots None = every slot in order."""
    import torch
    sp, n = _slots_arg(slots)
    _need(ids.numel() >= 3 * (n if slots is not None else store.num_slots), "ids must be [n][3]")
    _check(_lib.engram_store_read(store.handle, sp, n, _dev(ids, torch.int32, "ids"), _stream(stream)),
           "engram_store_read")


# ---------------------------------------------------------------------------
# the three hot calls
# ---------------------------------------------------------------------------

def engram_store_rollback(layout: Layout, tid2eid, store, slots, cu_seqlens, eids, keep_len, *,
                          snapshot=None, seq_start=None, dead=None, stream=None):
    """Roll the slots of a verify call back to the first keep_len[s] tokens of
    each sequence (see include/engram.h)."""
    import torch
    S = slots.numel()
    T = eids.numel()
    _need(cu_seqlens.numel() == S + 1 and keep_len.numel() == S, "cu_seqlens / keep_len size")
    _need(isinstance(store, Store), "store must be a Store")
    if snapshot is not None:
        _need(snapshot.numel() >= 3 * S, "snapshot must be [S][3]")
    if seq_start is not None:
        _need(seq_start.numel() == S, "seq_start must be [S]")
    if dead is not None:
        _need(dead.numel() >= T, "dead must cover the call's tokens")
    _check(_lib.engram_store_rollback(
        layout.handle, _dev(tid2eid, torch.int32, "tid2eid"), store.handle,
        _dev(slots, torch.int32, "slots"), S, _dev(cu_seqlens, torch.int32, "cu_seqlens"),
        T, _dev(eids, torch.int32, "eids"), None if dead is None else _dev(dead, torch.uint8, "dead"),
        None if seq_start is None else _dev(seq_start, torch.uint8, "seq_start"),
        None if snapshot is None else _dev(snapshot, torch.int32, "snapshot"),
        _dev(keep_len, torch.int32, "keep_len"), _stream(stream)), "engram_store_rollback")


def engram_compress_hash(layout: Layout, tid2eid, tokens, cu_seqlens, eids, row_ids, *,
                         seq_start=None, slots=None, store=None, dead=None, stream=None):
    import torch
    T = tokens.numel()
    S = cu_seqlens.numel() - 1
    info = layout.info
    _need(eids.numel() >= T and row_ids.numel() >= T * info.num_sites * info.cols,
          "eids / row_ids too small")
    _need(tid2eid.numel() == layout.desc.vocab_size, "tid2eid must hold vocab_size entries")
    _need(seq_start is None or seq_start.numel() >= S, "seq_start too small")
    _need(slots is None or slots.numel() >= S, "slots too small")
    _need(dead is None or dead.numel() >= T, "dead too small")
    _need(store is None or isinstance(store, Store), "store must be a Store (engram_store_create)")
    _check(_lib.engram_compress_hash(
        layout.handle, _dev(tid2eid, torch.int32, "tid2eid"), _dev(tokens, torch.int32, "tokens"), T,
        _dev(cu_seqlens, torch.int32, "cu_seqlens"), S, _dev(seq_start, torch.uint8, "seq_start"),
        _dev(slots, torch.int32, "slots"), None if store is None else store.handle,
        _dev(dead, torch.uint8, "dead"),
        _dev(eids, torch.int32, "eids"), _dev(row_ids, torch.int32, "row_ids"), _stream(stream)),
        "engram_compress_hash")


def _site_pointers(layout: Layout, tables: Sequence, scales: Optional[Sequence]):
    """ctypes arrays of the tables (and scales) one gather reads, after checking
    their sizes against the layout."""
    import torch
    info = layout.info
    per_site = info.table_split == ENGRAM_TABLE_PER_SITE
    used = 1 if per_site else 3
    _need(len(tables) >= used, f"{used} table(s) expected")
    pitch = layout.desc.row_pitch_bytes
    for n in range(used):
        _need(tables[n].numel() >= info.rows[n] * pitch, f"table {n} smaller than rows x pitch")
    tp = (_P * 3)(*[_dev(tables[min(n, used - 1)], torch.uint8, "table", host_ok=True) for n in range(3)])
    if scales is None:
        return tp, None
    _need(len(scales) >= used, f"{used} scale tensor(s) expected")
    sp = []
    for n in range(3):
        sc = scales[min(n, used - 1)]
        if info.scale_layout == ENGRAM_SCALE_BLOCK32_E8M0:
            _need(sc.numel() >= info.rows[min(n, used - 1)] * (info.row_dim // 32),
                  "e8m0 scales must be [rows][D/32]")
            sp.append(_dev(sc, torch.uint8, "scale", host_ok=True))
        else:
            _need(sc.numel() >= info.rows[min(n, used - 1)], "scales smaller than rows")
            sp.append(_dev(sc, torch.float32, "scale", host_ok=True))
    return tp, (_P * 3)(*sp)


def engram_gather_dequant(layout: Layout, tables: Sequence, scales: Optional[Sequence], row_ids,
                          out, *, site: int = 0, T: Optional[int] = None, stream=None):
    import torch
    if T is None:
        T = row_ids.shape[0]
    info = layout.info
    _need(0 <= site < info.num_sites, "site out of range")
    _need(row_ids.numel() >= T * info.num_sites * info.cols, "row_ids too small")
    _need(out.dim() == 2 and out.shape[0] >= T and out.shape[1] >= info.k_pad, "out too small")
    tp, sp = _site_pointers(layout, tables, scales)
    if out.dtype == torch.bfloat16:
        odt = ENGRAM_DTYPE_BF16
    elif out.dtype == torch.float32:
        odt = ENGRAM_DTYPE_F32
    else:
        raise TypeError("out must be bfloat16 or float32")
    _check(_lib.engram_gather_dequant(layout.handle, tp, sp, _dev(row_ids, torch.int32, "row_ids"), site,
                                      T, odt, _dev(out, None, "out"), out.shape[1], _stream(stream)),
           "engram_gather_dequant")


def engram_lookup_decode(layout: Layout, tid2eid, tokens, eids, row_ids, tables: Sequence,
                         scales: Sequence, rows, *, slots=None, store=None, dead=None, stream=None):
    """One decode step's compress + hash + gather (one token per sequence, token t in
    slot slots[t], -1 or no slots: it starts its sequence) into eids, row_ids, the
    store and the bf16 rows [T][>= k_pad]."""
    import torch
    T = tokens.numel()
    info = layout.info
    _need(eids.numel() >= T and row_ids.numel() >= T * info.num_sites * info.cols,
          "eids / row_ids too small")
    _need(tid2eid.numel() == layout.desc.vocab_size, "tid2eid must hold vocab_size entries")
    _need(slots is None or slots.numel() >= T, "slots too small")
    _need(dead is None or dead.numel() >= T, "dead too small")
    _need(store is None or isinstance(store, Store), "store must be a Store (engram_store_create)")
    _need(rows.dim() == 2 and rows.shape[0] >= T and rows.shape[1] >= info.k_pad, "rows too small")
    _need(rows.dtype == torch.bfloat16, "rows must be bfloat16")
    tp, sp = _site_pointers(layout, tables, scales)
    _check(_lib.engram_lookup_decode(
        layout.handle, _dev(tid2eid, torch.int32, "tid2eid"), _dev(tokens, torch.int32, "tokens"), T,
        _dev(slots, torch.int32, "slots"), None if store is None else store.handle,
        _dev(dead, torch.uint8, "dead"), _dev(eids, torch.int32, "eids"),
        _dev(row_ids, torch.int32, "row_ids"), tp, sp, _dev(rows, None, "rows"), rows.shape[1],
        _stream(stream)), "engram_lookup_decode")


def engram_project(layout: Layout, rows, w, v, *, T: Optional[int] = None, stream=None):
    import torch
    if T is None:
        T = rows.shape[0]
    _need(rows.dim() == 2 and rows.shape[0] >= T, "rows too small")
    _need(w.dim() == 2 and v.dim() == 2 and v.shape[0] >= T and v.shape[1] == w.shape[0],
          "v must be [T][hidden]")
    _check(_lib.engram_project(layout.handle, _dev(rows, torch.bfloat16, "rows"), rows.shape[1],
                               _dev(w, torch.bfloat16, "w"), w.shape[1], w.shape[0],
                               _dev(v, torch.float32, "v"), T, _stream(stream)), "engram_project")


def engram_packed_weight_bytes(layout: Layout, hidden: int) -> int:
    n = _i64(0)
    _check(_lib.engram_packed_weight_bytes(layout.handle, int(hidden), ctypes.byref(n)),
           "engram_packed_weight_bytes")
    return int(n.value)


def engram_pack_weight(layout: Layout, w, packed, stream=None):
    """packed: a device tensor of at least engram_packed_weight_bytes(layout, hidden) bytes."""
    import torch
    _need(w.dim() == 2, "w must be [hidden][w_ld]")
    need = engram_packed_weight_bytes(layout, w.shape[0])
    _need(packed.numel() * packed.element_size() >= need, f"packed smaller than {need} bytes")
    _check(_lib.engram_pack_weight(layout.handle, _dev(w, torch.bfloat16, "w"), w.shape[1], w.shape[0],
                                   _dev(packed, None, "packed"), _stream(stream)), "engram_pack_weight")


def engram_project_packed(layout: Layout, rows, packed, hidden: int, v, *, T: Optional[int] = None,
                          stream=None):
    import torch
    if T is None:
        T = rows.shape[0]
    _need(rows.dim() == 2 and rows.shape[0] >= T, "rows too small")
    _need(v.dim() == 2 and v.shape[0] >= T and v.shape[1] == hidden, "v must be [T][hidden]")
    need = engram_packed_weight_bytes(layout, hidden)
    _need(packed.numel() * packed.element_size() >= need, f"packed smaller than {need} bytes")
    _check(_lib.engram_project_packed(layout.handle, _dev(rows, torch.bfloat16, "rows"), rows.shape[1],
                                      _dev(packed, None, "packed"), int(hidden),
                                      _dev(v, torch.float32, "v"), T, _stream(stream)),
           "engram_project_packed")


def engram_gather_project(layout: Layout, tables: Sequence, scales: Sequence, row_ids, w, v, *,
                          site: int = 0, T: Optional[int] = None, stream=None):
    import torch
    if T is None:
        T = row_ids.shape[0]
    info = layout.info
    _need(0 <= site < info.num_sites, "site out of range")
    _need(row_ids.numel() >= T * info.num_sites * info.cols, "row_ids too small")
    _need(w.dim() == 2 and v.dim() == 2 and v.shape[0] >= T and v.shape[1] == w.shape[0],
          "v must be [T][hidden]")
    tp, sp = _site_pointers(layout, tables, scales)
    _check(_lib.engram_gather_project(layout.handle, tp, sp, _dev(row_ids, torch.int32, "row_ids"), site,
                                      T, _dev(w, torch.bfloat16, "w"), w.shape[1], w.shape[0],
                                      _dev(v, torch.float32, "v"), _stream(stream)),
           "engram_gather_project")


def engram_project_splitk(layout: Layout, rows, w, partials, splits: int, *, T: Optional[int] = None,
                          stream=None):
    """partials: float [splits][>=T][hidden] workspace (slice s at offset s*T*hidden)."""
    import torch
    if T is None:
        T = rows.shape[0]
    hidden = w.shape[0]
    _need(rows.dim() == 2 and rows.shape[0] >= T, "rows too small")
    _need(partials.numel() >= splits * T * hidden, "partials smaller than splits x T x hidden")
    _check(_lib.engram_project_splitk(layout.handle, _dev(rows, torch.bfloat16, "rows"), rows.shape[1],
                                      _dev(w, torch.bfloat16, "w"), w.shape[1], hidden,
                                      _dev(partials, torch.float32, "partials"), splits, T,
                                      _stream(stream)), "engram_project_splitk")


def engram_gate_add_partials(layout: Layout, partials, splits: int, streams, *, keep=None, v=None,
                             T: Optional[int] = None, stream=None):
    import torch
    if T is None:
        T = streams.shape[0]
    hidden = streams.shape[2]
    _need(streams.dim() == 3 and streams.shape[0] >= T, "streams must be [T][hc][hidden]")
    _need(partials.numel() >= splits * T * hidden, "partials smaller than splits x T x hidden")
    _need(v is None or (v.dim() == 2 and v.shape[0] >= T and v.shape[1] == hidden), "v must be [T][hidden]")
    _need(keep is None or keep.numel() >= T, "keep too small")
    _check(_lib.engram_gate_add_partials(layout.handle, _dev(partials, torch.float32, "partials"), splits,
                                         hidden, streams.shape[1], _dev(keep, torch.uint8, "keep"),
                                         _dev(streams, torch.bfloat16, "streams"),
                                         _dev(v, torch.float32, "v"), T, _stream(stream)),
           "engram_gate_add_partials")


def engram_gate_add(layout: Layout, v, streams, *, keep=None, T: Optional[int] = None, stream=None):
    import torch
    if T is None:
        T = streams.shape[0]
    _need(streams.dim() == 3 and streams.shape[0] >= T, "streams must be [T][hc][hidden]")
    _need(v.dim() == 2 and v.shape[0] >= T and v.shape[1] == streams.shape[2], "v must be [T][hidden]")
    _need(keep is None or keep.numel() >= T, "keep too small")
    _check(_lib.engram_gate_add(layout.handle, _dev(v, torch.float32, "v"), streams.shape[2],
                                streams.shape[1], _dev(keep, torch.uint8, "keep"),
                                _dev(streams, torch.bfloat16, "streams"), T, _stream(stream)),
           "engram_gate_add")


class engram_proj_plan(ctypes.Structure):
    _fields_ = [("kernel", _i32), ("splits", _i32)]


ENGRAM_PROJ_PLAIN, ENGRAM_PROJ_PACKED, ENGRAM_PROJ_SPLITK = 0, 1, 2
_PROJ_NAMES = {ENGRAM_PROJ_PLAIN: "plain", ENGRAM_PROJ_PACKED: "packed", ENGRAM_PROJ_SPLITK: "splitk"}


def engram_projection_plan(layout: Layout, hidden: int, T: int, *, packed: bool, splits: int = 0):
    """(kernel name, splits) a T-token projection runs (host logic, no device)."""
    p = engram_proj_plan()
    _check(_lib.engram_projection_plan(layout.handle, int(hidden), int(T), int(bool(packed)), int(splits),
                                       ctypes.byref(p)), "engram_projection_plan")
    return _PROJ_NAMES[p.kernel], int(p.splits)


class Wkv:
    """Owner of an ``engram_wkv*`` handle: a site's projection weight bound to the
    layout and the largest call, with the packed copy and split-K workspace the
    library allocates for it.  Keeps a reference to ``w`` (the library reads it)."""

    def __init__(self, layout: Layout, w, max_tokens: int, splits: int = 0, stream=None):
        import torch
        _need(w.dim() == 2, "w must be [hidden][w_ld]")
        h = _P()
        _check(_lib.engram_wkv_create(layout.handle, _dev(w, torch.bfloat16, "w"), w.shape[1], w.shape[0],
                                      int(max_tokens), int(splits), _stream(stream), ctypes.byref(h)),
               "engram_wkv_create")
        self.handle = h.value
        self.layout = layout
        self.w = w
        self.hidden = int(w.shape[0])
        self.max_tokens = int(max_tokens)

    def __del__(self, _destroy=_lib.engram_wkv_destroy):
        h, self.handle = getattr(self, "handle", None), None
        if h:
            _destroy(h)

    def plan(self, T: int):
        """(kernel name, splits) of a T-token call."""
        p = engram_proj_plan()
        _check(_lib.engram_wkv_plan(self.handle, int(T), ctypes.byref(p)), "engram_wkv_plan")
        return _PROJ_NAMES[p.kernel], int(p.splits)


def engram_wkv_create(layout: Layout, w, max_tokens: int, *, splits: int = 0, stream=None) -> Wkv:
    return Wkv(layout, w, max_tokens, splits=splits, stream=stream)


def _check_gate_args(wkv: Wkv, streams, v, keep, T):
    _need(streams.dim() == 3 and streams.shape[0] >= T and streams.shape[2] == wkv.hidden,
          "streams must be [T][hc][hidden]")
    _need(v.dim() == 2 and v.shape[0] >= T and v.shape[1] == wkv.hidden, "v must be [T][hidden]")
    _need(keep is None or keep.numel() >= T, "keep too small")


def engram_gated_residual(layout: Layout, rows, wkv: Wkv, streams, v, *, keep=None,
                          T: Optional[int] = None, stream=None):
    import torch
    if T is None:
        T = streams.shape[0]
    _need(rows.dim() == 2 and rows.shape[0] >= T, "rows too small")
    _check_gate_args(wkv, streams, v, keep, T)
    _check(_lib.engram_gated_residual(
        layout.handle, _dev(rows, torch.bfloat16, "rows"), rows.shape[1], wkv.handle, streams.shape[1],
        _dev(keep, torch.uint8, "keep"), _dev(streams, torch.bfloat16, "streams"),
        _dev(v, torch.float32, "v"), T, _stream(stream)), "engram_gated_residual")


def engram_gated_residual_noalloc(layout: Layout, rows, wkv: Wkv, streams, *, keep=None,
                                  T: Optional[int] = None, stream=None):
    """engram_gated_residual with its scratch in the library's per-GPU array (no
    allocation; v is not returned)."""
    import torch
    if T is None:
        T = streams.shape[0]
    _need(rows.dim() == 2 and rows.shape[0] >= T, "rows too small")
    _need(streams.dim() == 3 and streams.shape[0] >= T and streams.shape[2] == wkv.hidden,
          "streams must be [T][hc][hidden]")
    _need(keep is None or keep.numel() >= T, "keep too small")
    _check(_lib.engram_gated_residual_noalloc(
        layout.handle, _dev(rows, torch.bfloat16, "rows"), rows.shape[1], wkv.handle, streams.shape[1],
        _dev(keep, torch.uint8, "keep"), _dev(streams, torch.bfloat16, "streams"), T, _stream(stream)),
        "engram_gated_residual_noalloc")


def engram_wkv_project(layout: Layout, rows, wkv: Wkv, v, *, T: Optional[int] = None, stream=None):
    import torch
    if T is None:
        T = rows.shape[0]
    _need(rows.dim() == 2 and rows.shape[0] >= T, "rows too small")
    _need(v.dim() == 2 and v.shape[0] >= T and v.shape[1] == wkv.hidden, "v must be [T][hidden]")
    _check(_lib.engram_wkv_project(layout.handle, _dev(rows, torch.bfloat16, "rows"), rows.shape[1],
                                   wkv.handle, _dev(v, torch.float32, "v"), T, _stream(stream)),
           "engram_wkv_project")


def engram_wkv_gate_add(layout: Layout, wkv: Wkv, v, streams, *, keep=None, T: Optional[int] = None,
                        stream=None):
    import torch
    if T is None:
        T = streams.shape[0]
    _check_gate_args(wkv, streams, v, keep, T)
    _check(_lib.engram_wkv_gate_add(layout.handle, wkv.handle, _dev(v, torch.float32, "v"),
                                    streams.shape[1], _dev(keep, torch.uint8, "keep"),
                                    _dev(streams, torch.bfloat16, "streams"), T, _stream(stream)),
           "engram_wkv_gate_add")


def engram_get_error(stream=None) -> int:
    return int(_lib.engram_get_error(_stream(stream)))


def check_device_error(where: str = "device", stream=None):
    _check(engram_get_error(stream), where)


from .runtime import Engram, pad_weight  # noqa: E402  (needs the functions above)
