#!/usr/bin/env python3
"""Throughput of the Engram n-gram memory hot path on one MI355X.

A step is one pass of the whole path over one batch with every input resident
in HBM: engram_compress_hash -> engram_gather_dequant -> engram_project ->
engram_gate_add (the two halves of engram_gated_residual, called separately so
that each kernel is bracketed by its own HIP events on the launch stream).

Default workload ("full"): 8 x 8,192 Zipf(1.1) tokens against three
5,040,000-row e4m3fn tables (row dim 6,500 + an fp32 scale per row, 91.6 GiB),
one hash head per order, projection 19,500 -> 4,096 into 4 residual streams.

Prints one JSON line: tokens/s; `roofline`, the roofline of the kernel that takes
the most time per step (at full scale the projection: flops / measured average
launch time, against 2.5 PFLOP/s bf16); the rooflines of the gather (HBM bytes the
method must move / launch time, against 8 TB/s: the metric's HBM figure), the
projection and the gate under their own names; the per-kernel breakdown; and the
oracle's single-core throughput on a bounded token sample.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
[--config full|full_bf16|long|prefill|decode|tiny|v41|v41_small] [--path split|fused] [--graph] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Engram tokens/s at 1 GPU + achieved HBM GB/s as % of MI355X peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA

WORKLOAD_TEXT = {
    "full": "full scale: 8 x 8,192 Zipf(1.1) tokens; 3 tables x 5,040,000 rows (15.12M) of 6,500 "
            "e4m3fn + fp32 row scale (91.6 GiB); 1 head per order; wkv 19,500->4,096 bf16; hc 4",
    "full_bf16": "full scale, BF16 tables: 8 x 8,192 Zipf(1.1) tokens; 3 x 5,040,000 rows of 6,500 "
                 "bf16 (183.1 GiB); 1 head per order; wkv 19,500->4,096; hc 4",
    "long": "long prefill: 65,536 Zipf(1.1) tokens in Geometric(mean 2,048) documents; "
            "3 x 4,194,304 rows of 1,024 e4m3fn; 1 head per order; wkv 3,072->4,096; hc 4",
    "prefill": "prefill: 4 x 4,096 Zipf(1.1) tokens; 3 x 1,048,576 rows of 512 e4m3fn; "
               "2 heads per order; wkv 3,072->4,096; hc 4",
    "decode": "decode step: 256 slots x 1 token, rolling store; prefill's tables and wkv",
    "tiny": "tiny: 512 uniform tokens; 3 x 4,096 rows of 128 e4m3fn; 2 heads; wkv 768->256; hc 4",
    "v41": "released layout: 8 x 8,192 Zipf(1.1) tokens; 2 Engram sites sharing one hash pass; "
           "3 orders x 8 heads; one table per site of 384,006,168 / 384,016,682 rows of 256 e4m3fn "
           "with (1,32) e8m0 scales (2 x 98.3 GB); wkv 6,144->4,096 per site; hc 4",
    "v41_small": "released layout structure at bucket floor 20,000: 4 x 2,048 Zipf(1.1) tokens; "
                 "2 sites; 3 x 8 heads; D 256; (1,32) e8m0 scales; wkv 6,144->1,024; hc 4",
}


def algorithmic_per_token(cfg):
    """Bytes (or flops) each kernel must move per token, counting rows touched."""
    H, D, hidden = cfg.heads, cfg.row_dim, cfg.hidden
    K = 3 * H * D
    scale = 0 if cfg.table_dtype != "fp8" else (D // 32 if cfg.scale_block else 4)
    return {
        "project_weight_bytes": 2 * K * hidden,
        # token id, tid2eid entry, compressed id out, 3H row ids per site out
        "hash_bytes": 4 + 4 + 4 + 4 * 3 * H * cfg.n_sites,
        # per site: 3H rows of D elements + their scales in; K bf16 out
        "gather_bytes": 3 * H * (D * cfg.elt_bytes + scale) + 2 * K,
        "project_flops": 2 * K * hidden,
        # per token: its row of E (bf16) in and its row of v (fp32) out; the weight's
        # bytes (project_weight_bytes) are per call, not per token
        "project_token_bytes": 2 * K + 4 * hidden,
        # 4 bf16 streams read and written, v (fp32) read
        "gate_bytes": cfg.hc_mult * hidden * 2 * 2 + 4 * hidden,
    }


def measured_traffic(cfg, profile="gather_dequant_{tag}_traffic.txt", source="gather.hip"):
    """HBM bytes per launch of a kernel from the committed profiler counters
    (profiles/<profile>, by default the gather's), or None when there is no
    measurement for this workload or the kernel's code changed since it was taken."""
    tag = {"full": "full_fp8"}.get(cfg.name, cfg.name)
    path = os.path.join(ROOT, "profiles", profile.format(tag=tag))
    src = os.path.join(ROOT, "hashed_gram_memory_tid2eid_amd", "csrc", "kernels", source)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    with open(src) as f:
        sha = kernel_code_hash(f.read())
    if kv.get("kernel_code_sha256_16") != sha:
        return None
    return float(kv["traffic_bytes_per_launch"])


def measured_mfma_ceiling():
    """The bf16 matrix-core rate this part reached with no data movement
    (profiles/mfma_ceiling_probe.txt, from `bench.py --mfma-ceiling`), TFLOP/s, or
    None without that profile."""
    import re
    path = os.path.join(ROOT, "profiles", "mfma_ceiling_probe.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        m = re.search(r"^best: ([\d.]+) TFLOP/s", f.read(), re.M)
    return float(m.group(1)) if m else None


def kernel_code_hash(text: str) -> str:
    """First 16 hex digits of a SHA-256 over a kernel source with its comments removed
    and its whitespace collapsed: an edit of the code changes it, an edit of a comment
    does not."""
    import hashlib
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def cpu_baseline(cfg, batch, site_tables, weights, streams_host_bits, budget_s: float):
    """The oracle as it stands, single-threaded on a host core, on a bounded token
    sample of the same workload (rows read from the device tables by torch)."""
    import engram_inputs as ei
    import oracle

    tid2eid = ei.make_tid2eid(cfg.vocab, cfg.vc)
    per_site = cfg.table_split == "site"
    if cfg.n_sites > 1 or per_site:
        layouts = oracle.site_layouts(cfg.n_sites, cfg.heads, cfg.hash_floor, per_site)
    elif cfg.hash_floor:
        layouts = [oracle.layout_at_floor([cfg.rows] * 3, cfg.heads, cfg.hash_floor)]
    else:
        layouts = [oracle.fit_layout([cfg.rows] * 3, cfg.heads)]
    store = ei.make_store_init(cfg) if batch.slots is not None else None
    # the oracle runs on this thread: pin the calling thread (Linux applies an affinity
    # set for pid 0 to the caller alone) to one host core for the timed part, and restore
    # its mask afterwards
    old_mask = os.sched_getaffinity(0)
    core = min(old_mask)
    os.sched_setaffinity(0, {core})
    try:
        res = _cpu_baseline_pinned(cfg, batch, site_tables, weights, streams_host_bits, budget_s,
                                   layouts, tid2eid, store)
    finally:
        os.sched_setaffinity(0, old_mask)
    res["sample"] += f"; pinned to host core {core} of {len(old_mask)} in this process's mask"
    return res


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (else the machine type)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


def _cpu_baseline_pinned(cfg, batch, site_tables, weights, streams_host_bits, budget_s, layouts,
                         tid2eid, store):
    import numpy as np
    import torch

    import oracle

    t0 = time.perf_counter()
    site_rows = []
    for si, L in enumerate(layouts):
        st = store if si == 0 or store is None else store.copy()
        _, rows = oracle.compress_hash(L, vocab=cfg.vocab, vc=cfg.vc, pad_token_id=cfg.pad_token_id,
                                       tid2eid=tid2eid, tokens=batch.tokens,
                                       cu_seqlens=batch.cu_seqlens, seq_start=batch.seq_start,
                                       slots=batch.slots, store=st)
        site_rows.append(rows)
    t_hash_all = time.perf_counter() - t0
    Ws = [w.view(torch.int16).cpu().numpy().view(np.uint16) for w in weights]
    rng = np.random.default_rng(1234)
    order = rng.permutation(batch.T)
    H, D = cfg.heads, cfg.row_dim
    bf16 = cfg.table_dtype == "bf16"
    per_site = cfg.table_split == "site"
    done, t_rest = 0, 0.0
    chunk = 4
    while done < batch.T and t_rest + t_hash_all * done / batch.T < budget_s:
        idx = np.sort(order[done:done + chunk])
        for si in range(cfg.n_sites):
            tabs = site_tables[si]
            raw = np.zeros((len(idx), 3 * H, D), np.uint16 if bf16 else np.uint8)
            if bf16:
                sc = None
            elif cfg.scale_block:
                sc = np.zeros((len(idx), 3 * H, D // 32), np.uint8)
            else:
                sc = np.zeros((len(idx), 3 * H), np.float32)
            for o in range(3):
                n = 0 if per_site else o
                view = tabs.row_view(n)
                for h in range(H):
                    ii = torch.from_numpy(site_rows[si][idx, o, h].astype(np.int64)).to(view.device)
                    r = view.index_select(0, ii)
                    raw[:, o * H + h] = (r.view(torch.int16).cpu().numpy().view(np.uint16) if bf16
                                         else r.cpu().numpy())
                    if sc is not None:
                        sc[:, o * H + h] = tabs.scale[n].index_select(0, ii).cpu().numpy()
            x = streams_host_bits[si][idx]
            t1 = time.perf_counter()
            if cfg.scale_block:
                _, e16 = oracle.dequant_rows_block32(raw.reshape(-1, D), sc.reshape(-1, D // 32))
            else:
                _, e16 = oracle.dequant_rows(raw.reshape(-1, D), None if sc is None else sc.reshape(-1),
                                             bf16_table=bf16)
            v = oracle.project(e16.reshape(len(idx), -1), Ws[si])
            oracle.gate_add(x, v)
            t_rest += time.perf_counter() - t1
        done += len(idx)
    total = t_rest + t_hash_all * done / batch.T
    return {
        "value": done / total,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "sample": (f"{done} of {batch.T} tokens of the same batch (seeded), full path per token "
                   f"and site ({cfg.n_sites}): compress+hash (whole batch {t_hash_all:.3f}s, charged "
                   f"pro rata), dequant, fp64 projection, gate; {total:.1f}s of single-thread C on "
                   f"{cpu_model()}, {os.cpu_count()} host CPUs"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 200 for decode workloads, whose ~35 us steps "
                         "vary by a few us over 20)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 5; 20 for decode)")
    ap.add_argument("--config", default="full", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--path", default="split", choices=["split", "fused"],
                    help="split: gather_dequant + project (default, faster); fused: gather_project")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step in a HIP graph and time K replays; value = graph rate")
    ap.add_argument("--host-tables", action="store_true",
                    help="keep the tables in pinned host memory (read over the host link)")
    ap.add_argument("--prefetch", action="store_true",
                    help="also time the pipelined loop: hash + gather of step i+1 on a prefetch "
                         "stream while step i projects and gates; value = pipelined rate")
    ap.add_argument("--order", default="lookahead", choices=["lookahead", "sequential"],
                    help="lookahead (split path, prefill-style workloads): per step the next "
                         "call's hash, then per site this call's projection, the next call's "
                         "gather, this call's gate; sequential: hash, gather, projection, gate. "
                         "The other order is timed after the main line.")
    ap.add_argument("--decode-lookup", default="fused", choices=["fused", "split"],
                    help="decode steps: fused = compress, hash and gather in one launch "
                         "(engram_lookup_decode, where the layout allows it); split = "
                         "engram_compress_hash then engram_gather_dequant")
    ap.add_argument("--proj-splits", type=int, default=0,
                    help="split-K factor of the projection (0: chosen from the call size)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-alt-paths", action="store_true",
                    help="skip the fused-path comparison after the timed steps (profiler runs)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--compare-vendor", action="store_true",
                    help="after the timed steps, time torch.mm (the vendor bf16 GEMM) on the "
                         "projection's rows and weight")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only run the matrix-core ceiling probe (16x16x32 bf16 products on "
                         "operands in registers, every CU, no data movement) and print its rate")
    ap.add_argument("--hbm-reference", action="store_true",
                    help="only run the HBM streaming references (read, copy, 1:2 expand, and the "
                         "gated residual's traffic without its arithmetic) and print their rates")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run a plain 1 GiB fp32 copy kernel three times "
                         "(reference for the HBM byte counters of a profiler run)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(tables are replicated per GPU, tokens split across them); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    if args.mfma_ceiling:
        # a child process, started before this one touches the GPU
        import re
        import runpy
        import subprocess
        probe = runpy.run_path(os.path.join(ROOT, "hashed_gram_memory_tid2eid_amd",
                                            "build_lib.py"))["build_mfma_ceiling"]()
        out = subprocess.run([probe], capture_output=True, text=True, timeout=120)
        if out.returncode != 0:
            print(out.stdout + out.stderr, file=sys.stderr)
            sys.exit(out.returncode)
        runs = {}
        for m in re.finditer(r"mfma chain (\d+): ([\d.]+) ms, ([\d.]+) TFLOP/s", out.stdout):
            runs.setdefault(int(m.group(1)), []).append(float(m.group(3)))
        best = {c: max(v) for c, v in runs.items()}
        print(json.dumps({"metric": "bf16 matrix-core rate with no data movement",
                          "unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS,
                          "runs": runs, "best": best,
                          "frac_of_peak": max(best.values()) / BF16_PEAK_TFLOPS}), flush=True)
        return

    if args.hbm_reference:
        # a child process, started before this one touches the GPU
        import re
        import runpy
        import subprocess
        probe = runpy.run_path(os.path.join(ROOT, "hashed_gram_memory_tid2eid_amd",
                                            "build_lib.py"))["build_hbm_reference"]()
        out = subprocess.run([probe], capture_output=True, text=True, timeout=120)
        if out.returncode != 0:
            print(out.stdout + out.stderr, file=sys.stderr)
            sys.exit(out.returncode)
        runs = {}
        for m in re.finditer(r"hbm (\w+): ([\d.]+) ms, ([\d.]+) GB/s", out.stdout):
            runs.setdefault(m.group(1), []).append(float(m.group(3)))
        best = {k: max(v) for k, v in runs.items()}
        print(json.dumps({"metric": "HBM rate of plain streaming kernels", "unit": "GB/s",
                          "peak": HBM_PEAK_GBS, "runs": runs, "best": best,
                          "frac_of_peak": {k: v / HBM_PEAK_GBS for k, v in best.items()}}),
              flush=True)
        return

    import numpy as np
    import torch

    import engram_inputs as ei
    decode_cfg = bool(ei.get_config(args.config).decode_steps)
    if args.steps is None:
        args.steps = 200 if decode_cfg else 20
    if args.warmup is None:
        args.warmup = 20 if decode_cfg else 5
    import runpy
    # builds only when the library is missing or was built from other sources
    runpy.run_path(os.path.join(ROOT, "hashed_gram_memory_tid2eid_amd", "build_lib.py"))["ensure_built"]()
    import hashed_gram_memory_tid2eid_amd as eng

    dev = "cuda:0"
    torch.cuda.set_device(0)
    cfg = ei.get_config(args.config)
    if args.path == "fused" and (cfg.table_dtype != "fp8" or (cfg.scale_block and cfg.row_dim > 256)
                                 or args.host_tables):
        print("bench.py: the fused path reads e4m3fn tables from HBM (one fp32 scale per row, or e8m0 "
              f"block scales on rows of at most 256 elements); workload {cfg.name}"
              f"{' with host tables' if args.host_tables else ''} needs --path split", file=sys.stderr)
        sys.exit(2)
    t_setup = time.perf_counter()
    tid2eid = torch.from_numpy(ei.make_tid2eid(cfg.vocab, cfg.vc)).to(dev)
    if cfg.decode_steps:
        batches = ei.make_decode_steps(cfg, 1)
        batch = batches[0]
    else:
        batch = ei.make_batch(cfg)
    T = batch.T
    NS = cfg.n_sites
    site_tables = [ei.make_tables(cfg, dev, site=s) for s in range(NS)]
    weights = [ei.make_weight(cfg, dev, site=s) for s in range(NS)]
    one = NS == 1
    # the look-ahead order applies to the split path's many-token calls (not decode steps,
    # graph captures or the two-stream prefetch loop, which keep their own order)
    lookahead_ok = (args.order == "lookahead" and args.path == "split" and not cfg.decode_steps
                    and not args.graph and not args.prefetch)
    if args.host_tables:
        # tables move to pinned host memory; the device copies are dropped
        for t in site_tables:
            for lst in (t.data, t.scale):
                for j in range(len(lst or [])):
                    h = torch.empty(lst[j].shape, dtype=lst[j].dtype, pin_memory=True)
                    h.copy_(lst[j])
                    lst[j] = h
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    site = eng.Engram(vocab_size=cfg.vocab, compressed_vocab=cfg.vc, pad_token_id=cfg.pad_token_id,
                      heads_per_order=cfg.heads,
                      rows=[cfg.rows] if cfg.table_split == "site" else [cfg.rows] * 3,
                      row_dim=cfg.row_dim, table_dtype=cfg.table_dtype,
                      row_pitch_bytes=cfg.row_pitch_bytes, tid2eid=tid2eid,
                      tables=site_tables[0].data if one else [t.data for t in site_tables],
                      scales=site_tables[0].scale if one else [t.scale for t in site_tables],
                      weight=weights[0] if one else weights, hidden=cfg.hidden, hc_mult=cfg.hc_mult,
                      max_tokens=T, path=args.path, num_sites=NS, table_split=cfg.table_split,
                      scale_block=cfg.scale_block, hash_floor=cfg.hash_floor,
                      prefetch_slots=2 if args.prefetch else 0, proj_splits=args.proj_splits,
                      lookahead=lookahead_ok)
    site_streams = [ei.make_streams(cfg, T, dev, step=s) for s in range(NS)]
    streams_host = None
    if not args.no_cpu_baseline:
        streams_host = [x.view(torch.int16).cpu().numpy().view(np.uint16).copy() for x in site_streams]

    def d(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    tok, cu, ss, sl = d(batch.tokens), d(batch.cu_seqlens), d(batch.seq_start), d(batch.slots)
    store = site.make_store(cfg.n_seqs, ids=d(ei.make_store_init(cfg))) if cfg.decode_steps else None
    # decode steps (one token per sequence, continuing from its slot) take the
    # one-launch lookup where the layout allows it
    use_lookup = (bool(cfg.decode_steps) and cfg.seq_len == 1 and args.decode_lookup == "fused"
                  and args.path == "split" and site.decode_lookup_supported)
    L = site.layout
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    print(f"# setup {setup_s:.1f}s: {cfg.name}, T={T}, k_pad={site.info.k_pad}", file=sys.stderr, flush=True)

    # kernel sequence of one step: the hash, then per site gather (+) project, gate;
    # in the look-ahead order the hash is the next call's, and per site the projection
    # (this call's rows, gathered one step earlier) comes before the next call's gather
    if args.path == "fused":
        seq = ["compress_hash"] + ["gather_project", "gate_add"] * NS
    elif use_lookup:
        seq = ["lookup_decode", "project", "gate_add"]
    else:
        seq = ["compress_hash"] + ["gather_dequant", "project", "gate_add"] * NS
    seq_la = ["compress_hash"] + ["project", "gather_dequant", "gate_add"] * NS

    def step_lookahead(ev=None):
        k = 0

        def mark():
            nonlocal k
            if ev:
                ev[k].record()
            k += 1
        mark()
        eng.engram_compress_hash(L, tid2eid, tok, cu, site.eids, site.row_ids, seq_start=ss,
                                 slots=sl, store=store)
        mark()
        for si in range(NS):
            site.project(si, site.site_rows[si], T)
            mark()
            eng.engram_gather_dequant(L, site.site_tables[si], site.site_scales[si], site.row_ids,
                                      site.site_rows[si], site=si, T=T)
            mark()
            site.gate(si, site_streams[si], T)
            mark()

    def step_sequential(ev=None):
        k = 0

        def mark():
            nonlocal k
            if ev:
                ev[k].record()
            k += 1
        mark()
        if use_lookup:
            eng.engram_lookup_decode(L, tid2eid, tok, site.eids, site.row_ids, site.site_tables[0],
                                     site.site_scales[0], site.rows, slots=sl, store=store)
            mark()
            site.project(0, site.rows, T)
            mark()
            site.gate(0, site_streams[0], T)
            mark()
            return
        eng.engram_compress_hash(L, tid2eid, tok, cu, site.eids, site.row_ids, seq_start=ss,
                                 slots=sl, store=store)
        mark()
        for si in range(NS):
            if args.path == "fused":
                eng.engram_gather_project(L, site.site_tables[si], site.site_scales[si], site.row_ids,
                                          site.site_weights[si], site.v, site=si, T=T)
                mark()
            else:
                eng.engram_gather_dequant(L, site.site_tables[si], site.site_scales[si], site.row_ids,
                                          site.rows, site=si, T=T)
                mark()
                site.project(si, site.rows, T)
                mark()
            if args.path == "fused":
                eng.engram_gate_add(L, site.v, site_streams[si], T=T)
            else:
                site.gate(si, site_streams[si], T)
            mark()

    def timed(step_fn, sq):
        """Warm-up steps, then K timed steps with an event between kernels: total ms,
        ms per launch of each kernel, host wall seconds."""
        for _ in range(args.warmup):
            step_fn()
        torch.cuda.synchronize()
        eng.check_device_error("warmup")
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(sq) + 1)] for _ in range(args.steps)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        start.record()
        for i in range(args.steps):
            step_fn(evs[i])
        stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        eng.check_device_error("timed steps")
        # average time per launch of each kernel (a step launches the per-site kernels NS times)
        kms = {}
        for n in dict.fromkeys(sq):
            js = [j for j, m in enumerate(sq) if m == n]
            kms[n] = float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs for j in js]))
        return start.elapsed_time(stop), kms, wall

    if lookahead_ok:
        # the first call's lookup, so that every timed step projects rows gathered a step earlier
        site.gather_ahead(tok, cu, seq_start=ss, slots=sl, store=store)
        step, order_seq = step_lookahead, seq_la
    else:
        step, order_seq = step_sequential, seq
    total_ms, kern_ms, wall = timed(step, order_seq)
    ms_per_step = total_ms / args.steps

    per = algorithmic_per_token(cfg)
    def gbs(b, ms):
        return b / (ms * 1e-3) / 1e9
    gather_bytes = per["gather_bytes"] * T
    proj_flops = per["project_flops"] * T
    gate_gbs = gbs(per["gate_bytes"] * T, kern_ms["gate_add"])
    if use_lookup:
        # the lookup is the hash and the gather in one launch: its bytes are both kernels'
        kernels = {}
        lookup_bytes = (per["hash_bytes"] + per["gather_bytes"]) * T
        lookup_gbs = gbs(lookup_bytes, kern_ms["lookup_decode"])
        kernels["lookup_decode"] = {"ms": kern_ms["lookup_decode"], "bound": "hbm", "GB/s": lookup_gbs,
                                    "frac": lookup_gbs / HBM_PEAK_GBS, "launches_per_step": 1}
    else:
        hash_gbs = gbs(per["hash_bytes"] * T, kern_ms["compress_hash"])
        kernels = {"compress_hash": {"ms": kern_ms["compress_hash"], "bound": "alu", "GB/s": hash_gbs,
                                     "launches_per_step": 1}}
    if args.path == "fused":
        fused_tflops = proj_flops / (kern_ms["gather_project"] * 1e-3) / 1e12
        kernels["gather_project"] = {"ms": kern_ms["gather_project"], "bound": "mfma",
                                     "TFLOP/s": fused_tflops, "frac": fused_tflops / BF16_PEAK_TFLOPS}
        roofline = {"bound": "mfma", "kernel": "gather_project", "achieved": fused_tflops,
                    "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": fused_tflops / BF16_PEAK_TFLOPS,
                    "traffic": None, "flops_per_launch": proj_flops,
                    "avg_launch_ms": kern_ms["gather_project"]}
    else:
        proj_tflops = proj_flops / (kern_ms["project"] * 1e-3) / 1e12
        if not use_lookup:
            gather_gbs = gbs(gather_bytes, kern_ms["gather_dequant"])
            kernels["gather_dequant"] = {"ms": kern_ms["gather_dequant"], "bound": "hbm",
                                         "GB/s": gather_gbs, "frac": gather_gbs / HBM_PEAK_GBS}
        kernels["project"] = {"ms": kern_ms["project"], "bound": "mfma", "TFLOP/s": proj_tflops,
                              "frac": proj_tflops / BF16_PEAK_TFLOPS}
        traffic = None if use_lookup else measured_traffic(cfg)
        if use_lookup:
            roofline_gather = {"bound": "hbm", "kernel": "lookup_decode", "achieved": lookup_gbs,
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": lookup_gbs / HBM_PEAK_GBS,
                               "traffic": None, "bytes_per_launch": lookup_bytes,
                               "avg_launch_ms": kern_ms["lookup_decode"]}
        else:
            roofline_gather = {"bound": "hbm", "kernel": "gather_dequant", "achieved": gather_gbs,
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gather_gbs / HBM_PEAK_GBS,
                               "traffic": traffic, "bytes_per_launch": gather_bytes,
                               "avg_launch_ms": kern_ms["gather_dequant"]}
        if traffic is not None:
            # the HBM rate the counters imply for this run's launch time
            kernels["gather_dequant"]["hbm_GB/s_measured_bytes"] = gbs(traffic, kern_ms["gather_dequant"])
        pkind = site.projection_kind(0, T)
        proj_traffic = (measured_traffic(cfg, "gemm_bf16_nt_packed_{tag}_counters.txt", "gemm_packed.hip")
                        if pkind == "packed" else None)
        # bound by the matrix cores when its flops per algorithmic byte (the weight once,
        # E in, v out) reach the ridge of 2.5 PFLOP/s over 8 TB/s, else by HBM (few tokens:
        # a decode step streams the whole weight for 256 rows)
        proj_bytes = per["project_weight_bytes"] + per["project_token_bytes"] * T
        kname = "gemm_bf16_nt_packed" if pkind == "packed" else "gemm_bf16_nt"
        if proj_flops / proj_bytes >= BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
            roofline_projection = {"bound": "mfma", "kernel": kname, "achieved": proj_tflops,
                                   "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                   "frac": proj_tflops / BF16_PEAK_TFLOPS, "traffic": proj_traffic,
                                   "flops_per_launch": proj_flops, "avg_launch_ms": kern_ms["project"]}
            ceiling = measured_mfma_ceiling()
            if ceiling:
                # the same instruction's rate with its operands in registers on this part
                roofline_projection["measured_ceiling"] = ceiling
                roofline_projection["frac_of_measured_ceiling"] = proj_tflops / ceiling
        else:
            proj_gbs = gbs(proj_bytes, kern_ms["project"])
            kernels["project"].update({"bound": "hbm", "GB/s": proj_gbs})
            roofline_projection = {"bound": "hbm", "kernel": kname, "achieved": proj_gbs,
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": proj_gbs / HBM_PEAK_GBS,
                                   "traffic": proj_traffic, "bytes_per_launch": proj_bytes,
                                   "flops_per_launch": proj_flops, "avg_launch_ms": kern_ms["project"]}
    kernels["gate_add"] = {"ms": kern_ms["gate_add"], "bound": "hbm", "GB/s": gate_gbs,
                           "frac": gate_gbs / HBM_PEAK_GBS}
    if args.path != "fused":
        roofline_gate = {"bound": "hbm", "kernel": "gate_add", "achieved": gate_gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gate_gbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic(cfg, "gate_add_{tag}_traffic.txt", "gate.hip"),
                         "bytes_per_launch": per["gate_bytes"] * T,
                         "avg_launch_ms": kern_ms["gate_add"]}
        # `roofline` is the dominant kernel's: the one with the most time per step (the
        # hash is a few microseconds at every size and never dominates)
        roofline = max((roofline_gather, roofline_projection, roofline_gate),
                       key=lambda r: r["avg_launch_ms"])
    for n in kernels:
        kernels[n].setdefault("launches_per_step", NS)

    result = {
        "metric": METRIC,
        "value": T * args.steps / (total_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; see engram_inputs)",
        "config": {"workload": WORKLOAD_TEXT[cfg.name], "name": cfg.name, "tokens_per_step": T,
                   "table_dtype": cfg.table_dtype, "rows_per_table": cfg.rows, "row_dim": cfg.row_dim,
                   "heads_per_order": cfg.heads, "hidden": cfg.hidden, "hc_mult": cfg.hc_mult,
                   "k_pad": site.info.k_pad, "path": args.path, "sites": NS,
                   "table_split": cfg.table_split, "scale_block": cfg.scale_block,
                   "tables_in": "pinned host memory" if args.host_tables else "HBM",
                   "proj_splits": site.proj_splits,
                   "step_order": "lookahead" if lookahead_ok else "sequential",
                   "projection": site.projection_kind(0, T) if args.path != "fused" else "fused",
                   "lookup": "lookup_decode" if use_lookup else "compress_hash + gather_dequant"},
        "roofline": roofline,
        "kernels": kernels,
        "wall_s_timed": wall,
        "setup_s": setup_s,
        "library": eng.engram_build_id(),
    }
    if args.path != "fused":
        result["roofline_gather"] = roofline_gather
        result["roofline_projection"] = roofline_projection
        result["roofline_gate"] = roofline_gate
    if lookahead_ok:
        # the same K steps in the sequential order (hash, gather, projection, gate of one
        # call), on the same inputs, after the main line
        o_ms, o_kern, _ = timed(step_sequential, seq)
        result["sequential_order"] = {
            "value": T * args.steps / (o_ms * 1e-3), "ms_per_step": o_ms / args.steps,
            "kernels_ms": o_kern,
            "gather_frac": gbs(gather_bytes, o_kern["gather_dequant"]) / HBM_PEAK_GBS}
    if args.graph:
        # the same step captured once and replayed K times (launch overhead removed);
        # the decode step is launch-bound, so this is its production form
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g):
                step()
        torch.cuda.current_stream().wait_stream(side)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gs.record()
        for _ in range(args.steps):
            g.replay()
        ge.record()
        torch.cuda.synchronize()
        eng.check_device_error("graph replays")
        g_ms = gs.elapsed_time(ge) / args.steps
        result["eager"] = {"value": result["value"], "ms_per_step": result["ms_per_step"]}
        result["graph"] = {"value": T / (g_ms * 1e-3), "ms_per_step": g_ms}
        result["value"] = T / (g_ms * 1e-3)
        result["ms_per_step"] = g_ms
        result["config"]["hip_graph"] = True
        del g
    if args.prefetch:
        # steady state of the prefetch pipeline: step i+1's hash and gathers run on a
        # stream of their own while step i's projections and gates run on the main one
        if args.path != "split" or cfg.decode_steps:
            raise SystemExit("--prefetch applies to the split path of a prefill workload")
        side = torch.cuda.Stream()
        main = torch.cuda.current_stream()

        def pipelined(n):
            pre = site.prefetch(tok, cu, stream=side, seq_start=ss)
            for i in range(n):
                nxt = site.prefetch(tok, cu, stream=side, seq_start=ss) if i + 1 < n else None
                for si in range(NS):
                    site.apply(pre, si, site_streams[si], stream=main)
                pre = nxt
        side.wait_stream(main)
        pipelined(args.warmup)
        torch.cuda.synchronize()
        ps, pe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ps.record()
        side.wait_stream(main)
        pipelined(args.steps)
        main.wait_stream(side)
        pe.record()
        torch.cuda.synchronize()
        eng.check_device_error("prefetch pipeline")
        p_ms = ps.elapsed_time(pe) / args.steps
        result["sequential"] = {"value": result["value"], "ms_per_step": result["ms_per_step"]}
        result["prefetch_pipeline"] = {"value": T / (p_ms * 1e-3), "ms_per_step": p_ms}
        result["value"] = T / (p_ms * 1e-3)
        result["ms_per_step"] = p_ms
        result["config"]["prefetch_stream"] = True
    if (args.path == "split" and cfg.table_dtype == "fp8" and NS == 1 and not cfg.scale_block
            and not args.no_alt_paths and not args.host_tables):
        # the other path on the same inputs, outside the timed region: the fused
        # gather + projection against gather_dequant + project
        v_alt = torch.empty_like(site.v)
        reps = max(3, min(args.steps, 10))
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        eng.engram_gather_project(L, site.tables, site.scales, site.row_ids, site.weight, v_alt, T=T)
        e[0].record()
        for _ in range(reps):
            eng.engram_gather_project(L, site.tables, site.scales, site.row_ids, site.weight, v_alt, T=T)
        e[1].record()
        for _ in range(reps):
            eng.engram_gather_dequant(L, site.tables, site.scales, site.row_ids, site.rows, T=T)
            site.project(0, site.rows, T)
        e[2].record()
        torch.cuda.synchronize()
        eng.check_device_error("fused comparison")
        f_ms, s_ms = e[0].elapsed_time(e[1]) / reps, e[1].elapsed_time(e[2]) / reps
        if site.projection_kind(0, T) == "packed":
            # the projection from the unpacked weight (two operands through LDS) on the same rows
            v_plain = torch.empty_like(site.v)
            eng.engram_project(L, site.rows, site.weight, v_plain, T=T)
            e[0].record()
            for _ in range(reps):
                eng.engram_project(L, site.rows, site.weight, v_plain, T=T)
            e[1].record()
            torch.cuda.synchronize()
            result["alt_paths_projection"] = {
                "gemm_bf16_nt_unpacked_ms": e[0].elapsed_time(e[1]) / reps,
                "bitwise_equal_v": bool(torch.equal(v_plain.view(torch.int32), site.v.view(torch.int32))),
                "reps": reps}
        result["alt_paths"] = {
            "gather_project_fused": {"ms": f_ms, "TFLOP/s": proj_flops / (f_ms * 1e-3) / 1e12,
                                     "bitwise_equal_v": bool(torch.equal(v_alt.view(torch.int32),
                                                                         site.v.view(torch.int32)))},
            "gather_dequant_plus_project": {"ms": s_ms},
            "reps": reps,
        }
        del v_alt
    if args.path == "split" and not args.host_tables and not args.no_alt_paths:
        # reuse in this batch and a control gather without it, outside the timed region:
        # repeated n-grams look up the same rows, which the caches then serve; the
        # control draws every row id uniformly from its column's buckets (seeded)
        info = site.info
        H = cfg.heads
        rid = site.row_ids[:T].reshape(T, NS, 3, H)
        unique = {}
        for n in range(3):
            col = rid[:, 0, n, :].reshape(-1)
            unique[f"{n + 2}-gram"] = torch.unique(col).numel() / max(1, col.numel())
        rid_u = torch.empty_like(rid)
        gen = torch.Generator(device=dev)
        gen.manual_seed(1234)
        for si in range(NS):
            for n in range(3):
                for h in range(H):
                    lo, p = int(info.site_offsets[si][n][h]), int(info.site_primes[si][n][h])
                    rid_u[:, si, n, h] = torch.randint(lo, lo + p, (T,), generator=gen, device=dev,
                                                       dtype=torch.int32)
        reps = max(3, min(args.steps, 10))
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        eng.engram_gather_dequant(L, site.site_tables[0], site.site_scales[0], rid_u, site.rows, site=0, T=T)
        e[0].record()
        for _ in range(reps):
            eng.engram_gather_dequant(L, site.site_tables[0], site.site_scales[0], rid_u, site.rows,
                                      site=0, T=T)
        e[1].record()
        for _ in range(reps):
            eng.engram_gather_dequant(L, site.site_tables[0], site.site_scales[0], site.row_ids, site.rows,
                                      site=0, T=T)
        e[2].record()
        torch.cuda.synchronize()
        eng.check_device_error("gather controls")
        u_ms, h_ms = e[0].elapsed_time(e[1]) / reps, e[1].elapsed_time(e[2]) / reps

        # one gather launch right after a given predecessor, with or without a 1 ms pause
        # (host sleep after a synchronisation) in between: whether the in-step gather pays
        # for the write-back of what the kernel before it wrote
        def gather_after(pre, pause):
            ts = []
            for _ in range(reps):
                pre()
                if pause:
                    torch.cuda.synchronize()
                    time.sleep(0.001)
                a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a0.record()
                eng.engram_gather_dequant(L, site.site_tables[0], site.site_scales[0], site.row_ids,
                                          site.rows, site=0, T=T)
                a1.record()
                torch.cuda.synchronize()
                ts.append(a0.elapsed_time(a1))
            ms = float(np.median(ts))
            return {"ms": ms, "frac": gbs(gather_bytes, ms) / HBM_PEAK_GBS}

        def gate0():
            site.gate(0, site_streams[0], T)

        def proj0():
            site.project(0, site.rows, T)

        def gather0():
            eng.engram_gather_dequant(L, site.site_tables[0], site.site_scales[0], site.row_ids,
                                      site.rows, site=0, T=T)
        after = {"after_gather": gather_after(gather0, False),
                 "after_gate": gather_after(gate0, False),
                 "after_gate_then_1ms_pause": gather_after(gate0, True),
                 "after_projection": gather_after(proj0, False),
                 "after_projection_then_1ms_pause": gather_after(proj0, True)}
        eng.check_device_error("gather after predecessors")
        result["gather_controls"] = {
            "unique_row_frac": unique,
            "uniform_rows": {"ms": u_ms, "GB/s": gbs(gather_bytes, u_ms),
                             "frac": gbs(gather_bytes, u_ms) / HBM_PEAK_GBS},
            "hashed_rows_back_to_back": {"ms": h_ms, "GB/s": gbs(gather_bytes, h_ms),
                                         "frac": gbs(gather_bytes, h_ms) / HBM_PEAK_GBS},
            "single_launch_median": after,
            "reps": reps,
        }
        del rid_u
    if args.compare_vendor and args.path == "split" and not cfg.decode_steps:
        # the vendor library's bf16 GEMM (torch.mm, bf16 output) on the same rows and weight,
        # outside the timed region: a reference point for the projection, not the product
        wt = site.site_weights[0].t().contiguous()
        out = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device=dev)
        torch.mm(site.rows[:T], wt, out=out)
        reps = max(3, min(args.steps, 10))
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        for _ in range(reps):
            torch.mm(site.rows[:T], wt, out=out)
        e[1].record()
        torch.cuda.synchronize()
        v_ms = e[0].elapsed_time(e[1]) / reps
        result["vendor_gemm"] = {"ms": v_ms, "TFLOP/s": proj_flops / (v_ms * 1e-3) / 1e12,
                                 "frac": proj_flops / (v_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                 "reps": reps, "what": "torch.mm of the same bf16 rows and weight"}
        del wt, out
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)   # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, batch, site_tables, weights, streams_host,
                                              args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
