"""Decode-step throughput of the CSA2 FP4 sparse-decode path on one MI355X.

Workload (default): 32 sequences x 64K tokens (32,768 compressed entries
each), 576-dim E2M1 entries with group 64 and Student-t(3) values, indexer
64 heads x 128 dims with integer values in [-8, 8], top-512, 64 query heads,
128-token bf16 window.  One step = one Full-layer decode step for the whole
batch: append one token per sequence (stand-in compressor + FP4 quantise),
window append, indexer scan + exact top-512, gather/dequantise + attention.

Inputs are seeded synthetic data resident in HBM before timing.  Several
cache replicas are stepped in rotation so consecutive steps do not hit the
last-level cache with the previous step's data.  The timed steps are plain
launches.  The headline roofline is the whole step: its algorithmic bytes
over the HIP-event time of the timed steps, against 8 TB/s.  The indexer
scan, the largest kernel, has a roofline object of its own, timed live with
HIP events on its launch stream on one timed step in --scan-sample-every
(each event pair adds a few microseconds to its step).
The per-kernel breakdown comes from a separate eager pass after the timed
steps with every kernel timer on.  --graph instead captures each replica's
step in a HIP graph and times graph replays (the scan time then comes from
the separate pass).

Prints one JSON line (rank 0).  --copy-probe MIB instead runs a plain
device copy of known size, used to calibrate hardware byte counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA2 FP4 sparse decode: steps/s at 64K ctx; achieved % of 8 TB/s HBM"
HBM_PEAK_GBPS = 8000.0
PMC_FILE = os.path.join(ROOT, "profiles", "decode_step_64k_b32_pmc.json")
CSRC = os.path.join(ROOT, "compressed_sparse_kv_append_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_64k_b32")
    p.add_argument("--replicas", type=int, default=2)
    p.add_argument("--cpu-baseline-seqs", type=int, default=0, help="sequences in the oracle's sample "
                   "(0: the whole batch)")
    p.add_argument("--cpu-baseline-seconds", type=float, default=10.0,
                   help="the oracle repeats decode steps until this much time has passed")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true", help="time HIP graph replays of the step")
    p.add_argument("--scan-sample-every", type=int, default=4)
    p.add_argument("--copy-probe", type=int, default=0, help="MiB copied by a plain device copy")
    p.add_argument("--idx-format", choices=("bf16", "fp4"), default="bf16",
                   help="indexer-key storage: bf16, or the pages' FP4 form (E2M1 + E8M0 per 16 dims)")
    p.add_argument("--swa-format", choices=("bf16", "fp8"), default="bf16",
                   help="window rows: bf16, or the pages' FP8 (E4M3)")
    p.add_argument("--kv-format", choices=("f32", "mx16"), default="f32",
                   help="main entries: E2M1 with fp32 group scales, or the pages' form with one E8M0 "
                   "byte per 16 channels (the workload's groups become 16)")
    p.add_argument("--pool", default="", help="pool_blocks,pool_block: the hierarchical indexer's candidate "
                   "pool in a layer-group workload (reindex layers select inside it)")
    p.add_argument("--capacity", type=int, default=0, help="entries per sequence the caches are allocated "
                   "for (0: what the timed steps need); the same entries, in a larger allocation")
    p.add_argument("--paged", type=int, default=0, metavar="PAGE", help="mixed workload: paged cache "
                   "planes of PAGE entries, each sequence holding only the pages it needs")
    p.add_argument("--mfma-compressor", action="store_true", help="mixed workload: the prefill chunk "
                   "through cskv_kv_append_fp4_mfma (matrix-core compressor, stated error bound) instead "
                   "of the exact fixed-order compressor")
    p.add_argument("--pmc-summary", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                   "COPY_WRITE_DIR", "COPY_MIB"), help="write the step's HBM-traffic summary from four "
                   "rocprofv3 --pmc output folders (FETCH_SIZE and WRITE_SIZE of a default run and of "
                   "--copy-probe COPY_MIB) to " + os.path.relpath(PMC_FILE, ROOT) + "; no GPU use")
    return p.parse_args()


def copy_probe(mib: int):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


# The kernels one decode step of the default workload launches, with launches
# per step (a name, followed by its argument list, is looked for in the
# profiler's kernel name).
STEP_KERNELS = (("quantize_kernel<true, true, true>", 1), ("indexer_scan_kernel<128, 4, false, false>", 1),
                ("topk_bound_slice_carry_kernel<4096, 512, 1>", 1), ("topk_bound_final_carry_kernel<32>", 1),
                ("sparse_attn_kernel<64, false, 64, false>", 1), ("attn_merge_kernel", 1))
SCAN_KERNEL = "indexer_scan_kernel<128, 4, false, false>"


def _counter_means(folder: str, counter: str) -> dict:
    """Mean Counter_Value per dispatch (summed over the rows of a dispatch) of
    every kernel in the rocprofv3 counter-collection csv under folder."""
    import csv
    path = None
    for root, _, files in os.walk(folder):
        for f in files:
            if f.endswith("counter_collection.csv"):
                path = os.path.join(root, f)
    if path is None:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    per = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            key = (row["Kernel_Name"], row["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    sums = {}
    for (name, _), v in per.items():
        t, n = sums.get(name, (0.0, 0))
        sums[name] = (t + v, n + 1)
    return {name: (t / n, n) for name, (t, n) in sums.items()}


def pmc_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib):
    """HBM bytes per step of the default workload, from FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch) scaled by what they read for a plain copy of known size."""
    copy_kib = int(copy_mib) * 1024
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    cf, cw = _counter_means(copy_fetch_dir, "FETCH_SIZE"), _counter_means(copy_write_dir, "WRITE_SIZE")

    def copy_value(d):
        vals = [v for name, (v, n) in d.items() if "copy" in name.lower()]
        if not vals:
            raise SystemExit("no copy kernel in the copy-probe counters")
        return max(vals)

    f_scale, w_scale = copy_kib / copy_value(cf), copy_kib / copy_value(cw)

    def find(d, kname):
        hits = [(name, v) for name, v in d.items() if kname + "(" in name]
        if not hits:
            raise SystemExit(f"kernel {kname} not in the counters")
        return hits[0][1]

    kernels, step = {}, 0.0
    for kname, per_step in STEP_KERNELS:
        (fv, fn), (wv, wn) = find(fetch, kname), find(write, kname)
        b = (fv * f_scale + wv * w_scale) * 1024.0
        kernels[kname] = {"fetch_kib": round(fv, 1), "write_kib": round(wv, 1), "dispatches": [fn, wn],
                          "hbm_bytes": round(b), "per_step": per_step}
        step += b * per_step
    out = {"workload": "decode_64k_b32", "source_sha256": source_sha256(),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "copy_probe_mib": int(copy_mib),
           "kernels": kernels, "step_traffic_bytes": round(step),
           "scan_traffic_bytes": kernels[SCAN_KERNEL]["hbm_bytes"]}
    with open(PMC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps({"step_traffic_bytes": out["step_traffic_bytes"],
                      "scan_traffic_bytes": out["scan_traffic_bytes"]}))


def build_replicas(ck, synth, w, cap, dev, n, idx_format=0, swa_format=0, k_format=0, prefill=False):
    """Entries-mode build of n identical cache replicas, one sequence at a time
    (each sequence's entries are drawn once and appended to every replica);
    prefill: each sequence's prefill tokens through the compressor instead."""
    import torch
    reps = [ck.Cache.allocate(w.batch, cap, w.k_group, w.v_group, w.idx_dim, idx_format=idx_format,
                              swa_format=swa_format, k_format=k_format) for _ in range(n)]
    if prefill:
        W = dev(synth.w_comp(w))
        for b in range(w.batch):
            toks = dev(synth.prefill_tokens(w, b, w.prefill_tokens))
            rows = dev(synth.prefill_idx_rows(w, b, w.prefill_tokens))
            cu = np.zeros(w.batch + 1, np.int32)
            cu[b + 1:] = w.prefill_tokens
            for c in reps:
                ck.kv_append_fp4(c, toks, dev(cu), W, rows)
        torch.cuda.synchronize()
        return reps
    for b in range(w.batch):
        ents = dev(synth.cache_entries(w, b))
        keys = dev(synth.cache_idx_keys(w, b))
        cu = np.zeros(w.batch + 1, np.int32)
        cu[b + 1:] = ents.shape[0]
        cu = dev(cu)
        for c in reps:
            ck.kv_append_fp4(c, ents, cu, None, keys)
    torch.cuda.synchronize()
    return reps


def scans_per_step(w, pool):
    """(full scans, pooled scans) one layer-group step runs."""
    full = pooled = 0
    have_pool = False
    for mode in w.layers:
        if mode == "full":
            full += 1
            have_pool = have_pool or pool is not None
        elif mode == "reindex":
            if have_pool:
                pooled += 1
            else:
                full += 1
    return full, pooled


def step_bytes(w, entries: float, pool=None, idx_fp4=False, swa_fp8=False, mx16=False) -> dict:
    """Algorithmic bytes of one step (whole batch): every plane read or written
    once by the method's definition; score arrays are not counted.  Scans: the
    whole indexer-key plane per full scan, the pooled positions' keys per
    pooled scan."""
    B, D, Dv, Di = w.batch, w.dim, w.vdim, w.idx_dim
    sb = 1 if mx16 else 4                      # bytes per group scale
    entry_fp4 = D // 2 + sb * (D // w.k_group)
    if w.v_group:
        entry_fp4 += Dv // 2 + sb * (Dv // w.v_group)
    full, pooled = scans_per_step(w, pool)
    L = len(w.layers)
    sel = sum(1 for m in w.layers if m != "reuse")
    pool_pos = min(entries, pool[0] * pool[1]) if pool else 0
    key_bytes = Di // 2 + Di // 16 if idx_fp4 else 2 * Di
    parts = {
        "indexer_keys": B * (full * entries + pooled * pool_pos) * key_bytes,
        "indexer_q": B * sel * w.idx_heads * Di * 2,
        "gather": L * B * min(w.topk, entries) * entry_fp4,
        "window": L * B * w.window * D * (1 if swa_fp8 else 2),
        "q": L * B * w.q_heads * D * 4,
        "out": L * B * w.q_heads * (Dv + 1) * 4,
        "indices": (sel + L) * B * w.topk * 4,
        # one token per sequence; a pair completes every other step, then the
        # compressor weights are read and one entry + indexer key written
        "append": B * (D * 4 * 2 + 0.5 * (entry_fp4 + key_bytes)) + 0.5 * D * 2 * D * 4,
    }
    parts["total"] = sum(parts.values())
    return parts


def cpu_baseline(synth, w, nseq: int, seconds: float, pool=None, idx_format=0, swa_format=0, k_format=0):
    """The oracle, as it is, on a bounded sample: nseq of the batch's sequences
    at full length, consecutive decode steps until `seconds` have passed (at
    least one); the cache build is untimed."""
    import oracle as orc
    nseq = w.batch if nseq <= 0 else max(1, min(nseq, w.batch))
    seqs = list(range(nseq))
    sub = synth.scaled(w, batch=nseq)
    max_steps = 100
    cap = w.entries + max_steps // 2 + 8
    hc = orc.Cache.empty(nseq, cap, w.dim, w.rope_dim, w.k_group, w.v_group, w.idx_dim,
                         idx_format=idx_format, swa_format=swa_format, k_format=k_format)
    t0 = time.time()
    if w.prefill_tokens:                       # through the compressor, as on the GPU
        n = w.prefill_tokens
        orc.kv_append(hc, np.concatenate([synth.prefill_tokens(w, b, n) for b in seqs]),
                      (np.arange(nseq + 1) * n).astype(np.int32), synth.w_comp(w),
                      np.concatenate([synth.prefill_idx_rows(w, b, n) for b in seqs]))
        ents = None
    else:
        ents = np.concatenate([synth.cache_entries(w, b) for b in seqs])
        keys = np.concatenate([synth.cache_idx_keys(w, b) for b in seqs])
        cu = (np.arange(nseq + 1) * w.entries).astype(np.int32)
        orc.kv_append(hc, ents, cu, None, keys)
    log(f"cpu baseline: oracle cache build {time.time() - t0:.1f}s (untimed)")
    del ents
    st = synth.step_inputs(w, 0, seqs=seqs)
    W = synth.w_comp(w)
    rings = [r.copy() for r in st.swa_ring]
    if swa_format:                             # the same rows in E4M3, written by the oracle
        rings8 = []
        for r in rings:
            Bw, Ww, Dw = r.shape
            r8 = np.zeros((Bw, Ww, Dw), np.uint8)
            orc.swa_append(r8, (r.astype(np.uint32) << 16).view(np.float32).reshape(Bw * Ww, Dw),
                           (np.arange(Bw + 1) * Ww).astype(np.int32), np.full(Bw, Ww, np.int32))
            rings8.append(r8)
        rings = rings8
    n_steps = 0
    t0 = time.perf_counter()
    while True:
        orc.layer_group_decode(hc, sub.layers, st.token, st.idx_row, W, st.q, st.q_idx, rings,
                               st.swa_row, w.topk, 1 / math.sqrt(w.dim), pool=pool)
        n_steps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds or n_steps >= max_steps:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    per_full_step = dt / n_steps * w.batch / nseq
    cpu = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": 1.0 / per_full_step, "unit": "steps/s", "cores": min(threads, nseq),
            "kind": "oracle",
            "sample": f"{nseq} of {w.batch} sequences at full length ({w.entries} entries), {n_steps} "
                      f"consecutive {'+'.join(w.layers)} decode steps in {dt:.1f} s"
                      + (f", scaled by {w.batch}/{nseq}" if nseq != w.batch else "")
                      + f"; cache build untimed; OpenMP over sequences on {cpu}"}


def cpu_baseline_one_thread(workload: str, seconds: float):
    """The oracle on one host thread: a child process with OMP_NUM_THREADS=1
    runs cpu_baseline on one sequence of the workload (scaled to the batch)."""
    import subprocess
    code = ("import json, sys; sys.path.insert(0, %r); import bench, synth; w = synth.WORKLOADS[%r]\n"
            "if w.entries is None and w.prefill_tokens: w = synth.scaled(w, entries=(w.prefill_tokens + 1) // 2)\n"
            "print(json.dumps(bench.cpu_baseline(synth, w, 1, %r)))") % (ROOT, workload, seconds)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)
        r = json.loads(p.stdout.strip().splitlines()[-1])
        r["cores"] = 1
        return r
    except Exception as e:                      # reported, never fatal
        return {"error": str(e)[:200]}


def gpu_clocks(torch):
    """Current shader and memory clock levels of GPU 0 from its sysfs entry
    (best effort: None where they cannot be read)."""
    try:
        pr = torch.cuda.get_device_properties(0)
        dev = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (getattr(pr, "pci_domain_id", 0), pr.pci_bus_id,
                                                        pr.pci_device_id)
        out = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            with open(os.path.join(dev, name)) as f:
                cur = [ln.split(":", 1)[1].strip().rstrip("*").strip() for ln in f if ln.strip().endswith("*")]
            out[name[7:]] = cur[0] if cur else None
        return out
    except Exception:
        return None


def source_sha256() -> str:
    """SHA-256 over the library's kernel and ABI sources, in name order."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".cpp", ".hpp")):
            h.update(f.encode())
            h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def pmc_traffic():
    """HBM bytes of one 64K x 32 step and of one scan launch, from the
    committed counter summary (FETCH_SIZE and WRITE_SIZE scaled by a plain
    copy's readings), if it was taken on the current sources; else None."""
    if not os.path.exists(PMC_FILE):
        return None
    try:
        d = json.load(open(PMC_FILE))
        if d.get("source_sha256") != source_sha256():
            return None
        return d
    except Exception:
        return None


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the batch shards by sequence with no exchange, so N GPUs run N independent copies)",
              file=sys.stderr)
        sys.exit(2)
    if a.pmc_summary:
        pmc_summary(*a.pmc_summary)
        return
    if a.copy_probe:
        copy_probe(a.copy_probe)
        return

    import torch

    import compressed_sparse_kv_append_amd as ck
    import synth

    ck.lib()
    if a.workload == MODEL_PLAN:
        return main_model(a, ck, synth, torch)
    w = synth.WORKLOADS[a.workload]
    if w.chunk_tokens:
        return main_mixed(a, ck, synth, torch)
    prefill = w.entries is None and w.prefill_tokens
    if prefill:
        # the tiny workload: its cache is built from prefill tokens through
        # the compressor (an odd count: the last token waits as pending)
        w = synth.scaled(w, entries=(w.prefill_tokens + 1) // 2)
    assert w.entries is not None, "bench steps fixed-length workloads"
    mx16 = a.kv_format == "mx16"
    if mx16:
        w = synth.scaled(w, k_group=16, v_group=16 if w.v_group else 0)
    pool = tuple(int(x) for x in a.pool.split(",")) if a.pool else None
    timer_steps = min(a.steps, 100)
    dist_steps = min(a.steps, 100)
    total_steps = a.warmup + timer_steps + dist_steps + a.steps + a.replicas
    per_rep = (total_steps + a.replicas - 1) // a.replicas
    cap = w.entries + (per_rep + 1) // 2 + 16
    if a.capacity:
        assert a.capacity >= cap, f"--capacity {a.capacity} below the {cap} entries the steps need"
        cap = a.capacity

    def dev(x):
        x = np.ascontiguousarray(x)
        return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()

    t0 = time.time()
    idx_fp4 = a.idx_format == "fp4"
    swa_fp8 = a.swa_format == "fp8"
    reps = build_replicas(ck, synth, w, cap, dev, a.replicas, ck.IDX_FP4 if idx_fp4 else ck.IDX_BF16,
                          ck.SWA_FP8 if swa_fp8 else ck.SWA_BF16, ck.KV_MX16 if mx16 else ck.KV_F32,
                          prefill=prefill)
    log(f"built {a.replicas} cache replicas in {time.time() - t0:.1f}s (indexer keys {a.idx_format}, "
        f"window {a.swa_format}, main entries {a.kv_format})")

    def ring_of(r16):
        """A layer's window ring: the bf16 ring, or the same rows written in FP8
        by the library's own window append."""
        if not swa_fp8:
            return dev(r16)
        Bw, Ww, Dw = r16.shape
        rows = (r16.astype(np.uint32) << 16).view(np.float32).reshape(Bw * Ww, Dw)
        ring = torch.zeros(Bw, Ww, Dw, dtype=torch.uint8, device="cuda")
        ck.swa_append(ring, dev(rows), dev((np.arange(Bw + 1) * Ww).astype(np.int32)),
                      dev(np.full(Bw, Ww, np.int32)))
        return ring
    st = synth.step_inputs(w, 0)
    W = dev(synth.w_comp(w))
    scale = 1 / math.sqrt(w.dim)
    B = w.batch
    per_rep_io = []
    for r in range(a.replicas):
        layers = []
        for li, mode in enumerate(w.layers):
            layers.append(ck.Layer(mode=mode, q=dev(st.q[li]),
                                   q_idx=None if st.q_idx[li] is None else dev(st.q_idx[li]),
                                   swa=ring_of(st.swa_ring[li]), swa_row=dev(st.swa_row[li]),
                                   idx=torch.empty(B, w.topk, dtype=torch.int32, device="cuda")
                                   if mode != "reuse" else None,
                                   out=torch.empty(B, w.q_heads, w.vdim, device="cuda"),
                                   lse=torch.empty(B, w.q_heads, device="cuda")))
        per_rep_io.append(dict(layers=layers,
                               ws=ck.workspace(reps[r], w.topk, ck.OP_LAYER_GROUP, w.q_heads, w.window,
                                               pool=pool)))
    tok, irow = dev(st.token), dev(st.idx_row)

    def step(i):
        r = i % a.replicas
        io = per_rep_io[r]
        ck.layer_group_decode(reps[r], io["layers"], tok, W, irow, w.topk, w.window, scale, ws=io["ws"],
                              pool=pool)

    kinds = {"append": ck.KERNEL_APPEND, "swa_append": ck.KERNEL_SWA_APPEND,
             "indexer_scan": ck.KERNEL_INDEXER_SCAN, "topk_select": ck.KERNEL_TOPK_SELECT,
             "attention": ck.KERNEL_ATTENTION}
    i = 0
    for _ in range(a.warmup):
        step(i)
        i += 1
    torch.cuda.synchronize()

    graphs = []
    if a.graph:
        for r in range(a.replicas):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r)
            graphs.append(g)
        torch.cuda.synchronize()
        for r in range(a.replicas):          # one untimed replay per replica
            graphs[(i + r) % a.replicas].replay()
        i += a.replicas
        torch.cuda.synchronize()
    every = max(1, a.scan_sample_every)
    if not a.graph:
        ck.timer_enable(ck.KERNEL_INDEXER_SCAN, (a.steps + every - 1) // every)

    ent_before = np.mean([r.n_tokens.float().mean().item() for r in reps]) / 2
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for j in range(a.steps):
        if a.graph:
            graphs[(i + j) % a.replicas].replay()
        else:
            ck.timer_pause(ck.KERNEL_INDEXER_SCAN, j % every != 0)
            step(i + j)
    e1.record()
    torch.cuda.synchronize()
    i += a.steps
    ms = e0.elapsed_time(e1) / a.steps
    live = None
    if not a.graph:
        tot, n = ck.timer_read(ck.KERNEL_INDEXER_SCAN)
        live = {"avg_us": 1000 * tot / max(n, 1), "launches": n}
        ck.timer_disable_all()
    ent_after = np.mean([r.n_tokens.float().mean().item() for r in reps]) / 2

    # per-step distribution: events around each step of a separate pass
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(dist_steps)]
    torch.cuda.synchronize()
    for ev0, ev1 in evs:
        ev0.record()
        step(i)
        ev1.record()
        i += 1
    torch.cuda.synchronize()
    per_step = np.array([ev0.elapsed_time(ev1) * 1000.0 for ev0, ev1 in evs])

    # per-kernel breakdown: separate eager pass with every timer on
    for kd in kinds.values():
        ck.timer_enable(kd, timer_steps)
    for _ in range(timer_steps):
        step(i)
        i += 1
    torch.cuda.synchronize()
    kern = {}
    for name, kd in kinds.items():
        tot, n = ck.timer_read(kd)
        kern[name] = {"avg_us": 1000 * tot / max(n, 1), "launches": n}
    ck.timer_disable_all()
    status = [int(r.status[0].item()) for r in reps]
    assert all(s == 0 for s in status), f"cache status flags raised: {status}"

    # mean entries per sequence over the timed steps
    entries_mean = float(0.5 * (ent_before + ent_after))
    sb = step_bytes(w, entries_mean, pool, idx_fp4, swa_fp8, mx16)
    n_full, n_pooled = scans_per_step(w, pool)
    scan_bytes = (sb["indexer_keys"] + sb["indexer_q"]) / (n_full + n_pooled)   # per launch, averaged
    scan = live if live is not None else kern["indexer_scan"]
    scan_us = scan["avg_us"]
    achieved = scan_bytes / (scan_us * 1e-6) / 1e9
    steps_per_s = 1000.0 / ms
    step_gbps = sb["total"] / (ms * 1e-3) / 1e9
    plain = (w.name == "decode_64k_b32" and not idx_fp4 and pool is None and not swa_fp8 and not mx16
             and not a.capacity)
    pmc = pmc_traffic() if plain else None
    result = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; %s cache entries, integer indexer inputs)"
                % {"t3": "Student-t(3)", "normal": "N(0,1)", "outliers": "N(0,1) with 1% x20 outliers"}[w.entry_law]
                + (", built from prefill tokens through the compressor" if prefill else ""),
        "config": {"workload": w.name, "batch": B, "context_tokens": 2 * w.entries,
                   "entries_per_seq": w.entries, "k_group": w.k_group, "storage": "e2m1+e8m0/16" if mx16 else "e2m1+fp32 scales",
                   "idx_heads": w.idx_heads, "idx_dim": w.idx_dim, "q_heads": w.q_heads,
                   "topk": w.topk, "window": w.window, "replicas": a.replicas,
                   "launch": "hip_graph" if a.graph else "eager", "layers": list(w.layers),
                   "idx_storage": "e2m1+e8m0/16" if idx_fp4 else "bf16",
                   "window_storage": "e4m3" if swa_fp8 else "bf16",
                   "pool": list(pool) if pool else None,
                   "capacity": cap,
                   "tokens_per_s": round(steps_per_s * B, 1)},
        # the whole step: every kernel of one decode step
        "roofline": {"bound": "hbm", "achieved": round(step_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(step_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None if pmc is None else pmc["step_traffic_bytes"],
                     "traffic_source": None if pmc is None else "committed rocprofv3 FETCH_SIZE + WRITE_SIZE "
                     "summary of these sources (profiles/decode_step_64k_b32_pmc.json), not this run",
                     "kernel": "decode_step", "bytes_per_launch": round(sb["total"]), "avg_us": round(ms * 1000, 2),
                     "timing": "hip events around the timed steps"},
        # the largest kernel of the step
        "roofline_scan": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                          "traffic": None if pmc is None else pmc["scan_traffic_bytes"],
                          "kernel": "indexer_scan",
                          "bytes_per_launch": round(scan_bytes), "avg_us": round(scan_us, 2),
                          "timed_launches": scan["launches"], "scans_per_step": [n_full, n_pooled],
                          "timing": ("hip events in the timed region, 1 step in %d" % every) if live is not None
                          else "hip events, separate eager pass"},
        "step_us": {"p10": round(float(np.percentile(per_step, 10)), 2),
                    "p50": round(float(np.percentile(per_step, 50)), 2),
                    "p90": round(float(np.percentile(per_step, 90)), 2),
                    "steps": int(dist_steps), "timing": "hip events around each step, separate pass"},
        "step_bytes": round(sb["total"]),
        "step_hbm_frac": round(sb["total"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "kernels_us": {k: round(v["avg_us"], 2) for k, v in kern.items()},
    }
    if prefill:
        result["config"]["prefill_tokens"] = w.prefill_tokens
        result["config"]["context_tokens"] = w.prefill_tokens + 1
    result["gpu_clocks"] = gpu_clocks(torch)
    if not a.no_cpu_baseline:
        log("timing the oracle on a CPU sample ...")
        result["cpu_baseline"] = cpu_baseline(synth, w, a.cpu_baseline_seqs, a.cpu_baseline_seconds, pool,
                                              int(idx_fp4), int(swa_fp8), int(mx16))
        if w.name in ("tiny_t4096", "decode_64k_b32") and not (idx_fp4 or swa_fp8 or mx16 or pool):
            log("timing the oracle on one host thread ...")
            result["cpu_baseline_1thread"] = cpu_baseline_one_thread(w.name, 3.0)
    print(json.dumps(result), flush=True)


ALU_PEAK_TFLOPS = 157.3      # MI355X fp32 vector, packed FMAs: 256 CUs x 4 SIMDs x 16 lanes x 2 x 2 FLOP x 2.4 GHz
ALU_PEAK_UNPACKED_TFLOPS = 78.6   # the same without packed fp32 (the library compiles it off)
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix cores
MODEL_PLAN = "model_plan_64k_b32"


def filler_rows(torch, seed, n, dim, law):
    """fp32 [n, dim] on the GPU, seeded, with the workload's value law."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    z = torch.randn(n, dim, generator=g, device="cuda")
    if law == "t3":
        chi = torch.randn(n, dim, 3, generator=g, device="cuda").square().sum(-1)
        z = z / torch.sqrt(chi / 3)
    return z.contiguous()


def filler_keys(torch, seed, n, dim):
    """bf16 bits [n, dim] of integers uniform in [-8, 8], on the GPU, seeded."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(-8, 9, (n, dim), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16).contiguous()


def main_model(a, ck, synth, torch):
    """One decode step of the pages' whole CSA2 layer plan at the 64K x 32
    size: three encoder caches of 32,768 entries (2->1 compression, Full + 5
    Reuse each) and the decoder cache of 65,536 entries (one per token, the
    new entry from the CED projection of a 4096-wide hidden state), read by
    Full + 3 Reuse and four Reindex + 3 Reuse groups: 38 layers, one
    cskv_model_decode call per step.  Student-t(3) entries, integer indexer
    keys and queries, N(0,1) queries and window rows, drawn on the GPU with
    seeded generators (the caches are too large to draw on the host in
    reasonable time); token counts are restored between steps outside the
    timed region so every step sees the same caches."""
    B, T, kg, Di, Hi, Hq, K, W, dm = 32, 65536, 64, 128, 64, 64, 512, 128, 4096
    pool = tuple(int(x) for x in a.pool.split(",")) if a.pool else None
    plan = synth.CSA2_PLAN
    scale = 1 / math.sqrt(576)
    t0 = time.time()
    groups, seed = [], 7000
    Wc = filler_rows(torch, seed, 576, 1152, "normal") * 0.02
    n_layers = 0
    for gi, (name, ratio, modes) in enumerate(plan):
        E = T // ratio
        c = ck.Cache.allocate(B, E + 64, kg, 0, Di, ratio=ratio)
        for b in range(B):
            seed += 1
            cu = np.zeros(B + 1, np.int32)
            cu[b + 1:] = E
            ck.kv_append_fp4(c, filler_rows(torch, seed, E, 576, "t3"), torch.from_numpy(cu).cuda(), None,
                             filler_keys(torch, seed + 500_000, E, Di))
        layers = []
        for li, m in enumerate(modes):
            seed += 1
            layers.append(ck.Layer(mode=m, q=filler_rows(torch, seed, B * Hq, 576, "normal").view(B, Hq, 576),
                                   q_idx=None if m == "reuse" else filler_keys(torch, seed + 1, B * Hi, Di).view(B, Hi, Di),
                                   swa=filler_rows(torch, seed + 2, B * W, 576, "normal").to(torch.bfloat16)
                                   .view(torch.int16).view(B, W, 576).contiguous(),
                                   swa_row=filler_rows(torch, seed + 3, B, 576, "normal"),
                                   idx=None if m == "reuse" else torch.empty(B, K, dtype=torch.int32, device="cuda"),
                                   out=torch.empty(B, Hq, 512, device="cuda"), lse=torch.empty(B, Hq, device="cuda")))
        n_layers += len(modes)
        grp = ck.Group(cache=c, layers=layers, new_idx_rows=filler_keys(torch, seed + 4, B, Di),
                       pool=pool if "reindex" in modes else None)
        if ratio == 1:
            grp.ced_h = filler_rows(torch, seed + 5, B, dm, "normal").to(torch.bfloat16).view(torch.int16).contiguous()
            grp.ced_w = (filler_rows(torch, seed + 6, 576, dm, "normal") * 0.02).to(torch.bfloat16).view(torch.int16).contiguous()
        else:
            grp.new_tokens, grp.w_comp = filler_rows(torch, seed + 5, B, 576, "normal"), Wc
        groups.append(grp)
    torch.cuda.synchronize()
    log(f"built {len(plan)} caches for {n_layers} layers in {time.time() - t0:.1f}s")
    n0 = [g.cache.n_tokens.clone() for g in groups]
    ws = ck.model_workspace(groups, K, W)

    def step():
        ck.model_decode(groups, K, W, scale, ws=ws)

    def reset():
        for g, n in zip(groups, n0):
            g.cache.n_tokens.copy_(n)

    for _ in range(a.warmup):
        step()
        reset()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    for e0, e1 in ev:
        e0.record()
        step()
        e1.record()
        reset()
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) * 1000.0 for e0, e1 in ev])
    kinds = {"append": ck.KERNEL_APPEND, "indexer_scan": ck.KERNEL_INDEXER_SCAN,
             "topk_select": ck.KERNEL_TOPK_SELECT, "attention": ck.KERNEL_ATTENTION}
    reps = min(a.steps, 20)
    for kd in kinds.values():
        ck.timer_enable(kd, 64 * reps)
    for _ in range(reps):
        step()
        reset()
    torch.cuda.synchronize()
    kern, scan_launches = {}, 0
    for name, kd in kinds.items():
        tot, cnt = ck.timer_read(kd)
        kern[name] = 1000 * tot / reps
        if name == "indexer_scan":
            scan_us, scan_launches = 1000 * tot / max(cnt, 1), cnt // reps
    ck.timer_disable_all()
    status = [int(g.cache.status[0].item()) for g in groups]
    assert all(x == 0 for x in status), f"cache status flags raised: {status}"
    # algorithmic bytes of the step's scans: every full scan reads its cache's
    # indexer keys (entries after the append), pooled scans the pooled rows
    full_bytes, pooled_bytes = 0.0, 0.0
    for (name, ratio, modes), g in zip(plan, groups):
        E = T // ratio + 1
        have_pool = False
        for m in modes:
            if m == "full":
                full_bytes += B * (E * 2 * Di + Hi * Di * 2)
                have_pool = pool is not None
            elif m == "reindex":
                if have_pool:
                    pooled_bytes += B * (min(E, pool[0] * pool[1]) * 2 * Di + Hi * Di * 2)
                else:
                    full_bytes += B * (E * 2 * Di + Hi * Di * 2)
    scan_total = full_bytes + pooled_bytes
    achieved = scan_total / scan_launches / (scan_us * 1e-6) / 1e9 if scan_launches else 0.0
    ms = float(t.mean()) / 1000.0
    result = {
        "metric": "CSA2 FP4 layer-plan decode: steps/s (all 38 layers, 4 caches) at 64K ctx",
        "value": round(1000.0 / ms, 2), "unit": "steps/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded GPU generators; Student-t(3) entries, integer indexer inputs)",
        "config": {"workload": MODEL_PLAN, "batch": B, "context_tokens": T, "k_group": kg, "idx_heads": Hi,
                   "idx_dim": Di, "q_heads": Hq, "topk": K, "window": W, "ced_d_model": dm,
                   "caches": [[n, r, len(m)] for n, r, m in plan], "layers": n_layers,
                   "pool": list(pool) if pool else None, "launch": "eager",
                   "tokens_per_s": round(1000.0 / ms * B, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": "indexer_scan",
                     "bytes_per_step": round(scan_total), "scans_per_step": scan_launches,
                     "avg_us": round(scan_us, 2), "timing": "hip events, separate eager pass"},
        "step_us": {"p10": round(float(np.percentile(t, 10)), 2), "p50": round(float(np.percentile(t, 50)), 2),
                    "p90": round(float(np.percentile(t, 90)), 2), "timing": "hip events around each step"},
        "kernels_us_per_step": {k: round(v, 2) for k, v in kern.items()},
    }
    if not a.no_cpu_baseline:
        log("timing the oracle on a CPU sample ...")
        result["cpu_baseline"] = model_cpu_baseline(synth, plan, B, T, kg, Di, Hi, Hq, K, W, 512, pool)
    print(json.dumps(result), flush=True)


def model_cpu_baseline(synth, plan, B, T, kg, Di, Hi, Hq, K, W, dm, pool):
    """The oracle's model decode on a bounded sample: 2 of the batch's
    sequences at full length in every cache (drawn with the host generators),
    one step, scaled by B / 2; the cache build is untimed.  The CED width is
    512 on the host (its cost is negligible beside the scans)."""
    import oracle as orc
    nseq = 2
    g = np.random.default_rng(7000)
    hgroups = []
    for name, ratio, modes in plan:
        E = T // ratio
        hc = orc.Cache.empty(nseq, E + 8, 576, 64, kg, 0, Di, ratio=ratio)
        for b in range(nseq):
            cu = np.zeros(nseq + 1, np.int32)
            cu[b + 1:] = E
            orc.kv_append(hc, synth.student_t3(g, (E, 576)), cu, None, synth.int_bf16(g, (E, Di)))
        L = len(modes)
        hg = dict(cache=hc, modes=modes, q=[synth.normal(g, (nseq, Hq, 576)) for _ in range(L)],
                  q_idx=[None if m == "reuse" else synth.int_bf16(g, (nseq, Hi, Di)) for m in modes],
                  rings=[synth.normal_bf16_trunc(g, (nseq, W, 576)) for _ in range(L)],
                  swa_rows=[synth.normal(g, (nseq, 576)) for _ in range(L)], idx_row=synth.int_bf16(g, (nseq, Di)))
        if ratio == 1:
            hg.update(ced_h=synth.int_bf16(g, (nseq, dm)), ced_w=synth.int_bf16(g, (576, dm)))
        else:
            hg.update(token=synth.normal(g, (nseq, 576)), w_comp=(g.standard_normal((576, 1152)) * 0.02).astype(np.float32))
        hgroups.append(hg)
    t0 = time.perf_counter()
    orc.model_decode(hgroups, K, 1 / math.sqrt(576), pool=pool)
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": 1.0 / (dt * B / nseq), "unit": "steps/s", "cores": min(threads, nseq), "kind": "oracle",
            "sample": f"{nseq} of {B} sequences at full length in all {len(plan)} caches, one step of all layers "
                      f"in {dt:.1f} s, scaled by {B}/{nseq}; cache build untimed"}


def build_ragged(ck, synth, w, cap, dev, torch, page=0, need=None):
    """Entries-mode build of the ragged cache, one sequence per call; the
    sequences' rows are drawn on host threads while earlier ones upload.
    page > 0: paged planes holding only the pages each sequence needs
    (need[b] entries), handed out in sequence order; unmapped table entries
    are -1."""
    import concurrent.futures as cf
    E = synth.entry_counts(w)
    if page:
        max_pages = (cap + page - 1) // page
        cap = max_pages * page
        per = [(int(n) + page - 1) // page for n in need]
        table = np.full((w.batch, max_pages), -1, np.int32)
        nxt = 0
        for b, k in enumerate(per):
            table[b, :k] = np.arange(nxt, nxt + k)
            nxt += k
        gc = ck.Cache.allocate_paged(w.batch, cap, page, nxt, dev(table), w.k_group, w.v_group, w.idx_dim)
    else:
        gc = ck.Cache.allocate(w.batch, cap, w.k_group, w.v_group, w.idx_dim)

    def draw(b):
        return synth.cache_entries(w, b), synth.cache_idx_keys(w, b)
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        for b, (ents, keys) in enumerate(ex.map(draw, range(w.batch))):
            cu = np.zeros(w.batch + 1, np.int32)
            cu[b + 1:] = int(E[b])
            ck.kv_append_fp4(gc, dev(ents), dev(cu), None, dev(keys))
    torch.cuda.synchronize()
    return gc


def mixed_cpu_baseline(synth, w, seconds: float):
    """The oracle on a bounded sample of the mixed step: the whole chunk append
    of sequence 0 through the compressor, then the decode step of the first
    nseq sequences (nseq grown until the sample takes about `seconds`); the
    cache build is untimed."""
    import oracle as orc
    E = synth.entry_counts(w)
    W = synth.w_comp(w)
    n = w.chunk_tokens
    toks, irows = synth.prefill_tokens(w, 0, n), synth.prefill_idx_rows(w, 0, n)
    nseq = 16
    cap = int(E[:nseq].max()) + n // 2 + 8
    hc = orc.Cache.empty(nseq, cap, w.dim, w.rope_dim, w.k_group, w.v_group, w.idx_dim)
    for b in range(nseq):
        cu = np.zeros(nseq + 1, np.int32)
        cu[b + 1:] = int(E[b])
        orc.kv_append(hc, synth.cache_entries(w, b), cu, None, synth.cache_idx_keys(w, b))
    cu = np.zeros(nseq + 1, np.int32)
    cu[1:] = n
    t0 = time.perf_counter()
    orc.kv_append(hc, toks, cu, W, irows)
    t_app = time.perf_counter() - t0
    sub = synth.scaled(w, batch=nseq)
    st = synth.step_inputs(w, 0, seqs=range(nseq))
    rings = [r.copy() for r in st.swa_ring]
    t0 = time.perf_counter()
    orc.layer_group_decode(hc, sub.layers, st.token, st.idx_row, W, st.q, st.q_idx, rings, st.swa_row,
                           w.topk, 1 / math.sqrt(w.dim))
    t_dec = time.perf_counter() - t0
    # decode time scales with the batch's entries (the scan dominates)
    t_dec_full = t_dec * float(E.sum() + n // 2) / float(E[:nseq].sum() + n // 2)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": 1.0 / (t_app + t_dec_full), "unit": "steps/s", "cores": min(threads, nseq),
            "kind": "oracle",
            "sample": f"chunk append of {n} tokens through the compressor ({t_app:.1f} s, one thread: "
                      f"one sequence), then the decode step of {nseq} of {w.batch} sequences "
                      f"({t_dec:.1f} s), scaled to the batch's {int(E.sum())} entries by entry count; "
                      "cache build untimed"}


def main_mixed(a, ck, synth, torch):
    """Mixed append + decode on the ragged batch: one step = the chunk of
    w.chunk_tokens tokens appended to sequence 0 through the compressor
    together with one token on every other sequence (one kv_append call),
    then one Full-layer decode step of the whole batch.  The sequences'
    token counts are restored between steps, outside the timed intervals, so
    every step sees the same cache; each step is timed with HIP events on
    the launch stream (append, decode, both)."""
    w = synth.WORKLOADS[a.workload]
    E = synth.entry_counts(w)
    B, n = w.batch, w.chunk_tokens
    cap = int(E.max()) + n // 2 + 16

    def dev(x):
        x = np.ascontiguousarray(x)
        return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()

    t0 = time.time()
    # entries each sequence reaches: the chunk's on sequence 0, then one per
    # pair of decode tokens (a few spare)
    need = E + 16
    need[0] += n // 2
    gc = build_ragged(ck, synth, w, cap, dev, torch, page=a.paged, need=need)
    plane_bytes = sum(t.numel() * t.element_size() for t in (gc.k_codes, gc.k_scales, gc.v_codes, gc.v_scales,
                                                              gc.idx_keys) if t is not None)
    log(f"built the ragged cache ({int(E.sum())} entries over {B} sequences, "
        f"{plane_bytes / 2**30:.2f} GiB of planes{', paged' if a.paged else ''}) in {time.time() - t0:.1f}s")
    lens = np.array([n] + [1] * (B - 1), np.int64)
    cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    toks = torch.empty(int(cu_h[-1]), w.dim, device="cuda")
    irows = torch.empty(int(cu_h[-1]), w.idx_dim, dtype=torch.int16, device="cuda")
    toks[:n] = dev(synth.prefill_tokens(w, 0, n))
    irows[:n] = dev(synth.prefill_idx_rows(w, 0, n))
    for b in range(1, B):
        toks[cu_h[b]:cu_h[b + 1]] = dev(synth.prefill_tokens(w, b, 1))
        irows[cu_h[b]:cu_h[b + 1]] = dev(synth.prefill_idx_rows(w, b, 1))
    cu = dev(cu_h)
    W = dev(synth.w_comp(w))
    app_ws = ck.append_workspace(int(cu_h[-1]), W)
    st = synth.step_inputs(w, 0)
    layers = [ck.Layer(mode="full", q=dev(st.q[0]), q_idx=dev(st.q_idx[0]), swa=dev(st.swa_ring[0]),
                       swa_row=dev(st.swa_row[0]), idx=torch.empty(B, w.topk, dtype=torch.int32, device="cuda"),
                       out=torch.empty(B, w.q_heads, w.vdim, device="cuda"),
                       lse=torch.empty(B, w.q_heads, device="cuda"))]
    tok, irow = dev(st.token), dev(st.idx_row)
    scale = 1 / math.sqrt(w.dim)
    n0 = gc.n_tokens.clone()
    gws = ck.workspace(gc, w.topk, ck.OP_LAYER_GROUP, w.q_heads, w.window)

    def append():
        ck.kv_append_fp4(gc, toks, cu, W, irows, ws=app_ws, mfma=a.mfma_compressor)

    def decode():
        ck.layer_group_decode(gc, layers, tok, W, irow, w.topk, w.window, scale, ws=gws)

    def reset():
        gc.n_tokens.copy_(n0)

    for _ in range(a.warmup):
        append()
        decode()
        reset()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    for e in ev:
        e[0].record()
        append()
        e[1].record()
        decode()
        e[2].record()
        reset()
    torch.cuda.synchronize()
    t_app = np.array([e[0].elapsed_time(e[1]) * 1000.0 for e in ev])
    t_dec = np.array([e[1].elapsed_time(e[2]) * 1000.0 for e in ev])
    t_step = np.array([e[0].elapsed_time(e[2]) * 1000.0 for e in ev])

    # per-kernel pass: the compressor alone, then the other kinds
    kinds = {"compress": ck.KERNEL_COMPRESS, "append": ck.KERNEL_APPEND,
             "indexer_scan": ck.KERNEL_INDEXER_SCAN, "topk_select": ck.KERNEL_TOPK_SELECT,
             "attention": ck.KERNEL_ATTENTION}
    reps = min(a.steps, 50)
    for kd in kinds.values():
        ck.timer_enable(kd, 2 * reps)
    for _ in range(reps):
        append()
        decode()
        reset()
    torch.cuda.synchronize()
    kern = {}
    for name, kd in kinds.items():
        tot, cnt = ck.timer_read(kd)
        kern[name] = 1000 * tot / max(cnt, 1) * (cnt / reps)     # per step
    ck.timer_disable_all()
    status = int(gc.status[0].item())
    assert status == 0, f"cache status flag raised: {status}"

    # algorithmic work of one step.  The token counts start even, so the
    # append completes the chunk's n/2 entries and leaves the other sequences'
    # tokens pending; the decode step's token completes their pairs and waits
    # in sequence 0.
    D = w.dim
    entry_b = D // 2 + 4 * (D // w.k_group) + w.vdim // 2 + 4 * (w.vdim // w.v_group)
    key_b = 2 * w.idx_dim
    comp_entries = n // 2 + (B - 1)
    comp_flops = 2.0 * comp_entries * D * 2 * D
    E_dec = float(E.sum() + n // 2 + B - 1)     # entries the decode scans
    scan_bytes = E_dec * key_b + B * w.idx_heads * w.idx_dim * 2
    dec_bytes = (scan_bytes + B * w.topk * entry_b + B * w.window * D * 2 + B * w.q_heads * D * 4
                 + B * w.q_heads * (w.vdim + 1) * 4 + B * (D * 4 * 2 + key_b) + (B - 1) * (entry_b + key_b))
    app_bytes = int(cu_h[-1]) * (D * 4 + key_b) + D * 2 * D * 4 + (n // 2) * (entry_b + key_b)
    ms = float(t_step.mean()) / 1000.0
    scan_us, comp_us = kern["indexer_scan"], kern["compress"]
    comp_tflops = comp_flops / (comp_us * 1e-6) / 1e12
    scan_gbps = scan_bytes / (scan_us * 1e-6) / 1e9
    if a.mfma_compressor:
        # algorithmic FLOP over the bf16 matrix peak; each term is issued as
        # three bf16 products (hi*hi + hi*lo + lo*hi)
        comp_roof = {"bound": "mfma", "achieved": round(comp_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(comp_tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "issued_flops_per_step": round(3 * comp_flops),
                     "kernel": "compress_mfma", "flops_per_step": round(comp_flops), "avg_us": round(comp_us, 2),
                     "timing": "hip events on the compressor's launch, separate eager pass"}
    else:
        comp_roof = {"bound": "alu", "achieved": round(comp_tflops, 2), "peak": ALU_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(comp_tflops / ALU_PEAK_TFLOPS, 4), "traffic": None,
                     "peak_unpacked": ALU_PEAK_UNPACKED_TFLOPS,
                     "frac_unpacked": round(comp_tflops / ALU_PEAK_UNPACKED_TFLOPS, 4),
                     "kernel": "compress", "flops_per_step": round(comp_flops), "avg_us": round(comp_us, 2),
                     "timing": "hip events on the compressor's launch, separate eager pass"}
    result = {
        "metric": "CSA2 FP4 mixed append + decode: steps/s on the ragged batch",
        "value": round(1000.0 / ms, 2), "unit": "steps/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16x3 matrix-core compressor" if a.mfma_compressor else "f32 compressor")
        + ", bf16 scan and attention",
        "data": "synthetic (seeded; N(0,1) tokens and entries with 1% x20 outliers, integer indexer inputs)",
        "config": {"workload": w.name, "batch": B, "token_range": list(w.ragged_tokens),
                   "entries_total": int(E.sum()), "chunk_tokens": n, "k_group": w.k_group,
                   "v_group": w.v_group, "idx_heads": w.idx_heads, "idx_dim": w.idx_dim,
                   "q_heads": w.q_heads, "topk": w.topk, "window": w.window, "launch": "eager",
                   "layers": ["full"], "compressor": "mfma" if a.mfma_compressor else "exact",
                   "page_size": a.paged, "plane_bytes": plane_bytes},
        "roofline": comp_roof,
        "roofline_scan": {"bound": "hbm", "achieved": round(scan_gbps, 1), "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": round(scan_gbps / HBM_PEAK_GBPS, 4),
                          "bytes_per_launch": round(scan_bytes), "avg_us": round(scan_us, 2)},
        "step_us": {k: {"p10": round(float(np.percentile(v, 10)), 2), "p50": round(float(np.percentile(v, 50)), 2),
                        "p90": round(float(np.percentile(v, 90)), 2)}
                    for k, v in (("append", t_app), ("decode", t_dec), ("step", t_step))},
        "append_bytes": round(app_bytes), "decode_bytes": round(dec_bytes),
        "decode_hbm_frac": round(dec_bytes / (float(t_dec.mean()) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "kernels_us": {k: round(v, 2) for k, v in kern.items()},
    }
    if not a.no_cpu_baseline:
        log("timing the oracle on a CPU sample ...")
        result["cpu_baseline"] = mixed_cpu_baseline(synth, w, a.cpu_baseline_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
