"""Benchmark: bifocal prefill TFLOP/s on a 128K Qwen3-8B attention layer and
bifocal decode GB/s over a 128K KV cache, on one MI355X.

One step = one bifocal prefill (32 query / 8 KV heads, head_dim 128,
L = 131072, w_pre = 32768 so s = 4, w0 = 4096, rope_theta 1e6, frequency
interpolation, bf16) plus one bifocal decode of one query per head over the
same layer's cache of N = 131073 keys (the new token's own key included, so
s = 5). Inputs are seeded N(0,1) bf16 (synthetic), resident in HBM before the
timed region.

Prints one JSON line. `value` is the prefill effective TFLOP/s: algorithmic
flops 4 * D * Hq * L (L + 1) / 2 (one score and one PV product per causal
pair) over the measured prefill time. Extra fields report the decode
bandwidth, position aliasing, the library's plain causal attention on the
same shapes (overhead reference), chunks of the last 512 / 4096 / 16384
queries against the 128K cache (contiguous and, for 512 / 4096, over 16-key
pages; each also with a chunk store that holds k'' and V^T of the keys
before the chunk), roofline
fractions against MI355X peaks
(bf16 dense MFMA 2.5 PFLOP/s, HBM 8 TB/s) and the fp64 CPU oracle timed on a
bounded row sample of the prefill workload.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from rope_context_extension_bifocal_amd import bifocal as bfl  # noqa: E402
from rope_context_extension_bifocal_amd import workloads as wl  # noqa: E402

METRIC = "bifocal prefill TFLOP/s + % MFMA peak @128K Qwen3-8B layer; decode GB/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
_CSRC = "rope_context_extension_bifocal_amd/csrc/"
# sources each measured kernel is built from: its counters go stale when one changes
KERNEL_SOURCES = {"prefill_bf16_kernel_bifocal": [_CSRC + "prefill.hip", _CSRC + "capi.cpp", _CSRC + "bf_common.h"],
                  "decode_split_kernel_bifocal": [_CSRC + "decode.hip", _CSRC + "capi.cpp", _CSRC + "bf_common.h"],
                  "rope_kernel": [_CSRC + "rope.hip", _CSRC + "capi.cpp", _CSRC + "bf_common.h"]}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    only if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_hash") != source_hash(KERNEL_SOURCES[kernel_key]):
        return None
    return ent.get("bytes_per_launch")


COPY_BYTES = 256 * 1024 * 1024
# kernels whose HBM traffic is reported: key -> substring of the kernel name
TRAFFIC_KERNELS = {"prefill_bf16_kernel_bifocal": "prefill_bf16_kernel<true, false>",
                   "decode_split_kernel_bifocal": "decode_split_kernel<true, false, true, false>",
                   "rope_kernel": "rope_kernel",
                   "copy": "copyBuffer"}


def _pmc_kib_per_dispatch(run_dir, counter, name_part):
    """Average value of one counter per dispatch of the kernels whose name
    contains name_part, over every counter_collection.csv under run_dir."""
    import csv
    import glob
    vals = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter or name_part not in row.get("Kernel_Name", ""):
                    continue
                key = row.get("Dispatch_Id") or row.get("Correlation_Id")
                vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for '{name_part}' under {run_dir}")
    return sum(vals.values()) / len(vals), len(vals)


def write_traffic(root):
    """profiles/traffic.json from the rocprofv3 --pmc runs under root:
    {copy,prefill,decode,rope}_{fetch,write}. FETCH_SIZE and WRITE_SIZE are KiB per
    dispatch; each is scaled by the factor that makes the 256 MiB copy read and
    write 256 MiB."""
    kib = COPY_BYTES / 1024.0
    cf, _ = _pmc_kib_per_dispatch(os.path.join(root, "copy_fetch"), "FETCH_SIZE", TRAFFIC_KERNELS["copy"])
    cw, _ = _pmc_kib_per_dispatch(os.path.join(root, "copy_write"), "WRITE_SIZE", TRAFFIC_KERNELS["copy"])
    f_fetch, f_write = kib / cf, kib / cw
    out = {"fetch_factor": round(f_fetch, 4),
           "write_factor": round(f_write, 4),
           "copy_calibration_kib": {"fetch": round(cf, 1), "write": round(cw, 1), "true": kib}}
    for key, leg in (("prefill_bf16_kernel_bifocal", "prefill"), ("decode_split_kernel_bifocal", "decode"),
                     ("rope_kernel", "rope")):
        if not os.path.isdir(os.path.join(root, f"{leg}_fetch")):
            log(f"no {leg}_fetch run under {root}: {key} left out")
            continue
        fk, nf = _pmc_kib_per_dispatch(os.path.join(root, f"{leg}_fetch"), "FETCH_SIZE", TRAFFIC_KERNELS[key])
        wk, nw = _pmc_kib_per_dispatch(os.path.join(root, f"{leg}_write"), "WRITE_SIZE", TRAFFIC_KERNELS[key])
        out[key] = {"source_hash": source_hash(KERNEL_SOURCES[key]), "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                    "dispatches": [nf, nw],
                    "bytes_per_launch": round((fk * f_fetch + wk * f_write) * 1024.0)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def time_calls(fn, n, stream):
    """Average ms of fn() over n calls, hipEvents on the stream the library
    launches on (torch's current stream)."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(n):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n


def _oracle_sampled(q, k, v, cu, cfg, mode, target_s, seed, what):
    """The oracle on seeded samples of query rows (all heads) of a packed
    prefill workload. A small sample and a large one (grown until a run takes
    at least target_s) separate the oracle's fixed key / value setup (rotating
    every key up to the sampled rows) from its cost per causal pair; the
    value is the pair rate, and the full workload's time is extrapolated as
    setup + pairs x cost per pair."""
    import oracle

    kf, vf = k.float().numpy(), v.float().numpy()
    cu_a = np.asarray(cu)
    T, D = cu[-1], q.shape[-1]
    rng = np.random.default_rng(seed)

    last = cu_a[1:] - 1  # every sample holds each sequence's last row: the same key setup

    def run(n):
        rows = np.unique(np.concatenate([last, rng.choice(T, size=min(n, T), replace=False)]))
        rows = rows.astype(np.int64)
        q_rows = q[:, torch.from_numpy(rows)].float().numpy()
        t0 = time.perf_counter()
        oracle.prefill(q_rows, kf, vf, cu, cfg["w0"], cfg["w_pre"], cfg["theta"], mode,
                       1 / math.sqrt(D), rows=rows, gathered=True)
        dt = time.perf_counter() - t0
        seq = np.searchsorted(cu_a, rows, side="right") - 1
        return rows, int(q.shape[0] * (rows - cu_a[seq] + 1).sum()), dt

    _, pairs_a, t_a = run(16)
    n = 48
    while True:
        rows, pairs_b, t_b = run(n)
        if t_b >= target_s or n >= 4096:
            break
        n = int(min(4096, n * max(2.0, 1.2 * target_s / max(t_b, 1e-3))))
    per_pair = max((t_b - t_a) / max(pairs_b - pairs_a, 1), 1e-15)
    setup = max(t_a - per_pair * pairs_a, 0.0)
    full_pairs = q.shape[0] * sum((cu[i + 1] - cu[i]) * (cu[i + 1] - cu[i] + 1) / 2
                                  for i in range(len(cu) - 1))
    return {"mode": "sampled rows, extrapolated", "value": round(4.0 * D / per_pair / 1e12, 6),
            "unit": "TFLOP/s", "seconds": round(t_a + t_b, 2), "setup_seconds": round(setup, 2),
            "extrapolated_full_seconds": round(setup + per_pair * full_pairs, 1),
            "sample": f"{len(rows)} seeded query rows x {q.shape[0]} heads of {what} ({pairs_b} "
                      f"causal pairs), after a smaller run with the same last rows that separates the key setup"}


def cpu_baseline(q3, k3, v3, budget_s=15.0):
    """The fp64 oracle as it stands, timed on the host cores, per workload:
    the tiny fp32 prefill and the three decode caches in full, the 32K, 128K
    and ragged prefills on seeded row samples (time extrapolated to the whole
    workload). The headline value is the 128K FI prefill's."""
    import oracle

    per = {}
    c3 = wl.CONFIGS["qwen3_8b_prefill_128k"]
    L3 = c3["lens"][0]
    per["qwen3_8b_prefill_128k"] = _oracle_sampled(q3, k3, v3, [0, L3], c3, "fi", budget_s * 0.35, 7,
                                                   "the 128K FI prefill")
    c2 = wl.CONFIGS["qwen3_1p7b_prefill_32k_s1"]
    q2, k2, v2 = wl.prefill_inputs(c2["Hq"], c2["Hkv"], c2["lens"][0], c2["D"], "bf16", c2["seed"])
    per["qwen3_1p7b_prefill_32k_s1"] = _oracle_sampled(q2, k2, v2, [0, c2["lens"][0]], c2, "fi",
                                                       budget_s * 0.2, 8, "the 32K s = 1 prefill")
    del q2, k2, v2
    c5 = wl.CONFIGS["qwen3_4b_ragged_prefill"]
    lens5 = wl.ragged_lengths(c5["n_seqs"], c5["len_lo"], c5["len_hi"], c5["seed"])
    cu5 = wl.cu_seqlens(lens5)
    q5, k5, v5 = wl.prefill_inputs(c5["Hq"], c5["Hkv"], cu5[-1], c5["D"], "bf16", c5["seed"])
    per["qwen3_4b_ragged_prefill"] = _oracle_sampled(q5, k5, v5, cu5, c5, "fi", budget_s * 0.2, 9,
                                                     "the ragged 8-sequence prefill")
    del q5, k5, v5
    c1 = wl.CONFIGS["tiny_fp32_s2"]
    L1 = c1["lens"][0]
    q1, k1, v1 = (x.numpy() for x in wl.prefill_inputs(c1["Hq"], c1["Hkv"], L1, c1["D"], "fp32",
                                                       c1["seed"]))
    t0 = time.perf_counter()
    oracle.prefill(q1, k1, v1, [0, L1], c1["w0"], c1["w_pre"], c1["theta"], "fi",
                   1 / math.sqrt(c1["D"]))
    dt = time.perf_counter() - t0
    per["tiny_fp32_s2"] = {"mode": "full", "value": round(4.0 * 128 * c1["Hq"] * L1 * (L1 + 1) / 2 / dt / 1e12, 6),
                           "unit": "TFLOP/s", "seconds": round(dt, 3)}
    cd = wl.CONFIGS["qwen3_8b_decode"]
    for i, Lc in enumerate(cd["cache_lens"]):
        N = Lc + 1
        qd, kc, vc = (x.float().numpy() for x in wl.decode_inputs(1, cd["Hq"], cd["Hkv"], N, 128,
                                                                  "bf16", cd["seed"] + i))
        t0 = time.perf_counter()
        oracle.decode(qd, kc, vc, [N], cd["w0"], cd["w_pre"], cd["theta"], "fi", 1 / math.sqrt(128))
        dt = time.perf_counter() - t0
        per[f"qwen3_8b_decode_{N}"] = {"mode": "full", "value": round(2.0 * N * cd["Hkv"] * 128 * 2 / dt / 1e9, 3),
                                       "unit": "GB/s", "seconds": round(dt, 3)}
    head = per["qwen3_8b_prefill_128k"]
    return {"value": head["value"], "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "seconds": round(sum(r["seconds"] for r in per.values()), 2),
            "sample": head["sample"], "per_config": per}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "copy", "rope"], default=None,
                    help="run only this leg (W warmup + K calls, no JSON line); for profilers. "
                         "'copy' is a plain 256 MiB device copy that calibrates the HBM counters")
    ap.add_argument("--write-traffic", metavar="DIR", default=None,
                    help="read the rocprofv3 --pmc runs under DIR (see profiles/hbm_traffic.txt) "
                         "and write profiles/traffic.json; needs no GPU")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the per-GPU shard is the single-GPU workload). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.only == "copy":  # counter calibration: read 256 MiB, write 256 MiB per call
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"only copy: {args.warmup} + {args.steps} copies of {COPY_BYTES} bytes done")
        return
    bfl.lib()
    stream = torch.cuda.current_stream()

    cfg = wl.CONFIGS["qwen3_8b_prefill_128k"]
    dcfg = wl.CONFIGS["qwen3_8b_decode"]
    L = cfg["lens"][0]
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    scale = 1 / math.sqrt(D)
    log("generating 128K prefill inputs")
    q, k, v = wl.prefill_inputs(Hq, Hkv, L, D, "bf16", cfg["seed"])
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cu = [0, L]
    o = torch.empty_like(qd)
    ws_p = bfl.alloc_workspace(bfl.workspace_bytes(bfl.BF_PHASE_PREFILL, 1, L, Hq, Hkv), "cuda")
    N = dcfg["cache_lens"][2] + 1
    log("generating 128K decode inputs")
    qdc, kc, vc = wl.decode_inputs(1, Hq, Hkv, N, D, "bf16", dcfg["seed"] + 2)
    qdc, kc, vc = qdc.cuda(), kc.cuda(), vc.cuda()
    od = torch.empty_like(qdc)
    ws_d = bfl.alloc_workspace(bfl.workspace_bytes(bfl.BF_PHASE_DECODE, 1, N, Hq, Hkv), "cuda")

    def prefill(mode="fi"):
        bfl.prefill(qd, kd, vd, cu, cfg["w0"], cfg["w_pre"], cfg["theta"], mode, scale, out=o,
                    workspace=ws_p)

    def plain_prefill():
        bfl.plain_prefill(qd, kd, vd, cu, scale, out=o, workspace=ws_p)

    def decode(mode="fi"):
        bfl.decode(qdc, kc, vc, [N], dcfg["w0"], dcfg["w_pre"], dcfg["theta"], mode, scale,
                   out=od, workspace=ws_d)

    def plain_decode():
        bfl.plain_decode(qdc, kc, vc, [N], scale, out=od, workspace=ws_d)

    flops = 4.0 * D * Hq * L * (L + 1) / 2
    kv_bytes = 2.0 * N * Hkv * D * 2

    # raw-input pre-step at the prefill shape: original RoPE of raw q, k in
    # place (on copies), and the same with the cache fill of k' and v
    qr, kr = None, None

    def rope_pre(cache=None):
        bfl.rope_prefill(qr, kr, cu, cfg["theta"], q_out=qr, k_out=kr,
                         **({} if cache is None else dict(v=vd, k_cache=cache[0], v_cache=cache[1])))

    if args.only == "rope":
        qr, kr = qd.clone(), kd.clone()
        for _ in range(args.warmup + args.steps):
            rope_pre()
        torch.cuda.synchronize()
        log(f"only rope: {args.warmup} + {args.steps} calls done")
        return
    if args.only is not None:  # profiling mode: one leg only
        fn = prefill if args.only == "prefill" else decode
        for _ in range(args.warmup + args.steps):
            fn()
        torch.cuda.synchronize()
        log(f"only {args.only}: {args.warmup} + {args.steps} calls done")
        return

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    # timed region: K steps, each one prefill and one decode, events per part
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        prefill()
        e1.record(stream)
        decode()
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_list = [a.elapsed_time(b) for a, b, _ in ev]
    pre_ms = float(np.mean(pre_list))
    dec_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))
    log(f"timed: prefill {pre_ms:.3f} ms, decode {dec_ms * 1e3:.1f} us, wall {wall:.3f} s")

    # references outside the timed region
    prefill("pa")
    pa_ms = time_calls(lambda: prefill("pa"), 3, stream)
    plain_prefill()
    plain_ms = time_calls(plain_prefill, 3, stream)
    shift_ms = time_calls(lambda: prefill("fi+shift"), 2, stream)
    for _ in range(10):
        decode()
    dec_many_ms = time_calls(decode, 50, stream)
    for _ in range(10):
        plain_decode()
    plain_dec_ms = time_calls(plain_decode, 50, stream)
    def cold_us(qx, kx, vx, n, ws_x, copies, calls=200, plain=False):
        """Decode over `copies` distinct cache copies in turn (together more
        than twice the 256 MB MALL), so no call finds its cache resident
        (plain: the library's plain attention the same way)."""
        kcs = [kx] + [kx.clone() for _ in range(copies - 1)]
        vcs = [vx] + [vx.clone() for _ in range(copies - 1)]
        it = [0]

        def fn():
            i = it[0] % copies
            it[0] += 1
            if plain:
                bfl.plain_decode(qx, kcs[i], vcs[i], [n], scale, workspace=ws_x)
            else:
                bfl.decode(qx, kcs[i], vcs[i], [n], dcfg["w0"], dcfg["w_pre"], dcfg["theta"], "fi",
                           scale, workspace=ws_x)

        for _ in range(20):
            fn()
        t = time_calls(fn, calls, stream)
        del kcs, vcs
        return t * 1e3

    # the same 131073-key decode over a paged cache (16-key pages in shuffled
    # order, as a serving engine's page pool would hold them)
    PG = 16
    n_pages = -(-N // PG)
    def paged_pool(x):
        xp = torch.zeros((Hkv, n_pages * PG, D), dtype=x.dtype, device=x.device)
        xp[:, :N] = x[0, :, :N]
        return xp.view(Hkv, n_pages, PG, D).transpose(0, 1).contiguous()  # [page, Hkv, PG, D]
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(11))
    kpg, vpg = paged_pool(kc)[perm.cuda()], paged_pool(vc)[perm.cuda()]
    table = torch.empty(n_pages, dtype=torch.int32)
    table[perm] = torch.arange(n_pages, dtype=torch.int32)
    table = table[None].cuda()
    pfn = lambda: bfl.decode_paged(qdc, kpg, vpg, table, [N], dcfg["w0"], dcfg["w_pre"],
                                   dcfg["theta"], "fi", scale, out=od, workspace=ws_d)
    for _ in range(10):
        pfn()
    paged_ms = time_calls(pfn, 50, stream)
    del kpg, vpg

    def stored_us(qx, kx, vx, n, ws_x, calls=100):
        """Decode with a far-key store (bifocal_decode_stored) once the store
        holds the far keys: the steady state of a decode loop at one s."""
        store = bfl.DecodeStore(kx)
        fn = lambda: bfl.decode_stored(qx, kx, vx, store, [n], dcfg["w0"], dcfg["w_pre"],
                                       dcfg["theta"], "fi", scale, workspace=ws_x)
        for _ in range(10):
            fn()
        t = time_calls(fn, calls, stream)
        del store
        return t * 1e3

    MALL = 256 * 1024 * 1024
    dec_cold_us = cold_us(qdc, kc, vc, N, ws_d, max(2, math.ceil(2 * MALL / kv_bytes)))
    plain_cold_us = cold_us(qdc, kc, vc, N, ws_d, max(2, math.ceil(2 * MALL / kv_bytes)), plain=True)
    dec_stored_us = stored_us(qdc, kc, vc, N, ws_d)
    small = {}
    for Lc in dcfg["cache_lens"][:2]:
        n = Lc + 1
        qs, ks, vs = (x.cuda() for x in wl.decode_inputs(1, Hq, Hkv, n, D, "bf16", dcfg["seed"]))
        ws_s = bfl.alloc_workspace(bfl.workspace_bytes(bfl.BF_PHASE_DECODE, 1, n, Hq, Hkv), "cuda")
        fn = lambda: bfl.decode(qs, ks, vs, [n], dcfg["w0"], dcfg["w_pre"], dcfg["theta"], "fi",
                                scale, workspace=ws_s)
        pfn = lambda: bfl.plain_decode(qs, ks, vs, [n], scale, workspace=ws_s)
        # with a far-key store, timed in the same warm state as the other two
        store_s = bfl.DecodeStore(ks)
        sfn = lambda: bfl.decode_stored(qs, ks, vs, store_s, [n], dcfg["w0"], dcfg["w_pre"],
                                        dcfg["theta"], "fi", scale, workspace=ws_s)
        for _ in range(10):
            fn()
            pfn()
            sfn()
        t_b = time_calls(fn, 100, stream)
        t_p = time_calls(pfn, 100, stream)
        t_s = time_calls(sfn, 100, stream)
        del store_s
        nbytes = 2.0 * n * Hkv * D * 2
        t_c = cold_us(qs, ks, vs, n, ws_s, max(2, math.ceil(2 * MALL / nbytes))) * 1e-3
        t_pc = cold_us(qs, ks, vs, n, ws_s, max(2, math.ceil(2 * MALL / nbytes)), plain=True) * 1e-3
        small[str(n)] = {"bifocal_us": round(t_b * 1e3, 2), "plain_us": round(t_p * 1e3, 2),
                         "stored_us": round(t_s * 1e3, 2),
                         "bifocal_gbs": round(nbytes / (t_b * 1e-3) / 1e9, 1),
                         "bifocal_cold_us": round(t_c * 1e3, 2),
                         "plain_cold_us": round(t_pc * 1e3, 2),
                         "bifocal_cold_gbs": round(nbytes / (t_c * 1e-3) / 1e9, 1)}
        del qs, ks, vs

    log("batched decode")
    batched = {}
    for Bb, Nb in ((32, 8193), (128, 2049)):
        gq = torch.Generator(device="cuda").manual_seed(Bb)
        qb = torch.randn(Bb, Hq, D, generator=gq, device="cuda").to(torch.bfloat16)
        copies = max(2, math.ceil(2 * MALL / (2.0 * Bb * Hkv * Nb * D * 2)))
        cb = [(torch.randn(Bb, Hkv, Nb, D, generator=gq, device="cuda").to(torch.bfloat16),
               torch.randn(Bb, Hkv, Nb, D, generator=gq, device="cuda").to(torch.bfloat16))
              for _ in range(copies)]
        wsb = bfl.alloc_workspace(bfl.workspace_bytes(bfl.BF_PHASE_DECODE, Bb, Nb, Hq, Hkv), "cuda")
        ob = torch.empty_like(qb)
        itb = [0]

        def bfn():  # rotate over cache copies: every call streams its cache from HBM
            kx, vx = cb[itb[0] % copies]
            itb[0] += 1
            bfl.decode(qb, kx, vx, [Nb] * Bb, dcfg["w0"], dcfg["w_pre"], dcfg["theta"], "fi", scale,
                       out=ob, workspace=wsb)
        for _ in range(10):
            bfn()
        tb = time_calls(bfn, 50, stream)
        nbytes = 2.0 * Bb * Hkv * Nb * D * 2
        batched[f"{Bb}x{Nb}"] = {"us": round(tb * 1e3, 2), "gbs": round(nbytes / (tb * 1e-3) / 1e9, 1)}
        del cb, qb, wsb, ob

    log("band-only (sliding-window) prefill and decode")
    band_fn = lambda: prefill("band")
    band_fn()
    band_ms = time_calls(band_fn, 5, stream)
    w0b = cfg["w0"]
    band_flops = 4.0 * D * Hq * (w0b * (w0b + 1) / 2 + (L - w0b) * w0b)  # pairs with i - j < w0
    band_dec = lambda: decode("band")
    for _ in range(10):
        band_dec()
    band_dec_ms = time_calls(band_dec, 100, stream)
    band_dec_bytes = 2.0 * min(N, dcfg["w0"]) * Hkv * D * 2

    log("ragged 8-sequence prefill")
    rcfg = wl.CONFIGS["qwen3_4b_ragged_prefill"]
    rlens = wl.ragged_lengths(rcfg["n_seqs"], rcfg["len_lo"], rcfg["len_hi"], rcfg["seed"])
    rcu = wl.cu_seqlens(rlens)
    rq, rk, rv = (x.cuda() for x in wl.prefill_inputs(rcfg["Hq"], rcfg["Hkv"], rcu[-1], D, "bf16",
                                                      rcfg["seed"]))
    ro = torch.empty_like(rq)
    rws = bfl.alloc_workspace(bfl.workspace_bytes(bfl.BF_PHASE_PREFILL, len(rlens), rcu[-1],
                                                  rcfg["Hq"], rcfg["Hkv"]), "cuda")
    rfn = lambda: bfl.prefill(rq, rk, rv, rcu, rcfg["w0"], rcfg["w_pre"], rcfg["theta"], "fi",
                              scale, out=ro, workspace=rws)
    rfn()
    ragged_ms = time_calls(rfn, 3, stream)
    ragged_flops = 4.0 * D * rcfg["Hq"] * sum(x * (x + 1) / 2 for x in rlens)
    del rq, rk, rv, ro, rws

    log("32K s = 1 prefill (Qwen3-1.7B shapes) and the tiny fp32 workload")
    c2 = wl.CONFIGS["qwen3_1p7b_prefill_32k_s1"]
    L2 = c2["lens"][0]
    q2, k2, v2 = (x.cuda() for x in wl.prefill_inputs(c2["Hq"], c2["Hkv"], L2, D, "bf16", c2["seed"]))
    o2 = torch.empty_like(q2)
    ws2 = bfl.alloc_workspace(bfl.workspace_bytes(bfl.BF_PHASE_PREFILL, 1, L2, c2["Hq"], c2["Hkv"]),
                              "cuda")
    f2 = lambda: bfl.prefill(q2, k2, v2, [0, L2], c2["w0"], c2["w_pre"], c2["theta"], "fi", scale,
                             out=o2, workspace=ws2)
    p2 = lambda: bfl.plain_prefill(q2, k2, v2, [0, L2], scale, out=o2, workspace=ws2)
    f2()
    p2()
    t2 = time_calls(f2, 10, stream)
    t2p = time_calls(p2, 10, stream)
    flops2 = 4.0 * D * c2["Hq"] * L2 * (L2 + 1) / 2
    del q2, k2, v2, o2, ws2
    c1 = wl.CONFIGS["tiny_fp32_s2"]
    L1 = c1["lens"][0]
    q1, k1, v1 = (x.cuda() for x in wl.prefill_inputs(c1["Hq"], c1["Hkv"], L1, D, "fp32", c1["seed"]))
    f1 = lambda: bfl.prefill(q1, k1, v1, [0, L1], c1["w0"], c1["w_pre"], c1["theta"], "fi", scale)
    f1()
    t1 = time_calls(f1, 20, stream)
    flops1 = 4.0 * D * c1["Hq"] * L1 * (L1 + 1) / 2
    del q1, k1, v1

    log("batched prefill: 64 x 2048 and 16 x 8192 prompts")
    batched_pre = {}
    for nb, lb in ((64, 2048), (16, 8192)):
        bcu = wl.cu_seqlens([lb] * nb)
        bq, bk, bv = (x.cuda() for x in wl.prefill_inputs(Hq, Hkv, bcu[-1], D, "bf16", 31 + nb))
        bo = torch.empty_like(bq)
        bws = bfl.alloc_workspace(bfl.workspace_bytes(bfl.BF_PHASE_PREFILL, nb, bcu[-1], Hq, Hkv),
                                  "cuda")
        bfn = lambda: bfl.prefill(bq, bk, bv, bcu, cfg["w0"], cfg["w_pre"], cfg["theta"], "fi",
                                  scale, out=bo, workspace=bws)
        bfn()
        b_ms = time_calls(bfn, 5, stream)
        b_flops = 4.0 * D * Hq * nb * lb * (lb + 1) / 2
        batched_pre[f"{nb}x{lb}"] = {"ms": round(b_ms, 3),
                                     "tflops": round(b_flops / (b_ms * 1e-3) / 1e12, 2)}
        del bq, bk, bv, bo, bws

    log("chunked prefill: the last 512 / 4096 / 16384 queries against the 128K cache")
    kcc, vcc = kd.unsqueeze(0), vd.unsqueeze(0)  # [1, Hkv, L, D]: the cache layout, cap = L
    chunk = {}
    cstore = bfl.ChunkStore(kcc)
    # the same cache as a shuffled pool of 16-key pages
    npg = L // 16
    perm = torch.randperm(npg, generator=torch.Generator().manual_seed(17)).cuda()
    kpg = torch.empty((npg, Hkv, 16, D), dtype=torch.bfloat16, device="cuda")
    vpg = torch.empty_like(kpg)
    kpg[perm] = kd.view(Hkv, npg, 16, D).permute(1, 0, 2, 3)
    vpg[perm] = vd.view(Hkv, npg, 16, D).permute(1, 0, 2, 3)
    tbl = perm.to(torch.int32).view(1, npg)
    pstore = bfl.ChunkStore(kpg, batch=1, max_pages_per_seq=npg)
    for lq in (512, 4096, 16384):
        reps = 20 if lq <= 4096 else 5  # short calls: more of them, less noise
        qch = qd[:, L - lq:].contiguous()
        och = torch.empty_like(qch)
        wsc = bfl.alloc_workspace(bfl.chunk_workspace_bytes(1, lq, L, Hq, Hkv), "cuda")
        cfn = lambda: bfl.prefill_chunk(qch, kcc, vcc, [0, lq], [L], cfg["w0"], cfg["w_pre"],
                                        cfg["theta"], "fi", scale, out=och, workspace=wsc)
        cfn()
        c_ms = time_calls(cfn, reps, stream)
        c_flops = 4.0 * D * Hq * (lq * L - lq * (lq - 1) / 2)  # positions L - lq .. L - 1
        chunk[str(lq)] = {"ms": round(c_ms, 3), "tflops": round(c_flops / (c_ms * 1e-3) / 1e12, 2)}
        # with a chunk store holding the cache up to the chunk: each call forms
        # k'' and V^T of the chunk's own keys only (as a chunk-by-chunk prompt does)
        wss = bfl.alloc_workspace(bfl.chunk_workspace_bytes(1, lq, lq, Hq, Hkv), "cuda")

        def sfn():
            cstore.reset(keys=L - lq)
            bfl.prefill_chunk_stored(qch, kcc, vcc, cstore, [0, lq], [L], cfg["w0"], cfg["w_pre"],
                                     cfg["theta"], "fi", scale, out=och, workspace=wss)
        sfn()
        s_ms = time_calls(sfn, reps, stream)
        chunk[f"{lq}_stored"] = {"ms": round(s_ms, 3),
                                 "tflops": round(c_flops / (s_ms * 1e-3) / 1e12, 2)}
        del wss
        if lq <= 4096:  # the same chunk over the page pool, stateless and with a store
            wsp = bfl.alloc_workspace(bfl.chunk_workspace_bytes(1, lq, L, Hq, Hkv, paged=True), "cuda")
            pfn = lambda: bfl.prefill_chunk_paged(qch, kpg, vpg, tbl, [0, lq], [L], cfg["w0"],
                                                  cfg["w_pre"], cfg["theta"], "fi", scale, out=och,
                                                  workspace=wsp)
            pfn()
            p_ms = time_calls(pfn, reps, stream)
            chunk[f"{lq}_paged16"] = {"ms": round(p_ms, 3),
                                      "tflops": round(c_flops / (p_ms * 1e-3) / 1e12, 2)}

            def psfn():
                pstore.reset(keys=L - lq)
                bfl.prefill_chunk_stored_paged(qch, kpg, vpg, tbl, pstore, [0, lq], [L], cfg["w0"],
                                               cfg["w_pre"], cfg["theta"], "fi", scale, out=och,
                                               workspace=wsp)
            psfn()
            ps_ms = time_calls(psfn, reps, stream)
            chunk[f"{lq}_paged16_stored"] = {"ms": round(ps_ms, 3),
                                             "tflops": round(c_flops / (ps_ms * 1e-3) / 1e12, 2)}
            del wsp
        if lq == 4096:
            # band-only (a sliding-window layer): the same chunk sees only its
            # window; its work is the pairs with i - j < w0
            bfn = lambda: bfl.prefill_chunk(qch, kcc, vcc, [0, lq], [L], cfg["w0"], cfg["w_pre"],
                                            cfg["theta"], "band", scale, out=och, workspace=wsc)
            bfn()
            b_ms = time_calls(bfn, reps, stream)
            b_flops = 4.0 * D * Hq * lq * cfg["w0"]  # every chunk row is past the first w0 keys
            chunk["4096_band"] = {"ms": round(b_ms, 3),
                                  "tflops": round(b_flops / (b_ms * 1e-3) / 1e12, 2)}
        del qch, och, wsc
    del cstore, pstore, kpg, vpg, tbl

    log("raw-input pre-step")
    qr, kr = qd.clone(), kd.clone()
    rope_pre()
    rope_ms = time_calls(rope_pre, 10, stream)
    kcache = torch.empty((1, Hkv, L, D), dtype=torch.bfloat16, device="cuda")
    vcache = torch.empty_like(kcache)
    rope_pre((kcache, vcache))
    rope_c_ms = time_calls(lambda: rope_pre((kcache, vcache)), 10, stream)
    del kcache, vcache
    q1, k1, v1 = qdc.clone(), torch.randn(1, Hkv, D, device="cuda").to(torch.bfloat16), \
        torch.randn(1, Hkv, D, device="cuda").to(torch.bfloat16)
    kc_app, vc_app = kc.clone(), vc.clone()
    app = lambda: bfl.rope_append(q1, k1, v1, kc_app, vc_app, [N], dcfg["theta"], q_out=q1)
    for _ in range(10):
        app()
    app_ms = time_calls(app, 100, stream)
    # the same bytes moved by a plain device copy (read q, k; write copies):
    # the ceiling of a read-plus-write stream on this part
    qcp, kcp = torch.empty_like(qr), torch.empty_like(kr)
    cp = lambda: (qcp.copy_(qr), kcp.copy_(kr))
    cp()
    copy_ms = time_calls(cp, 10, stream)
    del q1, kc_app, vc_app, qr, kr, qcp, kcp
    # algorithmic bytes: read raw q, k and write q', k'; the cache fill adds
    # k' to the cache and the copy of v (read + write)
    rope_bytes = 2.0 * (Hq + Hkv) * L * D * 2
    rope_c_bytes = rope_bytes + 3.0 * Hkv * L * D * 2
    rope_gbs = rope_bytes / (rope_ms * 1e-3) / 1e9

    tflops = flops / (pre_ms * 1e-3) / 1e12
    gbs = kv_bytes / (dec_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre_ms + dec_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_prefill_128k (FI) + qwen3_8b_decode_128k",
                   "batch": 1, "seq_len": L, "n_heads_q": Hq, "n_heads_kv": Hkv, "head_dim": D,
                   "w_pre": cfg["w_pre"], "w0": cfg["w0"], "rope_theta": cfg["theta"],
                   "s_prefill": bfl.s_of_L(L, cfg["w_pre"]), "decode_keys": N,
                   "s_decode": bfl.s_of_L(N, dcfg["w_pre"]), "long_mode": "fi"},
        "prefill_ms": round(pre_ms, 3),
        "prefill_ms_median": round(float(np.median(pre_list)), 3),
        "prefill_ms_min": round(float(np.min(pre_list)), 3),
        "prefill_frac_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "prefill_pa_tflops": round(flops / (pa_ms * 1e-3) / 1e12, 2),
        "plain_prefill_tflops": round(flops / (plain_ms * 1e-3) / 1e12, 2),
        "prefill_overhead_vs_plain": round(pre_ms / plain_ms - 1, 4),
        "prefill_pa_overhead_vs_plain": round(pa_ms / plain_ms - 1, 4),
        "prefill_fi_shift_tflops": round(flops / (shift_ms * 1e-3) / 1e12, 2),
        "decode_us": round(dec_ms * 1e3, 2),
        "decode_gbs": round(gbs, 1),
        "decode_frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "decode_us_50_calls": round(dec_many_ms * 1e3, 2),
        "decode_cold_us": round(dec_cold_us, 2),
        "decode_paged16_us": round(paged_ms * 1e3, 2),
        "decode_cold_gbs": round(kv_bytes / (dec_cold_us * 1e-6) / 1e9, 1),
        "plain_decode_cold_us": round(plain_cold_us, 2),
        "decode_cold_overhead_vs_plain": round(dec_cold_us / plain_cold_us - 1, 4),
        "plain_decode_us": round(plain_dec_ms * 1e3, 2),
        "decode_overhead_vs_plain": round(dec_many_ms / plain_dec_ms - 1, 4),
        "decode_stored_us": round(dec_stored_us, 2),
        "decode_stored_gbs": round(kv_bytes / (dec_stored_us * 1e-6) / 1e9, 1),
        "decode_stored_overhead_vs_plain": round(dec_stored_us / (plain_dec_ms * 1e3) - 1, 4),
        "decode_small": small,
        "decode_batched_cold": batched,
        "band_only": {"prefill_ms": round(band_ms, 3),
                      "prefill_tflops": round(band_flops / (band_ms * 1e-3) / 1e12, 2),
                      "decode_us": round(band_dec_ms * 1e3, 2),
                      "decode_gbs": round(band_dec_bytes / (band_dec_ms * 1e-3) / 1e9, 1)},
        "ragged_prefill": {"lengths": rlens, "ms": round(ragged_ms, 3),
                           "tflops": round(ragged_flops / (ragged_ms * 1e-3) / 1e12, 2)},
        "prefill_32k_s1": {"workload": "qwen3_1p7b_prefill_32k_s1 (16/8 heads, s = 1)",
                           "ms": round(t2, 3), "tflops": round(flops2 / (t2 * 1e-3) / 1e12, 2),
                           "plain_ms": round(t2p, 3),
                           "overhead_vs_plain": round(t2 / t2p - 1, 4)},
        "tiny_fp32_s2": {"ms": round(t1, 4), "tflops": round(flops1 / (t1 * 1e-3) / 1e12, 3),
                         "note": "parity workload (fp32 MFMA 32x32x2), not a throughput target"},
        "batched_prefill": batched_pre,
        "chunk_prefill_at_128k": chunk,
        "rope_prefill_ms": round(rope_ms, 4),
        "rope_prefill_gbs": round(rope_gbs, 1),
        "rope_prefill_cache_ms": round(rope_c_ms, 4),
        "rope_prefill_cache_gbs": round(rope_c_bytes / (rope_c_ms * 1e-3) / 1e9, 1),
        "rope_append_us": round(app_ms * 1e3, 2),
        "copy_same_bytes_gbs": round(rope_bytes / (copy_ms * 1e-3) / 1e9, 1),
        "roofline": {"kernel": "bifocal_prefill call (correction prep + V^T + MFMA tile loop)",
                     "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for("prefill_bf16_kernel_bifocal")},
        "roofline_decode": {"kernel": "bifocal_decode call (split-K + combine)", "bound": "hbm",
                            "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs / PEAK_HBM_GBS, 4),
                            "traffic": traffic_for("decode_split_kernel_bifocal")},
        "roofline_rope": {"kernel": "bifocal_rope_prefill (raw-input pre-step, in place)",
                          "bound": "hbm", "achieved": round(rope_gbs, 1), "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": round(rope_gbs / PEAK_HBM_GBS, 4),
                          "traffic": traffic_for("rope_kernel")},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle per workload")
        result["cpu_baseline"] = cpu_baseline(q, k, v)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
