"""Benchmark: byte-level BPE encode throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload throughput] [--gpus 1]

One step is one bpe_encode_batch call over the whole batch (byte-class scan,
pre-token merge, ID compaction and per-document offsets), with the input
already resident in HBM.  Prints one JSON line.  The default workload is the
throughput workload: 4,096 documents of 64 KiB (256 MiB) with the
32,000-merge table.

The CPU baseline is the oracle as it stands ("Hugging Face Tokenizers v1",
section "Benchmarks": a fresh process per repetition, workers on distinct
physical cores, output checked by the FNV-1a of its IDs): on one physical
core, pinned, over the first documents of the same batch, and in one pinned
process per physical core (lscpu, SMT siblings excluded, at most 16), each the
median of 5 runs in fresh processes.  The oracle's sample is compared with
the GPU's IDs element by element, and the GPU's whole batch with the oracle's
stored whole-batch checksums (cpu_baseline.parity_ok).  The host-to-device
copy of the input and the device-to-host copy of the IDs are timed apart
(`transfers`); neither is part of `value` or of the roofline.

The roofline object covers one encode call: its kernels run back to back
on one stream, and the library's stage timing (HIP events recorded between
them) gives each kernel's average duration.  Those events cost time of their
own, so they are recorded in a second pass of the same number of steps right
after the timed one; `ms_per_step` comes from the pass without them.
Algorithmic bytes are the call's: the input read once, the IDs and the
per-document offsets written once (N + 4T + 16(D + 1)).  Measured memory
traffic comes from profiles/traffic_<workload>.json: the L2's read requests
to memory (rocprofv3 TCC_EA0_RDREQ, 128 bytes each on this chip, as a copy, a
reduction and an elementwise kernel of known size show) and its write
requests (WRITE_SIZE), summed over the encode kernels of one call, with the
per-kernel L2 hit rates (TCC_HIT / (TCC_HIT + TCC_MISS)); both are reported
only while the kernel sources still hash to the value recorded there.

Beside the timed encode the line carries the decode of the same IDs
(`decode`, a round trip) and the encode with a BOS and an EOS ID around each
document (`special`, bpe_encode_batch_special), each timed the same way and
checked against the plain encode, and (`train`) bpe_train on the workload's
training corpus, its table checked against the one stored in assets/.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure


def kernel_sources_sha256() -> str:
    """Hash of every source the kernels are built from."""
    files = sorted(glob.glob(os.path.join(ROOT, "byte_level_bpe_pretokenize_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "bpe.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_counters(workload: str):
    """The committed counter summary of one encode call (HBM bytes, per-kernel
    L2 hit rates), or None when it is missing or the kernels changed since it
    was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("sources_sha256") != kernel_sources_sha256():
        return None
    return rec


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 200 for the serving workload)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="throughput",
                    choices=["tiny", "throughput", "multilingual", "adversarial", "serving"])
    ap.add_argument("--cpu-seconds", type=float, default=2.5,
                    help="target CPU time of one oracle baseline run (each is repeated 5 times)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-train", action="store_true",
                    help="skip timing bpe_train on the workload's training corpus")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run kernels of known traffic on the input (copy, reduction, "
                         "elementwise, fill) for the counter runs")
    return ap.parse_args()


def physical_cores():
    """One logical CPU per physical core among the CPUs this process may run
    on (SMT siblings excluded), from `lscpu -p=CPU,CORE,SOCKET` (the sysfs
    topology when lscpu is missing), at most 16 (one GPU's share of a box)."""
    import subprocess
    allowed = sorted(os.sched_getaffinity(0))
    core_of = {}
    try:
        out = subprocess.run(["lscpu", "-p=CPU,CORE,SOCKET"], capture_output=True, text=True,
                             check=True).stdout
        for line in out.splitlines():
            if line.startswith("#") or not line.strip():
                continue
            cpu, core, sock = (int(x) if x else -1 for x in line.split(",")[:3])
            core_of[cpu] = (sock, core)
        source = "lscpu"
    except (OSError, subprocess.CalledProcessError, ValueError):
        for cpu in allowed:
            base = f"/sys/devices/system/cpu/cpu{cpu}/topology/"
            try:
                core_of[cpu] = (int(open(base + "physical_package_id").read()),
                                int(open(base + "core_id").read()))
            except OSError:
                core_of[cpu] = (0, cpu)
        source = "sysfs"
    seen, pick = set(), []
    for cpu in allowed:
        key = core_of.get(cpu, (0, cpu))
        if key not in seen:
            seen.add(key)
            pick.append(cpu)
    return pick[:16], source, len(allowed)


def _oracle_run(args):
    """One timed oracle encode in a fresh process pinned to one CPU: returns
    (bytes, ids, seconds) and, when asked, the IDs and offsets."""
    cpu, merges, data, doc_off, want_ids = args
    os.sched_setaffinity(0, {cpu})
    import oracle as O
    table = O.Table(merges)
    t0 = time.perf_counter()
    ids, off = table.encode_batch(data, doc_off)
    dt = time.perf_counter() - t0
    return int(data.size), int(ids.size), dt, (ids, off) if want_ids else None


def _fresh_pool(n):
    import concurrent.futures as cf
    import multiprocessing as mp
    return cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"))


REPEATS = 5


def cpu_baseline(merges, batch, target_s, cores):
    """The oracle, as it stands, on one physical core (pinned), over a bounded
    prefix of the batch's documents sized for about target_s seconds; the
    median of REPEATS runs, each in a fresh process.  Returns the record, the
    oracle's IDs and offsets for the sample, and its rate (bytes/s)."""
    import oracle as O
    nd = batch.n_docs
    table = O.Table(merges)
    probe = max(1, min(nd, 2))
    t0 = time.perf_counter()
    table.encode_batch(batch.data[:batch.doc_off[probe]], batch.doc_off[:probe + 1])
    rate = batch.doc_off[probe] / max(1e-6, time.perf_counter() - t0)
    k = int(np.searchsorted(batch.doc_off, rate * target_s, side="right"))
    k = max(1, min(nd, k))
    n = int(batch.doc_off[k])
    data, off = batch.data[:n], batch.doc_off[:k + 1]
    runs, ids = [], None
    for rep in range(REPEATS):
        with _fresh_pool(1) as pool:
            nb, nt, dt, got = pool.submit(_oracle_run, (cores[0], merges, data, off, rep == 0)).result()
        runs.append(dt)
        if got is not None:
            ids, ids_off = got
    dt = float(np.median(runs))
    rec = {
        "value": round(n / dt / 1e6, 3),
        "unit": "MB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"first {k} of {nd} documents ({n} bytes) of the same batch; median of "
                  f"{REPEATS} runs, each a fresh process pinned to CPU {cores[0]} "
                  f"(runs {', '.join(f'{x:.2f}' for x in runs)} s)",
        "tokens_per_s": round(ids.size / dt, 1),
    }
    return rec, ids, ids_off, n / dt


def cpu_baseline_all_cores(merges, batch, rate1, target_s, cores, source, n_logical):
    """The same oracle in one process per physical core (each pinned to one
    CPU; documents split in contiguous shards of equal bytes), on a sample
    sized for about target_s seconds; the median of REPEATS runs, each with a
    fresh pool of processes."""
    nc = len(cores)
    nd = batch.n_docs
    k = int(np.searchsorted(batch.doc_off, rate1 * target_s * nc, side="right"))
    k = max(1, min(nd, k))
    n = int(batch.doc_off[k])
    cuts = sorted(set([0, k] + [int(np.searchsorted(batch.doc_off[:k + 1], n * j / nc))
                                for j in range(1, nc)]))
    shards = [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    walls, tokens = [], 0
    limit = 20 * target_s + 60
    for rep in range(REPEATS):
        jobs = []
        for j, (a, b) in enumerate(shards):
            lo, hi = int(batch.doc_off[a]), int(batch.doc_off[b])
            jobs.append((cores[j % nc], merges, batch.data[lo:hi], batch.doc_off[a:b + 1] - lo, False))
        with _fresh_pool(len(jobs)) as pool:
            # each process loads the oracle before the clock starts
            warm = [(cores[j % nc], merges, batch.data[:1], np.array([0, 1], dtype=np.int64), False)
                    for j in range(len(jobs))]
            list(pool.map(_oracle_run, warm, timeout=limit))
            t0 = time.perf_counter()
            res = list(pool.map(_oracle_run, jobs, timeout=limit))
            walls.append(time.perf_counter() - t0)
        tokens = sum(r[1] for r in res)
    wall = float(np.median(walls))
    return {
        "value": round(n / wall / 1e6, 3),
        "unit": "MB/s",
        "cores": len(shards),
        "kind": "oracle",
        "sample": f"first {k} of {nd} documents ({n} bytes) in {len(shards)} processes, one per "
                  f"physical core ({source}: {len(cores)} physical cores among {n_logical} "
                  f"allowed CPUs, SMT siblings excluded), each pinned; median of {REPEATS} runs "
                  f"with fresh processes ({', '.join(f'{x:.2f}' for x in walls)} s wall)",
        "tokens_per_s": round(tokens / wall, 1),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(documents are independent: a batch shards by document ranges, one process per GPU)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from byte_level_bpe_pretokenize_amd import Model
    from workloads import WORKLOADS, encode_batch_input, make_lexicon

    cfg = WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    batch = encode_batch_input(cfg, make_lexicon(cfg))
    t_gen = time.perf_counter() - t_gen
    merges = np.load(os.path.join(ROOT, "assets", f"merges_{args.workload}.npy"), allow_pickle=False)
    print(f"# generated {batch.n_bytes} bytes in {batch.n_docs} documents in {t_gen:.1f} s",
          file=sys.stderr, flush=True)
    if args.steps is None:
        args.steps = 200 if args.workload == "serving" else 20

    # the CPU baselines run first, before this process touches the GPU
    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        cores, source, n_logical = physical_cores()
        cpu, cpu_ids, cpu_off, rate1 = cpu_baseline(merges, batch, args.cpu_seconds, cores)
        print(f"# oracle, one core: {cpu['value']} MB/s", file=sys.stderr, flush=True)
        try:
            cpu_all = cpu_baseline_all_cores(merges, batch, rate1, args.cpu_seconds, cores, source,
                                              n_logical)
            print(f"# oracle, {cpu_all['cores']} physical cores: {cpu_all['value']} MB/s",
                  file=sys.stderr, flush=True)
        except Exception as exc:  # the single-core baseline stands alone
            cpu_all = {"error": f"{type(exc).__name__}: {exc}"}

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    model = Model(merges)
    N, D = batch.n_bytes, batch.n_docs
    # the input staged from pinned host memory (timed apart: it is never part
    # of the encode's time or roofline)
    host_data = torch.from_numpy(batch.data).pin_memory()
    data = torch.empty(N, dtype=torch.uint8, device=dev)
    doc_off = torch.from_numpy(batch.doc_off).to(dev)
    data.copy_(host_data, non_blocking=True)
    torch.cuda.synchronize()
    h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0.record()
    data.copy_(host_data, non_blocking=True)
    h1.record()
    torch.cuda.synchronize()
    h2d_ms = h0.elapsed_time(h1)
    ids = torch.empty(N, dtype=torch.int32, device=dev)
    id_off = torch.empty(D + 1, dtype=torch.int64, device=dev)
    ws = torch.empty(model.encode_workspace_bytes(N, D), dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        model.encode_batch_into(data, doc_off, ids, id_off, ws, status, stream)

    # device-to-device copy bandwidth of this machine, for context
    copy = torch.empty_like(data)
    for _ in range(3):
        copy.copy_(data)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        copy.copy_(data)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * N * 10 / (c0.elapsed_time(c1) / 1e3) / 1e9
    del copy

    if args.copy_calibration:
        # kernels of known traffic for the counter runs: a device copy (reads
        # and writes N bytes), a reduction with 16-byte loads (reads N), an
        # elementwise kernel (reads and writes N) and a fill (writes N)
        copy = torch.empty_like(data)
        copy.copy_(data)
        _ = data[:N & ~7].view(torch.int64).sum()
        _ = data[:N & ~3].view(torch.float32) * 2.0
        copy.zero_()
        torch.cuda.synchronize()
        del copy, _
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    st = int(status.item())
    if st:
        raise SystemExit(f"device status {st:#x} after warm-up")
    T = int(id_off[-1].item())

    # the timed steps: events around each call only
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    start, stop = evs[0], evs[-1]
    torch.cuda.synchronize()
    for k in range(args.steps):
        evs[k].record(stream)
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    per_step = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps))
    st = int(status.item())
    if st:
        raise SystemExit(f"device status {st:#x} in the timed region")
    # the same number of steps again with the library's stage timing (an
    # event between every two kernels), for the per-kernel durations; the
    # events themselves cost time, so these steps are not the ones timed above
    model.stage_timing(True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    staged_ms = start.elapsed_time(stop) / args.steps
    stage_ms, calls = model.stage_times("encode")
    model.stage_timing(False)
    st = int(status.item())
    if st:
        raise SystemExit(f"device status {st:#x} in the stage-timed steps")
    kern = {k: v / max(1, calls) for k, v in stage_ms.items()}
    path_ms = sum(kern.values())
    dominant = max(kern, key=kern.get)

    sec = ms / 1e3
    alg_bytes = N + 4 * T + 16 * (D + 1)
    achieved = alg_bytes / (path_ms / 1e3) / 1e9
    counters = measured_counters(args.workload)
    traffic = None if counters is None else int(counters["fetch_bytes_per_call"] +
                                                counters["write_bytes_per_call"])
    l2_hit = None if counters is None else counters.get("l2_hit_rate")

    # decode of the same IDs (round trip), timed the same way
    dec = {}
    mtb = model.max_token_bytes
    if mtb > 0:
        out = torch.empty(N + 64, dtype=torch.uint8, device=dev)
        byte_off = torch.empty(D + 1, dtype=torch.int64, device=dev)
        dws = torch.empty(max(1, model.decode_workspace_bytes(T, D)), dtype=torch.uint8, device=dev)
        dstat = torch.zeros(1, dtype=torch.int32, device=dev)
        ids_t = ids[:T]
        for _ in range(2):
            model.decode_batch_into(ids_t, id_off, out, byte_off, dws, dstat, stream)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            model.decode_batch_into(ids_t, id_off, out, byte_off, dws, dstat, stream)
        stop.record(stream)
        torch.cuda.synchronize()
        dms = start.elapsed_time(stop) / args.steps
        rt = bool(int(dstat.item()) == 0 and torch.equal(out[:N], data)
                  and torch.equal(byte_off, doc_off))
        dec = {"ms": round(dms, 4), "output_MB_per_s": round(N / (dms / 1e3) / 1e6, 1),
               "achieved_GB_per_s": round((4 * T + N + 16 * (D + 1)) / (dms / 1e3) / 1e9, 1),
               "round_trip_ok": rt}

    # the same encode with reserved IDs around each document (post-processing:
    # bpe_encode_batch_special), timed the same way; with the reserved IDs
    # taken out its IDs must be the plain encode's
    V = model.vocab_size
    sp_ids = torch.empty(N + 2 * D, dtype=torch.int32, device=dev)
    sp_off = torch.empty(D + 1, dtype=torch.int64, device=dev)
    sws = torch.empty(model.encode_special_workspace_bytes(N, D), dtype=torch.uint8, device=dev)
    sstat = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        model.encode_batch_special_into(data, doc_off, V, V + 1, sp_ids, sp_off, sws, sstat, stream)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        model.encode_batch_special_into(data, doc_off, V, V + 1, sp_ids, sp_off, sws, sstat, stream)
    stop.record(stream)
    torch.cuda.synchronize()
    sms = start.elapsed_time(stop) / args.steps
    sp_t = sp_ids[:T + 2 * D]
    keep = (sp_t != V) & (sp_t != V + 1)
    sp_ok = bool(int(sstat.item()) == 0
                 and torch.equal(sp_off, id_off + 2 * torch.arange(D + 1, device=dev))
                 and torch.equal(sp_t[keep], ids[:T])
                 and torch.equal(sp_ids[sp_off[:-1]], torch.full((D,), V, dtype=torch.int32, device=dev))
                 and torch.equal(sp_ids[sp_off[1:] - 1],
                                 torch.full((D,), V + 1, dtype=torch.int32, device=dev)))
    special = {"ms": round(sms, 4), "bos_eos_per_document": 2, "ids_match_plain": sp_ok}
    del sws, sp_ids, sp_t, keep

    # the GPU trainer on the workload's training corpus (the throughput and
    # tiny workloads), its table checked against the one stored in assets/
    train_info = None
    if not args.no_train and args.workload in ("throughput", "tiny"):
        from byte_level_bpe_pretokenize_amd import train as bpe_train
        from workloads import training_corpus
        tc = training_corpus(cfg, make_lexicon(cfg))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        tm, _ = bpe_train(tc.data, tc.doc_off, cfg.n_merges)
        train_s = time.perf_counter() - t0
        train_info = {"s": round(train_s, 3), "merges": int(tm.shape[0]),
                      "corpus_bytes": int(tc.data.size),
                      "matches_stored_table": bool(np.array_equal(tm, merges))}

    # the IDs back to pinned host memory (timed apart, as the input's copy)
    host_ids = torch.empty(T, dtype=torch.int32).pin_memory()
    host_ids.copy_(ids[:T], non_blocking=True)
    torch.cuda.synchronize()
    h0.record()
    host_ids.copy_(ids[:T], non_blocking=True)
    h1.record()
    torch.cuda.synchronize()
    d2h_ms = h0.elapsed_time(h1)
    transfers = {
        "h2d_ms": round(h2d_ms, 4), "h2d_GBps": round(N / (h2d_ms / 1e3) / 1e9, 1),
        "d2h_ms": round(d2h_ms, 4), "d2h_GBps": round(4 * T / (d2h_ms / 1e3) / 1e9, 1),
        "pcie_inclusive_MB_per_s": round(N / ((h2d_ms + ms + d2h_ms) / 1e3) / 1e6, 1),
    }
    ids_np = host_ids.numpy()
    id_off_np = id_off.cpu().numpy()
    fnv = None
    if cpu is not None:
        # the oracle's own sample, element by element, and the whole batch
        # against the oracle's whole-batch checksums (tests/golden/fullsize.json)
        import oracle as O
        k = cpu_off.size - 1
        ok = bool(np.array_equal(cpu_ids, ids_np[:cpu_ids.size]) and
                  np.array_equal(cpu_off, id_off_np[:k + 1]))
        fnv = f"{O.ids_fnv(ids_np):016x}"
        off_fnv = f"{O.fnv1a64(np.ascontiguousarray(id_off_np, dtype='<i8')):016x}"
        gold = json.load(open(os.path.join(ROOT, "tests", "golden", "fullsize.json")))[cfg.name]
        whole = bool(T == gold["T"] and fnv == gold["ids_fnv1a64"]
                     and off_fnv == gold["id_off_fnv1a64"])
        cpu["parity_ok"] = ok and whole
        cpu["sample"] += (f"; sample IDs equal to the GPU's: {ok}; whole-batch T and FNV-1a of "
                          f"IDs and offsets equal to the oracle's: {whole}")

    line = {
        "metric": "BPE encode input MB/s and tokens/s on 1 MI355X; % of HBM roofline",
        "value": round(N / sec / 1e6, 1),
        "unit": "MB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {D} documents, {N} bytes, {merges.shape[0]} merges",
            "n_bytes": N, "n_docs": D, "n_merges": int(merges.shape[0]), "tokens": T,
        },
        "tokens_per_s": round(T / sec, 1),
        "ms_median": round(per_step[len(per_step) // 2], 4),
        "ms_min": round(per_step[0], 4),
        "ms_p99": round(per_step[min(len(per_step) - 1, int(0.99 * len(per_step)))], 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "l2_hit": l2_hit,
            "scope": "one encode call: " + " + ".join(kern),
            "algorithmic_bytes": alg_bytes,
            "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
            "dominant": dominant,
            "timed_calls": calls,
            "ms_per_step_stage_timed": round(staged_ms, 4),
            "copy_GBps": round(copy_gbs, 1),
            "frac_of_copy": round(achieved / copy_gbs, 4),
        },
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "transfers": transfers,
        "ids_fnv1a64": fnv,
        "decode": dec,
        "special": special,
        "train": train_info,
        "ids_sha256": hashlib.sha256(ids_np.tobytes()).hexdigest()[:16],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
