"""Benchmark: exact BPE encode throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2] [--only]
    python bench.py --summarize DIR --workload NAME   (rocprofv3 output -> profiles/)

One step = one full encode (pre-tokenization, BPE of every pre-token, token-id
emission) of the workload's text, already resident in HBM.  The timed region
is exactly K steps, each between its own pair of HIP events on the launch
stream with a synchronisation after it, so every step is a single-request
latency; the headline is chars / p50 of those K latencies.  Prints one JSON
line with the headline workload's figures, the roofline of its dominant
kernel, every other workload's figures under config.workloads, and the CPU
oracle timed on this host as a reported baseline.

Workloads (seeded, synthetic; the headline is the 1,000,000-char single text):
  c1   64 KiB ASCII code-like text, GPT-2-style rules, 4,096 merges
  c2   1,000,000-char code/log mix, GPT-2-style rules, 50,000 merges
  c3   1,000,000-char mix with 5 % multibyte chars, cl100k-style, 100,000 merges
  c4   64 log-normal fresh texts (~8M chars) in one batch call
  c5a..c5d adversarial 1,000,000-char texts (one giant piece, 100K-digit runs,
       50K-space runs, alternating letter/punctuation)
  w100k one 100,000-letter random word (a long piece with many distinct merges)
  o2   the c3 text under the o200k-style rules (case-split words, attached
       contractions, CR/LF/'/' tails)
  ds   the c3 text under the DeepSeek-style rules (digit groups and CJK runs cut
       out first)
Each is checked against the oracle's stored digests before it is timed.

Roofline (per workload, for its dominant kernel):
  alg_bytes = n + 4T (+ 16 (B + 1) for a batch): the text read once and the
  ids written once, the per-encode algorithmic bytes of the method; the HBM
  fraction is alg_bytes / kernel time / 8 TB/s.  Kernel times are the
  rocprofv3 averages stored in profiles/counters.json while the SHA-256 of
  tt_kernels.hip recorded there matches the source (the live event averages
  otherwise, always reported beside them); the dominant kernel is the one
  with the largest time.  The stored counter passes also give its HBM bytes
  (FETCH_SIZE, WRITE_SIZE, calibrated on a 64 MiB copy) and its VALU issue
  fraction, SQ_INSTS_VALU x 4 cycles / 1024 SIMDs / 2.4 GHz / kernel time;
  `bound` says which fraction is the larger.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "exact BPE encode throughput: chars/s and ms per 1M chars; % of HBM peak"
HEADLINE = "c2"
ALL_WORKLOADS = ["c1", "c2", "c3", "c4", "c5a", "c5b", "c5c", "c5d", "w100k", "o2", "ds"]
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
CLOCK_GHZ = 2.4         # MI355X peak engine clock (one clock for every figure here)
SIMDS = 256 * 4         # 256 CUs x 4 SIMDs
# a wave64 VALU instruction occupies a 16-lane SIMD for 4 cycles
VALU_PEAK_GINST = SIMDS * CLOCK_GHZ / 4  # 614.4 G wave-instructions/s
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SRC = os.path.join(ROOT, "exact_byte_level_amd", "csrc", "tt_kernels.hip")
PRETOK_KERNELS = ("k_tile_summary", "k_pretok<0>", "k_pretok<1>", "k_pretok<2>", "k_pretok<3>")


def _sha(a):
    import numpy as np
    return hashlib.sha256(np.ascontiguousarray(a, dtype="<i4").tobytes()).hexdigest()


def kernel_source_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _base_name(k):
    """Kernel name without template arguments and namespace (profiler names)."""
    k = k.split("(")[0].replace("void ", "").replace("tt::", "").strip()
    return k


def load_counters():
    """Stored counter summaries whose kernel source matches this tree, by workload."""
    if not os.path.exists(COUNTERS):
        return {}
    with open(COUNTERS) as f:
        c = json.load(f)
    if c.get("kernel_source_sha256") != kernel_source_sha():
        return {}
    return c.get("workloads", {})


def pct(sorted_vals, q):
    return sorted_vals[min(len(sorted_vals) - 1, int(round(q * (len(sorted_vals) - 1))))]


# ------------------------------------------------------------------ GPU side

def measure(name, steps, warmup, graph=True, detail=False, counters=None):
    """Time one workload; returns a dict of its figures (verified first)."""
    import numpy as np
    import torch

    import exact_byte_level_amd as tt
    from synth.text import WORKLOADS, workload

    data, offs, pat, voc = workload(name)
    n = len(data)
    chars = len(data.decode("utf-8"))
    merges = np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % voc))
    tt.load(merges, pattern_id=pat)
    nseq = 1 if offs is None else len(offs) - 1
    tt.reserve(n, nseq)
    dev = torch.device("cuda", 0)
    x = torch.frombuffer(bytearray(data), dtype=torch.uint8).to(dev)
    out = torch.empty(n, dtype=torch.int32, device=dev)
    cnt = torch.empty(nseq + 1 if offs is not None else 1, dtype=torch.int64, device=dev)
    off = None if offs is None else torch.tensor(offs, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        if off is None:
            tt.encode_into(x, out, cnt)
        else:
            tt.encode_batch_into(x, off, out, cnt)

    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t0) * 1e3
    # slow workloads (a long piece of many rounds) take fewer steps
    k = steps if first_ms < 5.0 else max(3, min(steps, int(2000.0 / first_ms)))
    for _ in range(warmup if first_ms < 5.0 else min(warmup, 2)):
        step()
    torch.cuda.synchronize()
    T = int(cnt[-1].item())
    if T < 0:
        raise RuntimeError("%s: encode reported error %d" % (name, T))
    ids = out[:T].cpu().numpy()
    with open(os.path.join(ROOT, "tests", "golden", "expected.json")) as f:
        exp = json.load(f)[name]
    if exp["tokens"] != T or exp["ids_sha256"] != _sha(ids):
        raise RuntimeError("GPU ids differ from the oracle digest for %s" % name)

    # the timed region: exactly k steps, each a single-request latency
    torch.cuda.synchronize()
    lat = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
    lat = sorted(a.elapsed_time(b) for a, b in evs)
    p50, p99 = statistics.median(lat), pct(lat, 0.99)

    # k encodes queued back to back (a stream of requests): mean per encode
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(k):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    b2b_ms = e0.elapsed_time(e1) / k

    res = {
        "desc": WORKLOADS[name][2],
        "chars": chars, "bytes": n, "tokens": T, "seqs": nseq, "steps": k,
        "p50_ms": p50, "p99_ms": p99,
        "chars_per_s": chars / (p50 * 1e-3),
        "ms_per_1M_chars": p50 * 1e6 / chars,
        "back_to_back_mean_ms": b2b_ms,
        "verified_against_oracle": True,
    }

    # HIP graph replay of one captured encode (the pages' single-request mode)
    if graph:
        try:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                step()
            stream.wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                step()
            torch.cuda.synchronize()
            gl = []
            for _ in range(k):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.replay()
                b.record(stream)
                b.synchronize()
                gl.append(a.elapsed_time(b))
            # k replays queued back to back: the host's graph launch overlaps
            # the previous replay, as the plain launches' back-to-back mean
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            for _ in range(k):
                g.replay()
            g1.record(stream)
            torch.cuda.synchronize()
            if int(cnt[-1].item()) != T or _sha(out[:T].cpu().numpy()) != _sha(ids):
                raise RuntimeError("graph replay result differs")
            gl.sort()
            res["graph_p50_ms"] = statistics.median(gl)
            res["graph_p99_ms"] = pct(gl, 0.99)
            res["graph_back_to_back_mean_ms"] = g0.elapsed_time(g1) / k
            del g
        except Exception as ex:  # graph capture is context, not the headline
            print("graph mode skipped for %s: %r" % (name, ex), file=sys.stderr)

    if detail:
        # host-inclusive latency: encode plus the D2H read of the count
        th = []
        for _ in range(min(k, 50)):
            t0 = time.perf_counter()
            step()
            int(cnt[-1].item())
            th.append((time.perf_counter() - t0) * 1e3)
        res["host_incl_p50_ms"] = statistics.median(th)
        # byte-offset export: the same ids plus every token's byte start
        starts_buf = torch.empty(n + 1, dtype=torch.int32, device=dev)

        def step_off():
            tt.encode_offsets_into(x, off, out, starts_buf, cnt)

        step_off()
        torch.cuda.synchronize()
        if int(cnt[-1].item()) != T or _sha(out[:T].cpu().numpy()) != _sha(ids):
            raise RuntimeError("tt_encode_offsets ids differ from tt_encode's")
        if _sha(starts_buf[:T + 1].cpu().numpy()) != exp["token_starts_sha256"]:
            raise RuntimeError("GPU token offsets differ from the oracle digest for %s" % name)
        ol = []
        for _ in range(k):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step_off()
            b.record(stream)
            b.synchronize()
            ol.append(a.elapsed_time(b))
        res["with_byte_offsets_p50_ms"] = statistics.median(ol)
        res["byte_offsets_verified"] = True

    # per-kernel durations, live: an event after each launch (tt_profile), k steps
    tt.profile(True)
    acc = {}
    for _ in range(k):
        step()
        for kn, ms in tt.profile_read():
            acc.setdefault(kn, []).append(ms)
    tt.profile(False)
    kern_us = {kn: 1e3 * statistics.mean(v) for kn, v in acc.items()}
    res["kernels_us"] = {kn: round(v, 2) for kn, v in sorted(kern_us.items(), key=lambda kv: -kv[1])}
    pre_us = sum(v for kn, v in kern_us.items() if kn in PRETOK_KERNELS)
    bpe_us = sum(v for kn, v in kern_us.items() if kn not in PRETOK_KERNELS)
    res["stage_split"] = {
        "pretokenize_us": round(pre_us, 2),
        "pretokenize_GBps": round(n / (pre_us * 1e-6) / 1e9, 1) if pre_us else None,
        "bpe_and_emit_us": round(bpe_us, 2),
        "bpe_and_emit_GBps": round(n / (bpe_us * 1e-6) / 1e9, 1) if bpe_us else None,
    }
    res["roofline"] = roofline(name, n, T, nseq if off is not None else 0, kern_us, counters or {})
    return res


def _counter_key(kname, table):
    """The stored kernel name that kname (a tt_profile name, template
    arguments dropped where the profile keeps none) stands for."""
    if kname in table:
        return kname
    cands = [k for k in table if "<" not in kname and k.split("<")[0] == kname]
    return cands[0] if len(cands) == 1 else None


def roofline(name, n, T, nseq, kern_us, counters):
    c = counters.get(name, {})
    rp_table = c.get("avg_us", {})
    # the dominant kernel and its time: rocprofv3 averages where a record of
    # this kernel source exists, else the live event averages
    rp = {k: rp_table[_counter_key(k, rp_table)] for k in kern_us if _counter_key(k, rp_table)}
    use_rp = len(rp) == len(kern_us)
    times = rp if use_rp else kern_us
    dom = max(times, key=times.get)
    t_us = times[dom]
    key = _counter_key(dom, rp_table)
    alg = n + 4 * T + (16 * (nseq + 1) if nseq else 0)
    achieved = alg / (t_us * 1e-6) / 1e9
    roof = {
        "bound": "hbm",
        "kernel": key or dom,
        "achieved": round(achieved, 3),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": achieved / HBM_PEAK_GBS,
        "traffic": None,
        "alg_bytes": alg,
        "time_source": "rocprofv3 average (profiles/counters.json)" if use_rp else "live HIP events",
        "kernel_us": round(t_us, 3),
        "kernel_us_live": round(kern_us[dom], 2),
        "clock_ghz": CLOCK_GHZ,
    }
    if key:
        tr = c.get("hbm_bytes", {}).get(key)
        if tr is not None:
            roof["traffic"] = int(tr)
        vi = c.get("valu_insts", {}).get(key)
        if vi:
            valu = vi / (t_us * 1e-6) / 1e9
            roof["valu"] = {"insts": int(vi), "achieved": round(valu, 1), "peak": VALU_PEAK_GINST,
                            "unit": "G wave64 VALU instructions/s", "frac": round(valu / VALU_PEAK_GINST, 3)}
            roof["bound"] = "alu" if valu / VALU_PEAK_GINST > achieved / HBM_PEAK_GBS else "hbm"
    return roof


def run_session(steps, append_chars=1400):
    """Incremental repair (tt_session_append) on the 1M-char text as the
    session's context: host-inclusive latency of appends of ``append_chars``
    chars (the pages' median interactive append), against a full
    tt_encode_offsets of the same grown text; the session's tokens are checked
    against that full encode."""
    import numpy as np
    import torch

    import exact_byte_level_amd as tt
    from synth.text import workload
    from synth import mix_text

    data, offs, pat, voc = workload("c2")
    merges = np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % voc))
    tt.load(merges, pattern_id=pat)
    extra = mix_text(append_chars * (steps + 8), 4321)
    cap = len(data) + len(extra) + 16
    tt.reserve(cap, 1)
    s = tt.Session(cap)
    x = torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda()
    ext = torch.frombuffer(bytearray(extra), dtype=torch.uint8).cuda()
    s.reset(x)
    lat, full, ways = [], [], {}
    out = torch.empty(cap, dtype=torch.int32, device="cuda")
    st = torch.empty(cap + 1, dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, dtype=torch.int64, device="cuda")
    pos = 0
    for k in range(steps + 3):
        d = ext[pos:pos + append_chars]
        pos += append_chars
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        info = s.append(d)
        t1 = time.perf_counter()
        ways[info["doublings"]] = ways.get(info["doublings"], 0) + 1
        n, T = s.sizes()
        text = s.text()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        tt.encode_offsets_into(text, None, out, st, cnt)
        int(cnt.item())
        t3 = time.perf_counter()
        if k >= 3:
            lat.append((t1 - t0) * 1e3)
            full.append((t3 - t2) * 1e3)
    ok = (int(cnt.item()) == T and torch.equal(out[:T], s.ids()) and torch.equal(st[:T + 1], s.starts()))
    if not ok:
        raise RuntimeError("session tokens differ from a full encode")
    s.close()
    return {
        "context_chars": len(data),
        "append_chars": append_chars,
        "appends": steps,
        "append_p50_ms": statistics.median(lat),
        "full_reencode_p50_ms": statistics.median(full),
        "ways": {str(k): v for k, v in sorted(ways.items())},
        "verified_against_full_encode": ok,
    }


# ------------------------------------------------------------------ CPU side
# The oracle timed on this host's cores.  It runs before anything touches the
# GPU, in forked worker processes (fork only: no program is replaced).

def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    allowed = sorted(os.sched_getaffinity(0))
    return {"nproc": os.cpu_count(), "cpus_allowed": len(allowed), "cpu_model": model}, allowed


# Inputs of the CPU runs, prepared in the parent before the workers fork
# (each worker then reads them from its copy of the parent's memory).
_CPU = {}


def _cpu_input(name):
    import numpy as np
    from oracle.bpe import Vocab
    from synth.text import workload
    if name not in _CPU:
        data, offs, pat, voc = workload(name)
        _CPU[name] = (data, offs, pat, Vocab(np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % voc))))
    return _CPU[name]


def _oracle_job(args):
    """Worker: (workload, core, runs) -> per-run seconds of the split alone and
    of the whole encode, after one warm-up run."""
    name, core, runs = args
    from oracle.bpe import encode
    from oracle.pretok import split_bytes
    os.sched_setaffinity(0, {core})
    data, _, pat, v = _CPU[name]
    split_s, total_s = [], []
    for _ in range(runs + 1):
        t0 = time.perf_counter()
        split_bytes(data, pat)
        t1 = time.perf_counter()
        encode(data, v, pat)
        t2 = time.perf_counter()
        split_s.append(t1 - t0)
        total_s.append(t2 - t1)
    return split_s[1:], total_s[1:]


def _batch_text_job(args):
    """Worker of the all-cores batch run: encode text s of the batch."""
    name, s = args
    from oracle.bpe import encode
    data, offs, pat, v = _CPU[name]
    encode(data[offs[s]:offs[s + 1]], v, pat)


def cpu_baseline(runs=3):
    import multiprocessing as mp
    info, allowed = host_info()
    ctx = mp.get_context("fork")
    core = allowed[-1]
    data, _, _, _ = _cpu_input(HEADLINE)
    chars = len(data.decode("utf-8"))
    with ctx.Pool(1) as pool:
        split_s, total_s = pool.map(_oracle_job, [(HEADLINE, core, runs)])[0]
    t_all = statistics.median(total_s)
    t_split = statistics.median(split_s)
    res = {
        "value": chars / t_all,
        "unit": "chars/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "the whole %s text (%d chars): plain Python oracle (regex split + classic merge loop, no piece "
                  "memo), one process pinned to core %d, 1 warm-up + %d timed runs, median" % (
                      HEADLINE, chars, core, runs),
        "host": info,
        "pinned_core": core,
        "encode_s": round(t_all, 4),
        "split_s": round(t_split, 4),
        "bpe_s": round(t_all - t_split, 4),
    }
    # the 64-text batch on all allowed cores (a process per core, at most 16),
    # texts handed out largest first
    name = "c4"
    data, offs, _, _ = _cpu_input(name)
    bchars = len(data.decode("utf-8"))
    workers = min(16, len(allowed))
    nseq = len(offs) - 1
    jobs = [(name, s) for s in sorted(range(nseq), key=lambda s: -(offs[s + 1] - offs[s]))]
    times = []
    with ctx.Pool(workers) as pool:
        for r in range(runs + 1):
            t0 = time.perf_counter()
            pool.map(_batch_text_job, jobs, chunksize=1)
            if r:
                times.append(time.perf_counter() - t0)
    tb = statistics.median(times)
    res["batch_all_cores"] = {
        "workload": name, "chars": bchars, "workers": workers, "s": round(tb, 3),
        "chars_per_s": bchars / tb,
        "sample": "the whole 64-text batch, one text per task over %d worker processes, 1 warm-up + %d timed runs, "
                  "median" % (workers, runs),
    }
    return res


# ------------------------------------------------------- profile summaries

def summarize(outdir, name):
    """Read rocprofv3 CSV output under outdir (a kernel-trace run and counter
    runs of `bench.py --only --workload name`) and write
    profiles/<name>_kernels.md plus this workload's entry of
    profiles/counters.json."""
    src_sha = kernel_source_sha()
    stats = {}
    for p in glob.glob(os.path.join(outdir, "**", "*kernel_stats.csv"), recursive=True):
        with open(p) as f:
            for row in csv.DictReader(f):
                stats[row["Name"]] = row
    pmc = {}
    grid = {}
    for p in glob.glob(os.path.join(outdir, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as f:
            for row in csv.DictReader(f):
                key = (row["Kernel_Name"], row["Counter_Name"])
                pmc.setdefault(key, {})
                d = row.get("Dispatch_Id") or row.get("Correlation_Id")
                pmc[key][d] = pmc[key].get(d, 0.0) + float(row["Counter_Value"])
                grid[(key, d)] = int(row["Grid_Size"])

    def avg(kname, counter):
        v = pmc.get((kname, counter))
        return (sum(v.values()) / len(v), len(v)) if v else (None, 0)

    def probe_avg(kname, counter):
        # the copy kernel also serves the run's small uploads and reads:
        # only the dispatches of the largest grid are the 64 MiB probe
        v = pmc.get((kname, counter))
        if not v:
            return None
        g = max(grid[((kname, counter), d)] for d in v)
        vals = [x for d, x in v.items() if grid[((kname, counter), d)] == g]
        return sum(vals) / len(vals)

    copy = [k for k in {k for k, _ in pmc} if "copyBuffer" in k]
    fetch_scale = write_scale = None
    if copy:
        fk = probe_avg(copy[0], "FETCH_SIZE")
        wk = probe_avg(copy[0], "WRITE_SIZE")
        probe_kib = 64 * 1024.0
        fetch_scale = probe_kib / fk if fk else None
        write_scale = probe_kib / wk if wk else None
    kernels = sorted({k for k in stats} | {k for k, _ in pmc if "copyBuffer" not in k})
    entry = {"avg_us": {}, "hbm_bytes": {}, "valu_insts": {}}
    rows = []
    for k in kernels:
        base = _base_name(k)
        st = stats.get(k)
        avg_us = float(st["AverageNs"]) / 1e3 if st else None
        fk, nd = avg(k, "FETCH_SIZE")
        wk, _ = avg(k, "WRITE_SIZE")
        vi, _ = avg(k, "SQ_INSTS_VALU")
        hbm = None
        if fk is not None and wk is not None and fetch_scale and write_scale:
            hbm = 1024.0 * (fk * fetch_scale + wk * write_scale)
        if avg_us is not None and "copyBuffer" not in k:
            entry["avg_us"][base] = round(avg_us, 3)
        if hbm is not None:
            entry["hbm_bytes"][base] = round(hbm)
        if vi is not None:
            entry["valu_insts"][base] = round(vi)
        rows.append((k, st, avg_us, fk, wk, hbm, vi))
    cur = {"kernel_source_sha256": src_sha, "workloads": {}}
    if os.path.exists(COUNTERS):
        with open(COUNTERS) as f:
            old = json.load(f)
        if old.get("kernel_source_sha256") == src_sha:
            cur = old
    cur["workloads"][name] = entry
    with open(COUNTERS, "w") as f:
        json.dump(cur, f, indent=1, sort_keys=True)
    from synth.text import WORKLOADS
    lines = ["# Kernels of one encode: %s (%s)" % (name, WORKLOADS[name][2]), "",
             "rocprofv3 on one MI355X, run from /tmp (`<repo>` is the repository root); each counter in its own run:", "",
             "    rocprofv3 --kernel-trace --stats -f csv -d <out>/trace -o run -- python3 <repo>/bench.py --only "
             "--workload %s --steps 50 --warmup 5 --no-cpu --no-graph" % name]
    for c in ("FETCH_SIZE", "WRITE_SIZE", "SQ_INSTS_VALU"):
        lines.append("    timeout -s KILL 150 rocprofv3 --pmc %s -f csv -d <out>/%s -o %s -- python3 <repo>/bench.py "
                     "--only --workload %s --steps 5 --warmup 2 --no-cpu --no-graph --copy-probe 64" % (c, c, c, name))
    lines += ["", "    python3 bench.py --summarize <out> --workload %s" % name, ""]
    if fetch_scale:
        lines.append("Calibration: a 64 MiB device-to-device copy reads FETCH_SIZE %.1f KiB and WRITE_SIZE %.1f KiB per "
                     "dispatch, so fetch counts are scaled by %.4f and write counts by %.4f." % (
                         64 * 1024 / fetch_scale, 64 * 1024 / write_scale, fetch_scale, write_scale))
        lines.append("")
    lines += ["| kernel | calls | avg us | min us | max us | FETCH KiB | WRITE KiB | HBM bytes (scaled) | SQ_INSTS_VALU | "
              "VALU issue frac at %.1f GHz |" % CLOCK_GHZ,
              "|---|---|---|---|---|---|---|---|---|---|"]
    for k, st, avg_us, fk, wk, hbm, vi in rows:
        if "copyBuffer" in k:
            continue
        frac = vi * 4 / SIMDS / (CLOCK_GHZ * 1e3) / avg_us if (vi and avg_us) else None
        lines.append("| %s | %s | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            _base_name(k), st["Calls"] if st else "-", "%.2f" % avg_us if avg_us else "-",
            "%.2f" % (float(st["MinNs"]) / 1e3) if st else "-", "%.2f" % (float(st["MaxNs"]) / 1e3) if st else "-",
            "%.1f" % fk if fk is not None else "-", "%.1f" % wk if wk is not None else "-",
            "%d" % hbm if hbm is not None else "-", "%d" % vi if vi is not None else "-",
            "%.3f" % frac if frac else "-"))
    lines += ["", "Kernel source: tt_kernels.hip sha256 %s." % src_sha, ""]
    path = os.path.join(ROOT, "profiles", "%s_kernels.md" % name)
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(path)


# ---------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only", action="store_true", help="time only --workload (no other workloads, no session)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-session", action="store_true", help="skip the incremental-repair latency line")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize", metavar="DIR", help="summarise rocprofv3 CSV output of --workload into profiles/")
    args = ap.parse_args()

    if args.summarize:
        summarize(args.summarize, args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this path runs on one GPU only (no sharding or collectives are built); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    # the CPU oracle first: its worker processes are forked before anything
    # touches the GPU
    cpu = None if args.no_cpu else cpu_baseline()

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.copy_probe:
        src = torch.empty(args.copy_probe << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    counters = load_counters()
    head = measure(args.workload, args.steps, args.warmup, graph=not args.no_graph, detail=not args.only,
                   counters=counters)
    others = {}
    if not args.only:
        for name in ALL_WORKLOADS:
            if name == args.workload:
                continue
            r = measure(name, args.steps, args.warmup, graph=not args.no_graph, counters=counters)
            others[name] = r
            print("%s: p50 %.4f ms, %.3g chars/s, graph p50 %s ms (back to back %s), kernels (us) %s" % (
                name, r["p50_ms"], r["chars_per_s"], "%.4f" % r["graph_p50_ms"] if "graph_p50_ms" in r else "-",
                "%.4f" % r["graph_back_to_back_mean_ms"] if "graph_back_to_back_mean_ms" in r else "-",
                r.get("kernels_us")), file=sys.stderr, flush=True)
    sess = run_session(min(args.steps, 50)) if args.workload == "c2" and not args.no_session and not args.only \
        else None

    config = {"workload": "%s: %s" % (args.workload, head["desc"])}
    config.update({k: v for k, v in head.items() if k not in ("desc", "roofline")})
    config["session"] = sess
    config["workloads"] = {k: {kk: vv for kk, vv in v.items() if kk not in ("kernels_us",)} for k, v in others.items()}
    config["parallelism"] = "single GPU"
    line = {
        "metric": METRIC,
        "value": head["chars_per_s"],
        "unit": "chars/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["p50_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": config,
        "roofline": head["roofline"],
    }
    if cpu:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
