"""Benchmark: KV tokens compacted per second (score + select + gather +
re-rotate) on one MI355X, with the dominant call's HBM roofline and the CPU
oracle's rate on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: the Qwen3-8B-shaped 100,000-token session. One step is one
compaction of the whole session: kvc_score, kvc_select and
kvc_compact_rerotate over every (layer, KV head) row, inputs resident in HBM.
Decode attention over the compacted cache is timed beside the step (not in
`value`).

Other workloads (parity cases, measured the same way call by call):
  tiny            1 layer, T=4096, B=512, renumbered
  qwen3_8b_1m     T=1,048,576, all 36 layers per call (154.6 GB of K+V resident)
  pask_llama3_8b  64 x 32 layers: prompt compaction, int8/bf16/release tiers, decode
  pask_llama3_8b_int4  the same with the pages' INT4 low tier (two nibbles per byte)
  commitkv_28l    16 x 28 layers: page effects, retirement, checkpoint, paged decode
  commitkv_events the same commit on event pages (events of 1..40 tokens, pages of at most
                  16): pages kept under the token budget, compacted by token list
  commitkv_multi  16 x 28 layers: four successive commits (pre/post effects, pending-page
                  protection, checkpoint, retirement); one step = the four commits
  pace_h2o_decode 36 layers x 8 KV heads of 2048 + 32 resident slots: one step is one
                  eviction cycle (32 decode steps adding H2O cumulative attention,
                  then top-B by cumulative score + foresight bonus and compaction);
                  value = resident tokens per second through the cycle

Prints one JSON line.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")
METRIC = "KV tokens compacted/sec (score+select+gather+rerotate), % of HBM peak, 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b_100k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the CPU oracle sample (0 disables it)")
    ap.add_argument("--flush-mb", type=int, default=1024,
                    help="scratch written before every timed step so no step starts from cached data "
                         "(the 256 MB memory-side cache); 0 disables it")
    ap.add_argument("--layers-per-call", type=int, default=0,
                    help="layers per kvc_score / kvc_select / kvc_compact_rerotate call (a divisor of 36; "
                         "default all of them); with several groups one is selected and compacted on a "
                         "second stream while the next is scored")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (three times), so that HBM "
                         "counters can be scaled against a transfer of known size")
    return ap.parse_args()


# Sources (and build flags) of the calls whose HBM counters profiles/ holds:
# the counters stay valid until one of these changes.
COUNTED_SOURCES = ["budgeted_retention_amd/csrc/" + n for n in
                   ("kvc_internal.h", "common.hip", "score.hip", "select.hip", "compact.hip")] + [
                   "budgeted_retention_amd/build.py"]


_C_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def _code_only(name, text):
    """The source with C/C++ comments and blank space removed (string and
    character literals kept), so that editing a comment leaves the hash alone."""
    if not name.endswith((".hip", ".h", ".cpp")):
        return text
    text = _C_TOKENS.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    """Hash of the code (comments excluded) the counters were taken on."""
    h = hashlib.sha256()
    for name in COUNTED_SOURCES:
        with open(os.path.join(ROOT, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(_code_only(name, f.read()).encode())
    return h.hexdigest()[:16]


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_bandwidth(dev, mib=2048):
    """Device-to-device copy rate on this machine (bytes read + written per second)."""
    import torch
    n = mib * (1 << 20) // 2
    src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(5):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 5 * 2 * n * 2 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    return round(gbs, 1)


def host_cores():
    """Cores of this host (os.cpu_count) and the share a job may use: the
    scheduler's thread limit when one is set (OMP_NUM_THREADS), else all."""
    n = os.cpu_count() or 1
    lim = os.environ.get("OMP_NUM_THREADS", "")
    share = min(n, int(lim)) if lim.isdigit() and int(lim) > 0 else n
    return n, share


def run_metadata(dev):
    """Where the line was measured: commit, ROCm and torch versions, GPU name,
    and the GPU's current and maximum shader clock."""
    import subprocess
    import torch
    meta = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None), "git": None}
    if os.path.isdir(os.path.join(ROOT, ".git")):
        try:
            meta["git"] = subprocess.run(["git", "rev-parse", "--short=12", "HEAD"], cwd=ROOT, capture_output=True,
                                         text=True, timeout=10).stdout.strip() or None
        except Exception:
            pass
    if meta["git"] is None:   # a tree without its history: the commit the library was built from
        try:
            info = json.load(open(os.path.join(ROOT, "budgeted_retention_amd", "build_info.json")))
            meta["git"] = info.get("git")
            meta["git_dirty_at_build"] = info.get("dirty")
        except (OSError, ValueError):
            pass
    try:
        meta["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        meta["rocm"] = None
    p = torch.cuda.get_device_properties(dev)
    meta["gpu"] = f"{p.name} ({getattr(p, 'gcnArchName', '')}, {p.multi_processor_count} CUs)"
    meta["sclk"] = shader_clock(p)
    return meta


def shader_clock(props):
    """The GPU's current shader clock level from the driver's sysfs table
    (the line marked '*' of pp_dpm_sclk), read directly rather than through a
    helper program; the device's own PCI address when torch reports it."""
    import glob
    paths = []
    bus = getattr(props, "pci_bus_id", None)
    if bus is not None:
        dom, dev = getattr(props, "pci_domain_id", 0), getattr(props, "pci_device_id", 0)
        paths.append(f"/sys/bus/pci/devices/{dom:04x}:{bus:02x}:{dev:02x}.0/pp_dpm_sclk")
    paths += sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    for path in paths:
        try:
            lines = open(path).read().splitlines()
        except OSError:
            continue
        for line in lines:
            if line.rstrip().endswith("*") and ":" in line:
                return line.split(":", 1)[1].replace("*", "").strip()
    return None


# ---------------------------------------------------------------- algorithmic bytes

def compaction_bytes(rows, T, d, G, W, B):
    """Bytes each call must move at least once, per row: score reads K
    (T*d bf16) and the group's window queries (G*W*d bf16) once and writes T
    fp32 scores; select reads the scores and the row's tags (T bytes) and
    writes B indices and the count; compaction reads and writes B keys and
    values (bf16) plus B input and output positions; decode reads the B kept
    keys and values and the group's queries and writes their outputs."""
    score = T * d * 2 + G * W * d * 2 + T * 4
    select = T * 4 + T + B * 4 + 4
    compact = 2 * B * d * 2 + 2 * B * d * 2 + B * 4 * 2
    path = T * d * 2 + G * W * d * 2 + 4 * B * d * 2 + 16 * B   # the whole path, scores kept on chip
    decode = 2 * B * d * 2 + 2 * G * d * 2
    return dict(kvc_score=score * rows, kvc_select=select * rows, kvc_compact_rerotate=compact * rows,
                path=path * rows, kvc_decode_attn=decode * rows)


def roofline(bytes_per_call, ms, counters_name, workload):
    achieved = bytes_per_call / (ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(COUNTERS_FILE):
        c = json.load(open(COUNTERS_FILE))
        ent = c.get("calls", {}).get(counters_name)
        if ent and c.get("source_hash") == kernel_source_hash() and c.get("workload") == workload:
            traffic = ent["hbm_bytes_per_call"]
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": counters_name,
            "algorithmic_bytes": bytes_per_call}


def per_call_rates(bytes_by_call, ms_by_call):
    return {k: {"ms": round(ms_by_call[k], 4),
                "GB_s": round(bytes_by_call[k] / (ms_by_call[k] * 1e-3) / 1e9, 1),
                "hbm_frac": round(bytes_by_call[k] / (ms_by_call[k] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            for k in ms_by_call if k in bytes_by_call and ms_by_call[k] > 0}


# ---------------------------------------------------------------- CPU oracle baselines

def cpu_compaction_rows(K, V, Q, G, W, T, B, tags, bonus_tbl, n_sink, n_recent, renumber_base, rope_base,
                        rows, budget_s, L, Hkv, threads=1):
    """Time the float64 oracle (score + select + gather/re-rotate) over the
    rows in order (D2H copies of the exact input bytes, made before the timed
    part) until all `rows` are done or about `budget_s` seconds have passed.
    `threads` rows run at once, each on one BLAS thread (numpy releases the
    interpreter lock inside its array operations); the time is the wall time
    of those parallel batches. Returns (rows done, seconds)."""
    import concurrent.futures
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    from oracle import compact as o_compact, numfmt, policy as o_policy, score as o_score
    from oracle import select as o_select
    fl = np.zeros_like(bonus_tbl, dtype=np.uint8)

    def fetch(r):
        n, l, h = r // (L * Hkv), (r // Hkv) % L, r % Hkv
        return (K[n, l, h].cpu().view(torch.int16).numpy().view(np.uint16),
                V[n, l, h].cpu().view(torch.int16).numpy().view(np.uint16),
                Q[n, l, h * G:(h + 1) * G].cpu().view(torch.int16).numpy().view(np.uint16),
                tags[n].cpu().numpy() if tags is not None else np.zeros(T, np.uint8))

    def one(row):
        Kb, Vb, Qb, tg = row
        s = o_score.obs_window_score(numfmt.bf16_bits_to_f64(Kb), numfmt.bf16_bits_to_f64(Qb), W)
        tot, prot = o_policy.totals_and_protection(s, tg, bonus_tbl, fl, 0, n_sink, n_recent)
        kept, _ = o_select.select_top_b(tot, prot, B)
        o_compact.compact_row(Kb, Vb, np.arange(T), kept, renumber_base, rope_base)

    done, spent = 0, 0.0
    with threadpool_limits(limits=1), concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        while spent < budget_s and done < rows:
            batch = [fetch(r) for r in range(done, min(rows, done + threads))]
            t0 = time.perf_counter()
            list(ex.map(one, batch))
            spent += time.perf_counter() - t0
            done += len(batch)
    return done, spent


def oracle_call_times(w, budget_s):
    """The float64 oracle's time for the session's decode attention over the
    compacted cache and for score pooling (kernel 7), measured on a prefix of
    rows of seeded inputs of the same shapes and scaled to all rows (ms)."""
    import numpy as np
    from oracle import decode as o_decode, score as o_score
    rng = np.random.default_rng(1)
    G, d, B, T = w.group, w.head_dim, w.budget, w.n_tokens
    out = {}
    done, spent = 0, 0.0
    while spent < budget_s and done < w.rows:
        K, V, q = rng.standard_normal((B, d)), rng.standard_normal((B, d)), rng.standard_normal((G, d))
        t0 = time.perf_counter()
        for g in range(G):
            o_decode.decode_head(q[g], K, V)
        spent += time.perf_counter() - t0
        done += 1
    out["kvc_decode_attn"] = {"cpu_ms": round(spent / done * w.rows * 1e3, 2), "rows_sampled": done}
    done, spent = 0, 0.0
    while spent < budget_s and done < w.rows:
        sc = rng.gamma(0.5, 1.0, T)
        t0 = time.perf_counter()
        o_score.pool_scores(sc, 7, "max")
        spent += time.perf_counter() - t0
        done += 1
    out["kvc_pool_scores"] = {"cpu_ms": round(spent / done * w.rows * 1e3, 2), "rows_sampled": done}
    return out


def oracle_bonus(steps_ahead):
    import numpy as np
    from oracle import policy as o_policy
    return np.array([[0.0]] + [[0.0 if s is None else o_policy.foresight_bonus(1e3, 0.35, s)]
                               for s in steps_ahead])


# ---------------------------------------------------------------- workloads

def bench_compaction(args, w, dev):
    """score -> select -> compact over every row, then decode over the
    compacted cache. The layers go in groups of --layers-per-call (all 36 in
    one call by default). With several groups the scores of group g+1 are
    computed on one stream while group g is selected and compacted on a
    second stream (both at the default priority). The step is timed from the
    first launch to the last compaction's end event."""
    import torch
    from budgeted_retention_amd import kvc, synth
    inp = synth.make_compaction_inputs(w, dev)
    N, L, Hkv, Hq, d, T, W, B = (w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim,
                                 w.n_tokens, w.window, w.budget)
    per_layer = w.n_tokens > (1 << 20) - 1
    Lc = args.layers_per_call or L
    if L % Lc:
        raise SystemExit(f"--layers-per-call {Lc} must divide {L} layers")
    chunks = [(l, l + Lc) for l in range(0, L, Lc)]
    nc = len(chunks)
    rows_c = N * Lc * Hkv
    dims = kvc.make_dims(N, Lc, Hkv, Hq, d, T)
    vals = [0.0] + [0.0 if s is None else kvc.kvc_foresight_bonus(1e3, 0.35, s) for s in inp.spans.steps_ahead]
    bonus = torch.tensor(vals, dtype=torch.float32, device=dev).reshape(-1, 1)
    pols = [kvc.Policy(w.n_sink, w.n_recent, B, len(vals), 1, l0, L, inp.tags, bonus) for l0, _ in chunks]
    ws = kvc.workspace(kvc.KVC_OP_SCORE, dims, W, 0, dev)
    n_sel = kvc.kvc_workspace_bytes(kvc.KVC_OP_SELECT, dims, 0, B)
    ws_sel = torch.empty(n_sel, dtype=torch.uint8, device=dev) if n_sel else None
    # every group its own buffers: the two streams never touch the same memory
    scores = torch.empty((nc, rows_c, T), dtype=torch.float32, device=dev)
    kept = torch.empty((nc, rows_c, B), dtype=torch.int32, device=dev)
    n_kept = torch.empty((nc, rows_c), dtype=torch.int32, device=dev)
    Ko = torch.empty((nc, rows_c, B, d), dtype=torch.bfloat16, device=dev)
    Vo = torch.empty_like(Ko)
    po = torch.empty((nc, rows_c, B), dtype=torch.int32, device=dev)
    nh = torch.empty((nc, rows_c), dtype=torch.int32, device=dev)
    outs = [kvc.CompactOut(B, Ko[c], Vo[c], po[c], nh[c]) for c in range(nc)]
    dims_d = kvc.make_dims(N, Lc, Hkv, Hq, d, B)
    wsd = torch.empty(max(1, kvc.kvc_decode_workspace_bytes(dims_d, B, 0)), dtype=torch.uint8, device=dev)
    o = torch.empty((nc, N, Lc, Hq, d), dtype=torch.bfloat16, device=dev)
    views = []
    for l0, l1 in chunks:
        Kc, Vc, Qc, qc = inp.K[:, l0:l1], inp.V[:, l0:l1], inp.Q_obs[:, l0:l1], inp.q_dec[:, l0:l1]
        assert all(t.is_contiguous() for t in (Kc, Vc, Qc, qc))
        views.append((Kc, Vc, Qc, qc))
    names = ["kvc_score", "kvc_select", "kvc_compact_rerotate", "kvc_decode_attn"]
    s_score = torch.cuda.current_stream()
    s_comp = torch.cuda.Stream()              # default priority
    last_comp = [torch.cuda.Event()]          # the previous step's last event on s_comp

    def ev(stream):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def step(rec=None):
        s_score.wait_event(last_comp[0])
        t = {n: [] for n in names}
        t["start"] = ev(s_score)
        for c, ((Kc, Vc, Qc, qc), pol) in enumerate(zip(views, pols)):
            a = ev(s_score)
            kvc.kvc_score(dims, Kc, Qc, W, scores[c], ws, stream=s_score)
            b = ev(s_score)
            t["kvc_score"].append((a, b))
            s_comp.wait_event(b)
            a = ev(s_comp)
            kvc.kvc_select(dims, scores[c], pol, kept[c], B, n_kept[c], ws_sel, stream=s_comp)
            b = ev(s_comp)
            t["kvc_select"].append((a, b))
            kvc.kvc_compact_rerotate(dims, Kc, Vc, None, kept[c], B, n_kept[c], w.renumber_base, w.rope_base,
                                     outs[c], stream=s_comp)
            e = ev(s_comp)
            t["kvc_compact_rerotate"].append((b, e))
        t["end"] = e
        for c, (_, _, _, qc) in enumerate(views):   # after the path, off its critical stream order
            a = ev(s_comp)
            kvc.kvc_decode_attn(dims_d, qc, Ko[c], Vo[c], nh[c], B, o[c], wsd, stream=s_comp)
            t["kvc_decode_attn"].append((a, ev(s_comp)))
        last_comp[0] = torch.cuda.Event()
        last_comp[0].record(s_comp)
        if rec is not None:
            rec.append(t)

    calibrate_copy(args, dev)
    flush = torch.empty(max(1, args.flush_mb) * (1 << 18), dtype=torch.float32, device=dev) if args.flush_mb else None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for k in range(args.steps):
        if flush is not None:
            s_score.wait_event(last_comp[0])
            flush.fill_(float(k))   # outside the step's events
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step, part = [], {n: 0.0 for n in names}
    for t in recs:
        one = {n: sum(a.elapsed_time(b) for a, b in t[n]) for n in names}
        one["path"] = t["start"].elapsed_time(t["end"])
        per_step.append(one)
        for n in names:
            part[n] += one[n]
    part = {n: v / args.steps for n, v in part.items()}
    path_ms = sorted(o_["path"] for o_ in per_step)
    median_ms = path_ms[len(path_ms) // 2] if len(path_ms) % 2 else \
        0.5 * (path_ms[len(path_ms) // 2 - 1] + path_ms[len(path_ms) // 2])
    if not (n_kept == B).all():
        raise SystemExit("bench: a row kept a number of tokens other than the budget")
    mean_ms = sum(path_ms) / len(path_ms)
    ms = median_ms
    ab = compaction_bytes(w.rows, T, d, w.group, W, B)
    path_calls = names[:3]
    dom = max(path_calls, key=lambda n: part[n])
    roof = roofline(ab[dom], part[dom], dom, w.name)
    cpu = None
    if args.cpu_seconds > 0:
        n_host, share = host_cores()
        orc = (inp.K, inp.V, inp.Q_obs, w.group, W, T, B, inp.tags, oracle_bonus(inp.spans.steps_ahead),
               w.n_sink, w.n_recent, w.renumber_base, w.rope_base, w.rows)
        done, spent = cpu_compaction_rows(*orc, args.cpu_seconds, L, Hkv, threads=share)
        limit = "all rows" if done == w.rows else f"the first {done} rows (the {args.cpu_seconds:.0f} s limit)"
        cpu = {"value": T * N * (done / w.rows) / spent, "unit": "tokens/s", "cores": share,
               "host_cores": n_host, "kind": "oracle",
               "sample": f"{limit} of the {w.rows} (layer, KV head) rows of one {T}-token session: the float64 "
                         f"numpy oracle (score+select+gather/re-rotate), {share} rows at a time on one BLAS "
                         f"thread each, {spent:.1f} s of wall time, scaled to the whole session",
               "cpu_model": cpu_model()}
        # the same oracle on one core, on a smaller sample
        d1, s1 = cpu_compaction_rows(*orc, args.cpu_seconds / 5, L, Hkv, threads=1)
        cpu["value_1core"] = T * N * (d1 / w.rows) / s1
        cpu["rows_1core"] = d1
        cpu["calls"] = oracle_call_times(w, args.cpu_seconds / 5)
    value = N * T / (ms * 1e-3)
    config = {"workload": w.name, "n_seq": N, "layers": L, "kv_heads": Hkv, "q_heads": Hq, "head_dim": d,
              "tokens": T, "window": W, "budget": B, "sink": w.n_sink, "recent": w.n_recent,
              "rope_base": w.rope_base, "layers_per_call": Lc, "parallelism": "none"}
    copy_gbs = copy_bandwidth(dev)
    extra = {"hbm_frac_path": round(ab["path"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "ms_mean": round(mean_ms, 4), "timing": f"median of {args.steps} steps, each after writing "
             f"{args.flush_mb} MiB of scratch; a step runs from the first score launch to the last "
             f"compaction's end event; {nc} group(s) of {Lc} layers"
             + (", each group selected and compacted on a second stream while the next is scored"
                if nc > 1 else ""),
             "copy_GB_s": copy_gbs, "roofline_frac_of_copy": round(roof["achieved"] / copy_gbs, 4),
             "breakdown_ms": {n: round(part[n], 4) for n in path_calls},
             "decode_ms": round(part["kvc_decode_attn"], 4),
             "calls": per_call_rates(ab, part),
             "wall_ms_per_step": round(wall * 1e3 / args.steps, 4)}
    if not per_layer and w.renumber_base >= 0:
        dims_all = kvc.make_dims(N, L, Hkv, Hq, d, T)      # every group at once: the whole session
        extra["ref_store"] = bench_ref_store(args, w, dims_all, inp.K, inp.V, kept.view(-1, B), n_kept.view(-1),
                                             Ko.view(-1, B, d), Vo.view(-1, B, d), po.view(-1, B), dev)
        extra["pool"] = bench_pool(args, dims_all, scores.view(-1, T))
    return value, ms, config, roof, cpu, extra


def bench_pool(args, dims, scores):
    """Max pooling (kernel 7) of the session's window scores, timed on its own:
    the optional smoothing step between scoring and selection."""
    import torch
    from budgeted_retention_amd import kvc
    pooled = torch.empty_like(scores)
    for _ in range(max(1, args.warmup)):
        kvc.kvc_pool_scores(dims, scores, 7, kvc.KVC_POOL_MAX, pooled)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(args.steps):
        kvc.kvc_pool_scores(dims, scores, 7, kvc.KVC_POOL_MAX, pooled)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    nbytes = scores.numel() * 8   # each score read once and written once
    return {"ms": round(ms, 4), "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
            "kernel": 7, "mode": "max"}


def bench_ref_store(args, w, dims, K, V, kept, n_kept, Ko, Vo, po, dev):
    """The next compaction of the resident set with the reference store on:
    the B kept slots (with the references a first compaction started) plus B
    newly appended tokens without references, of which every other slot is
    kept. Timed on its own; not part of the step."""
    import torch
    from budgeted_retention_amd import kvc, synth
    rows, B, d = Ko.shape
    R1 = torch.empty_like(Ko)
    q1 = torch.empty_like(po)
    first = kvc.CompactOut(B, Ko, Vo, po, None, K_ref_out=R1, p_ref_out=q1)
    kvc.kvc_compact_rerotate(dims, K, V, None, kept, B, n_kept, w.renumber_base, w.rope_base, first)
    rK = torch.cat([Ko, synth.normal_bf16((rows, B, d), 71, dev)], dim=1)
    rV = torch.cat([Vo, synth.normal_bf16((rows, B, d), 72, dev)], dim=1)
    rp = torch.cat([po, torch.arange(B, 2 * B, dtype=torch.int32, device=dev).repeat(rows, 1)], dim=1)
    rR = torch.cat([R1, torch.zeros_like(R1)], dim=1)
    rq = torch.cat([q1, torch.full_like(q1, -1)], dim=1)
    keep = torch.arange(0, 2 * B, 2, dtype=torch.int32, device=dev).repeat(rows, 1)
    cnt = torch.full((rows,), B, dtype=torch.int32, device=dev)
    outs = [torch.empty((rows, B, d), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    o2 = kvc.CompactOut(B, outs[0], outs[1], torch.empty_like(po), None, K_ref=rR, p_ref=rq,
                        K_ref_out=outs[2], p_ref_out=torch.empty_like(po))
    dims_r = kvc.make_dims(w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, d, 2 * B)
    call = lambda: kvc.kvc_compact_rerotate(dims_r, rK, rV, rp, keep, B, cnt, 0, w.rope_base, o2)  # noqa: E731
    for _ in range(max(1, args.warmup)):
        call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(args.steps):
        call()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    used = int((o2.p_ref_out[:, : B // 2] == q1[:, 0::2]).float().mean().item() * 100 + 0.5)
    # kept K, V and references read and written, plus index, positions and reference positions
    nbytes = rows * B * (12 * d + 20)
    return {"ms": round(ms, 4), "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
            "resident_slots": 2 * B, "kept": B, "old_slots_from_reference_pct": used}


def bench_pipeline(args, w, dev, kind):
    """The mixed-precision or page-lifecycle workload, every call timed."""
    import numpy as np
    import torch
    from budgeted_retention_amd import pipelines, synth
    if kind == "pask":
        inp = synth.make_pask_inputs(w, dev)
        run = lambda timer=None: pipelines.run_pask(w, inp, timer)   # noqa: E731
        tokens = w.n_seq * (w.n_prompt + w.n_gen)
    else:
        inp = synth.make_commit_inputs(w, dev)
        run = lambda timer=None: pipelines.run_commit(w, inp, [w.tau_joint], timer)   # noqa: E731
        tokens = w.n_seq * w.n_tokens
    calibrate_copy(args, dev)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    timer = pipelines.CallTimer()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        res = run(timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    part = timer.median_step_ms(args.steps)
    host = {k: round(v * 1e3 / args.steps, 3) for k, v in timer.host.items()}
    d, Hkv, G, W = w.head_dim, w.n_kv_heads, w.n_q_heads // w.n_kv_heads, w.window
    rows = w.rows
    if kind == "pask":
        Tp, Tg, B = w.n_prompt, w.n_gen, w.budget
        n_h = int(res["n_h"].sum().item())                  # bf16 pool tokens (kept prompt + bf16 tier)
        n_l = int(res["n_l"].sum().item())                  # int8 pool tokens
        n_hg = n_h - rows * B                               # generated tokens routed to bf16
        ab = {"kvc_score": rows * (Tp * d * 2 + G * W * d * 2 + Tp * 4),
              "kvc_select": rows * (Tp * 4 + B * 4),
              "kvc_compact_rerotate:prompt": rows * (2 * B * d * 2 * 2 + B * 4),
              # every generated token's K, V, action, index and position read; the bf16
              # tier written with positions, the int8 tier as codes, fp16 scales, positions
              "kvc_compact_rerotate:tiered": rows * Tg * (2 * d * 2 + 1 + 4 + 4) + n_hg * (2 * d * 2 + 4)
                                             + n_l * (2 * d * w.low_bits // 8 + 2 * 2 + 4),
              # both pools read once, queries read and outputs written
              "kvc_decode_attn": n_h * 2 * d * 2 + n_l * (2 * d * w.low_bits // 8 + 2 * 2)
                                 + w.n_seq * w.n_layers * w.n_q_heads * d * 2 * 2}
        path_calls = ["kvc_score", "kvc_select", "kvc_compact_rerotate:prompt", "kvc_compact_rerotate:tiered"]
    else:
        T, B, ps = w.n_tokens, w.budget, w.page_size
        lrows = w.n_seq * Hkv          # rows of the deciding layer
        ab = {"kvc_page_effect:pre": lrows * (2 * T * d * 2 + G * W * d * 2),
              "kvc_page_effect:post": lrows * (2 * T * d * 2 + G * W * d * 2),
              "kvc_page_retire": lrows * (2 * T * d * 2 + G * W * d * 2),
              "kvc_score": rows * (T * d * 2 + G * W * d * 2 + T * 4)}
        if w.event_max:
            # event pages: (first, length) read wherever pages are read; the kept token count
            # per trajectory is what the budget admitted
            P = int(res["page_first"].shape[1])
            kept_pages = int(res["n_kept"].sum().item())
            kept_tok = res["n_tokens"].cpu().numpy().astype(np.int64)
            per_row_tok = int(kept_tok.sum()) * w.n_layers * Hkv
            ab.update({"kvc_page_scores": rows * T * 4 + w.n_seq * P * (4 + 8),
                       "kvc_page_select": w.n_seq * P * (4 + 8) + kept_pages * 4,
                       "kvc_page_tokens": kept_pages * (4 + 8) + int(kept_tok.sum()) * 4,
                       "kvc_compact_rerotate": per_row_tok * (2 * d * 2 * 2 + 4),
                       "kvc_decode_attn:pool": per_row_tok * 2 * d * 2,
                       "kvc_decode_attn:paged": per_row_tok * 2 * d * 2})
            path_calls = ["kvc_page_effect:pre", "kvc_page_effect:post", "kvc_page_retire", "kvc_score",
                          "kvc_page_scores", "kvc_page_select", "kvc_page_tokens", "kvc_compact_rerotate"]
        else:
            P = w.n_pages_all
            ab.update({"kvc_page_scores": rows * T * 4 + w.n_seq * P * 4,
                       "kvc_select": w.n_seq * (P * 4 + (B // ps) * 4),
                       "kvc_compact_rerotate": rows * (2 * B * d * 2 * 2 + B * 4),
                       "kvc_decode_attn:pool": rows * 2 * B * d * 2,
                       "kvc_decode_attn:paged": rows * 2 * B * d * 2})
            path_calls = ["kvc_page_effect:pre", "kvc_page_effect:post", "kvc_page_retire", "kvc_score",
                          "kvc_page_scores", "kvc_select", "kvc_compact_rerotate"]
    ms = sum(part[k] for k in path_calls)
    dom = max(path_calls, key=lambda k: part[k])
    roof = roofline(ab[dom], part[dom], dom, w.name)
    cpu = None
    if args.cpu_seconds > 0:
        n_host, share = host_cores()
        if kind == "pask":
            done, spent = cpu_compaction_rows(inp.K, inp.V, inp.Q_obs, G, W, w.n_prompt, w.budget, None,
                                              np.zeros((1, 1)), w.n_sink, w.n_recent, -1, w.rope_base, rows,
                                              args.cpu_seconds, w.n_layers, Hkv, threads=share)
            cpu = {"value": w.n_seq * w.n_prompt * (done / rows) / spent, "unit": "tokens/s",
                   "cores": share, "host_cores": n_host, "kind": "oracle",
                   "sample": f"{done} of {rows} prompt rows (score+select+gather), float64 numpy oracle, "
                             f"{share} rows at a time on one BLAS thread each, {spent:.1f} s of wall time "
                             f"scaled to all prompt tokens"}
        else:
            done, spent = cpu_compaction_rows(inp.K, inp.V, inp.Q_post, G, W, w.n_tokens, w.budget, None,
                                              np.zeros((1, 1)), 0, 0, -1, 1e6, rows, args.cpu_seconds,
                                              w.n_layers, Hkv, threads=share)
            cpu = {"value": w.n_seq * w.n_tokens * (done / rows) / spent, "unit": "tokens/s",
                   "cores": share, "host_cores": n_host, "kind": "oracle",
                   "sample": f"{done} of {rows} rows: post-commit window score + per-row top-B and gather "
                             f"(float64 numpy oracle, {share} rows at a time on one BLAS thread each), "
                             f"{spent:.1f} s of wall time scaled to all rows; the page effects are not in "
                             f"the sample"}
    value = tokens / (ms * 1e-3)
    if kind == "pask":
        config = {"workload": w.name, "n_seq": w.n_seq, "layers": w.n_layers, "layer_groups": w.n_groups,
                  "kv_heads": Hkv, "q_heads": w.n_q_heads, "head_dim": d, "prompt": w.n_prompt,
                  "generated": w.n_gen, "window": W, "budget": w.budget, "byte_budget": w.budget_fraction, "low_bits": w.low_bits,
                  "parallelism": "none"}
    else:
        config = {"workload": w.name, "n_seq": w.n_seq, "layers": w.n_layers, "kv_heads": Hkv,
                  "q_heads": w.n_q_heads, "head_dim": d, "tokens": w.n_tokens, "page": w.page_size,
                  "window": W, "budget": w.budget, "decision_layer": w.layer, "parallelism": "none"}
        if w.event_max:
            config.update(pages=f"event pages: history events of 1..{w.event_max} tokens cut into pages of "
                                f"at most {w.page_size}", n_pages=P,
                          kept_tokens_mean=round(float(res["n_tokens"].float().mean().item()), 1))
    extra = {"timing": f"per call, the median over {args.steps} runs of its HIP-event time; ms_per_step "
                       f"sums the path's calls",
             "breakdown_ms": {k: round(part[k], 4) for k in path_calls},
             "other_ms": {k: round(v, 4) for k, v in part.items() if k not in path_calls},
             "host_ms": host, "calls": per_call_rates(ab, part),
             "wall_ms_per_step": round(wall * 1e3 / args.steps, 4)}
    return value, ms, config, roof, cpu, extra


def cpu_h2o_rows(w, inp, budget_s):
    """Time the float64 oracle's cycle (E decode steps of cumulative attention,
    eviction, gather) over a prefix of rows. Returns (rows done, seconds)."""
    import numpy as np
    import torch
    from oracle import h2o, numfmt, policy
    B, E, G, L, Hkv = w.budget, w.interval, w.group, w.n_layers, w.n_kv_heads
    from budgeted_retention_amd.pipelines import H2O_SIGMA
    bonus = np.array([0.0] + [policy.foresight_bonus(H2O_SIGMA, 0.35, s) for s in inp.steps_ahead]).reshape(-1, 1)
    floor = np.zeros_like(bonus, np.uint8)
    done, spent = 0, 0.0
    while done < w.rows and spent < budget_s:
        r = done
        l, h = (r // Hkv) % L, r % Hkv
        K = inp.K[r].cpu().view(torch.int16).numpy().view(np.uint16).copy()
        K[B:] = inp.K_new[0, r].cpu().view(torch.int16).numpy().view(np.uint16)
        q = inp.q[0, :, 0, l, h * G:(h + 1) * G].float().cpu().numpy().astype(np.float64)
        acc = inp.acc[r].cpu().numpy().astype(np.float64)
        tags = inp.tags[r].cpu().numpy().astype(np.int64)
        t0 = time.perf_counter()
        Kf = numfmt.bf16_bits_to_f64(K)
        for e in range(E):
            acc[:B + e + 1] = h2o.accumulate(acc[:B + e + 1], q[e], Kf[:B + e + 1])
        kept = h2o.evict(acc, tags, bonus, floor, 0, w.n_sink, w.n_recent, B)
        _ = (K[kept], acc[kept], tags[kept])
        spent += time.perf_counter() - t0
        done += 1
    return done, spent


def bench_h2o(args, w, dev):
    """PACE-style decode with H2O eviction: one step = one cycle."""
    import torch
    from budgeted_retention_amd import pipelines, synth
    cycles = args.warmup + args.steps
    inp = synth.make_h2o_inputs(w, max(cycles, 1), dev)
    calibrate_copy(args, dev)
    timer = pipelines.CallTimer()
    # one run over warm-up + timed cycles; the warm-up cycles' events are dropped
    marks = []

    class Cut:
        def __call__(self, name):
            if name == "append":
                marks.append(len(timer.events))
            return timer(name)
    res = pipelines.run_h2o(w, inp, cycles, Cut())
    torch.cuda.synchronize()
    first = marks[args.warmup] if args.warmup < len(marks) else len(timer.events)
    timer.events = timer.events[first:]
    part = {k: v / args.steps for k, v in timer.totals_ms().items()}
    rows, S, B, E, d, G = w.rows, w.slots, w.budget, w.interval, w.head_dim, w.group
    path_calls = ["kvc_decode_attn_h2o", "kvc_select", "kvc_compact_rerotate"]
    ms = sum(part[k] for k in path_calls)
    # decode: every resident key's K and V read once per step (B+1 .. B+E keys) and its score
    # read and written; select: scores and tags read, B indices written; compaction: kept K, V,
    # reference keys, positions, reference positions, scores and tags read and written, index read
    keys = rows * sum(B + e + 1 for e in range(E))
    ab = {"kvc_decode_attn_h2o": keys * (2 * d * 2 + 8) + E * w.n_seq * w.n_layers * w.n_q_heads * d * 2 * 2,
          "kvc_select": rows * (S * 5 + B * 4),
          "kvc_compact_rerotate": rows * B * (12 * d + 30)}
    dom = max(path_calls, key=lambda k: part[k])
    roof = roofline(ab[dom], part[dom], dom, w.name)
    cpu = None
    if args.cpu_seconds > 0:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            done, spent = cpu_h2o_rows(w, inp, args.cpu_seconds)
        cpu = {"value": w.n_seq * S * (done / rows) / spent, "unit": "tokens/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{done} of {rows} rows through one cycle ({E} decode steps of cumulative attention, "
                         f"eviction, gather), float64 numpy oracle on one BLAS thread, {spent:.1f} s scaled "
                         f"to all rows"}
    config = {"workload": w.name, "n_seq": w.n_seq, "layers": w.n_layers, "kv_heads": w.n_kv_heads,
              "q_heads": w.n_q_heads, "head_dim": d, "budget": B, "interval": E, "sink": w.n_sink,
              "recent": w.n_recent, "parallelism": "none"}
    extra = {"breakdown_ms": {k: round(part[k], 4) for k in path_calls},
             "other_ms": {k: round(v, 4) for k, v in part.items() if k not in path_calls},
             "decoded_tokens_per_s": round(w.n_seq * E / (ms * 1e-3), 1),
             "calls": per_call_rates(ab, part)}
    del res
    return w.n_seq * S / (ms * 1e-3), ms, config, roof, cpu, extra


def bench_commit_multi(args, w, dev):
    """Successive CommitKV commits: one step = every commit of the workload."""
    import torch
    from budgeted_retention_amd import pipelines, synth
    inp = synth.make_commit_multi_inputs(w, dev)
    calibrate_copy(args, dev)
    for _ in range(args.warmup):
        pipelines.run_commit_multi(w, inp)
    torch.cuda.synchronize()
    timer = pipelines.CallTimer()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        pipelines.run_commit_multi(w, inp, timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    part = timer.median_step_ms(args.steps)
    host = {k: round(v * 1e3 / args.steps, 3) for k, v in timer.host.items()}
    C, N, L, Hkv, d, W, ps = w.commits, w.n_seq, w.n_layers, w.n_kv_heads, w.head_dim, w.window, w.page_size
    G = w.n_q_heads // Hkv
    rows, Ta, Tb, B = w.rows, w.t_pre, w.t_post, w.budget
    lrows = N * Hkv
    # per step (all commits): the deciding layer's K and V read once per effect call, every row's K
    # read by the window score, page scores, the page list, and the kept pages gathered and written
    ab = {"kvc_page_effect:pre": C * lrows * (2 * Ta * d * 2 + G * W * d * 2),
          "kvc_page_effect:post": C * lrows * (2 * Tb * d * 2 + G * W * d * 2),
          "kvc_page_retire": C * lrows * (2 * Tb * d * 2 + G * W * d * 2),
          "kvc_score": C * rows * (Ta * d * 2 + G * W * d * 2 + Ta * 4),
          "kvc_page_scores": C * (rows * Ta * 4 + N * (Ta // ps) * 4),
          "kvc_select": C * N * ((Ta // ps) * 5 + (B // ps) * 4),
          "kvc_compact_rerotate": C * rows * (2 * B * d * 2 * 2 + B * 4 * 2)}
    path_calls = list(ab)
    ms = sum(part[k] for k in path_calls)
    dom = max(path_calls, key=lambda k: part[k])
    roof = roofline(ab[dom], part[dom], dom, w.name)
    config = {"workload": w.name, "n_seq": N, "layers": L, "kv_heads": Hkv, "q_heads": w.n_q_heads,
              "head_dim": d, "commits": C, "turn": w.n_call, "observation": w.n_obs, "window": W,
              "page": ps, "budget": B, "eta": w.eta, "decision_layer": w.layer, "parallelism": "none"}
    extra = {"timing": f"per call, the median over {args.steps} runs of its HIP-event time; ms_per_step "
                       f"sums the path's calls",
             "breakdown_ms": {k: round(part[k], 4) for k in path_calls},
             "other_ms": {k: round(v, 4) for k, v in part.items() if k not in path_calls},
             "host_ms": host, "calls": per_call_rates(ab, part),
             "wall_ms_per_step": round(wall * 1e3 / args.steps, 4)}
    # tokens: every commit compacts the sequence's pre-commit cache
    return C * N * Ta / (ms * 1e-3), ms, config, roof, None, extra


def calibrate_copy(args, dev):
    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 2
        src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the compaction of a row "
              "needs no communication, so N GPUs would each run their own rows.", file=sys.stderr)
        sys.exit(2)
    import torch
    from budgeted_retention_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in synth.WORKLOADS:
        w = synth.WORKLOADS[args.workload]
        value, ms, config, roof, cpu, extra = bench_compaction(args, w, dev)
    elif args.workload in synth.PASK_WORKLOADS:
        w = synth.PASK_WORKLOADS[args.workload]
        value, ms, config, roof, cpu, extra = bench_pipeline(args, w, dev, "pask")
    elif args.workload in synth.COMMIT_WORKLOADS:
        w = synth.COMMIT_WORKLOADS[args.workload]
        value, ms, config, roof, cpu, extra = bench_pipeline(args, w, dev, "commit")
    elif args.workload in synth.COMMIT_MULTI_WORKLOADS:
        w = synth.COMMIT_MULTI_WORKLOADS[args.workload]
        value, ms, config, roof, cpu, extra = bench_commit_multi(args, w, dev)
    elif args.workload in synth.H2O_WORKLOADS:
        w = synth.H2O_WORKLOADS[args.workload]
        value, ms, config, roof, cpu, extra = bench_h2o(args, w, dev)
    else:
        raise SystemExit(f"unknown workload {args.workload}")
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": config,
        **extra, "roofline": roof, "cpu_baseline": cpu, "run": run_metadata(dev),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
