"""Benchmark: KV tokens compacted per second (score + select + gather +
re-rotate) on one MI355X, with the dominant kernel's HBM roofline and the CPU
oracle's rate on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one compaction of a whole session: kvc_score, kvc_select and
kvc_compact_rerotate over every (layer, KV head) row, inputs resident in HBM.
Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b_100k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the CPU oracle sample (0 disables it)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (three times), so that HBM "
                         "counters can be scaled against a transfer of known size")
    return ap.parse_args()


def kernel_source_hash():
    """Hash of the HIP sources the counters were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "budgeted_retention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w):
    """Bytes the path must move at least once, per row and per call (the design doc
    gives the derivation): score reads K once and Q once and writes the fp32
    scores; select reads scores (and tags) and writes B indices; compaction
    reads and writes B keys and values plus positions."""
    G = w.group
    T, d, W, B = w.n_tokens, w.head_dim, w.window, w.budget
    score = T * d * 2 + G * W * d * 2 + T * 4
    select = T * 4 + T + B * 4 + 4
    compact = 2 * B * d * 2 + 2 * B * d * 2 + B * 4 * 2
    path = T * d * 2 + G * W * d * 2 + 4 * B * d * 2 + 16 * B   # the whole path, scores kept on chip
    return dict(score=score * w.rows, select=select * w.rows, compact=compact * w.rows,
                path=path * w.rows)


def cpu_baseline(w, inp, budget_s):
    """Time the float64 oracle over a prefix of the session's rows (D2H copies of
    the exact input bytes), until about `budget_s` seconds of oracle work."""
    import numpy as np
    import torch
    from oracle import compact as o_compact, numfmt, policy as o_policy, score as o_score
    from oracle import select as o_select
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
    G, W, T, B = w.group, w.window, w.n_tokens, w.budget
    tbl = np.array([[0.0]] + [[0.0 if s is None else o_policy.foresight_bonus(1e3, 0.35, s)]
                              for s in inp.spans.steps_ahead])
    fl = np.zeros_like(tbl, dtype=np.uint8)
    L, Hkv = w.n_layers, w.n_kv_heads
    done, spent = 0, 0.0
    while spent < budget_s and done < w.rows:
        r = done
        n, l, h = r // (L * Hkv), (r // Hkv) % L, r % Hkv
        Kb = inp.K[n, l, h].cpu().view(torch.int16).numpy().view(np.uint16)
        Vb = inp.V[n, l, h].cpu().view(torch.int16).numpy().view(np.uint16)
        Qb = inp.Q_obs[n, l, h * G:(h + 1) * G].cpu().view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        s = o_score.obs_window_score(numfmt.bf16_bits_to_f64(Kb), numfmt.bf16_bits_to_f64(Qb), W)
        tot, prot = o_policy.totals_and_protection(s, inp.spans.tags, tbl, fl, 0, w.n_sink, w.n_recent)
        kept, _ = o_select.select_top_b(tot, prot, B)
        o_compact.compact_row(Kb, Vb, np.arange(T), kept, w.renumber_base, w.rope_base)
        spent += time.perf_counter() - t0
        done += 1
    rate = T * (done / w.rows) / spent
    return {"value": rate, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {w.rows} (layer, KV head) rows of one {T}-token session, "
                      f"float64 numpy oracle (score+select+gather/re-rotate), "
                      f"{spent:.1f} s of oracle time scaled to the whole session"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the compaction of a row "
              "needs no communication, so N GPUs would each run their own rows.", file=sys.stderr)
        sys.exit(2)
    import torch
    from budgeted_retention_amd import kvc, synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = synth.make_compaction_inputs(w, dev)
    N, L, Hkv, Hq, d, T, W, B = (w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim,
                                 w.n_tokens, w.window, w.budget)
    rows = w.rows
    dims = kvc.make_dims(N, L, Hkv, Hq, d, T)
    vals = [0.0] + [0.0 if s is None else kvc.kvc_foresight_bonus(1e3, 0.35, s)
                    for s in inp.spans.steps_ahead]
    bonus = torch.tensor(vals, dtype=torch.float32, device=dev).reshape(-1, 1)
    pol = kvc.Policy(w.n_sink, w.n_recent, B, len(vals), 1, 0, L, inp.tags, bonus)
    ws = kvc.workspace(kvc.KVC_OP_SCORE, dims, W, 0, dev)
    scores = torch.empty((rows, T), dtype=torch.float32, device=dev)
    kept = torch.empty((rows, B), dtype=torch.int32, device=dev)
    n_kept = torch.empty(rows, dtype=torch.int32, device=dev)
    Ko = torch.empty((rows, B, d), dtype=torch.bfloat16, device=dev)
    Vo = torch.empty_like(Ko)
    po = torch.empty((rows, B), dtype=torch.int32, device=dev)
    nh = torch.empty(rows, dtype=torch.int32, device=dev)
    out = kvc.CompactOut(B, Ko, Vo, po, nh)

    def step(ev=None):
        if ev:
            ev[0].record()
        kvc.kvc_score(dims, inp.K, inp.Q_obs, W, scores, ws)
        if ev:
            ev[1].record()
        kvc.kvc_select(dims, scores, pol, kept, B, n_kept)
        if ev:
            ev[2].record()
        kvc.kvc_compact_rerotate(dims, inp.K, inp.V, None, kept, B, n_kept, w.renumber_base,
                                 w.rope_base, out)
        if ev:
            ev[3].record()

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 2
        src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [[e[i].elapsed_time(e[i + 1]) for i in range(3)] for e in evs]
    step_ms = [sum(p) for p in per]
    ms = sum(step_ms) / len(step_ms)
    part_ms = [sum(p[i] for p in per) / len(per) for i in range(3)]
    if not (n_kept == B).all():
        raise SystemExit("bench: a row kept a number of tokens other than the budget")

    ab = algorithmic_bytes(w)
    names = ["kvc_score", "kvc_select", "kvc_compact_rerotate"]
    keys = ["score", "select", "compact"]
    dom = max(range(3), key=lambda i: part_ms[i])
    achieved = ab[keys[dom]] / (part_ms[dom] * 1e-3) / 1e9
    traffic = None
    if os.path.exists(COUNTERS_FILE):
        c = json.load(open(COUNTERS_FILE))
        ent = c.get("calls", {}).get(names[dom])
        if ent and c.get("source_hash") == kernel_source_hash() and c.get("workload") == w.name:
            traffic = ent["hbm_bytes_per_call"]
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": names[dom],
            "algorithmic_bytes": ab[keys[dom]]}

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, inp, args.cpu_seconds)

    value = N * T / (ms * 1e-3)
    line = {
        "metric": "KV tokens compacted/sec (score+select+gather+rerotate), % of HBM peak, 1 GPU",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "n_seq": N, "layers": L, "kv_heads": Hkv, "q_heads": Hq,
                   "head_dim": d, "tokens": T, "window": W, "budget": B, "sink": w.n_sink,
                   "recent": w.n_recent, "rope_base": w.rope_base, "parallelism": "none"},
        "hbm_frac_path": round(ab["path"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "breakdown_ms": {n: round(t, 4) for n, t in zip(names, part_ms)},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
