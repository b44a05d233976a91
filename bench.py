"""Benchmark of the LoSA hot path on one MI355X.

One step = the whole path on the Wan2.1-1.3B-shaped layer (B1 H12 N32760
D128, block 64, bf16, tau 0.99): the construction step (dense attention with
the block mass map in one sweep, then threshold selection) on the step-3
inputs, then block-sparse attention over the frozen lists on the 47
later-step inputs (steps 4..50, each a fresh 5 % perturbation of Q, K and V),
all resident in HBM before timing starts.  The headline value is the
sparse-attention time per call; the dense kernel is timed on the same 47
inputs for the speedup, and the two-pass construction (dense pass, then the
separate mass pass) once more for comparison.

Prints one JSON line.  ``--gpus`` above 1 is refused: this path runs on one
GPU.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-attn ms/call + MFMA util at Wan2.1-1.3B shape (99% mass); x vs dense"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_wan13_traffic.json")
SELECT_COUNTERS_FILE = os.path.join(ROOT, "profiles", "select_kernel_counters.json")
CLOCK_FILE = os.path.join(ROOT, "profiles", "sustained_clock.json")
CSRC = os.path.join(ROOT, "block_sparse_attention_losa_amd", "csrc")
KERNEL_SOURCES = [os.path.join(CSRC, f)
                  for f in ("attn_bf16.hip", "attn_common.h", "losa_device.h",
                            "losa_launch.h", "frozen_lists.hip")]
SELECT_SOURCES = [os.path.join(CSRC, f) for f in ("select.hip", "losa_device.h", "losa_launch.h")]
# MI355X: 256 CUs x 4 SIMDs; a wave64 VALU instruction (fp32 or fp64 at full
# rate) occupies its SIMD for 4 cycles; nominal clock 2.4 GHz
SIMDS = 1024
VALU_CYCLES_PER_INSTR = 4
CLOCK_GHZ = 2.4


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_hash(sources=None):
    """Hash of the code of the timed kernel, its launch shapes and its launch
    plan (identifies the build a counter summary was taken on).  Comments
    and whitespace are left out, so editing a comment keeps the summary."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES if sources is None else sources:
        with open(path, encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def kept_flops(count, idx, n, block, d):
    """Sum over kept (query block, key block) pairs of 4*|I|*|J|*D."""
    import numpy as np

    nb = count.shape[-1]
    sizes = np.array([min(n, (j + 1) * block) - j * block for j in range(nb)], np.int64)
    total = 0
    cnt = count.reshape(-1, nb)
    ids = idx.reshape(-1, nb, nb)
    for r in range(cnt.shape[0]):
        for i in range(nb):
            c = int(cnt[r, i])
            total += int(sizes[i]) * int(sizes[ids[r, i, :c]].sum())
    return 4.0 * total * d


def dense_flops(b, h, n, d):
    return 4.0 * b * h * n * n * d


def read_traffic(n_launch_units):
    """HBM bytes per sparse launch from the committed counter summary, or
    None when absent or taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    if rec.get("kernel_sha") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def read_sustained_clock(workload, achieved_tflops):
    """The shader clock the timed sparse kernel sustains on this workload
    (rocprofv3: GRBM_GUI_ACTIVE per XCD over the dispatch time, mean over
    boxes), and the achieved rate against the MFMA peak at that clock.  None
    when absent, for another workload, or taken on another kernel source."""
    if not os.path.exists(CLOCK_FILE):
        return None
    with open(CLOCK_FILE) as fh:
        rec = json.load(fh)
    if rec.get("kernel_sha") != kernel_hash():
        return None
    entry = rec.get("workloads", {}).get(workload)
    if not entry:
        return None
    ghz = float(entry["ghz"])
    peak = PEAK_BF16_TFLOPS * ghz / CLOCK_GHZ
    return {"ghz": ghz, "peak_at_clock": round(peak, 1),
            "frac_at_clock": round(achieved_tflops / peak, 4),
            "source": "profiles/sustained_clock.json"}


def select_floor_ms(rows, nkb):
    """Compute floor of the selection kernel for `rows` rows of `nkb` key
    blocks: the VALU instructions it issues per row (counted with rocprofv3,
    SQ_INSTS_VALU / rows, for the row length's sort size) at one wave64
    instruction per 4 cycles on each of the 1024 SIMDs at 2.4 GHz.  None when
    the committed counter summary is absent or was taken on other sources."""
    if not os.path.exists(SELECT_COUNTERS_FILE):
        return None
    with open(SELECT_COUNTERS_FILE) as fh:
        rec = json.load(fh)
    if rec.get("kernel_sha") != kernel_hash(SELECT_SOURCES):
        return None
    sort_size = 16
    while sort_size < nkb:
        sort_size *= 2
    per_row = rec.get("valu_instructions_per_row", {}).get(str(sort_size))
    if per_row is None:
        return None
    return rows * per_row * VALU_CYCLES_PER_INSTR / SIMDS / (CLOCK_GHZ * 1e9) * 1e3


def cpu_baseline(cfg, q, k, v, idx, count, budget_s):
    """The fp64 oracle's sparse attention on a bounded sample of query
    blocks of the same workload, scaled to ms per full call."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - informational only
        threads = os.cpu_count() or 1
    nb = cfg.num_blocks
    rng = np.random.default_rng(0)
    items = [(h, i) for h in range(cfg.heads) for i in range(nb)]
    order = rng.permutation(len(items))
    done = 0
    t0 = time.perf_counter()
    for j in order:
        h, i = items[j]
        oracle.sparse_attention(q[0, h], k[0, h], v[0, h], idx[0, h], count[0, h], cfg.block,
                                qblocks=[i])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    ms_per_call = dt / done * len(items) * 1e3
    return {"value": round(ms_per_call, 1), "unit": "ms/call", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {len(items)} query blocks (random heads) of one sparse call "
                      f"on the step-4 input, {dt:.1f} s, scaled to the full call"}


def host_info():
    """Host facts the oracle timings depend on: BLAS threads, CPU model and
    numpy's BLAS."""
    import numpy as np

    threads, blas = os.cpu_count() or 1, "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            threads = max(i.get("num_threads", 1) for i in info)
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
    except Exception:  # pragma: no cover - informational only
        pass
    if blas == "unknown":
        try:
            cfg = np.show_config(mode="dicts")
            blas = cfg["Build Dependencies"]["blas"]["name"]
        except Exception:  # pragma: no cover - informational only
            pass
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover - informational only
        pass
    return {"cores": int(threads), "cpu_model": model, "blas": blas,
            "affinity": len(os.sched_getaffinity(0))}


def oracle_profile(cfg, step3, later, mass, idx, count, tau, budget_s):
    """Each oracle function of the path on a bounded random sample of its
    work (query blocks of random heads; rows of the mass map for the
    selection), scaled to seconds per full call on the workload: the dense
    pass, the mass map and the selection on the construction-step inputs
    ``step3``, sparse attention on a later-step input ``later``."""
    import numpy as np

    import oracle

    nb, blk = cfg.num_blocks, cfg.block
    rng = np.random.default_rng(1)
    bh = [(bb, hh) for bb in range(cfg.batch) for hh in range(cfg.heads)]
    units = len(bh) * nb

    def sample(fn):
        done, t0 = 0, time.perf_counter()
        for j in rng.permutation(units):
            (bb, hh), i = bh[j // nb], int(j % nb)
            fn(bb, hh, i)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return {"s_per_call": round(dt / done * units, 2),
                "sample": f"{done} of {units} query blocks, {dt:.1f} s"}

    def rows_of(i):
        lo, hi = oracle.block_rows(i, cfg.seq_len, blk)
        return np.arange(lo, hi)

    def mass_of_block(bb, hh, i):
        # both passes for one query block: its rows' lse, then its mass row
        rows = rows_of(i)
        lse = np.zeros(cfg.seq_len)
        lse[rows] = oracle.row_lse(q[bb, hh], k[bb, hh], rows=rows)
        return oracle.block_mass(q[bb, hh], k[bb, hh], blk, lse=lse, qblocks=[i])

    (q, k, v), (q4, k4, v4) = step3, later
    res = {"dense_attention": sample(lambda bb, hh, i: oracle.dense_attention(
               q[bb, hh], k[bb, hh], v[bb, hh], rows=rows_of(i))),
           "block_mass": sample(lambda bb, hh, i: mass_of_block(bb, hh, i)),
           "sparse_attention": sample(lambda bb, hh, i: oracle.sparse_attention(
               q4[bb, hh], k4[bb, hh], v4[bb, hh], idx[bb, hh], count[bb, hh], blk,
               qblocks=[i]))}
    rows = mass.reshape(-1, nb)
    pick = rng.permutation(rows.shape[0])
    done, t0 = 0, time.perf_counter()
    while done < len(pick) and time.perf_counter() - t0 <= budget_s:
        oracle.select(rows[pick[done:done + 64]], tau)
        done += min(64, len(pick) - done)
    dt = time.perf_counter() - t0
    res["select"] = {"s_per_call": round(dt / done * rows.shape[0], 2),
                     "sample": f"{done} of {rows.shape[0]} rows, {dt:.1f} s"}
    res.update(host_info())
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--later", type=int, default=None,
                    help="later-step inputs per step (default 47 for the Wan2.1-1.3B layer, 4 otherwise)")
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--oracle-profile", type=float, default=0.0, metavar="SECONDS",
                    help="also time every oracle function on a sample of about this many "
                         "seconds each (off by default)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards over heads with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_attention_losa_amd as losa
    from block_sparse_attention_losa_amd import synth

    cfg = synth.CONFIGS[args.config]
    tau = args.tau if args.tau is not None else cfg.tau
    n_later = args.later if args.later is not None else (len(cfg.later_steps) or 4)
    later_steps = list(cfg.later_steps) or list(range(4, 4 + n_later))
    later_steps = later_steps[:n_later]
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    b, h, n, d, blk = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.block
    nb = cfg.num_blocks

    log(f"[bench] generating {cfg.name} (step 3) on the host")
    t0 = time.perf_counter()
    q3, k3, v3 = synth.make_inputs(cfg)
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s; perturbing {len(later_steps)} later steps on the GPU")
    tq3, tk3, tv3 = (torch.from_numpy(x).to(dev).to(tdt) for x in (q3, k3, v3))
    later = []
    for t in later_steps:
        later.append(tuple(synth.perturb_on_device(cfg, x, t, i) for i, x in enumerate((tq3, tk3, tv3))))
    o = torch.empty_like(tq3)
    o_dense = torch.empty_like(tq3)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=dev)
    mass = torch.empty((b, h, nb, nb), dtype=torch.float32, device=dev)
    mass2 = torch.empty_like(mass)
    ws = torch.empty(losa.dense_attn_mass_workspace_bytes(tq3, blk), dtype=torch.uint8,
                     device=dev)
    plan = losa.sparse_plan(torch.zeros((b, h, nb), dtype=torch.int32, device=dev), block=blk,
                            head_dim=d)
    idx = torch.empty((b, h, nb, nb), dtype=torch.int32, device=dev)
    count = torch.empty((b, h, nb), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def one_step(record):
        marks = {}
        e = [ev() for _ in range(4)]
        e[0].record()
        losa.dense_attn_mass(tq3, tk3, tv3, block=blk, o=o_dense, lse=lse, mass=mass,
                             workspace=ws)
        e[1].record()
        losa.select(mass, tau, idx=idx, count=count)
        e[2].record()
        losa.sparse_plan(count, block=blk, head_dim=d, plan=plan)
        e[3].record()
        sp = []
        for (q, k, v) in later:
            s0, s1 = ev(), ev()
            s0.record()
            losa.sparse_attn(q, k, v, idx, count, block=blk, o=o, plan=plan)
            s1.record()
            sp.append((s0, s1))
        if record is not None:
            record.append((e, sp))

    log(f"[bench] warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        one_step(None)
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} step(s)")
    recs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    fused_ms = [r[0][0].elapsed_time(r[0][1]) for r in recs]
    select_ms = [r[0][1].elapsed_time(r[0][2]) for r in recs]
    plan_ms = [r[0][2].elapsed_time(r[0][3]) for r in recs]
    sparse_ms = [a.elapsed_time(z) for r in recs for (a, z) in r[1]]
    sparse_mean = float(np.mean(sparse_ms))

    # dense kernel on the same later-step inputs, for the speedup
    dense_later = []
    if not args.no_dense:
        log("[bench] dense kernel on the later-step inputs")
        for (q, k, v) in later:
            s0, s1 = ev(), ev()
            s0.record()
            losa.dense_attn(q, k, v, block=blk, o=o_dense, want_lse=False)
            s1.record()
            dense_later.append((s0, s1))
        torch.cuda.synchronize()
    dense_later_ms = [a.elapsed_time(z) for (a, z) in dense_later]

    # the same sparse calls without the plan (default head-major order)
    unplanned = []
    if not args.no_dense:
        log("[bench] sparse kernel without the plan")
        for (q, k, v) in later:
            s0, s1 = ev(), ev()
            s0.record()
            losa.sparse_attn(q, k, v, idx, count, block=blk, o=o)
            s1.record()
            unplanned.append((s0, s1))
        torch.cuda.synchronize()
    unplanned_ms = [a.elapsed_time(z) for (a, z) in unplanned]

    # the two-pass construction (dense pass with lse, then the mass pass) on
    # the same step-3 input, for comparison with the one-sweep path
    log("[bench] two-pass construction")
    two = []
    for _ in range(3):
        e = [ev() for _ in range(3)]
        e[0].record()
        losa.dense_attn(tq3, tk3, tv3, block=blk, o=o_dense, lse=lse)
        e[1].record()
        losa.block_mass(tq3, tk3, block=blk, lse=lse, mass=mass2)
        e[2].record()
        two.append(e)
    torch.cuda.synchronize()
    two_dense_ms = [e[0].elapsed_time(e[1]) for e in two]
    two_mass_ms = [e[1].elapsed_time(e[2]) for e in two]
    mass_gap = float((mass2 - mass).abs().max())

    # drift of the frozen lists: share of each later step's dense attention
    # mass they still cover, at the first and the last later step
    drift = {}
    for name, pos in (("first_later_step", 0), ("last_later_step", len(later) - 1)):
        q, k, v = later[pos]
        _, lse_d = losa.dense_attn(q, k, v, block=blk)
        _, lse_k = losa.sparse_attn(q, k, v, idx, count, block=blk, want_lse=True)
        r = losa.retained_mass(lse_k, lse_d, block=blk, head_dim=d).cpu().numpy()
        drift[name] = {"step": later_steps[pos], "mean": round(float(r.mean()), 5),
                       "p1": round(float(np.percentile(r, 1)), 5),
                       "min": round(float(r.min()), 5)}
        del lse_d, lse_k

    cnt_h = count.cpu().numpy()
    idx_h = idx.cpu().numpy()
    f = float(cnt_h.sum()) / (b * h * nb * nb)
    flops = kept_flops(cnt_h, idx_h, n, blk, d)
    achieved = flops / (sparse_mean * 1e-3) / 1e12
    dflops = dense_flops(b, h, n, d)
    dense_mean = float(np.mean(dense_later_ms)) if dense_later_ms else None
    traffic = read_traffic(1)
    # the selection reads the mass map and writes the lists (its HBM
    # roofline), and sorts every row (its VALU floor, from counted
    # instructions)
    rows = b * h * nb
    select_bytes = 4 * nb * rows + 4 * int(cnt_h.sum()) + 4 * rows
    select_mean = float(np.mean(select_ms))
    select_floor = select_floor_ms(rows, nb)
    props = torch.cuda.get_device_properties(dev)

    out = {
        "metric": METRIC,
        "value": round(sparse_mean, 4),
        "unit": "ms/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": b, "heads": h, "seq_len": n, "head_dim": d,
                   "block": blk, "tau": tau, "later_steps_per_step": len(later),
                   "step": "one-sweep dense+mass, select and plan on step 3, planned sparse on each later step"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "sustained_clock": read_sustained_clock(cfg.name, achieved),
        "kept_fraction": round(f, 4),
        "mfma_util": round(achieved / PEAK_BF16_TFLOPS, 4),
        "x_vs_dense": round(dense_mean / sparse_mean, 3) if dense_mean else None,
        "ideal_speedup": round(1.0 / f, 3),
        "speedup_bar": round(0.85 / f, 3),
        "sparse_ms_median": round(float(np.median(sparse_ms)), 4),
        "sparse_ms_without_plan": round(float(np.mean(unplanned_ms)), 4) if unplanned_ms else None,
        "sparse_kept_tflop": round(flops / 1e12, 4),
        "dense_ms_per_call": round(dense_mean, 4) if dense_mean else None,
        "dense_tflops": round(dflops / (dense_mean * 1e-3) / 1e12, 1) if dense_mean else None,
        "construction_ms": {"dense_attn_mass": round(float(np.mean(fused_ms)), 4),
                            "select": round(float(np.mean(select_ms)), 4),
                            "sparse_plan": round(float(np.mean(plan_ms)), 4),
                            "two_pass_dense": round(float(np.mean(two_dense_ms)), 4),
                            "two_pass_block_mass": round(float(np.mean(two_mass_ms)), 4),
                            "max_mass_gap_one_sweep_vs_two_pass": mass_gap},
        "retained_mass": drift,
        "select": {"ms": round(select_mean, 4), "algorithmic_mb": round(select_bytes / 1e6, 2),
                   "gbps": round(select_bytes / (select_mean * 1e-3) / 1e9, 1),
                   "hbm_peak_gbps": PEAK_HBM_GBS,
                   "hbm_frac": round(select_bytes / (select_mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                   "valu_floor_ms": round(select_floor, 4) if select_floor else None,
                   "valu_floor_frac": round(select_floor / select_mean, 4) if select_floor else None},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count,
                   "memory_gib": round(props.total_memory / 2**30, 1)},
        "kernel_sha": kernel_hash(),
    }
    if not args.no_cpu_baseline:
        log(f"[bench] oracle cpu baseline (~{args.cpu_budget:.0f} s)")
        q4, k4, v4 = (x.float().cpu().numpy() for x in later[0])
        out["cpu_baseline"] = cpu_baseline(cfg, q4, k4, v4, idx_h, cnt_h, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    if args.oracle_profile > 0:
        log(f"[bench] oracle profile (~{4 * args.oracle_profile:.0f} s)")
        step4 = tuple(x.float().cpu().numpy() for x in later[0])
        out["oracle_profile"] = oracle_profile(cfg, (q3, k3, v3), step4, mass.cpu().numpy(),
                                               idx_h, cnt_h, tau, args.oracle_profile)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
