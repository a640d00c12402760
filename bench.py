"""Benchmark of the verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--algo auto|multipass|fused]
    python bench.py --workload lmhead [--steps K] [--warmup W]

Workload: B=64 sequences, gamma=4 drafts, V=128256, bf16 logits, T=1.  Target
logits are N(0, 3^2) with 8 peaked tokens per row (+8).  Draft logits are the
target plus N(0, sigma_b^2), with sigma_b ~ U(0.2, 2) per sequence (seeded,
synthetic).  One step is one spec_verify call over the whole batch.  The inputs
are resident in HBM; NSETS copies rotate so that the working set exceeds the
256 MB last-level cache and every step streams from HBM.

With --workload lmhead the step is instead the LM heads of both models plus
the verification (spec_lmhead_verify): B=8, gamma=4, hidden size d=4096,
V=128256, bf16 hidden states and weights (W_p ~ N(0, 0.02^2), W_q = W_p +
N(0, 0.005^2)), fp32 logits.  The weights (2 x 1.05 GB) exceed the last-level
cache, so every step streams them from HBM.

Prints one JSON line (rank 0) with the throughput in verified target rows/s
(B*(gamma+1) per step).  It also carries:
  roofline:     algorithmic bytes of one launch / its average duration
                (one pair of HIP events on the launch stream around the
                back-to-back timed steps), against 8 TB/s;
  cpu_baseline: the fp64 oracle (test infrastructure) timed on the same
                workload on this host's cores (at most 16 threads), with the
                CPU model named.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified logit rows/s (B*(gamma+1) x V) and % of peak HBM GB/s at V=128256"
HBM_PEAK_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "speculative_sampling_verification_02_amd", "csrc")
WORKLOAD_TEXT = {
    "verify": "Gaussian rows with 8 peaked tokens, per-sequence draft noise",
    "small1": "target N(0, 2^2), draft = target + N(0, 1)",
    "small2": "target N(0, 3^2), draft = 0.8 target + N(0, 0.5^2)",
    "large5": "target N(0, 4^2) with a Zipf(1.1)-ranked bias, draft noise N(0, 1.5^2), "
              "5% confidently wrong draft rows",
}


def kernel_source_hash() -> str:
    """Hash of every kernel source: a counter record taken on other sources is
    not reported."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(n_accepted: np.ndarray, gamma: int, V: int, elem: int, gamma_seq=None,
                      filtered: bool = False) -> int:
    """Bytes the method must read per call: the 2*gamma_b draft/target rows of every
    sequence (all overlaps are reported), the bonus row only where every draft was
    kept (always, with top-k / top-p: every row's threshold needs the whole row),
    plus tokens, uniforms and outputs."""
    B = len(n_accepted)
    gb = np.full(B, gamma) if gamma_seq is None else np.asarray(gamma_seq)
    rows = 2 * int(gb.sum()) + (B if filtered else int((n_accepted == gb).sum()))
    small = 4 * B * gamma + 4 * B * (gamma + 1) + 4 * B * (2 + 3 * gamma)
    return rows * V * elem + small


def host_threads() -> int:
    """Threads for the CPU baseline: the CPUs this process may run on, at most
    16 (one GPU's share of a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, budget_s: float = 10.0) -> dict:
    """The fp64 oracle as it stands, on the whole batch, repeated until
    `budget_s` of wall time has passed (after one untimed call); its blocks of
    sequences run on host_threads() threads."""
    from oracle import verify as ov
    threads = host_threads()
    ov.verify_case(case, workers=threads)            # untimed: first-touch page faults
    rows = calls = 0
    t0 = time.perf_counter()
    while True:
        ov.verify_case(case, workers=threads)
        rows += case.B * (case.gamma + 1)
        calls += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"the whole batch ({case.B} sequences, rows of {case.V} {case.dtype} logits), "
                      f"{calls} call(s) in {dt:.1f} s, NumPy fp64 on {threads} threads"}


def load_counters(key: str) -> dict:
    """The rocprofv3 counter record of one workload (profiles/counters.json:
    HBM bytes per launch from FETCH_SIZE and WRITE_SIZE scaled by a copy of
    known size, vector-ALU or matrix-core busy), or {} when it is missing or
    was taken on other kernel sources."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    entry = rec.get(key) or {}
    return entry if entry.get("source_hash") == kernel_source_hash() else {}


class LoopTime:
    def __init__(self, mean_us: float, wall_s: float):
        self.mean = mean_us   # average launch duration on the stream, µs
        self.wall_s = wall_s  # host wall time of the timed region, s


def timed_loop(torch, steps: int, step) -> LoopTime:
    """Runs `steps` steps back to back between one pair of HIP events on the
    launch stream (torch's current stream, which every step launches on).
    Events between the steps would each add a marker packet and several µs
    of idle time to the stream, so the per-launch duration is the events'
    interval over the steps: the kernels' own durations plus the (sub-µs)
    dispatch gaps between them."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for k in range(steps):
        step(k)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return LoopTime(1e3 * e0.elapsed_time(e1) / steps, wall)


def copy_calibration(torch, dev) -> None:
    """One plain 1 GiB device-to-device copy: under rocprofv3 --pmc it gives the
    scale of FETCH_SIZE and WRITE_SIZE for bytes of known count."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def stream_read_rate(torch, sv, dev, nbytes: int = 1 << 30, reps: int = 20) -> float:
    """GB/s of a plain streaming read (spec_stream_read) of a 1 GiB buffer, four
    times the last-level cache: the HBM read rate this device sustains, for
    context beside the 8 TB/s peak."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    # two 256-thread workgroups per compute unit: the fastest shape of a sweep
    # of 256..16384 workgroups on the MI355X (7.1 TB/s; more workgroups read
    # more scattered pages at once and fall back to 5.7-6.2 TB/s)
    blocks = 2 * 256
    sink = torch.empty(blocks, dtype=torch.int32, device=dev)
    for _ in range(3):
        sv.stream_read(buf, sink, blocks)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        sv.stream_read(buf, sink, blocks)
    e.record()
    e.synchronize()
    gbs = nbytes * reps / (s.elapsed_time(e) * 1e-3) / 1e9
    del buf, sink
    return gbs


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--algo", default="auto", choices=["auto", "multipass", "fused"])
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--workload", default="verify",
                    choices=["verify", "lmhead", "small1", "small2", "large5", "kvcrop"],
                    help="verify: B=64, gamma=4, V=128256 bf16 (the headline); lmhead: LM heads + verify at "
                         "B=8, d=4096; small1 / small2: B=1, gamma=3 / 7, V=32128 fp32; large5: B=256, "
                         "gamma=8, V=256000 bf16; kvcrop: the KV-cache crop after the headline verification "
                         "(64 K/V caches of B=64 x 8 heads x 512 positions x 128 bf16)")
    ap.add_argument("--temperature", type=float, default=1.0,
                    help="temperature of the verify workloads (0: argmax mode)")
    ap.add_argument("--lenience", type=float, default=1.0, help="lenience factor l in (0, 1] (spec_verify_ex)")
    ap.add_argument("--ragged", action="store_true",
                    help="per-sequence draft counts gamma_b ~ U{1..gamma} (seeded; spec_verify_ex)")
    ap.add_argument("--vocab", type=int, default=0,
                    help="the verify workload's recipe at another vocabulary size (e.g. 50257, whose rows are "
                         "not 16-byte aligned and take the multipass path)")
    ap.add_argument("--top-k", type=int, default=0, help="top-k filter of p and q (0: off; spec_verify_ex)")
    ap.add_argument("--top-p", type=float, default=1.0, help="top-p filter of p and q (1: off; spec_verify_ex)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the verification step shards by sequence with no communication)", file=sys.stderr)
        return 2
    if args.workload == "lmhead":
        return run_lmhead(args)
    if args.workload == "kvcrop":
        return run_kvcrop(args)

    import torch

    import speculative_sampling_verification_02_amd as sv
    import workloads as W

    dev = torch.device("cuda:0")
    algo = {"auto": sv.ALGO_AUTO, "multipass": sv.ALGO_MULTIPASS, "fused": sv.ALGO_FUSED}[args.algo]
    T = float(args.temperature)
    if args.vocab and args.workload == "verify":
        case = W.config3(0, T, V=args.vocab)
    else:
        case = {"verify": W.config3, "small1": W.config1, "small2": W.config2, "large5": W.config5}[args.workload](0, T)
    B, G, V = case.B, case.gamma, case.V
    bf16 = case.dtype == "bf16"
    elem = 2 if bf16 else 4
    print(f"[bench] generated B={B} gamma={G} V={V} {case.dtype}", file=sys.stderr, flush=True)

    def to_dev(a):
        if bf16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    base = (to_dev(case.target), to_dev(case.draft))
    sets = [base] + [(base[0].clone(), base[1].clone()) for _ in range(args.sets - 1)]
    tokens = torch.from_numpy(case.tokens).to(dev)
    uniforms = torch.from_numpy(case.uniforms).to(dev)
    ws = torch.zeros(sv.workspace_size(B, G, V, sv.SPEC_BF16 if bf16 else sv.SPEC_F32), dtype=torch.uint8,
                     device=dev)
    gseq_np = np.random.default_rng([0, 0x6A]).integers(1, G + 1, size=B) if args.ragged else None
    gseq = None if gseq_np is None else torch.from_numpy(gseq_np.astype(np.int32)).to(dev)
    outs = [{k: torch.empty(s, dtype=dt, device=dev) for k, s, dt in (
        ("n_accepted", (B,), torch.int32), ("next_token", (B,), torch.int32),
        ("alpha", (B, G), torch.float32), ("p_draft", (B, G), torch.float32),
        ("q_draft", (B, G), torch.float32))} for _ in sets]

    # one prepared launch per buffer set: the timed loop then spends only the
    # C call on the host, well under the kernel's duration
    launches = [sv.prepare_verify(t, d, tokens, uniforms, T, algo=algo, workspace=ws, outputs=o,
                                  lenience=args.lenience, gamma_seq=gseq, top_k=args.top_k, top_p=args.top_p)
                for (t, d), o in zip(sets, outs)]

    def step(k):
        launches[k % len(sets)]()

    if args.copy_calibration:
        copy_calibration(torch, dev)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    launch_us = timed_loop(torch, args.steps, step)
    elapsed = launch_us.wall_s
    stream_gbs = stream_read_rate(torch, sv, dev)

    ms_per_step = 1e3 * elapsed / args.steps
    rows = B * (G + 1)
    n0 = outs[0]["n_accepted"].cpu().numpy()
    filtered = T > 0 and (0 < args.top_k < V or args.top_p < 1.0)
    default_path = args.lenience == 1.0 and not args.ragged and not filtered
    alg = algorithmic_bytes(n0, G, V, elem, gseq_np, filtered)
    avg_launch_s = launch_us.mean * 1e-6
    achieved = alg / avg_launch_s / 1e9
    algo_name = {sv.ALGO_AUTO: "auto", sv.ALGO_MULTIPASS: "multipass", sv.ALGO_FUSED: "fused"}[algo]
    # AUTO dispatches the headline workload (aligned bf16 rows, 16 workgroups
    # per row) to the fused kernel at T = 1 and to the multipass path at T = 0;
    # the counter record holds both
    counters = {}
    if args.workload == "verify" and default_path and not args.vocab:
        if T == 1.0 and algo_name in ("auto", "fused"):
            counters = load_counters("fused_verify_T1")
        elif T == 0.0 and algo_name in ("auto", "multipass"):
            counters = load_counters("multipass_verify_T0")
    line = {
        "metric": METRIC,
        "value": rows / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"spec_verify B={B} gamma={G} V={V} {case.dtype} logits T={T:g}, "
                               + WORKLOAD_TEXT[args.workload],
                   "B": B, "gamma": G, "V": V, "logits": case.dtype, "temperature": T,
                   "algo": algo_name, "buffer_sets": len(sets), "lenience": args.lenience,
                   "gamma_seq": None if gseq_np is None else "U{1..gamma}, mean %.2f" % gseq_np.mean(),
                   "top_k": args.top_k, "top_p": args.top_p},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": counters.get("traffic_bytes"),
                     "launch_us_mean": launch_us.mean,
                     "alg_bytes": alg, "full_bytes": (2 * G + 1) * V * elem * B,
                     "stream_read_GBps": stream_gbs, "frac_of_stream_read": achieved / stream_gbs,
                     "valu_busy_pct": counters.get("valu_busy_pct")},
    }
    if not args.no_cpu_baseline and default_path and not args.vocab:
        line["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(line), flush=True)
    return 0


def lmhead_step_bytes(n_accepted: np.ndarray, B: int, gamma: int, d: int, V: int) -> int:
    """Bytes one spec_lmhead_verify call must move: both weight matrices once,
    the hidden states, the fp32 logits written once and read back by the
    verification (its algorithmic rows, as for spec_verify), and the small I/O."""
    weights = 2 * d * V * 2
    hidden = (B * (gamma + 1) + B * gamma) * d * 2
    logits_out = B * (2 * gamma + 1) * V * 4
    return weights + hidden + logits_out + algorithmic_bytes(n_accepted, gamma, V, 4)


def run_lmhead(args) -> int:
    import torch

    import speculative_sampling_verification_02_amd as sv
    import workloads as W

    dev = torch.device("cuda:0")
    case = W.config4(0, 1.0)
    B, G, d, V = case.B, case.gamma, case.d, case.V
    print(f"[bench] generated LM-head workload B={B} gamma={G} d={d} V={V}", file=sys.stderr, flush=True)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    hidden, wp, wq = to_dev(case.hidden), to_dev(case.w_target), to_dev(case.w_draft)
    tokens = torch.from_numpy(case.tokens).to(dev)
    uniforms = torch.from_numpy(case.uniforms).to(dev)
    ws = torch.zeros(max(1, sv.lmhead_workspace_size(B, G, d, V)), dtype=torch.uint8, device=dev)
    out = {"target_logits": torch.empty(B, G + 1, V, dtype=torch.float32, device=dev),
           "draft_logits": torch.empty(B, G, V, dtype=torch.float32, device=dev),
           "n_accepted": torch.empty(B, dtype=torch.int32, device=dev),
           "next_token": torch.empty(B, dtype=torch.int32, device=dev),
           "alpha": torch.empty(B, G, dtype=torch.float32, device=dev),
           "p_draft": torch.empty(B, G, dtype=torch.float32, device=dev),
           "q_draft": torch.empty(B, G, dtype=torch.float32, device=dev)}

    def step():
        sv.lmhead_verify(hidden, wp, wq, B, G, tokens, uniforms, 1.0, workspace=ws, outputs=out)

    if args.copy_calibration:
        copy_calibration(torch, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    launch_us = timed_loop(torch, args.steps, lambda k: step())
    ms_per_step = 1e3 * launch_us.wall_s / args.steps
    step_bytes = lmhead_step_bytes(out["n_accepted"].cpu().numpy(), B, G, d, V)
    achieved = step_bytes / (launch_us.mean * 1e-6) / 1e9
    # counters of the step's two kernels (the LM-head GEMM and the
    # verification), and the GEMM's matrix-core busy share of its span
    counters = load_counters("lmhead")
    line = {
        "metric": METRIC,
        "value": B * (G + 1) / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"spec_lmhead_verify B={B} gamma={G} d={d} V={V}, bf16 hidden states "
                               "and weights, fp32 logits, T=1",
                   "B": B, "gamma": G, "d": d, "V": V, "temperature": 1.0},
        # one step is one matrix-core launch for both heads plus the
        # verification launch on its fp32 logits; the bytes and the duration
        # are those of the whole step
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": counters.get("traffic_bytes"),
                     "launch_us_mean": launch_us.mean,
                     "step_bytes": step_bytes,
                     "lmhead_traffic_bytes": counters.get("lmhead_traffic_bytes"),
                     "mfma_util_pct": counters.get("mfma_util_pct")},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = lmhead_cpu_baseline(case, out)
    print(json.dumps(line), flush=True)
    return 0


def run_kvcrop(args) -> int:
    """The KV-cache crop (spec_kv_crop) that follows the headline verification:
    32 layers' K and V caches (64 contiguous caches of B=64 sequences x 8 heads
    x 512 positions x 128 bf16), the pass having written gamma + 1 = 5 entries
    per sequence (the previous step's final token and the 4 drafts; keep_extra
    1), the discarded entries zero-filled.  n_accepted comes from one
    verification of the B=64, gamma=4, V=128256 batch.  Every timed step crops
    its own copy of the committed lengths, so each does the same work."""
    import ctypes

    import torch

    import speculative_sampling_verification_02_amd as sv
    import workloads as W

    dev = torch.device("cuda:0")
    B, G, H, S_max, D, n_caches = 64, 4, 8, 512, 128, 64
    appended, keep_extra = G + 1, 1
    case = W.config3(0, 1.0)
    t = {k: v for k, v in zip(("target", "draft"),
                              (torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
                               for a in (case.target, case.draft)))}
    out = sv.verify(t["target"], t["draft"], torch.from_numpy(case.tokens).to(dev),
                    torch.from_numpy(case.uniforms).to(dev), 1.0)
    n_acc = out["n_accepted"]
    n_np = n_acc.cpu().numpy()
    del t
    caches = [torch.ones(B, H, S_max, D, dtype=torch.bfloat16, device=dev) for _ in range(n_caches)]
    rng = np.random.default_rng([0, 0x4B])
    committed = torch.from_numpy(rng.integers(0, S_max - appended, size=B).astype(np.int32)).to(dev)
    total = args.warmup + args.steps
    lens = [committed.clone() for _ in range(total)]   # one copy of the lengths per step
    print(f"[bench] KV crop: {n_caches} caches [{B}, {H}, {S_max}, {D}] bf16, n_accepted from the verification "
          f"(mean {n_np.mean():.2f})", file=sys.stderr, flush=True)
    ptrs = (ctypes.c_void_p * n_caches)(*[c.data_ptr() for c in caches])
    fn, entry = sv.lib.spec_kv_crop, D * 2

    def step(k, stream):
        st = fn(ptrs, n_caches, B, H, S_max, entry, ctypes.c_void_p(lens[k].data_ptr()),
                ctypes.c_void_p(n_acc.data_ptr()), appended, keep_extra, 1, stream)
        if st != 0:
            raise RuntimeError(f"spec_kv_crop: status {st}")

    cur = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for k in range(args.warmup):
        step(k, cur)
    torch.cuda.synchronize()
    # The crop is two short launches, shorter than their host-side launch cost
    # from Python; in a serving loop they queue behind the verification.  The
    # timed steps are therefore captured once into a HIP graph and replayed,
    # so the stream runs them back to back as it would there.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        for k in range(args.steps):
            step(args.warmup + k, cap)
    for l in lens:
        l.copy_(committed)
    torch.cuda.synchronize()
    launch_us = timed_loop(torch, 1, lambda k: graph.replay())
    launch_us.mean /= args.steps
    ms_per_step = 1e3 * launch_us.wall_s / args.steps
    # algorithmic bytes: the zero-filled entries, plus lengths read and written
    # and n_accepted read
    discarded = int((appended - keep_extra - n_np).sum())
    alg = discarded * H * entry * n_caches + 3 * 4 * B
    achieved = alg / (launch_us.mean * 1e-6) / 1e9
    # the new lengths must be the oracle's (checked on the last step's copy)
    want = committed.cpu().numpy() + keep_extra + n_np
    assert np.array_equal(lens[-1].cpu().numpy(), want), "crop lengths"
    line = {
        "metric": METRIC,
        "value": B * (G + 1) / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"spec_kv_crop after spec_verify B={B} gamma={G} V=128256: {n_caches} contiguous "
                               f"caches [{B}, {H}, {S_max}, {D}] bf16, appended {appended}, keep_extra "
                               f"{keep_extra}, discarded entries zero-filled",
                   "B": B, "gamma": G, "H": H, "S_max": S_max, "D": D, "caches": n_caches},
        # rows/s here: the verified rows whose cache state one crop settles
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "launch_us_mean": launch_us.mean,
                     "alg_bytes": alg, "discarded_entries": discarded * H * n_caches},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = kvcrop_cpu_baseline(caches[0].shape, n_caches, committed.cpu().numpy(), n_np,
                                                   appended, keep_extra)
    print(json.dumps(line), flush=True)
    return 0


def kvcrop_cpu_baseline(shape, n_caches, committed, n_np, appended, keep_extra, budget_s: float = 5.0) -> dict:
    """The crop oracle on host copies of the same caches (bf16 as uint16):
    whole calls over all caches, repeated for `budget_s`."""
    from oracle import kvcache as okv
    caches = [np.ones(shape, np.uint16) for _ in range(n_caches)]
    B = shape[0]
    calls = 0
    t0 = time.perf_counter()
    while True:
        okv.crop_contiguous(caches, committed, n_np, appended, keep_extra, True)
        calls += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": B * appended * calls / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"the whole crop ({n_caches} caches of {shape}), {calls} call(s) in {dt:.1f} s, NumPy, "
                      "one thread"}


def lmhead_cpu_baseline(case, out, cols: int = 4096) -> dict:
    """The oracle's LM-head step on this host: the fp64 products of both heads
    over `cols` columns (timed, then scaled to all V columns) plus the fp64
    verification of the whole batch on the GPU's fp32 logits (timed)."""
    from oracle import lmhead as olm
    from oracle import verify as ov
    import workloads as W
    threads = host_threads()
    t0 = time.perf_counter()
    sl = slice(0, cols)
    olm.logits(case.hidden, case.w_target, cols=sl)
    olm.logits(case.hidden[case.draft_hidden_rows()], case.w_draft, cols=sl)
    heads = (time.perf_counter() - t0) * case.V / cols
    vc = W.VerifyCase("lmhead", out["target_logits"].cpu().numpy(), out["draft_logits"].cpu().numpy(), "f32",
                      case.tokens, case.uniforms, case.temperature)
    t1 = time.perf_counter()
    ov.verify_case(vc, workers=threads)
    verify_s = time.perf_counter() - t1
    step = heads + verify_s
    return {"value": case.B * (case.gamma + 1) / step, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"both heads' fp64 products over {cols} of {case.V} columns (scaled to all: {heads:.2f} s) "
                      f"plus the fp64 verification of the whole batch ({verify_s:.2f} s); NumPy, "
                      f"{threads} threads for the verification"}


if __name__ == "__main__":
    sys.exit(main())
