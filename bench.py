"""Benchmark: sparse-MLA forward + backward on one MI355X.

One step = the index plan (built once: forward and backward take the same
indices), the forward and the backward (dq pass, dkv pass) over the whole
workload, inputs resident in HBM.  The backward runs in its stored-P form
(the dq pass stores P and scale * dS, the dkv pass reads them: one recompute
of the scores per backward); --dkv-scores recompute selects the form whose
dkv pass recomputes them.  The default workload
is the packed ragged batch: S=4096 tokens as sequences {512, 1024, 1536,
1024}, H=8 heads, topk=2048 full causal rows (2,361,344 valid pairs).

Prints ONE JSON line with the metric (useful TFLOP/s, i.e. 7680*H flops per
valid (token, slot) pair over the fwd+bwd step time), the roofline of the
dominant kernel (timed with HIP events on the library's stream) and the CPU
baseline (the fp64 oracle on a bounded token sample, on the host cores).
Outside the timed step it also reports the index-production top-k, the
finite check of dq / dkv, the forward over fp8 kv records and a step with
two kv groups.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
METRIC = "sparse-MLA fwd+bwd useful TFLOP/s at H=8 topk=2048; % of bf16 MFMA peak"

# Algorithmic flops per valid (token, slot) pair and head, per kernel.
FLOPS_PER_PAIR_HEAD = {
    "fwd": 2 * (576 + 512),                  # scores + PV
    "bwd_dq": 2 * (576 + 512 + 576),         # recomputed scores, dP, dQ
    "bwd_dkv": 2 * (576 + 512 + 576 + 512),  # recomputed scores, dP, dK, dV
}
FLOPS_STORED_DKV = 2 * (576 + 512)          # dK, dV only (stored-P backward)
USEFUL_PER_PAIR_HEAD = 7680                  # fwd 2176 + bwd 5504 (one recompute)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="packed_ragged",
                    choices=["tiny", "packed_ragged", "padding_stress", "recency", "long_context",
                             "heads128"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dkv-mode", default="deterministic", choices=["deterministic", "atomic"],
                    help="dkv reduction: the bitwise-reproducible per-row reduction (default) or "
                         "fp32 atomic adds")
    ap.add_argument("--dkv-scores", default="stored", choices=["stored", "recompute"],
                    help="dkv pass: read P and scale * dS stored by the dq pass (default: one "
                         "recompute of the scores per backward) or recompute the scores and dP")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="time the steps without per-kernel HIP events")
    ap.add_argument("--no-topk", action="store_true",
                    help="skip the index-production (top-k) measurement")
    ap.add_argument("--no-kv-groups", action="store_true",
                    help="skip the two-kv-group step (its launches share the kernels' names)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads reported beside the headline")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (three times) and "
                         "exit: the calibration run for the HBM byte counters")
    return ap.parse_args()


def source_digest() -> str:
    """sha256 over the kernel sources (csrc/*.hip, *.h, include/*.h, sorted)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "bwd_sparse_mla_amd", "csrc", "*")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain
    copy's reading), or None when there is none for the current sources."""
    digest = source_digest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for ln in fh:
                if not ln.startswith("traffic: "):
                    continue
                rec = json.loads(ln[len("traffic: "):])
                if (rec.get("kernel") == kernel and rec.get("workload") == workload
                        and rec.get("source_sha256") == digest):
                    return rec
    return None


def copy_probe(mib: int) -> None:
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


TOPK_S, TOPK_K = 8192, 2048


def topk_measure(steps: int):
    """The index-production step on one causal sequence of TOPK_S tokens,
    K = TOPK_K, fp32 logits (seeded normal): mean time per call over `steps`
    calls, and its bytes against HBM.  Rows no longer than K read no logits;
    a longer row reads its range once, and every row writes K indices."""
    import torch

    import bwd_sparse_mla_amd as smla
    from workloads.synth import causal_ranges
    gen = torch.Generator(device="cuda").manual_seed(20)
    lg = torch.randn(TOPK_S, TOPK_S, device="cuda", generator=gen, dtype=torch.float32)
    ks_np, ke_np = causal_ranges([TOPK_S])
    ks, ke = torch.from_numpy(ks_np).cuda(), torch.from_numpy(ke_np).cuda()
    out = torch.empty(TOPK_S, TOPK_K, dtype=torch.int32, device="cuda")
    for _ in range(3):
        smla.topk_indices(lg, ks, ke, TOPK_K, out=out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        smla.topk_indices(lg, ks, ke, TOPK_K, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    n = (ke_np - ks_np).astype(np.int64)
    nbytes = int(4 * n[n > TOPK_K].sum() + 4 * TOPK_S * TOPK_K)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"one causal sequence, S={TOPK_S}, K={TOPK_K}, fp32 logits",
            "ms": round(ms, 5), "bytes_per_call": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def nonfinite_measure(run, steps: int):
    """The finite check of the backward's outputs: NaN / Inf counted over dq
    and dkv of the step just run (one counter, two launches per check), mean
    time per check and its bytes against HBM (each buffer read once)."""
    import torch

    import bwd_sparse_mla_amd as smla
    cnt = torch.zeros(1, dtype=torch.int64, device=run.dq.device)

    def check():
        smla.count_nonfinite(run.dq, cnt)
        smla.count_nonfinite(run.dkv, cnt)

    for _ in range(3):
        check()
    torch.cuda.synchronize()
    cnt.zero_()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        check()
    e1.record()
    torch.cuda.synchronize()
    if int(cnt.item()) != 0:
        raise RuntimeError("nonfinite entries in dq / dkv")
    ms = e0.elapsed_time(e1) / steps
    nbytes = run.dq.numel() * run.dq.element_size() + run.dkv.numel() * run.dkv.element_size()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"what": "NaN/Inf count over dq and dkv", "ms": round(ms, 5), "bytes_per_check": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def fp8_fwd_measure(run, w, q, kv, idx, steps: int):
    """The forward over fp8 kv records of the same workload (e4m3 latent with
    fp32 per-128-column scales, bf16 rope: 656 bytes per row instead of 1152)
    against the bf16 forward, both on the plan the timed steps built: mean
    time per launch of each, and the fp8 forward's useful rate."""
    import torch

    from workloads import synth
    rec = torch.from_numpy(synth.quantize_kv_fp8(w.kv, pow2_scales=False)).to(kv.device)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    rec2 = torch.from_numpy(synth.quantize_kv_fp8(w.kv, pow2_scales=True)).to(kv.device)
    run.plan(idx)
    ms8 = timed(lambda: run.fwd_fp8(q, rec, idx, w.sm_scale, planned=True))
    if not bool(torch.isfinite(run.out.float()).all()):
        raise RuntimeError("nonfinite values in the fp8 forward's out")
    ms8p = timed(lambda: run.fwd_fp8(q, rec2, idx, w.sm_scale, planned=True, pow2_scales=True))
    ms16 = timed(lambda: run.fwd(q, kv, idx, w.sm_scale, planned=True))
    flops = FLOPS_PER_PAIR_HEAD["fwd"] * w.H * w.n_valid
    return {"what": "forward over fp8 kv records (656 B per row) vs the bf16 forward",
            "ms": round(ms8, 5), "ms_pow2_scales": round(ms8p, 5), "bf16_fwd_ms": round(ms16, 5),
            "useful_tflops": round(flops / (ms8 * 1e-3) / 1e12, 1)}


def kv_groups_measure(dev, steps: int, stored: bool):
    """Two kv groups of 8 heads each (H = 16) at the packed ragged batch's
    sizes: one grouped call (kv [S_kv, 2, 576], indices [S, 2, K]) against two
    single-group calls on the same data, each a full step (plan, forward,
    backward).  Seeded N(0, 1) bf16 q / kv / dout; each group's indices are
    full causal rows over the sequences {512, 1024, 1536, 1024}, shuffled
    independently."""
    import torch

    import bwd_sparse_mla_amd as smla
    from workloads import synth
    rng = np.random.default_rng(11)
    seqlens = [512, 1024, 1536, 1024]
    S, K, G, Hg = sum(seqlens), 2048, 2, 8
    idx_np = np.stack([synth.causal_full_rows(rng, seqlens, K) for _ in range(G)], axis=1)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)

    def randn(*shape):
        return torch.randn(*shape, device=dev, generator=gen).to(torch.bfloat16)

    q, kv, dout = randn(S, G * Hg, 576), randn(S, G, 576), randn(S, G * Hg, 512)
    idx = torch.from_numpy(idx_np).to(dev).contiguous()
    scale = 1.0 / 192 ** 0.5

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    run = smla.SparseMLARunner(S, S, G * Hg, K, dev, dkv_stored_p=stored, kv_groups=G)

    def grouped():
        run.plan(idx)
        run.fwd(q, kv, idx, scale, planned=True)
        run.bwd(q, kv, dout, idx, scale, planned=True)

    ms_g = timed(grouped)
    if not (bool(torch.isfinite(run.dq.float()).all()) and bool(torch.isfinite(run.dkv.float()).all())):
        raise RuntimeError("nonfinite values in the grouped backward")
    runs = [smla.SparseMLARunner(S, S, Hg, K, dev, dkv_stored_p=stored) for _ in range(G)]
    parts = [(q[:, g * Hg:(g + 1) * Hg].contiguous(), kv[:, g].contiguous(),
              dout[:, g * Hg:(g + 1) * Hg].contiguous(), idx[:, g].contiguous()) for g in range(G)]

    def separate():
        for r, (qg, kvg, dog, ixg) in zip(runs, parts):
            r.plan(ixg)
            r.fwd(qg, kvg, ixg, scale, planned=True)
            r.bwd(qg, kvg, dog, ixg, scale, planned=True)

    ms_s = timed(separate)
    useful = 7680 * Hg * int((idx_np >= 0).sum())
    return {"workload": "packed ragged batch sizes, 2 kv groups x 8 heads (H=16)",
            "ms_per_step": round(ms_g, 5), "useful_tflops": round(useful / (ms_g * 1e-3) / 1e12, 2),
            "two_single_group_calls_ms": round(ms_s, 5)}


def host_info():
    """Host cores this process may run on, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model}


def cpu_threads() -> int:
    """Threads for the oracle's BLAS pool: every core the process may run on,
    capped by OMP_NUM_THREADS when the environment sets a CPU share."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def cpu_baseline(w, target_s: float):
    """The fp64 oracle as it stands, on a seeded sample of tokens of the same
    workload (their forward + backward, dkv scattered into the full kv), with
    its BLAS pool on cpu_threads() threads."""
    import threadpoolctl

    from oracle import sparse_mla_bwd, sparse_mla_fwd
    from workloads import synth

    threads = cpu_threads()
    kv = synth.bf16_bits_to_f64(w.kv)
    rng = np.random.default_rng(1234)
    order = rng.permutation(w.S)

    def run(toks):
        toks = np.sort(toks)
        q = synth.bf16_bits_to_f64(w.q[toks])
        do = synth.bf16_bits_to_f64(w.dout[toks])
        ix = w.idx[toks]
        t = time.perf_counter()
        sparse_mla_fwd(q, kv, ix, w.sm_scale)
        sparse_mla_bwd(q, kv, do, ix, w.sm_scale)
        dt = time.perf_counter() - t
        nv = int(np.count_nonzero((ix >= 0) & (ix < w.S_kv)))
        return dt, nv, len(toks)

    with threadpoolctl.threadpool_limits(limits=threads):
        dt0, nv0, n0 = run(order[:64])
        per_pair = dt0 / max(nv0, 1)
        nv_mean = w.n_valid / w.S
        n = int(min(w.S, max(64, target_s / max(per_pair * nv_mean, 1e-9))))
        dt, nv, n = run(order[:n])
    flops = USEFUL_PER_PAIR_HEAD * w.H * nv
    host = host_info()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} of {w.S} tokens (seeded), {nv} valid pairs, fwd+bwd fp64, "
                      f"{dt:.1f} s wall",
            "affinity_cores": host["affinity_cores"], "cpu_model": host["cpu_model"]}


def gpu_tensors(w, dev):
    import torch
    to_bf16 = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(
        torch.bfloat16).to(dev)
    return (to_bf16(w.q), to_bf16(w.kv), to_bf16(w.dout),
            torch.from_numpy(np.ascontiguousarray(w.idx)).to(dev))


class Case:
    """One workload on the preallocated runner: the step and its timings."""

    def __init__(self, w, dev, atomic: bool, stored: bool):
        import bwd_sparse_mla_amd as smla
        self.w = w
        self.q, self.kv, self.dout, self.idx = gpu_tensors(w, dev)
        self.run = smla.SparseMLARunner(w.S, w.S_kv, w.H, w.K, dev, dkv_atomic=atomic,
                                        dkv_stored_p=stored)
        self.run._check(self.q, self.kv, self.idx, self.dout)
        self.stored = stored

    def fwd(self):
        # the index plan (once: forward and backward take the same indices), then the forward
        self.run.plan(self.idx)
        self.run.fwd(self.q, self.kv, self.idx, self.w.sm_scale, planned=True)

    def bwd(self):
        self.run.bwd(self.q, self.kv, self.dout, self.idx, self.w.sm_scale, planned=True)

    def step(self):
        # one step of the path: plan, forward, backward
        self.fwd()
        self.bwd()

    def timed_mean(self, steps: int, warmup: int):
        """Mean ms per step over `steps` steps between two events on the
        library's stream (torch's current stream), after `warmup` steps."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            self.step()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, time.perf_counter() - t0

    def per_step(self, n: int, cold: bool = False):
        """Per-step event timings (plan + forward, backward, total) of n
        steps, ms each; cold: a 1 GiB buffer is written before every step
        (outside the events), so the L2 and MALL start without the inputs."""
        import torch
        flush = torch.empty(1 << 28, dtype=torch.float32, device=self.q.device) if cold else None
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        for i in range(n):
            if cold:
                flush.fill_(float(i))
            ev[i][0].record()
            self.fwd()
            ev[i][1].record()
            self.bwd()
            ev[i][2].record()
        torch.cuda.synchronize()
        f = [e[0].elapsed_time(e[1]) for e in ev]
        b = [e[1].elapsed_time(e[2]) for e in ev]
        t = [e[0].elapsed_time(e[2]) for e in ev]
        med = lambda x: float(np.median(x))
        return {"fwd_ms": round(med(f), 5), "bwd_ms": round(med(b), 5),
                "fwd_bwd_ms": round(med(t), 5), "samples": n}

    def kernel_ms(self, steps: int):
        """Per-kernel mean durations: `steps` more steps with the library
        bracketing each of its launches by HIP events on its stream."""
        import torch

        import bwd_sparse_mla_amd as smla
        smla.timing_start(32 * steps)
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        smla.timing_stop()
        kernels = {}
        for name in ("plan", "order", "fwd", "bwd_dq", "dkv_schedule", "dkv_clear", "bwd_dkv",
                     "dkv_finalize"):
            n, tot = smla.timing_read(name)
            if n:
                kernels[name] = {"launches": n, "avg_ms": tot / n}
        return kernels

    def check_finite(self):
        import torch
        for name, t in (("out", self.run.out), ("lse", self.run.lse), ("dq", self.run.dq),
                        ("dkv", self.run.dkv)):
            bad = int((~torch.isfinite(t.float())).sum())
            if bad:
                raise RuntimeError(f"{self.w.name}: {bad} nonfinite values in {name}")


def useful_flops(w) -> int:
    return USEFUL_PER_PAIR_HEAD * w.H * w.n_valid


def gather_block(w, ms: float):
    """Effective gather rate: the algorithmic kv-row gathers of one forward and
    one backward (1152 bytes per valid pair each) over the step time, against
    HBM peak; it can exceed 1 because the L2 / MALL serve repeated rows."""
    nbytes = 2 * 1152 * w.n_valid
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bytes_per_step": nbytes, "GBs": round(gbs, 1), "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 3)}


# Other configurations of the same path, reported beside the headline: the
# tiny correctness case, the padding-stress batch, one GPU's share at the
# production shape (recency-biased picks), the long context in both dkv
# modes, and the packed batch with 0.1% repeated slots (the cost of the
# repeated-slot path).  (name, dkv atomic, timed steps, warm-up steps)
CONFIGS = [("tiny", False, 20, 3), ("padding_stress", False, 20, 3), ("recency", False, 5, 2),
           ("long_context", False, 3, 1), ("long_context", True, 3, 1), ("repeated_slots", False, 5, 2)]


def config_line(w, dev, atomic: bool, stored: bool, steps: int, warmup: int):
    import torch
    case = Case(w, dev, atomic, stored)
    ms, _ = case.timed_mean(steps, warmup)
    case.check_finite()
    parts = case.per_step(max(3, steps))
    kernels = case.kernel_ms(steps)
    useful = useful_flops(w)
    value = useful / (ms * 1e-3) / 1e12
    rec = {"workload": w.name, "S": w.S, "H": w.H, "topk": w.K, "valid_pairs": w.n_valid,
           "dkv_mode": "atomic" if atomic else "deterministic", "steps": steps,
           "ms_per_step": round(ms, 5), "median": parts, "useful_tflops": round(value, 2),
           "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 3),
           "kernels_ms": {k: round(v["avg_ms"], 5) for k, v in kernels.items()},
           "effective_gather": gather_block(w, ms)}
    del case
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a measured configuration.",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return

    import torch

    from workloads import synth

    w = synth.WORKLOADS[args.workload]()
    print(f"[bench] workload {w.name}: S={w.S} H={w.H} K={w.K} S_kv={w.S_kv} "
          f"valid pairs={w.n_valid}", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    stored = args.dkv_scores == "stored"
    case = Case(w, dev, args.dkv_mode == "atomic", stored)
    run, q, kv, idx = case.run, case.q, case.kv, case.idx

    # The timed region: K steps between two events on the library's stream
    # (torch's current stream), no other work inside.
    ms, wall = case.timed_mean(args.steps, args.warmup)
    print(f"[bench] timed {args.steps} steps: {ms:.4f} ms/step (wall {wall:.3f} s)",
          file=sys.stderr, flush=True)
    case.check_finite()
    # Medians of per-step event timings, warm and with the caches flushed.
    warm = case.per_step(args.steps)
    cold = case.per_step(max(5, min(args.steps, 20)), cold=True)
    print(f"[bench] median warm {warm} cold {cold}", file=sys.stderr, flush=True)
    # Per-kernel durations: the same K steps again, with the library
    # bracketing each of its launch steps by HIP events on that stream (the
    # event records add a few microseconds per launch, so this pass is not the
    # one the headline number comes from).
    timing = not args.no_kernel_timing
    kernels = case.kernel_ms(args.steps) if timing else {}

    nv = w.n_valid
    useful = useful_flops(w)
    value = useful / (ms * 1e-3) / 1e12

    roofline = None
    if timing:
        dom = max((k for k in kernels if k in FLOPS_PER_PAIR_HEAD),
                  key=lambda k: kernels[k]["avg_ms"])
        per_pair = FLOPS_PER_PAIR_HEAD[dom]
        if dom == "bwd_dkv" and stored:
            per_pair = FLOPS_STORED_DKV   # P and dS come from the dq pass
        flops = per_pair * w.H * nv
        ach = flops / (kernels[dom]["avg_ms"] * 1e-3) / 1e12
        rec = recorded_traffic(dom, w.name)
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": None if rec is None else rec["bytes_per_launch"],
                    "flops_per_launch": flops, "avg_ms": round(kernels[dom]["avg_ms"], 5)}
        if rec is not None:
            roofline["traffic_GBs"] = round(
                rec["bytes_per_launch"] / (kernels[dom]["avg_ms"] * 1e-3) / 1e9, 1)
        print(f"[bench] kernels {kernels}", file=sys.stderr, flush=True)

    print("[bench] finite check of dq / dkv ...", file=sys.stderr, flush=True)
    finite = nonfinite_measure(run, max(10, args.steps))

    print("[bench] fp8 kv forward ...", file=sys.stderr, flush=True)
    fp8 = fp8_fwd_measure(run, w, q, kv, idx, max(10, args.steps))

    kvgroups = None
    if not args.no_kv_groups:
        print("[bench] kv groups ...", file=sys.stderr, flush=True)
        kvgroups = kv_groups_measure(dev, max(10, args.steps), stored)

    topk = None
    if not args.no_topk:
        print("[bench] index production (top-k) ...", file=sys.stderr, flush=True)
        topk = topk_measure(max(5, args.steps // 2))
    del case, run, q, kv, idx
    torch.cuda.empty_cache()

    configs = None
    if not args.no_configs:
        configs = []
        for name, atomic, steps, warmup in CONFIGS:
            if name == args.workload and not atomic:
                continue
            wc = synth.WORKLOADS[name]()
            print(f"[bench] config {wc.name} dkv {'atomic' if atomic else 'deterministic'} "
                  f"({steps} steps) ...", file=sys.stderr, flush=True)
            configs.append(config_line(wc, dev, atomic, stored, steps, warmup))
            del wc

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "S": w.S, "S_kv": w.S_kv, "H": w.H, "topk": w.K,
                   "seqlens": w.seqlens, "valid_pairs": nv, "useful_gflop": useful / 1e9,
                   "parallelism": "none (one GPU)", "dkv_mode": args.dkv_mode,
                   "dkv_scores": args.dkv_scores},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 3),
        "median": {"warm": warm, "cold_caches": cold},
        "kernels_ms": {k: round(v["avg_ms"], 5) for k, v in kernels.items()},
        "kernel_timing": ("per-launch HIP events on the library's stream, in a second pass of "
                          "the same steps after the timed region" if timing else None),
        "roofline": roofline,
        "effective_gather": gather_block(w, ms),
        "cpu_baseline": cpu,
        "host": host_info(),
        "configs": configs,
        "index_topk": topk,
        "nonfinite_check": finite,
        "fwd_fp8_kv": fp8,
        "kv_groups": kvgroups,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
