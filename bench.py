"""Throughput of the split-KV / FLARE softmax hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--cpu-seconds S]
                    [--backward] [--shared] [--fused] [--graph] [--flush-mall]

A step is one pass of the whole path over one batch of synthetic input that
already sits in HBM.  For the default workload (FLARE++, B=1, H=16, N=262144,
M=128, D=64, R=16, bf16) that is: encoder 1 over (Q~, K~, V~) -> merge ->
encoder 2 over (Q(X), K, V) -> merge -> decode of every token.  The line
printed is one JSON object: tokens/s (B*N*H per step; mean, median and
minimum step times), the roofline of the binding kernel (of the encoder and
the decode, the one furthest below the HBM roofline: achieved algorithmic HBM
bytes per launch over its event-timed duration), the step-level fraction of
the roofline, and the CPU oracle timed on a bounded sample.

Only one GPU is used; --gpus above 1 is refused.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import split_kv_softmax_amd as fl  # noqa: E402
import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores, published
# committed rocprofv3 counter summaries (profiles/<name>_counters.md) per workload
COUNTER_FILES = {
    W.FLAREPP.name: "flarepp_fwd_N262144_counters.md",
    W.FLARE_BLOCK.name: "flare_block_N65536_counters.md",
    W.SPLITKV_Q1.name: "splitkv_q1_N131072_counters.md",
    W.MASKED_FWD_BWD.name: "masked_fwd_bwd_N262144_counters.md",
    W.FLAREPP_D16.name: "flarepp_fwd_D16_N1048576_counters.md",
    W.FLARE_ENCODE_F32_SMALL.name: "encode_fp32_small_N1024_counters.md",
}
# the sources each kernel family is built from (the summaries record their hash)
KERNEL_SOURCES = {"encode_ilv": ["encode.hip"], "encode_mfma": ["encode.hip"], "encode_q1": ["encode.hip"],
                  "encode_generic": ["encode.hip"], "mask_words": ["encode.hip"], "heavy_first": ["encode.hip"],
                  "decode_mfma": ["decode.hip"], "decode_generic": ["decode.hip"], "fold": ["merge.hip"],
                  "bwd_kv_mfma": ["encode_bwd.hip"], "bwd_kv_ws": ["encode_bwd.hip"], "bwd_dq_mfma": ["encode_bwd.hip"],
                  "bwd_dq_reduce": ["encode_bwd.hip"], "bwd_rowdot": ["encode_bwd.hip"], "dbwd_": ["decode_bwd.hip"]}


def source_hash(kernel: str) -> str:
    import hashlib
    key = next(k for k in KERNEL_SOURCES if k in kernel)
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[key] + ["common.h", "kernels.h"]:
        h.update(open(os.path.join(HERE, "split_kv_softmax_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def counter_summary(workload: str, kernel: str):
    """HBM bytes and matrix-core use per launch of `kernel` from the committed counter summary of
    `workload`, or None when there is none or its sources changed since the counters were taken."""
    try:
        txt = open(os.path.join(HERE, "profiles", COUNTER_FILES[workload])).read()
        d = json.loads(txt.split("```json", 1)[1].split("```", 1)[0])
        key = next(k for k in d["kernels"] if kernel in k)
        e = d["kernels"][key]
        if e["source_hash"] != source_hash(kernel):
            return None
        return e
    except (KeyError, OSError, StopIteration, ValueError, IndexError):
        return None


def _ev():
    return torch.cuda.Event(enable_timing=True)


class Step:
    """A step as named phases run back to back."""

    def _phases(self, phases):
        self.phases = phases
        self.names = [n for n, _ in phases]
        self.phase_ms = [[] for _ in phases]   # per-launch milliseconds of each phase

    def __call__(self):
        for _, fn in self.phases:
            fn()

    def run_marked(self, k, a, b):
        """One step with events a and b recorded around its phase k."""
        for i, (_, fn) in enumerate(self.phases):
            if i == k:
                a.record()
            fn()
            if i == k:
                b.record()


class FlareppStep(Step):
    """The FLARE++ forward chain with preallocated outputs; fused: each encoder
    and its merge as one call (flare_encode_merge)."""

    def __init__(self, w: W.Workload, x, fused=False, shared=False):
        self.w, self.x = w, x
        self.shared = shared
        B, H, N, M, D, R = w.B, w.H, w.N, w.M, w.D, w.R
        dev = x["K"].device
        f32 = dict(dtype=torch.float32, device=dev)
        # shared projections: the query-synthesis encoder reads K and V themselves
        Kt, Vt = (x["K"], x["V"]) if shared else (x["Kt"], x["Vt"])
        self.O1 = torch.empty((R, B, H, M, D), **f32)
        self.L1 = torch.empty((R, B, H, M), **f32)
        self.QX = torch.empty((B, H, M, D), **f32)
        self.QXL = torch.empty((B, H, M), **f32)
        self.QXb = torch.empty((B, H, M, D), dtype=torch.bfloat16, device=dev)
        self.O2 = torch.empty_like(self.O1)
        self.L2 = torch.empty_like(self.L1)
        self.Z = torch.empty((B, H, M, D), **f32)
        self.L = torch.empty((B, H, M), **f32)
        self.Y = torch.empty_like(x["K"])
        dec = ("decode", lambda: fl.decode(x["K"], self.QXb, self.Z, w.scale, None, self.Y))
        if fused:
            self._phases([
                ("encode_merge1", lambda: fl.encode_merge(x["Qt"], Kt, Vt, w.offsets, None, w.scale, True,
                                                          self.O1, self.L1, self.QX, self.QXL, self.QXb)),
                ("encode_merge2", lambda: fl.encode_merge(self.QXb, x["K"], x["V"], w.offsets, None, w.scale, False,
                                                          self.O2, self.L2, self.Z, self.L)),
                dec])
        else:
            self._phases([
                ("encode1", lambda: fl.encode(x["Qt"], Kt, Vt, w.offsets, None, w.scale, self.O1, self.L1)),
                ("merge1", lambda: fl.lse_merge(self.O1, self.L1, Z=self.QX, L=self.QXL, Z_bf16=self.QXb)),
                ("encode2", lambda: fl.encode(self.QXb, x["K"], x["V"], w.offsets, None, w.scale, self.O2, self.L2)),
                ("merge2", lambda: fl.lse_merge(self.O2, self.L2, Z=self.Z, L=self.L)),
                dec])


class EncodeMergeStep(Step):
    """Encoder over every partition, then the tree merge (single-query split-KV, small encoder)."""

    def __init__(self, w: W.Workload, x, fused=False, extra=()):
        self.w, self.x = w, x
        B, H, N, M, D, R = w.B, w.H, w.N, w.M, w.D, w.R
        f32 = dict(dtype=torch.float32, device=x["K"].device)
        self.O = torch.empty((R, B, H, M, D), **f32)
        self.Lp = torch.empty((R, B, H, M), **f32)
        self.Z = torch.empty((B, H, M, D), **f32)
        self.L = torch.empty((B, H, M), **f32)
        mask = x.get("mask")
        if fused:
            phases = [("encode_merge", lambda: fl.encode_merge(x["Q"], x["K"], x["V"], w.offsets, mask, w.scale,
                                                               False, self.O, self.Lp, self.Z, self.L))]
        else:
            phases = [("encode", lambda: fl.encode(x["Q"], x["K"], x["V"], w.offsets, mask, w.scale, self.O,
                                                   self.Lp)),
                      ("merge", lambda: fl.lse_merge(self.O, self.Lp, Z=self.Z, L=self.L))]
        self._phases(phases + list(extra))


class FlareStep(EncodeMergeStep):
    """FLARE block: encode -> merge -> decode of every token (K as token queries, Q as latent keys)."""

    def __init__(self, w: W.Workload, x, fused=False):
        self.Y = torch.empty_like(x["K"])
        super().__init__(w, x, fused, [("decode", lambda: fl.decode(x["K"], x["Q"], self.Z, w.scale, None,
                                                                     self.Y))])


class FwdBwdStep(EncodeMergeStep):
    """Masked encoder forward + merge, then the encoder backward with the global statistics."""

    def __init__(self, w: W.Workload, x, fused=False):
        B, H, M, D = w.B, w.H, w.M, w.D
        dev = x["K"].device
        self.dQ = torch.empty((B, H, M, D), dtype=torch.float32, device=dev)
        self.dK = torch.empty_like(x["K"])
        self.dV = torch.empty_like(x["V"])
        bwd = ("backward", lambda: fl.encode_bwd(x["Q"], x["K"], x["V"], w.offsets, x.get("mask"), w.scale, self.Z,
                                                 self.L, x["dZ"], self.dQ, self.dK, self.dV))
        super().__init__(w, x, fused, [bwd])


def _oracle_cores():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def _host(t, b, h):
    return t[h:h + 1].cpu() if t.dim() == 3 else t[b:b + 1, h:h + 1].cpu()


def cpu_baseline(w: W.Workload, x, budget_s: float, shared: bool = False):
    """Time the float64 oracle on whole (batch, head) slices of the same inputs, full N each,
    until about ``budget_s`` seconds of CPU work are done; tokens/s = sliced tokens / wall."""
    from oracle import flare_ref as ref
    todo = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, spent = 0, 0.0
    for b, h in todo:
        xs = {k: _host(v, b, h) for k, v in x.items() if k != "mask"}
        mk = x["mask"][b:b + 1].cpu() if "mask" in x else None
        t0 = time.perf_counter()
        if w.kind == "flarepp":
            kt, vt = (xs["K"], xs["V"]) if shared else (xs["Kt"], xs["Vt"])
            ref.flarepp_ref(xs["Qt"], kt, vt, xs["K"], xs["V"], w.offsets, w.scale)
        elif w.kind == "flare":
            e = ref.encode_ref(xs["Q"], xs["K"], xs["V"], w.offsets, None, w.scale)
            ref.decode_ref(xs["K"], xs["Q"], e["Z"], w.scale)
        elif w.kind == "encode_bwd":
            e = ref.encode_ref(xs["Q"], xs["K"], xs["V"], w.offsets, mk, w.scale)
            ref.encode_bwd_ref(xs["Q"], xs["K"], xs["V"], mk, w.scale, e["Z"], e["L"], xs["dZ"])
        else:
            ref.encode_ref(xs["Q"], xs["K"], xs["V"], w.offsets, None, w.scale)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    what = {"flarepp": "FLARE++ chain (2 encoders + decode)", "flare": "FLARE block (encode + decode)",
            "encode_bwd": "masked encoder forward + backward", "splitkv": "split-KV encoder + merge",
            "encode": "encoder + merge"}[w.kind]
    return {"value": w.N * done / spent, "unit": "tokens/s", "cores": int(_oracle_cores()), "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"{what} on {done} of {w.B * w.H} (batch, head) slices, full N={w.N} each; "
                      f"{spent:.2f} s wall"}


def roofline_candidates(w: W.Workload, x, step, ph):
    """(kernel name, ms per launch, algorithmic bytes per launch, kernel key of the committed counter
    summary or None) of each kernel that can bind the step; the caller reports the one furthest below
    the roofline."""
    kvb = 2 if w.dtype == "bf16" else 4
    row = w.D * kvb                               # bytes of one K, V, Y, dK or dV row
    rows = w.B * w.H * w.N
    if w.kind == "flarepp" and "encode2_bwd" in ph:
        # physical-value encoder backward: K, V read, dV written, dK read and written (it adds into the
        # decoder's key gradient); query-synthesis encoder backward: Kt, Vt read, dKt, dVt written, or
        # with shared projections K, V read and dK, dV read and written (it adds into both)
        ms = 0.5 * (ph["encode2_bwd"] + ph["encode1_bwd"])
        enc1_rows = 6 if getattr(step, "shared", False) else 4
        return [("flare_encode_bwd call (row term, key/value-gradient kernel with fused query gradient, reduce); "
                 "both encoder backwards averaged", ms, (5 + enc1_rows) * rows * row // 2, None)]
    if w.kind == "flarepp":
        plain = not getattr(step, "shared", False)
        if "encode_merge1" in ph:
            enc = ("encode_ilv_kernel with the merge inside (flare_encode_merge, one launch; both encoders "
                   "averaged)", 0.5 * (ph["encode_merge1"] + ph["encode_merge2"]), 2 * rows * row, None)
        else:
            enc = ("encode_ilv_kernel (flare_encode, one launch; both encoders averaged)",
                   0.5 * (ph["encode1"] + ph["encode2"]), 2 * rows * row, "encode_ilv_kernel" if plain else None)
        dec = ("decode_mfma_kernel (flare_decode, one launch)", ph["decode"], 2 * rows * row,
               "decode_mfma_kernel" if plain else None)
        return [enc, dec]
    if w.kind == "flare":
        enc = ph.get("encode", ph.get("encode_merge"))
        return [("encode_ilv_kernel (flare_encode, one launch)", enc, 2 * rows * row,
                 "encode_ilv_kernel" if "encode" in ph else None),
                ("decode_mfma_kernel (flare_decode, one launch)", ph["decode"], 2 * rows * row, "decode_mfma_kernel")]
    if w.kind == "encode_bwd":
        valid = int(x["mask"].sum().item()) * w.H if "mask" in x else rows
        return [("flare_encode_bwd call (row term, query-gradient, key/value-gradient and reduce kernels)",
                 ph["backward"], 2 * valid * row + 2 * rows * row, None)]
    key = {"splitkv": "encode_q1_kernel", "encode": "encode_generic_kernel"}.get(w.kind)
    return [("flare_encode call (one encoder launch)", ph.get("encode", ph.get("encode_merge")), 2 * rows * row,
             key if "encode" in ph else None)]


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_reference(nbytes=1 << 30, reps=5):
    """Context for the HBM roofline: a plain device-to-device copy of 1 GiB
    (read + write bytes over its event-timed duration)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = _ev(), _ev()
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"GB_s": 2 * nbytes / (ms * 1e-3) / 1e9, "ms": ms, "what": "1 GiB device-to-device copy, read+write bytes"}


class FlareppTrainStep(FlareppStep):
    """FLARE++ forward chain followed by its backward chain (decoder, physical-value
    encoder, query-synthesis encoder) with preallocated gradients."""

    def __init__(self, w: W.Workload, x, fused=False, shared=False):
        super().__init__(w, x, fused, shared)
        dev = x["K"].device
        B, H, M, D = w.B, w.H, w.M, w.D
        f32 = dict(dtype=torch.float32, device=dev)
        self.dY = W.normal((B, H, w.N, D), w.wid, W.T_DZ, 1.0, torch.bfloat16, dev)
        self.dK = torch.empty_like(x["K"])
        self.dV = torch.empty_like(x["V"])
        self.dKt = torch.empty_like(x["Kt"])
        self.dVt = torch.empty_like(x["Vt"])
        self.dQX = torch.empty((B, H, M, D), **f32)
        self.dZ2 = torch.empty((B, H, M, D), **f32)
        self.dQt = torch.empty((B, H, M, D), **f32)
        self.dZ2c = torch.empty((B, H, M, D), dtype=torch.bfloat16, device=dev)
        self.dQXc = torch.empty((B, H, M, D), dtype=torch.bfloat16, device=dev)
        self._phases(self.phases + [
            ("decode_bwd", lambda: fl.decode_bwd(x["K"], self.QXb, self.Z, w.scale, self.dY, None, self.dK, self.dQX,
                                                 self.dZ2, self.dZ2c)),
            ("encode2_bwd", lambda: fl.encode_bwd(self.QXb, x["K"], x["V"], w.offsets, None, w.scale, self.Z, self.L,
                                                  self.dZ2c, dQ=self.dQX, dK=self.dK, dV=self.dV, dQ_cast=self.dQXc,
                                                  flags=fl.ACCUMULATE_DQ | fl.ACCUMULATE_DK)),
            ("encode1_bwd", (lambda: fl.encode_bwd(x["Qt"], x["K"], x["V"], w.offsets, None, w.scale, self.QX,
                                                   self.QXL, self.dQXc, dQ=self.dQt, dK=self.dK, dV=self.dV,
                                                   flags=fl.ACCUMULATE_DK | fl.ACCUMULATE_DV)) if shared else
             (lambda: fl.encode_bwd(x["Qt"], x["Kt"], x["Vt"], w.offsets, None, w.scale, self.QX,
                                    self.QXL, self.dQXc, dQ=self.dQt, dK=self.dKt, dV=self.dVt)))])


STEPS = {"flarepp": FlareppStep, "flare": FlareStep, "splitkv": EncodeMergeStep, "encode": EncodeMergeStep,
         "encode_bwd": FwdBwdStep}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The clocks ramp up over the first ~50 ms of sustained work (about 60
    # steps of the FLARE++ chain); the untimed warm-up covers that ramp.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=W.FLAREPP.name, choices=sorted(W.BY_NAME))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="about this much oracle work on whole (batch, head) slices")
    ap.add_argument("--backward", action="store_true",
                    help="FLARE++ only: time the forward chain plus its backward chain (a training step "
                         "of the mixer); not the headline metric")
    ap.add_argument("--fused", action="store_true",
                    help="each encoder and its merge as one call (flare_encode_merge: the merge runs in the "
                         "encoder launch)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and replay it for the warm-up and timed steps "
                         "(the per-kernel times come from eager launches after the timed region)")
    ap.add_argument("--shared", action="store_true",
                    help="FLARE++ only: the shared-projection variant (the query-synthesis encoder reads K and V; "
                         "with --backward its key and value gradients add into dK and dV)")
    ap.add_argument("--flush-mall", action="store_true",
                    help="after the timed region, run the steps again with a 512 MiB scratch write before "
                         "every step, so that no input is served from the 256 MB last-level cache, and report "
                         "their step times")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, copy 1 GiB device-to-device 3 times "
                         "(the plain copy that scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the path is per-GPU and there is no multi-GPU leg.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(2)
    w = W.BY_NAME[args.workload]
    torch.cuda.set_device(0)
    x = w.make("cuda")
    if args.backward and w.kind != "flarepp":
        print("--backward is defined for the FLARE++ workload only", file=sys.stderr)
        sys.exit(2)
    if args.shared and w.kind != "flarepp":
        print("--shared is defined for the FLARE++ workload only", file=sys.stderr)
        sys.exit(2)
    if w.kind == "flarepp":
        step = (FlareppTrainStep if args.backward else FlareppStep)(w, x, args.fused, args.shared)
    else:
        step = STEPS[w.kind](w, x, args.fused)
    run = step
    if args.graph:
        # one eager step on a side stream sizes the library's cached workspace
        # and counters outside the capture
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        run = graph.replay
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides.  An event after every step
    # gives the per-step durations (median, minimum); eager step i also records an event pair
    # around its phase i mod (number of phases), so every kernel's average launch duration comes
    # from the timed launches themselves (two more events per step cost the step about 1 %;
    # events between every kernel of a step slow the following steps by up to a quarter on this
    # GPU).  A graph replay is one launch: with --graph, and for phases that K steps leave
    # without a sample, the per-kernel durations come from the same scheme on eager steps run
    # after the timed region.
    nph = len(step.phases)
    in_region = not args.graph
    t_start, t_end = _ev(), _ev()
    step_ev = [_ev() for _ in range(args.steps)]
    marks = [(_ev(), _ev()) for _ in range(args.steps)] if in_region else []
    torch.cuda.synchronize()
    t_start.record()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        if in_region:
            step.run_marked(i % nph, *marks[i])
        else:
            run()
        step_ev[i].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps
    per_step = [t_start.elapsed_time(step_ev[0])] + [step_ev[i - 1].elapsed_time(step_ev[i])
                                                    for i in range(1, args.steps)]
    for i, (a, b) in enumerate(marks):
        step.phase_ms[i % nph].append(a.elapsed_time(b))
    missing = [k for k in range(nph) if not step.phase_ms[k]]
    if missing:
        # three untimed steps first keep the GPU busy while the host queues the rest
        extra = [(k, _ev(), _ev()) for _ in range(max(args.steps, 10)) for k in missing]
        for _ in range(3):
            step()
        for k, a, b in extra:
            step.run_marked(k, a, b)
        torch.cuda.synchronize()
        for k, a, b in extra:
            step.phase_ms[k].append(a.elapsed_time(b))
    pass_steps = None
    if args.flush_mall:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        ends = [(_ev(), _ev()) for _ in range(args.steps)]
        for _ in range(3):
            run()
        for a, b in ends:
            scratch.fill_(1)
            a.record()
            step()
            b.record()
        torch.cuda.synchronize()
        pass_steps = [a.elapsed_time(b) for a, b in ends]
        del scratch
    ph = {n: sum(p) / len(p) for n, p in zip(step.names, step.phase_ms)}
    cands = roofline_candidates(w, x, step, ph)
    # the binding kernel: the one furthest below the HBM roofline
    kern_name, kern_ms, kern_bytes, kern_key = min(cands, key=lambda c: c[2] / c[1])
    achieved = kern_bytes / (kern_ms * 1e-3) / 1e9
    summ = counter_summary(w.name, kern_key) if kern_key else None
    tokens = w.B * w.N * w.H
    kvb = 2 if w.dtype == "bf16" else 4
    is_main = w.name == W.FLAREPP.name and not args.backward and not args.shared

    line = {
        "metric": "FLARE encode+decode tokens/sec (B*N*H) at N=256K; % of HBM/MFMA roofline" if is_main
        else (("FLARE++ forward+backward tokens/sec (B*N*H)" if args.backward else f"{w.kind} tokens/sec (B*N*H)")
              + (", shared projections" if args.shared else "")),
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": f"synthetic (seeded N(0,1) inputs{' rounded to bf16' if w.dtype == 'bf16' else ''})",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "M": w.M, "D": w.D, "R": w.R,
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "single GPU",
                   "encode_merge": "one call" if args.fused else "two calls",
                   **({"projections": "shared"} if args.shared else {}),
                   "launch": "hip graph replay" if args.graph else "eager"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": summ["hbm_bytes_per_launch"] if summ else None,
                     "mfma_util": summ["mfma_util"] if summ else None,
                     "kernel": kern_name, "kernel_ms": kern_ms, "algorithmic_bytes": kern_bytes},
        "step_ms": {"mean": ms_per_step, "median": statistics.median(per_step), "min": min(per_step)},
        "phases_ms": ph,
        "phases_timed_in_region": in_region,
        "wall_s_timed": wall,
    }
    if len(cands) > 1:
        line["kernels"] = []
        for n, ms, b, key in cands:
            cs = counter_summary(w.name, key) if key else None
            line["kernels"].append({"kernel": n, "ms": ms, "algorithmic_bytes": b,
                                    "traffic": cs["hbm_bytes_per_launch"] if cs else None,
                                    "mfma_util": cs["mfma_util"] if cs else None,
                                    "frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
    if pass_steps:
        line["step_ms_mall_flushed"] = {"mean": sum(pass_steps) / len(pass_steps),
                                        "median": statistics.median(pass_steps), "min": min(pass_steps)}
    if is_main:
        step_bytes = 6 * tokens * w.D * kvb        # 2 encoders (K,V) + decode (read K, write Y)
        if kern_key:
            line["roofline"]["source_hash"] = source_hash(kern_key)
        line["step_roofline"] = {"algorithmic_bytes": step_bytes,
                                 "achieved_GBs": step_bytes / (ms_per_step * 1e-3) / 1e9,
                                 "frac": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                 "frac_median_step": step_bytes / (line["step_ms"]["median"] * 1e-3) / 1e9
                                 / HBM_PEAK_GBS}
    if "mask" in x:
        line["config"]["valid_fraction"] = float(x["mask"].float().mean().item())
    line["copy_reference"] = copy_reference()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds, args.shared)
    print(json.dumps(line), flush=True)
    if args.calibrate_copy:
        del x, step
        torch.cuda.empty_cache()
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
