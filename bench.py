"""Benchmark of the OSR forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one chunk-wise OSR forward over the headline workload, the
long-context one (B=1, H=16, T=65536, m=d=128, chunk 128, forget gate
sigmoid(N(3,1)), bf16 inputs, fp32 state and y) with every input already
resident in HBM; the whole step runs in the library's HIP kernels, called
through the C ABI.  The metric is head-tokens per second (B*H*T per step).
Printed: one JSON line with the headline value, the roofline of the chunk
path measured live with HIP events on the launch stream, the fp64 CPU oracle
timed on this host, and secondary lines for the decode, recurrent and other
chunked workloads, the backward and the layer glue around the recurrence.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
FP32_VALU_PEAK_TFLOPS = 157.3

HEADLINE = "chunked_b1h16_t65536_m128d128_c128"
HEADLINE_CHUNK = 128
SMALL = "chunked_b4h8_t2048_m64d64_c64"


def algorithmic_bytes(w: dict, y_bytes: int = 4) -> float:
    """Compulsory HBM bytes of one forward: every input read once, y written
    once, the fp32 state read once and written once per (b,h)."""
    e = 2 if w["in_dtype"] == "bf16" else 4
    tok = w["B"] * w["H"] * w["T"]
    per_tok = e * (3 * w["m"] + w["d"] + 1) + y_bytes * w["d"]
    return float(tok * per_tok + 2 * 4 * w["B"] * w["H"] * w["m"] * w["d"])


def algorithmic_flops(w: dict, chunk: int) -> float:
    """Algorithmic flops of one forward (multiply-add = 2), decoding objective:
    chunk C > 1: 8md + (C+1)(m+d) + 4md/C + 16m + 3d per head-token;
    C = 1 (recurrent, decode): 12md + 16m + 3d per head-token."""
    m, d = w["m"], w["d"]
    if chunk > 1:
        f = 8 * m * d + (chunk + 1) * (m + d) + 4 * m * d / chunk + 16 * m + 3 * d
    else:
        f = 12 * m * d + 16 * m + 3 * d
    return float(f * w["B"] * w["H"] * w["T"])


def algorithmic_bytes_bwd(w: dict) -> float:
    """Compulsory HBM bytes of one backward: the forward's inputs and fp32 dy
    read once, the fp32 gradients of every input written once, and per (b,h)
    the state, its upstream gradient and its gradient moved once each."""
    e = 2 if w["in_dtype"] == "bf16" else 4
    tok = w["B"] * w["H"] * w["T"]
    per_tok = (e + 4) * (3 * w["m"] + w["d"] + 1) + 4 * w["d"]
    return float(tok * per_tok + 3 * 4 * w["B"] * w["H"] * w["m"] * w["d"])


def chain_reference_ms(w: dict, chunk: int) -> float:
    """Dependency-chain reference: the chunks of one (b,h) run in sequence, so
    the step cannot beat (T/C) x (per-chunk flops at one CU's bf16 MFMA peak)."""
    per_chunk = algorithmic_flops(dict(w, B=1, H=1, T=chunk), chunk)
    return (w["T"] / chunk) * per_chunk / (BF16_MFMA_PEAK_TFLOPS * 1e12 / 256) * 1e3


# Sources of the backward kernels (every csrc/osr_bwd* file): not part of the
# forward and decode kernels whose traffic counters are keyed by the hash below.
BWD_PREFIX = "osr_bwd"
# Source of the layer-glue kernels: not part of either.
GLUE_SOURCES = ("osr_glue.hip",)


def source_hash() -> str:
    """Hash of the sources the forward and decode kernels are built from."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "compressed_memory_linear_amd", "csrc", "*"))):
        base = os.path.basename(p)
        if base.startswith(BWD_PREFIX) or base in GLUE_SOURCES:
            continue
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


class Case:
    """Device-resident inputs and outputs for one entry point on one workload
    (entry: chunked, chunked_gated, recurrent, decode, backward, or train: the
    saving forward and the backward from its saved values, one training step).
    With copies > 1 the steps rotate over that many separately allocated input
    sets, so a working set larger than the 256 MB Infinity Cache is read from
    HBM rather than from the cache."""

    def __init__(self, name: str, entry: str, chunk: int, y_dtype=None, copies: int = 1, mode: int = 0,
                 linearisation: int = 0):
        import torch
        from compressed_memory_linear_amd import osr, synth
        self.name, self.entry, self.chunk, self.mode, self.lin = name, entry, chunk, mode, linearisation
        self.w = dict(synth.WORKLOADS[name])
        inp = synth.workload_inputs(name)
        self.inp = inp
        self.sets = [osr.to_device(inp) for _ in range(copies)]
        self.copies = copies
        self.i = 0
        self.y_dtype = y_dtype or torch.float32
        self.y = torch.empty((inp.B, inp.T, inp.H, inp.d), dtype=self.y_dtype, device="cuda")
        self.state_out = torch.empty_like(self.sets[0]["state"])
        self.ws = None
        if entry in ("backward", "train"):
            desc = osr.make_desc(inp.B, inp.T, inp.H, inp.m, inp.d, 1,
                                 osr.BF16 if inp.in_dtype == "bf16" else osr.F32, osr.F32, mode, linearisation)
            self.ws = torch.empty(osr.lattice_osr_bwd_workspace_bytes(desc, chunk), dtype=torch.uint8,
                                  device="cuda")
            g = torch.Generator(device="cuda").manual_seed(7)
            self.dy = torch.randn(self.y.shape, generator=g, device="cuda")
            self.dso = torch.randn(self.state_out.shape, generator=g, device="cuda")
            t0 = self.sets[0]
            self.grads = {"d" + n: torch.empty(t0[n].shape, dtype=torch.float32, device="cuda")
                          for n in ("q", "k", "v", "gamma", "mu")}
            self.grads["dstate_in"] = torch.empty_like(t0["state"])
        if entry == "chunked_gated":
            g = torch.Generator(device="cuda").manual_seed(9)
            self.gate = (torch.randn(self.y.shape, generator=g, device="cuda") * 2).to(self.sets[0]["q"].dtype)
        if entry in ("chunked", "chunked_gated"):
            desc = osr.make_desc(inp.B, inp.T, inp.H, inp.m, inp.d, 1,
                                 osr.BF16 if inp.in_dtype == "bf16" else osr.F32, osr.F32, mode, linearisation)
            need = osr.lattice_osr_workspace_bytes(desc, chunk)
            if need:
                self.ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def step(self):
        from compressed_memory_linear_amd import osr
        t = self.sets[self.i % self.copies]
        self.i += 1
        args = (t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"])
        if self.entry == "chunked":
            osr.lattice_osr_fwd_chunked(*args, self.chunk, mode=self.mode, y_dtype=self.y_dtype,
                                        state_out=self.state_out, y=self.y, workspace=self.ws,
                                        linearisation=self.lin)
        elif self.entry == "chunked_gated":
            osr.lattice_osr_fwd_chunked_gated(t["q"], t["k"], t["v"], t["gamma"], t["mu"], self.gate, t["state"],
                                              self.chunk, mode=self.mode, y_dtype=self.y_dtype,
                                              state_out=self.state_out, y=self.y, workspace=self.ws,
                                              linearisation=self.lin)
        elif self.entry == "backward":
            osr.lattice_osr_bwd_chunked(*args, self.dy, self.dso, self.chunk, mode=self.mode, grads=self.grads,
                                        workspace=self.ws)
        elif self.entry == "train":
            # one training step of the layer at a small chunk: the forward that saves what the
            # backward needs, then the backward from those values
            osr.lattice_osr_fwd_chunked_save(*args, self.chunk, mode=self.mode, y_dtype=self.y_dtype,
                                             state_out=self.state_out, y=self.y, saved=self.ws)
            osr.lattice_osr_bwd_chunked_saved(*args, self.dy, self.dso, self.chunk, saved=self.ws, mode=self.mode,
                                              grads=self.grads)
        elif self.entry == "recurrent":
            osr.lattice_osr_fwd_recurrent(*args, mode=self.mode, y_dtype=self.y_dtype, state_out=self.state_out,
                                          y=self.y)
        else:
            # decode keeps stepping the same state in place, as a decoder would
            osr.lattice_osr_decode_step(*args, mode=self.mode, y_dtype=self.y_dtype, state_out=t["state"], y=self.y)

    @property
    def head_tokens(self) -> int:
        return self.inp.B * self.inp.H * self.inp.T


class GlueCase:
    """Device-resident inputs of the layer glue on a workload's shape (bf16 projections,
    fp32 filters, fp32 y): entry "glue_pre" (short convolutions of q and k, sigmoid
    writing intensity) or "glue_post" (GeLU post-gate)."""

    def __init__(self, name: str, entry: str):
        import torch
        from compressed_memory_linear_amd import osr, synth
        self.name, self.entry = name, entry
        self.w = dict(synth.WORKLOADS[name])
        w = self.w
        g = synth.make_glue_inputs(w["B"], w["T"], w["H"], w["m"], w["d"], seed=w["seed"] + 50)

        def dev(a):
            t = torch.from_numpy(a)
            return (t.view(torch.bfloat16) if a.dtype.itemsize == 2 else t).to("cuda")

        if entry == "glue_pre":
            self.args = [dev(a) for a in (g.xq, g.xk, g.logit, g.wq, g.wk, g.bq, g.bk, g.hist_q, g.hist_k)]
            self.outs = dict(q=torch.empty_like(self.args[0]), k=torch.empty_like(self.args[1]),
                             gamma=torch.empty_like(self.args[2]), hist_q_out=torch.empty_like(self.args[7]),
                             hist_k_out=torch.empty_like(self.args[8]))
        else:
            self.y, self.gate = dev(g.y), dev(g.gate)
            self.out = torch.empty_like(self.y)
        del g
        self.osr = osr

    def step(self):
        if self.entry == "glue_pre":
            self.osr.lattice_osr_glue_pre(*self.args, **self.outs, return_history=True)
        else:
            self.osr.lattice_osr_glue_post(self.y, self.gate, out=self.out)

    @property
    def head_tokens(self) -> int:
        return self.w["B"] * self.w["H"] * self.w["T"]


def algorithmic_bytes_glue(w: dict, entry: str) -> float:
    """Compulsory HBM bytes of one glue call (bf16 projections and gates, fp32 y):
    pre reads xq, xk and the per-slot logits and writes q, k and gamma (each
    B T H m bf16), plus the filters, biases and histories; post reads y (fp32)
    and the gate (bf16) and writes y * GeLU(gate) (fp32)."""
    rows = w["B"] * w["T"] * w["H"]
    if entry == "glue_pre":
        n = w["H"] * w["m"]
        return rows * w["m"] * 2 * 3 * 2 + 2 * n * 5 * 4 + 2 * 2 * w["B"] * 3 * n * 2
    return rows * w["d"] * (4 + 2 + 4)


def time_case(case: Case, steps: int, warmup: int):
    """Average ms per step, timed with HIP events on the launch stream."""
    import torch
    for _ in range(warmup):
        case.step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        case.step()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def step_percentiles(case: Case, steps: int):
    """p10 / p50 / p90 of single-step times (ms), each step bracketed by its
    own HIP events on the launch stream; a pass of its own after the timed
    region, so the headline figure is untouched by the extra events."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        case.step()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
    return {"p10": q(0.1), "p50": q(0.5), "p90": q(0.9), "steps": steps}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name: str, chunk: int, budget_s: float = 12.0) -> dict:
    """The fp64 oracle on this host, over the whole workload, repeated until
    about budget_s seconds have passed (at least once)."""
    import oracle
    from compressed_memory_linear_amd import synth
    inp = synth.workload_inputs(name)
    args = inp.values_f64()
    reps, total, threads = 0, 0.0, 0
    while reps == 0 or (total < budget_s and reps < 2000):
        t0 = time.perf_counter()
        _, _, threads = oracle.osr_forward(*args, chunk_size=chunk, return_threads=True)
        total += time.perf_counter() - t0
        reps += 1
    out = {"value": inp.head_tokens * reps / total, "unit": "head-tokens/s", "cores": threads,
           "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
           "sample": f"whole workload {name} (B*H*T = {inp.head_tokens} head-tokens), "
                     f"{reps} repetition(s), {total:.2f} s, fp64 C with {threads} threads over the "
                     f"{inp.B * inp.H} (b,h) sequences (one thread per sequence at most)"}
    # the tiny fp32 workload on one thread, at each of its chunk sizes
    tiny = synth.workload_inputs("tiny_f32_m16d32_t64")
    targs = tiny.values_f64()
    single = {}
    for c in (1, 4, 16, 64):
        reps, total = 0, 0.0
        while reps == 0 or (total < 0.5 and reps < 10000):
            t0 = time.perf_counter()
            oracle.osr_forward(*targs, chunk_size=c, nthreads=1)
            total += time.perf_counter() - t0
            reps += 1
        single[f"C{c}"] = tiny.head_tokens * reps / total
    out["tiny_f32_m16d32_t64_one_thread"] = {"unit": "head-tokens/s", "cores": 1, **single}
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--only", default=None, help="time a single workload/entry (profiling runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the OSR path shards over "
                                   "(batch, head) with no communication, and multi-GPU runs are "
                                   "not part of it; use --gpus 1"}))
        return 2

    import torch
    from compressed_memory_linear_amd import osr
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    osr.load_library()

    if args.only == "copy":
        # Plain device-to-device copy of 256 MiB: the reference for scaling the
        # FETCH_SIZE / WRITE_SIZE counters (it moves exactly 256 MiB each way).
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_each_way": 256 << 20, "launches": args.warmup + args.steps}))
        return 0
    if args.only:
        name, entry, chunk = args.only.split(":")
        case = GlueCase(name, entry) if entry.startswith("glue") else Case(name, entry, int(chunk))
        ms = time_case(case, args.steps, args.warmup)
        print(json.dumps({"only": args.only, "ms_per_step": ms,
                          "head_tokens_per_s": case.head_tokens / (ms * 1e-3)}), flush=True)
        return 0

    head = Case(HEADLINE, "chunked", HEADLINE_CHUNK, copies=1)
    ms = time_case(head, args.steps, args.warmup)
    pct = step_percentiles(head, max(args.steps, 20))
    value = head.head_tokens / (ms * 1e-3)
    abytes = algorithmic_bytes(head.w)
    achieved = abytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "tokens/s for OSR fwd (BxHxT, m, d) + % of MFMA/HBM roofline",
        "value": value,
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "step_ms_percentiles": pct,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-in/f32",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "B": head.w["B"], "H": head.w["H"], "T": head.w["T"], "m": head.w["m"],
                   "d": head.w["d"], "chunk": HEADLINE_CHUNK, "inputs": "bf16", "state": "f32", "y": "f32",
                   "objective": "decoding", "forget_gate": "sigmoid(N(3,1))", "input_copies": head.copies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(f"chunked:{HEADLINE}"),
                     "algorithmic_bytes_per_launch": abytes,
                     "algorithmic_flops_per_launch": algorithmic_flops(head.w, HEADLINE_CHUNK),
                     "mfma_frac_algorithmic": algorithmic_flops(head.w, HEADLINE_CHUNK) / (ms * 1e-3) / 1e12
                                              / BF16_MFMA_PEAK_TFLOPS,
                     "chain_reference_ms": chain_reference_ms(head.w, HEADLINE_CHUNK),
                     "kernels": "one call = state-passing kernel + read-out kernel (split per kernel in "
                                "the rocprofv3 summary)",
                     "measured": "HIP events on the launch stream around the timed steps"},
    }
    del head
    torch.cuda.empty_cache()

    if not args.no_secondary:
        sec = []
        for name, entry, chunk, steps, mode, lin in ((SMALL, "chunked", 64, 20, 0, 0),
                                                     ("decode_s256h32_m128d128", "decode", 1, 50, 0, 0),
                                                     ("chunked_b8h16_t4096_m64d128_c64", "chunked", 64, 5, 0, 0),
                                                     ("chunked_b8h16_t4096_m64d128_c64", "chunked_gated", 64, 5, 0,
                                                      0),
                                                     (SMALL, "recurrent", 1, 2, 0, 0),
                                                     (SMALL, "chunked", 4, 3, 0, 0),
                                                     (SMALL, "chunked", 64, 10, 2, 0),
                                                     (SMALL, "chunked", 64, 10, 0, 1),
                                                     (SMALL, "backward", 64, 2, 0, 0),
                                                     (SMALL, "backward", 4, 1, 0, 0),
                                                     (SMALL, "train", 4, 1, 0, 0),
                                                     (HEADLINE, "backward", HEADLINE_CHUNK, 2, 0, 0)):
            # the small workload (51 MB) fits the 256 MB Infinity Cache: rotate 8 input copies
            c = Case(name, entry, chunk, copies=8 if name == SMALL and entry == "chunked" else 1,
                     mode=mode, linearisation=lin)
            t_ms = time_case(c, steps, 1)
            ab = {"backward": algorithmic_bytes_bwd(c.w),
                  "train": algorithmic_bytes(c.w) + algorithmic_bytes_bwd(c.w)}.get(entry, algorithmic_bytes(c.w))
            if entry == "chunked_gated":  # the gate is read once more (in the inputs' dtype)
                ab += c.head_tokens * c.w["d"] * (2 if c.w["in_dtype"] == "bf16" else 4)
            sec.append({"workload": name, "entry": entry, "chunk": chunk,
                        "objective": {0: "decoding", 1: "similarity", 2: "encoding"}[mode],
                        "linearisation": "recurrence_linear1" if lin else "recurrence_linear2", "ms_per_step": t_ms,
                        "head_tokens_per_s": c.head_tokens / (t_ms * 1e-3),
                        "hbm_gbs_algorithmic": ab / (t_ms * 1e-3) / 1e9,
                        "hbm_frac": ab / (t_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "tflops_algorithmic": None if entry in ("backward", "train")
                        else algorithmic_flops(c.w, chunk) / (t_ms * 1e-3) / 1e12,
                        "chain_reference_ms": chain_reference_ms(c.w, chunk) if entry == "chunked" and chunk >= 16
                        else None})
            del c
            torch.cuda.empty_cache()
        for entry in ("glue_pre", "glue_post"):
            name = "chunked_b8h16_t4096_m64d128_c64"
            c = GlueCase(name, entry)
            t_ms = time_case(c, 10, 2)
            ab = algorithmic_bytes_glue(c.w, entry)
            sec.append({"workload": name, "entry": entry, "ms_per_step": t_ms,
                        "head_tokens_per_s": c.head_tokens / (t_ms * 1e-3),
                        "hbm_gbs_algorithmic": ab / (t_ms * 1e-3) / 1e9,
                        "hbm_frac": ab / (t_ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
            del c
            torch.cuda.empty_cache()
        out["secondary"] = sec

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(HEADLINE, HEADLINE_CHUNK)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
