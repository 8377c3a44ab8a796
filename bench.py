"""KDA benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--chunk 16|64] [--no-cpu]
                    [--no-decode] [--no-varlen] [--no-prologue] [--no-backward]
                    [--no-long] [--decode-reps R] [--calib-mib M]

A step is one chunkwise prefill over the K3 head-shape workload (B=1, H=96,
T=4096, dk=dv=128, bf16 inputs, fp32 state, S0 ~ N(0, 0.02^2)) with inputs
resident in HBM; ``value`` is tokens/s over the K timed steps.  The same run
also times the fused decode step on the batched decode workload (B=64, H=96,
d=128, 256 steps on a persistent fp32 state) and reports head-state updates/s
under ``decode``.  Times come from HIP events recorded on the stream the
kernels are launched on (torch's current stream).

Roofline: both kernels are HBM-bound at these shapes.  ``achieved`` is the
algorithmic bytes one launch must move divided by its average duration:
  prefill: B*T*H*(4*d*2 + d*2 + 2) + 2*B*H*d*d*4 + H*4 bytes
           (q, k, z, v read, o written, beta read; S0 read and S_T written; A)
  decode : B*H*(2*d*d*4 + 4*d*2 + 2 + d*2) + H*4 bytes per step
The fp64 oracle is timed on the host cores over the full prefill workload
(``cpu_baseline``), reported in the same unit.  Prints ONE JSON line.

``mfma`` reports the same prefill against the bf16 matrix-core peak: the
algorithmic flops of a launch (6d^2 + 5Cd + C^2/3 per token-head) over its
time, and the MFMA flops a counter run measured for this kernel source
(``SQ_INSTS_VALU_MFMA_MOPS_BF16`` x 512; masked and duplicated tiles
included), read from the kernel's summary under profiles/.

``long`` times the long-context (B1 H96 T65536, z ~ N(2,1)) and million-token
(B1 H16 T2^20) prefill workloads at 64- and 16-token chunks over 3 launches
each, inputs drawn on the device; the million-token head share also split
into 4, 8 and 9 segments at 16-token chunks and 9 and 17 at 64
(kda_prefill_split).
Each entry's ``roofline.traffic`` is the HBM bytes per call from its counter
summary under profiles/ (for a split call, both passes), null once the kernel
source has changed.  ``timing`` gives the median and minimum per-launch time
of 10 equal segments of the timed steps.

``backward`` times kda_prefill_bwd_ex on the same workload: gradients of q,
k, v, z, beta, A and S0 from seeded dL/do and dL/dS_T (the forward is rerun
with 16-token state checkpoints inside the call, beside the backward's prep on
a second stream of the caller's).

``prologue`` times the layer's prologue on raw inputs of the same shapes
(short convolutions of width 4, SiLU, q/k L2 norm, continued sequences): the
prologue kernel alone (HBM-bound: q, k, v read and written once, states and
taps), prologue + prefill end to end, and the decode step with the prologue
fused in.

``--calib-mib M`` adds, after the timed region, one elementwise copy of M MiB
(read M, write M): the reference a hardware byte counter (FETCH_SIZE,
WRITE_SIZE) is scaled by when the kernels' HBM traffic is measured.
``roofline.traffic`` is the measured HBM bytes per launch recorded in the
kernel's summary under profiles/, reported only while the kernel source still
hashes to the one the counters were taken on (null otherwise).

Order: packed, prologue, backward, long, decode, then the headline prefill,
timed last so that its W warm-up and K timed steps run on a GPU that has been
under load for a while (the decode timing, 16 runs of 256 steps, ends right
before it), whatever W is.  The clocks of an MI355X drop within about a second
of idling, and the K3 prefill then reads ~25% slower until they ramp up again
(measured: 225-230 us per launch just after 1 s idle, 187 us after 2 s of
decode steps, 180 us after 0.5 s of back-to-back prefills).  The oracle
baseline runs after every GPU timing.
"""
from __future__ import annotations

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

HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "linear_recurrent_attention_chunkwise_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "KDA prefill tokens/s (H=96,d=128,bf16) + decode state-updates/s; % roofline"


def prefill_bytes(B, T, H, d, esz=2):
    return B * T * H * (4 * d * esz + d * esz + esz) + 2 * B * H * d * d * 4 + H * 4


MFMA_PEAK_TFLOPS = 2500.0   # dense bf16


def prefill_flops(B, T, H, d, chunk):
    """Algorithmic flops of one prefill: 6d^2 + 5Cd + C^2/3 per token-head (the
    state products, the chunk-local products and the triangular inverse)."""
    return B * T * H * (6 * d * d + 5 * chunk * d + chunk * chunk / 3.0)


def decode_bytes(B, H, d, esz=2):
    return B * H * (2 * d * d * 4 + 4 * d * esz + esz + d * esz) + H * 4


def prefill_kernel_name(chunk):
    """Name of the kernel a default-configured prefill of the K3 workload runs."""
    return "kda_prefill16_kernel" if chunk == 16 else "kda_prefill_kernel"


def source_hash(files):
    """sha256 over the given kernel sources (in order), as hex."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


KERNEL_SOURCES = {
    "kda_prefill16_kernel": ["kda_prefill16.hip", "kda_device.h"],
    "kda_prefill_kernel": ["kda_prefill.hip", "kda_device.h"],
    "kda_decode_kernel": ["kda_decode.hip", "kda_device.h"],
    "kda_conv_norm_kernel": ["kda_conv.hip", "kda_device.h"],
}


def recorded_counter(kernel, summary, key="traffic_bytes_per_launch"):
    """A per-launch counter figure (`key: value` line) from a committed counter
    summary, or None when the summary is missing or was taken on a different
    kernel source."""
    path = os.path.join(PROFILES, summary)
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    text = open(path).read()
    mb = re.search(r"^" + re.escape(key) + r":\s*([0-9]+)", text, re.M)
    mh = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not mb or not mh or mh.group(1) != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return int(mb.group(1))


def recorded_traffic(kernel, summary):
    """HBM bytes per launch from a committed counter summary (see recorded_counter)."""
    return recorded_counter(kernel, summary)


def calibration_copy(torch, mib):
    """One elementwise copy of `mib` MiB on the current stream (not timed)."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _events(torch):
    return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))


SEGMENTS = 10


def time_prefill(torch, kda, inp, chunk, steps, warmup, segments=1):
    """ms per launch over the timed steps, plus the median and minimum of the
    per-launch times of SEGMENTS equal segments (events between segments)."""
    out = torch.empty_like(inp["v"])
    S_T = torch.empty_like(inp["S0"]) if inp["S0"] is not None else None

    ws = None
    if segments > 1:
        B, T, H, d = inp["q"].shape
        ws = torch.empty(kda.prefill_split_workspace_size(inp["q"].dtype, B, T, H, d, d, chunk,
                                                          segments),
                         dtype=torch.uint8, device=inp["q"].device)

    def run():
        kda.prefill(inp["q"], inp["k"], inp["v"], inp["z"], inp["beta"], inp["A"], inp["S0"],
                    chunk=chunk, out=out, S_T=S_T, segments=segments, workspace=ws)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    nseg = min(SEGMENTS, steps)
    bounds = [steps * i // nseg for i in range(nseg + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nseg + 1)]
    ev[0].record()
    for i in range(nseg):
        for _ in range(bounds[i + 1] - bounds[i]):
            run()
        ev[i + 1].record()
    torch.cuda.synchronize()
    seg = sorted(ev[i].elapsed_time(ev[i + 1]) / (bounds[i + 1] - bounds[i]) for i in range(nseg))
    return ev[0].elapsed_time(ev[nseg]) / steps, seg[len(seg) // 2], seg[0]


VARLEN_LENGTHS = [4096, 1000, 37, 2500, 16, 513, 64, 3000]   # mixed, ragged, 11226 tokens
VARLEN_CKPT_EVERY = 1024


def time_varlen(torch, kda, vin, ckpt_every, steps, warmup):
    """ms per launch of the packed prefill (optionally with checkpoints)."""
    o = torch.empty_like(vin["v"])
    S_T = torch.empty_like(vin["S0"])
    cu = vin["cu_seqlens"]
    ck = None
    if ckpt_every > 0:
        _, n = kda.checkpoint_rows(VARLEN_LENGTHS, ckpt_every)
        ck = torch.empty((n,) + tuple(vin["S0"].shape[1:]), dtype=torch.float32,
                         device=vin["S0"].device)

    def run():
        kda.prefill_varlen(vin["q"], vin["k"], vin["v"], vin["z"], vin["beta"], vin["A"], cu,
                           S0=vin["S0"], chunk=16, ckpt_every=ckpt_every, out=o, S_T=S_T,
                           ckpt=ck, seq_lens=VARLEN_LENGTHS)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_decode(torch, kda, dinp, reps):
    S = dinp["S"]
    steps = dinp["q"].shape[0]
    out = torch.empty_like(dinp["v"][0])

    def one_pass():
        for t in range(steps):
            kda.decode_step(dinp["q"][t], dinp["k"][t], dinp["v"][t], dinp["z"][t],
                            dinp["beta"][t], dinp["A"], S, out=out)

    one_pass()   # warm-up pass
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(reps):
        one_pass()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * steps)   # ms per decode step


PROLOGUE_WIDTH, PROLOGUE_ACT = 4, "silu"


def conv_norm_bytes(B, T, H, d, W, esz=2):
    """q, k, v read and written once, convolution states read and written, taps."""
    return 6 * B * T * H * d * esz + 2 * 3 * B * (W - 1) * H * d * esz + 3 * H * d * W * 4


def time_layer(torch, kda, lin, steps, warmup):
    """ms per launch of kda_conv_norm alone and of kda_prefill_conv (prologue +
    prefill) on the raw layer inputs."""
    dev = lin["q"].device
    st_in = (lin["sq"], lin["sk"], lin["sv"])
    st_out = tuple(torch.empty_like(t) for t in st_in)
    outs = tuple(torch.empty_like(lin[n]) for n in ("q", "k", "v"))
    o = torch.empty_like(lin["v"])
    S_T = torch.empty_like(lin["S0"])
    B, T, H, d = lin["q"].shape
    ws = torch.empty(kda.prefill_conv_workspace_size(lin["q"].dtype, B, T, H, d, d, 16),
                     dtype=torch.uint8, device=dev)
    taps = (lin["wq"], lin["wk"], lin["wv"])

    def conv():
        kda.conv_norm(lin["q"], lin["k"], lin["v"], *taps, state=st_in, act=PROLOGUE_ACT,
                      out=outs, state_out=st_out)

    def layer():
        kda.prefill_conv(lin["q"], lin["k"], lin["v"], lin["z"], lin["beta"], lin["A"], *taps,
                         state=st_in, act=PROLOGUE_ACT, S0=lin["S0"], chunk=16, out=o, S_T=S_T,
                         state_out=st_out, workspace=ws)

    res = []
    for fn in (conv, layer):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = _events(torch)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / steps)
    return res


def time_decode_conv(torch, kda, dl, reps):
    """ms per fused decode step with the prologue (kda_decode_step_conv)."""
    S = dl["S"]
    steps = dl["q"].shape[0]
    out = torch.empty_like(dl["v"][0])
    st = (dl["sq"], dl["sk"], dl["sv"])
    taps = (dl["wq"], dl["wk"], dl["wv"])

    def one_pass():
        for t in range(steps):
            kda.decode_step_conv(dl["q"][t], dl["k"][t], dl["v"][t], dl["z"][t], dl["beta"][t],
                                 dl["A"], *taps, st, S, act=PROLOGUE_ACT, out=out)

    one_pass()
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(reps):
        one_pass()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * steps)


def _host_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(w, inp_cpu):
    """The fp64 oracle on the host cores: the full prefill workload on all
    threads, and two heads on one thread (per-core rate)."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    threads = max(1, min(threads, os.cpu_count() or 1, w.B * w.H))
    f = lambda t: None if t is None else t.float().numpy()
    args = [f(inp_cpu[n]) for n in ("q", "k", "v", "z", "beta", "A", "S0")]
    t0 = time.perf_counter()
    oracle.prefill(*args, threads=threads)
    dt = time.perf_counter() - t0
    heads = [0, 1]
    sub = [a[:, :, heads] if a.ndim == 4 else a[:, :, heads] for a in args[:5]]
    sub += [args[5][heads], args[6][:, heads] if args[6] is not None else None]
    t1 = time.perf_counter()
    oracle.prefill(*sub, threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": w.B * w.T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"full {w.name} prefill (B{w.B} H{w.H} T{w.T} d{w.dk}), fp64 sequential "
                      f"recurrence, {dt:.2f} s wall",
            "single_thread": {"value": w.B * w.T * len(heads) / dt1, "unit": "token-heads/s/core",
                              "sample": f"heads {heads} of the same workload on 1 thread, "
                                        f"{dt1:.2f} s wall"},
            "host": _host_info()}


LONG_CASES = [("long_prefill_bf16", 64, 1), ("long_prefill_bf16", 16, 1),
              ("million_prefill_bf16", 64, 1), ("million_prefill_bf16", 16, 1),
              ("million_prefill_bf16", 16, 4), ("million_prefill_bf16", 16, 8),
              ("million_prefill_bf16", 16, 9), ("million_prefill_bf16", 64, 9),
              ("million_prefill_bf16", 64, 17)]


def time_backward(torch, kda, inp, dO, dST, steps, warmup):
    """ms per call of the chunk-parallel backward (kda_prefill_bwd: forward
    rerun with per-chunk state checkpoints, then the reverse chunk kernels),
    outputs and workspace allocated once outside the timed region."""
    B, T, H, d = inp["q"].shape
    dev = inp["q"].device
    ws = torch.empty(kda.prefill_bwd_workspace_size(inp["q"].dtype, B, T, H, d, d),
                     dtype=torch.uint8, device=dev)

    def run():
        kda.prefill_bwd(inp["q"], inp["k"], inp["v"], inp["z"], inp["beta"], inp["A"],
                        inp["S0"], dO, dST, workspace=ws)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, ws.numel()


def time_long(torch, kda, steps):
    """The long-context (B1 H96 T65536) and million-token (B1 H16 T2^20) prefill
    workloads, inputs drawn on the device (same recipe and seed, device
    generator), timed over a few launches at each chunk size."""
    from linear_recurrent_attention_chunkwise_amd.inputs import WORKLOADS, make_prefill_inputs
    dev = torch.device("cuda:0")
    res = {}
    cache = {}
    for name, chunk, segments in LONG_CASES:
        w = WORKLOADS[name]
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            cache[name] = make_prefill_inputs(w, device=dev)
        inp = cache[name]
        ms, med, mn = time_prefill(torch, kda, inp, chunk, steps, 1, segments)
        b = prefill_bytes(w.B, w.T, w.H, w.dk)
        key = f"{name}_c{chunk}" + (f"_split{segments}" if segments > 1 else "")
        kernel = prefill_kernel_name(chunk)
        if segments > 1:   # the split call's two passes of the prefill kernel
            summary = f"kda_prefill_split_{name}" + ("" if chunk == 16 else f"_c{chunk}") + ".md"
            traffic = recorded_counter(kernel, summary, f"traffic_bytes_per_launch_split{segments}")
        else:
            traffic = recorded_traffic(kernel, f"{kernel}_{name}_c{chunk}.md")
        res[key] = {
            "value": w.B * w.T / (ms * 1e-3), "unit": "tokens/s", "ms_per_launch": ms,
            "median_ms": med, "min_ms": mn, "chunk": chunk, "segments": segments,
            "workload": f"{name}: B={w.B} H={w.H} T={w.T} d={w.dk} bf16, z mean {w.z_mean}",
            "hbm_frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "roofline": {"bound": "hbm", "achieved": b / (ms * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
                         "kernel": kernel, "bytes_per_launch": b}}
    cache.clear()
    torch.cuda.empty_cache()
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=8000)
    ap.add_argument("--chunk", type=int, default=16, choices=(16, 64))
    ap.add_argument("--decode-reps", type=int, default=16,
                    help="runs of the 256-step decode workload in its timing")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-prologue", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the chunk-parallel backward timing")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context and million-token prefill timings")
    ap.add_argument("--calib-mib", type=int, default=0,
                    help="also run one elementwise copy of this many MiB (byte-counter reference)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (got --gpus {args.gpus}); "
              "multi-GPU runs are not part of it", file=sys.stderr)
        return 2

    import torch

    import linear_recurrent_attention_chunkwise_amd as kda
    from linear_recurrent_attention_chunkwise_amd.inputs import (WORKLOADS, make_decode_inputs,
                                                                 make_prefill_inputs)

    dev = torch.device("cuda:0")
    w = WORKLOADS["k3_prefill_bf16"].with_(chunk=args.chunk)
    inp_cpu = make_prefill_inputs(w)
    inp = {k: (v.to(dev) if v is not None else None) for k, v in inp_cpu.items()}
    sections = {}
    if not args.no_varlen:
        from linear_recurrent_attention_chunkwise_amd.inputs import make_varlen_inputs
        wv = WORKLOADS["k3_prefill_bf16"].with_(seed=5)
        vin = {k: (v.to(dev) if v is not None else None)
               for k, v in make_varlen_inputs(wv, VARLEN_LENGTHS).items()}
        ntok = sum(VARLEN_LENGTHS)
        nseq = len(VARLEN_LENGTHS)
        vbytes = (ntok * wv.H * (5 * wv.dk * 2 + 2) + 2 * nseq * wv.H * wv.dk * wv.dk * 4
                  + wv.H * 4)
        vms = time_varlen(torch, kda, vin, 0, max(1, args.steps // 4), max(1, args.warmup // 40))
        cms = time_varlen(torch, kda, vin, VARLEN_CKPT_EVERY, max(1, args.steps // 4),
                          max(1, args.warmup // 40))
        nck = sum(L // VARLEN_CKPT_EVERY for L in VARLEN_LENGTHS)
        cbytes = vbytes + nck * wv.H * wv.dk * wv.dk * 4
        sections["varlen"] = {
            "value": ntok / (vms * 1e-3), "unit": "tokens/s", "ms_per_launch": vms,
            "workload": f"packed prefill, {nseq} sequences of lengths {VARLEN_LENGTHS} "
                        f"({ntok} tokens), H={wv.H}, d={wv.dk}, bf16, chunk 16",
            "roofline": {"bound": "hbm", "achieved": vbytes / (vms * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": vbytes / (vms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "bytes_per_launch": vbytes},
            "with_checkpoints": {"ckpt_every": VARLEN_CKPT_EVERY, "checkpoints": nck,
                                 "ms_per_launch": cms, "value": ntok / (cms * 1e-3),
                                 "bytes_per_launch": cbytes}}
    if not args.no_prologue:
        from linear_recurrent_attention_chunkwise_amd.inputs import (make_layer_decode_inputs,
                                                                     make_layer_inputs)
        Wc = PROLOGUE_WIDTH
        lin = {k: (v.to(dev) if v is not None else None)
               for k, v in make_layer_inputs(w, Wc).items()}
        cms_, lms = time_layer(torch, kda, lin, max(1, args.steps // 4), max(1, args.warmup // 40))
        del lin
        cb = conv_norm_bytes(w.B, w.T, w.H, w.dk, Wc)
        wd = WORKLOADS["k3_decode_bf16"]
        dl = make_layer_decode_inputs(wd, Wc, device=dev)
        dcms = time_decode_conv(torch, kda, dl, args.decode_reps)
        del dl
        dcb = (decode_bytes(wd.B, wd.H, wd.dk) + 2 * 3 * wd.B * (Wc - 1) * wd.H * wd.dk * 2
               + 3 * wd.H * wd.dk * Wc * 4)
        sections["prologue"] = {
            "width": Wc, "activation": PROLOGUE_ACT,
            "workload": f"{w.name} raw layer inputs (B={w.B} H={w.H} T={w.T} d={w.dk} bf16), "
                        f"short convolutions of width {Wc} + {PROLOGUE_ACT} + q/k L2 norm, "
                        f"continued sequence",
            "conv_norm": {"us_per_launch": cms_ * 1e3, "kernel": "kda_conv_norm_kernel",
                          "roofline": {"bound": "hbm", "achieved": cb / (cms_ * 1e-3) / 1e9,
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": cb / (cms_ * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                       "traffic": recorded_traffic(
                                           "kda_conv_norm_kernel",
                                           f"kda_conv_norm_kernel_{w.name}.md"),
                                       "bytes_per_launch": cb}},
            "prefill_conv": {"value": w.B * w.T / (lms * 1e-3), "unit": "tokens/s",
                             "ms_per_launch": lms},
            "decode_step_conv": {
                "value": wd.B * wd.H / (dcms * 1e-3), "unit": "head-state-updates/s",
                "us_per_step": dcms * 1e3,
                "workload": f"{wd.name} with the fused prologue (B={wd.B} H={wd.H})",
                "roofline": {"bound": "hbm", "achieved": dcb / (dcms * 1e-3) / 1e9,
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": dcb / (dcms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "traffic": recorded_traffic(
                                 "kda_decode_kernel", f"kda_decode_kernel_conv_{wd.name}.md"),
                             "kernel": "kda_decode_kernel (prologue fused)",
                             "bytes_per_launch": dcb}}}
    if not args.no_backward:
        from linear_recurrent_attention_chunkwise_amd.inputs import make_cotangents
        dO, dST = make_cotangents(w, device=dev)
        bms, wsb = time_backward(torch, kda, inp, dO, dST,
                                 max(1, args.steps // 20), max(1, args.warmup // 400))
        del dO, dST
        torch.cuda.empty_cache()
        sections["backward"] = {
            "value": w.B * w.T / (bms * 1e-3), "unit": "tokens/s", "ms_per_call": bms,
            "workload": f"{w.name}: gradients of q, k, v, z, beta, A, S0 from dL/do and "
                        f"dL/dS_T (B={w.B} H={w.H} T={w.T} d={w.dk}, bf16 in, fp32 gradients)",
            "workspace_bytes": wsb,
            "kernels": "forward rerun with 16-token checkpoints, then kda_bwd_prep, "
                       "kda_bwd_dstate, kda_bwd_part, kda_bwd_grad, kda_bwd_dA"}
    if not args.no_long:
        sections["long"] = time_long(torch, kda, 3)
    if not args.no_decode:
        wd = WORKLOADS["k3_decode_bf16"]
        dinp = make_decode_inputs(wd, device=dev)
        dms = time_decode(torch, kda, dinp, args.decode_reps)
        dbytes = decode_bytes(wd.B, wd.H, wd.dk)
        dach = dbytes / (dms * 1e-3) / 1e9
        sections["decode"] = {
            "value": wd.B * wd.H / (dms * 1e-3), "unit": "head-state-updates/s",
            "us_per_step": dms * 1e3,
            "workload": f"{wd.name}: B={wd.B} H={wd.H} d={wd.dk}, {wd.steps} steps, fp32 state",
            "roofline": {"bound": "hbm", "achieved": dach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dach / HBM_PEAK_GBS,
                         "traffic": recorded_traffic("kda_decode_kernel",
                                                     f"kda_decode_kernel_{wd.name}.md"),
                         "kernel": "kda_decode_kernel", "bytes_per_launch": dbytes}}
    # The headline is timed last: the sections above keep the GPU busy for
    # several seconds, so its W warm-up and K timed steps run at the clocks a
    # GPU under load holds, not the ramp out of idle (timed first on an idle
    # GPU, the K3 prefill reads ~25% slower for its first few hundred launches).
    ms, ms_med, ms_min = time_prefill(torch, kda, inp, args.chunk, args.steps, args.warmup)
    pbytes = prefill_bytes(w.B, w.T, w.H, w.dk)
    achieved = pbytes / (ms * 1e-3) / 1e9
    pkernel = prefill_kernel_name(args.chunk)
    ptraffic = recorded_traffic(pkernel, f"{pkernel}_{w.name}_c{args.chunk}.md")
    result = {
        "metric": METRIC,
        "value": w.B * w.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "timing": {"segments": min(SEGMENTS, args.steps), "median_ms_per_step": ms_med,
                   "min_ms_per_step": ms_min, "clock": "HIP events on the launch stream"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: KDA chunkwise prefill B={w.B} H={w.H} T={w.T} "
                               f"dk=dv={w.dk} chunk={args.chunk} bf16 in, fp32 state",
                   "B": w.B, "H": w.H, "T": w.T, "d": w.dk, "chunk": args.chunk},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": ptraffic,
                     "kernel": pkernel, "bytes_per_launch": pbytes},
    }
    # the prefill against the matrix cores as well: algorithmic flops, and the
    # MFMA flops a counter run measured (masked and duplicated tiles included)
    pflops = prefill_flops(w.B, w.T, w.H, w.dk, args.chunk)
    counted = recorded_counter(pkernel, f"{pkernel}_{w.name}_c{args.chunk}.md",
                               "mfma_flops_per_launch")
    result["mfma"] = {
        "algorithmic_flops_per_launch": pflops,
        "achieved": pflops / (ms * 1e-3) / 1e12, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
        "frac": pflops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
        "counted_flops_per_launch": counted,
        "counted_frac": (counted / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS
                         if counted is not None else None)}
    result.update(sections)
    if args.calib_mib > 0:
        calibration_copy(torch, args.calib_mib)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, inp_cpu)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
