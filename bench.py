#!/usr/bin/env python3
"""Cold-cache benchmark of the skinny decode GEMV on one MI355X (gfx950).

Headline: bf16 weights x bf16 activation, M=1, K=4096, N=12288 (100.7 MB of
weights per launch), the decode shape of "The Shape That Actually Matters"
(The shape a decode step actually runs).  Following its instrument (The
instrument came first): enough distinct weight buffers rotate per launch that
the working set (>= 2 GB) is far past the 256 MB Infinity Cache, so every
launch streams its weights from HBM; at least 1 s of warm-up on the same
rotation; then repeats of 200 timed launches, and no ratio is claimed unless
there are at least 10 repeats and their run-to-run spread is under 5%
(`config.protocol_ok`).

One step = one repeat of 200 GEMV launches, each on the next rotation buffer;
--steps repeats are timed after --warmup untimed ones (plus whatever tops the
warm-up up to 1 s).  `value` is achieved HBM GB/s = algorithmic bytes (weights
+ x + y) per launch / time per launch.  Times come from HIP events recorded on
the stream the kernels run on.  Before any workload is timed, sampled outputs
of five of its rotation buffers are checked against the CPU oracle; a failure
stops the run (no number is reported for a wrong kernel).

Further arms (same protocol): the launch floor (an empty kernel back to back,
eager and from a graph, and the streaming read at 33 MB .. 1 GiB), the
streaming-read ceiling, q8_0 / q4_0 x fp32 and q4_0 / q8_0 x Q8_1 at M=1..8
(K=4096, N=14336; fp32-activation defaults that carry the activation as one
fp16 term are timed beside the two-term kernel), the Llama-2-7B-shaped q4_0 x
Q8_1 decode layer over 32 distinct layers (plain, with the SwiGLU launch
writing Q8_1, and with the layer's RMSNorm as its own launch or writing Q8_1
itself), the fused RMSNorm -> Q8_1 launch alone, the q8_0 M=1 K=256 N=512
launch-bound case, the M=512 MFMA prefill tile (q4_0, q8_0, q4_K and q6_K
weights), and the K-quant (q4_K, q6_K super-block) weights x fp32 and x Q8_1
at the same decode shape.  The `sweep` arm (not part of `all`) times the
default of each (format, M) named by --sweep / --ms against every compiled
alternative, each gated against the oracle first.  The CPU oracle is timed on
a bounded sample of the headline workload on this host's cores.

Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 5] [--arms all|none|a,b] [--ms 1,2,4,8]
                      [--sweep q4_0_f32,...]
Prints one JSON line on stdout; per-arm details go to the --details file when
one is given.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, vendor figure
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
PEAK_INT8_TOPS = 5000.0        # MI355X dense int8 MFMA, vendor figure
ROTATION_BYTES = 2 * 1000**3   # >= 2 GB working set per arm
METRIC = "achieved HBM GB/s (% of peak) + µs per M=1 GEMV, cold-cache rotation"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_bf16_m1_k4096_n12288_hbm_traffic.md")


def counter_traffic():
    """HBM bytes per headline launch from the committed hardware-counter
    summary, or None when that summary is missing or was taken on GEMV sources
    other than the ones built now (the counters would describe another kernel)."""
    from skinny_gemm_decode_amd.rocprof_summary import gemv_source_hash
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(line.strip().split(": ", 1) for line in text.splitlines() if line.strip().startswith(
        ("traffic_bytes_per_launch:", "gemv_source_sha256:")))
    if fields.get("gemv_source_sha256") != gemv_source_hash():
        return None
    return int(fields["traffic_bytes_per_launch"])


# --------------------------------------------------------------------------
# timing helpers
# --------------------------------------------------------------------------

class Telemetry:
    """Clock levels, temperatures and power of the GPU torch uses, read from
    sysfs (the amdgpu driver's pp_dpm_* levels and hwmon sensors of the PCI
    device whose bus number torch reports).  Reading is host-side file I/O and
    puts nothing on the GPU's queues."""

    def __init__(self, torch, root: str = "/sys/class/drm"):
        import glob
        self.dev = None
        try:
            bus = int(torch.cuda.get_device_properties(0).pci_bus_id)
        except Exception:
            return
        for d in sorted(glob.glob(os.path.join(root, "card*", "device"))):
            try:
                slot = [l.split("=", 1)[1].strip() for l in open(os.path.join(d, "uevent")) if
                        l.startswith("PCI_SLOT_NAME=")][0]
            except (OSError, IndexError):
                continue
            if int(slot.split(":")[1], 16) == bus and os.path.exists(os.path.join(d, "pp_dpm_sclk")):
                self.dev, self.slot = d, slot
                self.hwmon = sorted(glob.glob(os.path.join(d, "hwmon", "hwmon*")))
                break

    @staticmethod
    def _level(path):
        try:
            for line in open(path):
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            pass
        return None

    def read(self):
        if self.dev is None:
            return None
        out = {"sclk_mhz": self._level(os.path.join(self.dev, "pp_dpm_sclk")),
               "mclk_mhz": self._level(os.path.join(self.dev, "pp_dpm_mclk"))}
        for h in self.hwmon:
            for name, key, scale in (("temp2", "t_junction_c", 1e-3), ("temp3", "t_mem_c", 1e-3),
                                     ("power1", "power_w", 1e-6)):
                f = os.path.join(h, name + "_input")
                if key not in out and os.path.exists(f):
                    try:
                        out[key] = float(open(f).read()) * scale
                    except (OSError, ValueError):
                        pass
        return out

    @staticmethod
    def summary(samples):
        samples = [s for s in samples if s]
        if not samples:
            return None
        res = {"samples": len(samples)}
        for k in ("sclk_mhz", "mclk_mhz", "t_junction_c", "t_mem_c", "power_w"):
            v = [s[k] for s in samples if s.get(k) is not None]
            if v:
                res[k] = [round(min(v), 1), round(max(v), 1)]
        return res


class Timer:
    """Times `launch(i, stream)` calls on torch's current stream with HIP events."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, launch, n_rot: int, repeats: int = 10, per_repeat: int = 200, warm_repeats: int = 0,
            warm_s: float | None = None, telemetry: Telemetry | None = None):
        """`warm_repeats` untimed repeats, topped up to at least `warm_s`
        seconds of untimed launches, then `repeats` timed repeats of
        `per_repeat` launches, each bracketed by events; launch i uses
        rotation slot i % n_rot."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        sh = stream.cuda_stream
        i = 0
        t0 = time.time()
        done = 0
        while done < warm_repeats or (warm_s is not None and time.time() - t0 < warm_s):
            for _ in range(per_repeat):
                launch(i % n_rot, sh)
                i += 1
            done += 1
            torch.cuda.synchronize()
        warm_time = time.time() - t0
        events = [torch.cuda.Event(enable_timing=True) for _ in range(repeats + 1)]
        torch.cuda.synchronize()
        samples = []
        events[0].record(stream)
        for r in range(repeats):
            for _ in range(per_repeat):
                launch(i % n_rot, sh)
                i += 1
            events[r + 1].record(stream)
            # the host runs ahead of the queue: this sample falls while earlier
            # timed launches execute, and adds no gap between them
            if telemetry is not None:
                samples.append(telemetry.read())
        torch.cuda.synchronize()
        rep_us = [events[r].elapsed_time(events[r + 1]) * 1000.0 / per_repeat for r in range(repeats)]
        total_ms = events[0].elapsed_time(events[-1])
        res = summarize(rep_us, total_ms, repeats * per_repeat)
        res.update(repeats=repeats, launches_per_repeat=per_repeat, warm_repeats=done,
                   warm_s=round(warm_time, 3))
        if telemetry is not None:
            res["telemetry_per_repeat"] = samples
            res["telemetry"] = Telemetry.summary(samples)
        return res


#: the instrument of "The Shape That Actually Matters" (The instrument came
#: first): at least 1 s of warm-up, 200 launches per repeat, 10 repeats, and no
#: ratio claimed unless the spread of the repeats is under 5%
PROTOCOL = {"min_warm_s": 1.0, "per_repeat": 200, "min_repeats": 10, "max_spread": 0.05}


def summarize(rep_us, total_ms, launches):
    """Per-launch time of a run of repeats.  spread = (max - min) / mean of
    the repeats, None with fewer than two (no spread can be claimed then)."""
    mean = statistics.fmean(rep_us)
    spread = (max(rep_us) - min(rep_us)) / mean if (len(rep_us) >= 2 and mean > 0) else None
    return {
        "us_per_launch": total_ms * 1000.0 / launches,
        "us_median": statistics.median(rep_us),
        "us_min": min(rep_us),
        "us_max": max(rep_us),
        "spread": spread,
        "spread_ok": spread is not None and spread < PROTOCOL["max_spread"],
        "repeats_us": [round(v, 4) for v in rep_us],
        "total_ms": total_ms,
    }


def protocol_ok(res) -> bool:
    """The run followed the instrument: enough warm-up, enough repeats of
    enough launches, and a spread under 5%."""
    return (res["warm_s"] >= PROTOCOL["min_warm_s"] and res["repeats"] >= PROTOCOL["min_repeats"]
            and res["launches_per_repeat"] >= PROTOCOL["per_repeat"] and res["spread_ok"])


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

def rotation_count(bytes_per_buffer: int, minimum: int = 1) -> int:
    return max(minimum, -(-ROTATION_BYTES // bytes_per_buffer))


def make_packed_rotation(skg, si, torch, kind, fmt, N, K, n_rot, seed0, keep_rows=None, keep_bufs=()):
    """n_rot packed weight buffers generated on the device; keeps host copies
    of the canonical rows `keep_rows` of the buffers `keep_bufs` (for the
    oracle gate)."""
    bufs, kept = [], {}
    idx = None if keep_rows is None else torch.as_tensor(keep_rows, device="cuda")
    for b in range(n_rot):
        W = si.torch_weights(kind, N, K, seed0 + b, "cuda")
        P = skg.pack_weights(fmt, N, K, W)
        if idx is not None and b in keep_bufs:
            kept[b] = W[idx].cpu().numpy()
        bufs.append(P)
        del W
    torch.cuda.synchronize()
    return bufs, kept


def gate_rows(N, n=24, seed=0):
    """Rows checked against the oracle before an arm is timed: both ends, the
    last workgroup's tail and a seeded sample."""
    import numpy as np
    rows = {0, 1, N - 2, N - 1} | set(range(max(0, N - 20), N))
    rows |= set(np.random.default_rng(seed).choice(N, min(n, N), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < N))


def compare_abba(timer, launch_a, launch_b, n_rot, launches, cycles=3):
    """Interleaved comparison of two launch functions: `cycles` independent
    cycles in the fixed order A1 B1 B2 A2, and the ratio B / A as the mean of
    the per-cycle ratios (the RX 6700 XT write-up, Approach & Methodology;
    "Six hypotheses, four refutations", How the agents searched: A/B/A rather
    than A/B).  Clock or temperature drift within a cycle cancels."""
    out = []
    for _ in range(cycles):
        legs = [timer.run(f, n_rot, repeats=max(1, launches // 200))["us_per_launch"]
                for f in (launch_a, launch_b, launch_b, launch_a)]
        a, b = (legs[0] + legs[3]) / 2, (legs[1] + legs[2]) / 2
        out.append({"a_us": [round(legs[0], 4), round(legs[3], 4)], "b_us": [round(legs[1], 4), round(legs[2], 4)],
                    "b_over_a": b / a})
    return {"order": "A1 B1 B2 A2", "cycles": out, "launches_per_leg": launches,
            "b_over_a": statistics.fmean(c["b_over_a"] for c in out)}


def bench_gemv_arm(skg, si, torch, timer, name, kind, fmt, M, N, K, x_host, repeats=10, warm_repeats=0,
                   warm_s=1.0, graph=False, telemetry=None, abba=0, variants=()):
    """One GEMV workload over a >= 2 GB rotation: oracle gate on sampled rows
    of five rotation buffers, then the timed repeats, the streaming read of
    the same buffers, and optionally an ABBA check against that read, graph
    replay and further kernel variants (each gated before it is timed)."""
    wbytes = skg.packed_size(fmt, N, K)
    n_rot = rotation_count(wbytes)
    log(f"[{name}] {n_rot} rotation buffers x {wbytes / 1e6:.1f} MB")
    rows = gate_rows(N, seed=M)
    keep_bufs = sorted({0, 1, 2, 3, n_rot - 1})
    bufs, kept = make_packed_rotation(skg, si, torch, kind, fmt, N, K, n_rot, seed0=1000 * (fmt + 1) + 10 * M,
                                      keep_rows=rows, keep_bufs=keep_bufs)
    x = torch.from_numpy(x_host).cuda()
    q8 = fmt in skg.Q8_1_FMTS
    if q8:
        xin = skg.quantize_act_q8_1(x)
        xbytes = xin.numel()
    else:
        xin = x
        xbytes = x.numel() * x.element_size()
    ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _ in range(2)]
    wp = [b.data_ptr() for b in bufs]
    xp, yp = xin.data_ptr(), [y.data_ptr() for y in ys]
    lib = skg.lib
    sh = torch.cuda.current_stream().cuda_stream
    idx = torch.as_tensor(rows, device="cuda")

    def launch(i, sh):
        lib.skg_gemv(fmt, M, K, N, wp[i], xp, yp[i & 1], sh)

    def gate(label):
        """Finite, deterministic on every rotation buffer, and within the
        oracle's tolerance on the sampled rows of the kept buffers."""
        outs = {}
        for i in range(n_rot):
            skg.check(lib.skg_gemv(fmt, M, K, N, wp[i], xp, yp[0], sh))
            a = ys[0].clone()
            skg.check(lib.skg_gemv(fmt, M, K, N, wp[i], xp, yp[1], sh))
            if not torch.equal(a, ys[1]):
                raise RuntimeError(f"[{label}] GEMV not deterministic on buffer {i}; refusing to time")
            if not bool(torch.isfinite(a).all()):
                raise RuntimeError(f"[{label}] non-finite GEMV output on buffer {i}; refusing to time")
            if i in kept:
                outs[i] = a[:, idx].cpu().numpy()
        xq_gpu = xin.cpu().numpy() if q8 else None
        return oracle_gate_gemv(label, kind, fmt, skg, x_host, xq_gpu, [(kept[b], outs[b]) for b in keep_bufs])

    worst = gate(name)
    res = timer.run(launch, n_rot, repeats=repeats, warm_repeats=warm_repeats, warm_s=warm_s, telemetry=telemetry)
    alg = wbytes + xbytes + M * N * 4
    res.update(name=name, fmt=skg.FMT_NAMES[fmt], M=M, N=N, K=K, rotation_buffers=n_rot,
               working_set_bytes=n_rot * wbytes, algorithmic_bytes=alg,
               gbs=alg / (res["us_per_launch"] * 1e-6) / 1e9, oracle_gate_worst_err_over_tol=worst,
               variant=skg.gemv_default_variant(fmt, M, skg.EPI_NONE, K))
    res["frac_peak"] = res["gbs"] / PEAK_HBM_GBS
    # achievable reference: the streaming-read kernel over the same buffers
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    skp = sink.data_ptr()

    def read(i, sh):
        lib.skg_stream_read(wp[i], wbytes, skp, sh)

    ceil = timer.run(read, n_rot, repeats=repeats, warm_s=0.1)
    res["ceiling_us"] = ceil["us_per_launch"]
    res["ceiling_gbs"] = wbytes / (ceil["us_per_launch"] * 1e-6) / 1e9
    res["frac_ceiling"] = ceil["us_per_launch"] / res["us_per_launch"]
    if abba:
        res["abba_vs_read"] = compare_abba(timer, launch, read, n_rot, abba)
    if graph:
        res["graph"] = bench_graph(torch, launch, n_rot)
        res["graph"]["gbs"] = alg / (res["graph"]["us_per_launch"] * 1e-6) / 1e9
    res["variants"] = []
    for v in variants:
        skg.gemv_select(v)
        try:
            vw = gate(f"{name} variant {v}")
            vr = timer.run(launch, n_rot, repeats=repeats, warm_s=0.3)
        finally:
            skg.gemv_set_variant(fmt, M, skg.EPI_NONE, 0)
        res["variants"].append({"variant": v, "us_per_launch": vr["us_per_launch"], "spread": vr["spread"],
                                "gbs": alg / (vr["us_per_launch"] * 1e-6) / 1e9,
                                "oracle_gate_worst_err_over_tol": vw})
    del bufs
    torch.cuda.empty_cache()
    return res


def bench_graph(torch, launch, n_rot, per_graph=200, repeats=10):
    """Same launches captured into a HIP graph of 200 and replayed: removes
    host launch overhead, so back-to-back kernel time shows."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):
            launch(i % n_rot, s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        for i in range(per_graph):
            launch(i % n_rot, s.cuda_stream)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(repeats + 1)]
    cur = torch.cuda.current_stream()
    ev[0].record(cur)
    for r in range(repeats):
        g.replay()
        ev[r + 1].record(cur)
    torch.cuda.synchronize()
    rep_us = [ev[r].elapsed_time(ev[r + 1]) * 1000.0 / per_graph for r in range(repeats)]
    return summarize(rep_us, ev[0].elapsed_time(ev[-1]), per_graph * repeats)


def bench_ceiling(skg, torch, timer, warm_s):
    """Streaming-read ceiling over a >= 2 GB rotation of 100.7 MB buffers."""
    nbytes = 12288 * 4096 * 2
    n_rot = rotation_count(nbytes)
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 255) for _ in range(n_rot)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    bp = [b.data_ptr() for b in bufs]
    sp = sink.data_ptr()
    sh = torch.cuda.current_stream().cuda_stream
    lib = skg.lib

    def launch(i, sh):
        lib.skg_stream_read(bp[i], nbytes, sp, sh)

    skg.check(lib.skg_stream_read(bp[0], nbytes, sp, sh))
    res = timer.run(launch, n_rot, repeats=10, warm_s=warm_s)
    res.update(name="stream_read_ceiling", bytes=nbytes, rotation_buffers=n_rot,
               gbs=nbytes / (res["us_per_launch"] * 1e-6) / 1e9)
    res["frac_peak"] = res["gbs"] / PEAK_HBM_GBS
    del bufs
    torch.cuda.empty_cache()
    return res


LAYER_MODES = {
    # name suffix, launches per layer
    "plain": ("", 5),
    "q8_1_epilogue": ("_q8_1_epilogue", 4),
    "norm_unfused": ("_rmsnorm_unfused", 6),
    "norm_fused": ("_rmsnorm_fused", 4),
    "full_unfused": ("_full_rmsnorm_unfused", 10),
    "full_fused": ("_full_rmsnorm_fused", 7),
}


def bench_layer(skg, si, torch, timer, warm_s, mode="plain"):
    """Llama-2-7B-shaped q4_0 x Q8_1 decode layer, M=1, 32 distinct layers.
    One step = one layer.
      plain (5 launches): quantize(x) -> QKV (one launch) -> gate/up + SwiGLU
        (one launch) -> quantize(h) -> down (K=11008).
      q8_1_epilogue (4): the gate/up launch also writes the Q8_1 blocks of h
        (the bits quantize(h) would write), so down reads them directly.
      norm_unfused (6): the layer's RMSNorm (per-layer gain) as its own launch
        writing fp32, then quantize -> QKV -> gate/up + SwiGLU -> quantize(h)
        -> down.
      norm_fused (4): RMSNorm writes the Q8_1 blocks of its output itself,
        then QKV -> gate/up + SwiGLU with Q8_1 output -> down.
      full_unfused (10) / full_fused (7): every weight product of the layer,
        with the 4096 x 4096 attention-output projection O and both RMSNorms
        (attention, then feed-forward).  Attention and the residual adds are
        not part of the path: O reads the Q8_1 blocks of a fixed stand-in for
        the attention output, quantised each layer, and the second norm reads
        a fixed stand-in for the residual stream."""
    suffix, launches = LAYER_MODES[mode]
    full = mode.startswith("full")
    D, F = 4096, 11008
    fmt = skg.Q4_0_Q8_1
    layers = []
    for l in range(32):
        q, k, v = (si.torch_weights("q4_0", D, D, 50_000 + 10 * l + j, "cuda") for j in range(3))
        g, u = (si.torch_weights("q4_0", F, D, 50_005 + 10 * l + j, "cuda") for j in range(2))
        d = si.torch_weights("q4_0", D, F, 50_009 + 10 * l, "cuda")
        o = si.torch_weights("q4_0", D, D, 60_000 + l, "cuda") if full else None
        gains = [torch.from_numpy(si.norm_gain_f32(si.rng_for(l, 3, 8 + j), D)).cuda() for j in range(2)]
        layers.append((skg.pack_weights_multi(fmt, [D, D, D], D, [q, k, v]),
                       skg.pack_weights_multi(fmt, [F, F], D, [g, u]),
                       skg.pack_weights(fmt, D, F, d),
                       skg.pack_weights(fmt, D, D, o) if full else None, gains))
        del q, k, v, g, u, d, o
    torch.cuda.synchronize()
    x = torch.from_numpy(si.activations_f32(si.rng_for(0, 3, 7), 1, D)).cuda()
    x2 = torch.from_numpy(si.activations_f32(si.rng_for(0, 3, 10), 1, D)).cuda()
    att = torch.from_numpy(si.activations_f32(si.rng_for(0, 3, 11), 1, D)).cuda()
    xn = torch.empty((1, D), dtype=torch.float32, device="cuda")
    xq = torch.empty((1, D // 32, 36), dtype=torch.uint8, device="cuda")
    aq = torch.empty((1, D // 32, 36), dtype=torch.uint8, device="cuda")
    yq, yk, yv, ya = (torch.empty((1, D), dtype=torch.float32, device="cuda") for _ in range(4))
    h = torch.empty((1, F), dtype=torch.float32, device="cuda")
    hq = torch.empty((1, F // 32, 36), dtype=torch.uint8, device="cuda")
    yo = torch.empty((1, D), dtype=torch.float32, device="cuda")
    import ctypes
    lib = skg.lib
    sh = torch.cuda.current_stream().cuda_stream
    N3 = (ctypes.c_int64 * 3)(D, D, D)
    N2 = (ctypes.c_int64 * 2)(F, F)
    Y3 = (ctypes.c_void_p * 3)(yq.data_ptr(), yk.data_ptr(), yv.data_ptr())
    Y1 = (ctypes.c_void_p * 1)(h.data_ptr())
    Y2 = (ctypes.c_void_p * 2)(h.data_ptr(), hq.data_ptr())
    ptrs = [(a.data_ptr(), b.data_ptr(), c.data_ptr(), o.data_ptr() if o is not None else None,
             [gn.data_ptr() for gn in gs]) for a, b, c, o, gs in layers]
    xp, x2p, attp, xnp, xqp, aqp = (t.data_ptr() for t in (x, x2, att, xn, xq, aq))
    hp, hqp, yop, yap = h.data_ptr(), hq.data_ptr(), yo.data_ptr(), ya.data_ptr()
    eps = 1e-5
    xqb, hqb = D // 32 * 36, F // 32 * 36

    # Each step: (function of (layer, stream), algorithmic bytes read + written).
    def quantize(src, dst, K, qb):
        return (lambda i, s: lib.skg_quantize_act_q8_1(1, K, src, dst, s), 4 * K + qb)

    def norm_fp32(src, j):
        return (lambda i, s: lib.skg_rmsnorm_q8_1(1, D, src, ptrs[i][4][j], eps, xnp, None, s), 3 * 4 * D)

    def norm_q8_1(src, j):
        return (lambda i, s: lib.skg_rmsnorm_q8_1(1, D, src, ptrs[i][4][j], eps, None, xqp, s), 2 * 4 * D + xqb)

    qkv = (lambda i, s: lib.skg_gemv_multi(fmt, 1, D, 3, N3, ptrs[i][0], xqp, Y3, 0, s), xqb + 3 * 4 * D)
    swiglu = (lambda i, s: lib.skg_gemv_multi(fmt, 1, D, 2, N2, ptrs[i][1], xqp, Y1, skg.EPI_SWIGLU, s),
              xqb + 4 * F)
    swiglu_q = (lambda i, s: lib.skg_gemv_multi(fmt, 1, D, 2, N2, ptrs[i][1], xqp, Y2, skg.EPI_SWIGLU_Q8_1, s),
                xqb + 4 * F + hqb)
    down = (lambda i, s: lib.skg_gemv(fmt, 1, F, D, ptrs[i][2], hqp, yop, s), hqb + 4 * D)
    oproj = (lambda i, s: lib.skg_gemv(fmt, 1, D, D, ptrs[i][3], aqp, yap, s), xqb + 4 * D)

    chains = {
        "plain": [quantize(xp, xqp, D, xqb), qkv, swiglu, quantize(hp, hqp, F, hqb), down],
        "q8_1_epilogue": [quantize(xp, xqp, D, xqb), qkv, swiglu_q, down],
        "norm_unfused": [norm_fp32(xp, 0), quantize(xnp, xqp, D, xqb), qkv, swiglu, quantize(hp, hqp, F, hqb), down],
        "norm_fused": [norm_q8_1(xp, 0), qkv, swiglu_q, down],
        "full_unfused": [norm_fp32(xp, 0), quantize(xnp, xqp, D, xqb), qkv, quantize(attp, aqp, D, xqb), oproj,
                         norm_fp32(x2p, 1), quantize(xnp, xqp, D, xqb), swiglu, quantize(hp, hqp, F, hqb), down],
        "full_fused": [norm_q8_1(xp, 0), qkv, quantize(attp, aqp, D, xqb), oproj, norm_q8_1(x2p, 1), swiglu_q,
                       down],
    }
    chain = chains[mode]
    assert len(chain) == launches
    fns = [f for f, _ in chain]

    def launch(i, sh):
        for f in fns:
            f(i, sh)

    launch(0, sh)
    torch.cuda.synchronize()
    if not bool(torch.isfinite(yo).all()) or (full and not bool(torch.isfinite(ya).all())):
        raise RuntimeError("layer chain produced non-finite output")
    res = timer.run(launch, 32, repeats=20, per_repeat=32, warm_s=warm_s)
    wbytes = (skg.packed_size_multi(fmt, [D, D, D], D) + skg.packed_size_multi(fmt, [F, F], D)
              + skg.packed_size(fmt, D, F) + (skg.packed_size(fmt, D, D) if full else 0))
    alg = wbytes + sum(b for _, b in chain)
    res.update(name="llama2_7b_q4_0_q8_1_layer" + suffix, layers=32,
               working_set_bytes=32 * (wbytes + 2 * 4 * D), weight_bytes_per_layer=wbytes,
               algorithmic_bytes=alg, launches_per_layer=launches)
    res["us_per_layer"] = res.pop("us_per_launch")
    res["gbs"] = alg / (res["us_per_layer"] * 1e-6) / 1e9
    res["frac_peak"] = res["gbs"] / PEAK_HBM_GBS
    res["graph"] = bench_graph(torch, launch, 32, per_graph=32)
    res["graph"]["gbs"] = alg / (res["graph"]["us_per_launch"] * 1e-6) / 1e9
    del layers
    torch.cuda.empty_cache()
    return res


def bench_norm(skg, si, torch, timer, warm_s, M=1, K=4096):
    """The fused RMSNorm -> Q8_1 launch alone (M x K fp32 in, Q8_1 out), over
    32 distinct inputs and gains.  Launch-bound: 2 x 16 KB in, 4.6 KB out."""
    n = 32
    xs = [torch.from_numpy(si.activations_f32(si.rng_for(i, 6, 10), M, K)).cuda() for i in range(n)]
    gs = [torch.from_numpy(si.norm_gain_f32(si.rng_for(i, 6, 11), K)).cuda() for i in range(n)]
    xq = torch.empty((M, K // 32, 36), dtype=torch.uint8, device="cuda")
    lib = skg.lib
    sh = torch.cuda.current_stream().cuda_stream
    ptrs = [(a.data_ptr(), b.data_ptr()) for a, b in zip(xs, gs)]
    qp = xq.data_ptr()

    def launch(i, sh):
        xp, gp = ptrs[i]
        lib.skg_rmsnorm_q8_1(M, K, xp, gp, 1e-5, None, qp, sh)

    skg.check(lib.skg_rmsnorm_q8_1(M, K, ptrs[0][0], ptrs[0][1], 1e-5, None, qp, sh))
    torch.cuda.synchronize()
    # gate: the same launch also writing xn, its Q8_1 blocks the oracle's
    # quantisation of that xn and xn within the RMSNorm tolerance
    xn = torch.empty((M, K), dtype=torch.float32, device="cuda")
    skg.check(lib.skg_rmsnorm_q8_1(M, K, ptrs[0][0], ptrs[0][1], 1e-5, xn.data_ptr(), qp, sh))
    oracle_gate_norm(f"rmsnorm_q8_1_m{M}_k{K}", xs[0].cpu().numpy(), gs[0].cpu().numpy(), 1e-5, xn.cpu().numpy(),
                     xq.cpu().numpy())
    res = timer.run(launch, n, repeats=10, per_repeat=200, warm_s=warm_s)
    res.update(name=f"rmsnorm_q8_1_m{M}_k{K}", algorithmic_bytes=4 * M * K + 4 * K + M * (K // 32) * 36)
    res["graph"] = bench_graph(torch, launch, n, per_graph=200)
    return res


def bench_prefill(skg, si, torch, timer, warm_s, kind="q4_0", act="bf16"):
    """The M=512 tile: bf16 activations on the bf16 matrix cores, or (act
    "q8_1") Q8_1 activation blocks on the integer matrix cores."""
    M, N, K = 512, 14336, 4096
    if act == "q8_1":
        fmt = {"q4_0": skg.Q4_0_Q8_1, "q8_0": skg.Q8_0_Q8_1}[kind]
    else:
        fmt = {"q4_0": skg.Q4_0_BF16, "q8_0": skg.Q8_0_BF16, "q4_K": skg.Q4_K_BF16, "q6_K": skg.Q6_K_BF16}[kind]
    wbytes = skg.packed_size(fmt, N, K)
    n_rot = rotation_count(wbytes)
    cols = gate_rows(N, n=40, seed=11)
    bufs, kept = make_packed_rotation(skg, si, torch, kind, fmt, N, K, n_rot, seed0=70_000, keep_rows=cols,
                                      keep_bufs=(0, n_rot - 1))
    if act == "q8_1":
        x_host = si.activations_f32(si.rng_for(0, 5, 9), M, K)
        A = skg.quantize_act_q8_1(torch.from_numpy(x_host).cuda())
        A_host = A.cpu().numpy().reshape(M, K // 32, 36)   # checked against the oracle's quantiser below
    else:
        A_host = si.activations_bf16(si.rng_for(0, 5, 9), M, K)
        A = torch.from_numpy(A_host.view("int16")).cuda()
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    lib = skg.lib
    sh = torch.cuda.current_stream().cuda_stream
    wp = [b.data_ptr() for b in bufs]
    ap, yp = A.data_ptr(), y.data_ptr()

    def launch(i, sh):
        lib.skg_gemm_tiled(fmt, M, K, N, wp[i], ap, yp, sh)

    mrows = gate_rows(M, n=24, seed=12)
    if act == "q8_1":
        import numpy as np
        import oracle
        if not np.array_equal(A_host, oracle.quantize_q8_1(x_host).reshape(A_host.shape)):
            raise RuntimeError("Q8_1 activation differs from the oracle; refusing to time")
    for b in (0, n_rot - 1):
        skg.check(lib.skg_gemm_tiled(fmt, M, K, N, wp[b], ap, yp, sh))
        torch.cuda.synchronize()
        if not bool(torch.isfinite(y).all()):
            raise RuntimeError("prefill tile produced non-finite output; refusing to time")
        oracle_gate_prefill(f"prefill_{kind}_{act} buffer {b}", kind, kept[b], A_host[mrows], act,
                            y[torch.as_tensor(mrows, device="cuda")][:, torch.as_tensor(cols, device="cuda")]
                            .cpu().numpy())
    res = timer.run(launch, n_rot, repeats=10, per_repeat=50, warm_s=warm_s)
    flops = 2.0 * M * N * K
    res.update(name=f"prefill_{kind}_{act}_m512", M=M, N=N, K=K, rotation_buffers=n_rot, flop=flops,
               tflops=flops / (res["us_per_launch"] * 1e-6) / 1e12)
    res["frac_peak_mfma_bf16"] = res["tflops"] / PEAK_BF16_TFLOPS
    if act == "q8_1":
        res["frac_peak_mfma_int8"] = res["tflops"] / PEAK_INT8_TOPS
    del bufs
    torch.cuda.empty_cache()
    return res


def bench_floor(skg, torch, timer, warm_s):
    """What every launch costs before it moves a byte, and what a plain read
    achieves per launch as the buffer grows: an empty kernel launched back to
    back (one workgroup, and the headline's grid of 6144 x 512 threads),
    eagerly and from a HIP graph, then the streaming read over rotations of
    33.0 MB, 62.4 MB, 100.7 MB and 1 GiB buffers (>= 2 GB each)."""
    lib = skg.lib
    out = {"empty": [], "read": []}
    for grid, block in ((1, 64), (6144, 512)):
        def launch(i, sh, grid=grid, block=block):
            lib.skg_empty_launch(grid, block, sh)

        skg.check(lib.skg_empty_launch(grid, block, torch.cuda.current_stream().cuda_stream))
        r = timer.run(launch, 1, repeats=10, warm_s=warm_s)
        g = bench_graph(torch, launch, 1)
        out["empty"].append({"grid": grid, "block": block, "us_per_launch": r["us_per_launch"],
                             "spread": r["spread"], "graph_us_per_launch": g["us_per_launch"]})
        log(f"[floor] empty kernel {grid} x {block}: {r['us_per_launch']:.2f} us eager, "
            f"{g['us_per_launch']:.2f} us from a graph")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for nbytes in (33_030_144, 62_390_272, 100_663_296, 1 << 30):
        n_rot = rotation_count(nbytes, minimum=2)
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n_rot)]
        for b in bufs:
            b.fill_(1)
        bp = [b.data_ptr() for b in bufs]

        def read(i, sh, nbytes=nbytes):
            lib.skg_stream_read(bp[i], nbytes, sink.data_ptr(), sh)

        r = timer.run(read, n_rot, repeats=10, per_repeat=200 if nbytes < (1 << 30) else 20, warm_s=0.2)
        out["read"].append({"bytes": nbytes, "rotation_buffers": n_rot, "us_per_launch": r["us_per_launch"],
                            "spread": r["spread"], "gbs": nbytes / (r["us_per_launch"] * 1e-6) / 1e9})
        log(f"[floor] read {nbytes / 1e6:.1f} MB: {r['us_per_launch']:.2f} us "
            f"({nbytes / (r['us_per_launch'] * 1e-6) / 1e9:.0f} GB/s)")
        del bufs
        torch.cuda.empty_cache()
    # fixed cost per launch of the read: t(bytes) - bytes / (asymptotic rate of the 1 GiB read)
    big = out["read"][-1]
    rate = big["bytes"] / big["us_per_launch"]
    for r in out["read"]:
        r["fixed_us_vs_1gib_rate"] = r["us_per_launch"] - r["bytes"] / rate
    return out


# --------------------------------------------------------------------------
# The oracle leg: the CPU oracle checks sampled outputs of every timed
# workload before it is timed (no timing on a failure), and is itself timed
# on a bounded sample of the headline workload on this host's cores.  Nothing
# else in this file touches the oracle, and the GPU path never does.
# --------------------------------------------------------------------------

def oracle_gate_gemv(label, kind, fmt, skg, x_host, xq_gpu, pairs):
    """pairs: (canonical weight rows, GPU outputs [M, rows]) per kept rotation
    buffer.  Q8_1 activations must equal the oracle's quantisation bit for
    bit; every output must lie within the oracle's tolerance.  Returns the
    worst error / tolerance; raises on any failure."""
    import numpy as np

    import oracle
    q8 = fmt in skg.Q8_1_FMTS
    if q8:
        xq_ref = oracle.quantize_q8_1(x_host)
        if not np.array_equal(xq_gpu.reshape(xq_ref.shape), xq_ref):
            raise RuntimeError(f"[{label}] Q8_1 activation differs from the oracle; refusing to time")
    worst = 0.0
    for rows_w, y_gpu in pairs:
        if kind == "bf16":
            rows_w = rows_w.view(np.uint16)
        if fmt == skg.Q4_0_Q8_1:
            y_ref, _, bound = oracle.gemv_q4_0_q8_1_ref(rows_w, xq_ref)
        elif fmt == skg.Q8_0_Q8_1:
            y_ref, bound = oracle.gemv_q8_0_q8_1_ref(rows_w, xq_ref)
        elif q8:
            y_ref, bound = oracle.gemv_ref(oracle.dequantize(kind, rows_w), oracle.decode_q8_1(xq_ref))
        else:
            x_kind = "bf16" if fmt == skg.BF16_BF16 else "f32"
            xv = x_host.view(np.uint16) if x_kind == "bf16" else x_host
            y_ref, bound = oracle.gemv_ref_fmt(kind, rows_w, xv, x_kind=x_kind)
        ok, w = oracle.check_close(y_gpu, y_ref, oracle.tolerance(bound))
        worst = max(worst, w)
        if not ok:
            raise RuntimeError(f"[{label}] GPU output outside the oracle's tolerance (worst err/tol {w:.3g}); "
                               f"refusing to time")
    return worst


def oracle_gate_prefill(label, kind, cols_w, A_rows, act, y_gpu):
    import oracle
    if act == "q8_1":
        if kind == "q4_0":
            y_ref, _, bound = oracle.gemv_q4_0_q8_1_ref(cols_w, A_rows)
        else:
            y_ref, bound = oracle.gemv_q8_0_q8_1_ref(cols_w, A_rows)
    else:
        y_ref, bound, _ = oracle.gemm_tiled_ref(cols_w, A_rows, kind)
    ok, w = oracle.check_close(y_gpu, y_ref, oracle.tolerance(bound))
    if not ok:
        raise RuntimeError(f"[{label}] outside the oracle's tolerance (worst err/tol {w:.3g}); refusing to time")
    return w


def oracle_gate_norm(label, x, g, eps, xn_gpu, xq_gpu):
    import numpy as np

    import oracle
    xn_ref = oracle.rmsnorm(x, g, eps)
    if not np.all(np.abs(xn_gpu - xn_ref) <= oracle.rmsnorm_tolerance(xn_ref)):
        raise RuntimeError(f"[{label}] RMSNorm outside the oracle's tolerance; refusing to time")
    if not np.array_equal(xq_gpu.reshape(-1), oracle.quantize_q8_1(xn_gpu).reshape(-1)):
        raise RuntimeError(f"[{label}] Q8_1 blocks differ from the oracle's quantisation; refusing to time")


def cpu_baseline(si, x_host, budget_s=12.0):
    """The oracle as it stands, timed on this host's cores on a bounded
    sample of the headline workload: whole bf16 GEMVs (exact decode to fp64,
    numpy fp64 matvec) over two generated weight buffers, repeated until about
    budget_s seconds of oracle time; generation is not timed."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    N, K = 12288, 4096
    x = x_host
    Ws = [si.bf16_weights(si.rng_for(0, 2, 100 + b), N, K) for b in range(2)]
    times = []
    while sum(times) < budget_s and len(times) < 400:
        W = Ws[len(times) % 2]
        t1 = time.perf_counter()
        oracle.gemv_ref_fmt("bf16", W, x, x_kind="bf16")
        times.append(time.perf_counter() - t1)
    per = sum(times) / len(times)
    alg = N * K * 2 + K * 2 + N * 4
    # the same GEMVs with the BLAS pool held to one thread (a few, for scale)
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            for r in range(3):
                oracle.gemv_ref_fmt("bf16", Ws[r % 2], x, x_kind="bf16")
            one = (time.perf_counter() - t1) / 3
    except ImportError:
        pass
    return {
        "value": alg / per / 1e9,
        "unit": "GB/s",
        "cores": blas_threads if blas_threads else os.cpu_count(),
        "kind": "oracle",
        "sample": (f"{len(times)} whole bf16 GEMVs M=1 K=4096 N=12288 over 2 generated weight buffers "
                   f"({sum(times):.1f} s of oracle time: exact decode to fp64, single-threaded, then numpy "
                   f"fp64 matvec on the BLAS threads given in cores); host has {os.cpu_count()} logical CPUs"),
        "us_per_gemv": per * 1e6,
        "one_blas_thread": None if one is None else {"us_per_gemv": one * 1e6, "value": alg / one / 1e9},
    }


# --------------------------------------------------------------------------

def takes_k4096(v, nb=128):
    """Whether a compiled GEMV variant handles K = 4096 (nb = 128 blocks):
    the library's own shape rules, restated for choosing what to time."""
    if v["x_lds"] in (3, 5):
        return v["waves"] * v["kw"] == nb
    if v["x_lds"] == 2:
        return nb % v["kw"] == 0 and nb <= v["waves"] * v["kw"]
    if v["x_lds"] == 4:
        return nb % 16 == 0
    if v["x_lds"] == 1 and v["kw"] > 1:
        return ((nb + 64 * v["j"] - 1) // (64 * v["j"])) % v["kw"] == 0
    return True


def sweep_variants(skg, fmt, M):
    """Every compiled plain-output variant of (fmt, M) that takes K = 4096,
    the default excluded (it is timed as the arm itself)."""
    dv = skg.gemv_default_variant(fmt, M, skg.EPI_NONE, 4096)
    seen, out = {tuple(dv[k] for k in skg.VARIANT_KEYS)}, []
    for v in skg.gemv_variants():
        key = tuple(v[k] for k in skg.VARIANT_KEYS)
        if v["fmt"] == fmt and v["M"] == M and v["epi"] == skg.EPI_NONE and takes_k4096(v) and key not in seen:
            seen.add(key)
            out.append(v)
    return out


def two_term_variants(skg, fmt, M, K=4096):
    """Compiled matrix-core variants of (fmt, M) that carry the fp32
    activation as two fp16 terms (~22 significant bits) and take K, fastest
    kind first: the LDS-ring kernel with grouped blocks, then the ring with
    one block per MFMA, the register-fed kernel and the per-wave rings."""
    vs = [v for v in skg.gemv_variants() if v["fmt"] == fmt and v["M"] == M and v["epi"] == skg.EPI_NONE
          and v["x_lds"] in (2, 3, 4, 5) and v["j"] == 2
          and (v["x_lds"] not in (3, 5) or v["waves"] * v["kw"] == K // 32)
          and (v["x_lds"] in (3, 5) or ((K // 32) % v["kw"] == 0 and K // 32 <= v["waves"] * v["kw"]))]
    order = {5: 0, 3: 1, 2: 2, 4: 3}
    return sorted(vs, key=lambda v: order[v["x_lds"]])[:1]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10,
                    help="timed steps of the headline; one step = one repeat of 200 GEMV launches")
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed warm-up steps of the headline (topped up to at least 1 s)")
    ap.add_argument("--arms", default="all", help="all, none, or a comma list of: floor,ceiling,q8_0,q4_0,q8_1,"
                                                  "multi_m,layer,small,norm,prefill,kquant,sweep (not in all)")
    ap.add_argument("--ms", default="1,2,4,8", help="activation rows M of the multi_m and sweep arms (comma list, 1..8)")
    ap.add_argument("--sweep", default="q4_0_f32",
                    help="formats of the sweep arm (comma list of names: bf16_bf16, q8_0_f32, q4_0_f32, q4_0_q8_1, "
                         "q8_0_q8_1, q4_K_f32, q6_K_f32, q4_K_q8_1, q6_K_q8_1)")
    ap.add_argument("--arm-warm-s", type=float, default=1.0, help="warm-up seconds of every further arm")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (its pre-timing parity gates still run)")
    ap.add_argument("--details", default=None, help="write the full results JSON here")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run 5 plain 256 MiB device-to-device copies (a known-size reference for "
                         "hardware traffic counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path is single-GPU "
              f"by design: no sharding or collectives).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import skinny_gemm_decode_amd as skg
    from synth import inputs as si

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")
    timer = Timer(torch)
    all_arms = {"floor", "ceiling", "q8_0", "q4_0", "q8_1", "multi_m", "layer", "small", "norm", "prefill", "kquant",
                "sweep"}
    arms = set() if args.arms == "none" else (all_arms - {"sweep"} if args.arms == "all" else set(args.arms.split(",")))
    unknown = arms - all_arms
    if unknown:
        print(f"unknown arms {sorted(unknown)}", file=sys.stderr)
        sys.exit(2)
    warm = args.arm_warm_s

    # ---- headline: bf16 M=1 K=4096 N=12288; step = 200 launches ----
    N, K = 12288, 4096
    x_host = si.activations_bf16(si.rng_for(0, 2, 0), 1, K)
    head = bench_gemv_arm(skg, si, torch, timer, "bf16_m1_k4096_n12288", "bf16", skg.BF16_BF16, 1, N, K,
                          x_host.view(np.int16), repeats=args.steps, warm_repeats=args.warmup,
                          warm_s=PROTOCOL["min_warm_s"], graph=True, telemetry=Telemetry(torch), abba=1000)
    head["protocol_ok"] = protocol_ok(head)
    if head.get("telemetry"):
        log(f"[headline] telemetry over the timed repeats: {head['telemetry']}")
    log(f"[headline] ABBA against the streaming read of the same buffers: {head['abba_vs_read']}")
    sp = "n/a" if head["spread"] is None else f"{100 * head['spread']:.2f}%"
    log(f"[headline] {head['us_per_launch']:.2f} us/launch  {head['gbs']:.0f} GB/s  "
        f"({100 * head['frac_peak']:.1f}% of 8 TB/s)  {head['repeats']} repeats of 200 after "
        f"{head['warm_s']:.2f} s warm-up, spread {sp}  graph {head['graph']['us_per_launch']:.2f} us  "
        f"read-ceiling {head['ceiling_us']:.2f} us")

    details = {"headline": head, "arms": {}}
    if "floor" in arms:
        details["arms"]["floor"] = bench_floor(skg, torch, timer, warm)
    if "ceiling" in arms:
        details["arms"]["ceiling"] = bench_ceiling(skg, torch, timer, warm)
        log(f"[ceiling] {details['arms']['ceiling']['gbs']:.0f} GB/s")
    for kind, fmt, key in (("q8_0", skg.Q8_0_F32, "q8_0"), ("q4_0", skg.Q4_0_F32, "q4_0"),
                           ("q4_0", skg.Q4_0_Q8_1, "q8_1"), ("q8_0", skg.Q8_0_Q8_1, "q8_1"),
                           ("q4_K", skg.Q4_K_F32, "kquant"), ("q6_K", skg.Q6_K_F32, "kquant"),
                           ("q4_K", skg.Q4_K_Q8_1, "kquant"), ("q6_K", skg.Q6_K_Q8_1, "kquant")):
        if key not in arms:
            continue
        Ms = tuple(int(v) for v in args.ms.split(",")) if "multi_m" in arms else (1,)
        for M in Ms:
            xh = si.activations_f32(si.rng_for(0, 4, M), M, 4096)
            # fp32-activation matrix-core defaults that round the activation to
            # one fp16 term are timed beside the two-term (~22-bit) kernel
            dv = skg.gemv_default_variant(fmt, M, skg.EPI_NONE, 4096)
            mf_f32 = fmt in (skg.Q8_0_F32, skg.Q4_0_F32, skg.Q4_K_F32, skg.Q6_K_F32)
            extra = (two_term_variants(skg, fmt, M) if mf_f32 and dv["x_lds"] in (2, 3, 5) and dv["j"] == 1 else [])
            r = bench_gemv_arm(skg, si, torch, timer, f"{skg.FMT_NAMES[fmt]}_m{M}_k4096_n14336", kind, fmt, M,
                               14336, 4096, xh, warm_s=warm, graph=True, variants=extra)
            r["activation"] = ("fp32 rounded to one fp16 term per element" if mf_f32 and dv["x_lds"] in (2, 3, 5)
                               and dv["j"] == 1 else
                               "fp32 as two fp16 terms" if mf_f32 and dv["x_lds"] in (2, 3, 5)
                               else "Q8_1" if fmt in skg.Q8_1_FMTS else "fp32")
            details["arms"][r["name"]] = r
            vs = "".join(f"  two-term {v['us_per_launch']:.2f} us" for v in r["variants"])
            log(f"[{r['name']}] {r['us_per_launch']:.2f} us  {r['gbs']:.0f} GB/s  ({r['activation']})  graph "
                f"{r['graph']['us_per_launch']:.2f} us  read-ceiling {r['ceiling_us']:.2f} us{vs}")
    if "sweep" in arms:
        # the default of each (format, M) against every compiled alternative,
        # each gated against the oracle before it is timed: how the defaults
        # were chosen, reproducible from this file
        for name in args.sweep.split(","):
            fmt = {v: k for k, v in skg.FMT_NAMES.items()}[name]
            for M in (int(v) for v in args.ms.split(",")):
                xh = si.activations_f32(si.rng_for(0, 4, M), M, 4096)
                r = bench_gemv_arm(skg, si, torch, timer, f"sweep_{name}_m{M}_k4096_n14336", skg.WEIGHT_KIND[fmt],
                                   fmt, M, 14336, 4096, xh, warm_s=warm, variants=sweep_variants(skg, fmt, M))
                details["arms"][r["name"]] = r
                log(f"[{r['name']}] default {r['variant']}: {r['us_per_launch']:.2f} us")
                for v in sorted(r["variants"], key=lambda v: v["us_per_launch"]):
                    log(f"    {v['variant']}: {v['us_per_launch']:.2f} us")
    if "small" in arms:
        xh = si.activations_f32(si.rng_for(0, 1, 0), 1, 256)
        r = bench_gemv_arm(skg, si, torch, timer, "q8_0_f32_m1_k256_n512", "q8_0", skg.Q8_0_F32, 1, 512, 256, xh,
                           warm_s=warm, graph=True)
        details["arms"][r["name"]] = r
        log(f"[{r['name']}] {r['us_per_launch']:.2f} us (graph {r['graph']['us_per_launch']:.2f} us)")
    if "norm" in arms:
        for M in (1, 8):
            r = bench_norm(skg, si, torch, timer, warm, M=M)
            details["arms"][r["name"]] = r
            log(f"[{r['name']}] {r['us_per_launch']:.2f} us (graph {r['graph']['us_per_launch']:.2f} us)")
    if "layer" in arms:
        for mode in LAYER_MODES:
            r = bench_layer(skg, si, torch, timer, warm, mode=mode)
            details["arms"][r["name"]] = r
            log(f"[{r['name']}] {r['us_per_layer']:.2f} us/layer {r['gbs']:.0f} GB/s  graph "
                f"{r['graph']['us_per_launch']:.2f} us/layer ({r['graph']['gbs']:.0f} GB/s)")
    if "prefill" in arms:
        for kind, act in (("q4_0", "bf16"), ("q8_0", "bf16"), ("q4_K", "bf16"), ("q6_K", "bf16"),
                          ("q4_0", "q8_1"), ("q8_0", "q8_1")):
            r = bench_prefill(skg, si, torch, timer, warm, kind=kind, act=act)
            details["arms"][r["name"]] = r
            log(f"[{r['name']}] {r['us_per_launch']:.1f} us  {r['tflops']:.0f} TFLOP/s "
                f"({100 * r['frac_peak_mfma_bf16']:.1f}% of bf16 peak)")

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[calibration] 5 x 256 MiB device copies")
        del src, dst

    cpu = None if args.no_cpu_baseline else cpu_baseline(si, x_host)
    if cpu:
        log(f"[cpu oracle] {cpu['value']:.2f} GB/s ({cpu['us_per_gemv']:.0f} us per GEMV, {cpu['cores']} threads)")
        if cpu["one_blas_thread"]:
            o = cpu["one_blas_thread"]
            log(f"[cpu oracle] {o['value']:.2f} GB/s ({o['us_per_gemv']:.0f} us per GEMV) with one BLAS thread")

    traffic = counter_traffic()
    floor = details["arms"].get("floor")
    line = {
        "metric": METRIC,
        "value": round(head["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_launch"] * head["launches_per_repeat"] / 1000.0,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: bf16 weights N(0,0.02), bf16 activation N(0,1), seeded; generated on device",
        "config": {
            "workload": "bf16 GEMV M=1 K=4096 N=12288, cold-cache rotation",
            "M": 1, "K": 4096, "N": 12288,
            "step": "one repeat of 200 GEMV launches, each on the next rotation buffer",
            "rotation_buffers": head["rotation_buffers"],
            "working_set_bytes": head["working_set_bytes"],
            "repeats": head["repeats"],
            "launches_per_repeat": head["launches_per_repeat"],
            "warm_s": head["warm_s"],
            "us_per_launch": round(head["us_per_launch"], 3),
            "frac_of_8TBs": round(head["frac_peak"], 4),
            "spread": None if head["spread"] is None else round(head["spread"], 4),
            "spread_ok": head["spread_ok"],
            "protocol_ok": head["protocol_ok"],
            "oracle_gate_worst_err_over_tol": round(head["oracle_gate_worst_err_over_tol"], 4),
            "stream_read_ceiling_us": round(head["ceiling_us"], 3),
            "frac_of_stream_read_ceiling": round(head["frac_ceiling"], 4),
            "stream_read_over_gemv_abba": round(head["abba_vs_read"]["b_over_a"], 4),
            "graph_us_per_launch": round(head["graph"]["us_per_launch"], 3),
            "empty_launch_us": None if floor is None else
            {f"{e['grid']}x{e['block']}": [round(e["us_per_launch"], 3), round(e["graph_us_per_launch"], 3)]
             for e in floor["empty"]},
            "timer": "HIP events on the launch stream, eager launches, 200 per repeat",
        },
        "telemetry": head.get("telemetry"),
        "roofline": {
            "bound": "hbm",
            "achieved": round(head["gbs"], 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(head["frac_peak"], 4),
            "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes": head["algorithmic_bytes"],
        },
        "cpu_baseline": None if cpu is None else {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")},
    }
    details["line"] = line
    details["cpu_baseline"] = cpu
    path = args.details
    if path:
        with open(path, "w") as f:
            json.dump(details, f, indent=1, default=lambda o: o.tolist() if hasattr(o, "tolist") else str(o))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
