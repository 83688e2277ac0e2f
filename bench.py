"""Benchmark of the hot path on one MI355X; prints ONE JSON line.

Step (the timed unit): one pass of the MLA decode hot path over the
variable-length batch -- weight absorption (q_lat = q_nope W_UK), then
mla_decode_fwd (split plan, split kernel, log-sum-exp combine) -- on
B = 256 sequences x 128 heads with cache lengths uniform in [256, 8192]
(seeded synthetic inputs, already resident in HBM).

value = KV-cache bytes read per step (sum of len_b x 1152 B) / step time,
        in GB/s (absorption included in the step time).
roofline = the decode call alone (plan + split + combine, timed with HIP
        events on the stream the library launches on) against 8 TB/s.
decode_fixed = the decode alone on 16 sequences x 4096 tokens (inputs
        rotated over 8 copies so the Infinity Cache cannot serve them).
prefill = bf16 causal prefill (B=4 H=16 N=4096 D=128) and the fp32
        vector-ALU prefill (B=4 H=8 N=8192 D=64), TFLOP/s vs their peaks.
cpu_baseline = the fp64 oracle on a bounded sample of the same decode
        workload, timed on this host's cores.
power = socket power, shader clock and energy per call of each GPU leg,
        sampled (read-only amdsmi queries) over a separate ~1 s loop of the
        leg after its timed region, and the bf16 MFMA rate this board
        sustains under its power limit (a calibration kernel of back-to-back
        MFMAs on register data, libmla_calib.so); null without amdsmi.

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 100] [--no-cpu] [--no-prefill]

Warm-up: besides the --warmup steps, every timed leg first runs its workload
for a fixed time (--warm-seconds, default 2 s for the decode and 0.5 s for
the others): the first calls after a start run slower than the steady state
(the shader clock ramps up under load), however few steps --warmup asks for.
The decode leg reports the seconds and calls it warmed up for.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6   # dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
FP32_VALU_PEAK_TFLOPS = 157.3
METRIC = "MLA decode HBM GB/s (% of peak) + prefill attention TFLOPS (% MFMA peak)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--warm-seconds", type=float, default=2.0,
                    help="time-based warm-up of the decode leg before the --warmup steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurements")
    ap.add_argument("--only", choices=["decode", "decode_fixed", "prefill_bf16", "prefill_fp32", "prefill_chunk",
                                       "copy"],
                    default=None,
                    help="run only one workload (for profiling); 'copy' is a plain 256 MiB device copy "
                         "used to calibrate the HBM byte counters")
    return ap.parse_args()


def attn_flops(B, H, N, D, causal):
    """Algorithmic FLOPs: 2 products of 2*D per visible (query, key) pair."""
    pairs = N * (N + 1) // 2 if causal else N * N
    return 4.0 * B * H * D * pairs


def warm(fn, seconds, min_calls=3):
    """Run fn until `seconds` of wall time have passed (and at least
    min_calls times); returns (seconds, calls)."""
    import torch
    t0, calls = time.perf_counter(), 0
    while True:
        fn()
        calls += 1
        if calls % 8 == 0 or calls >= min_calls:
            torch.cuda.synchronize()
            if calls >= min_calls and time.perf_counter() - t0 >= seconds:
                return time.perf_counter() - t0, calls


def time_events(fn, reps):
    import torch
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


class PowerSampler:
    """Socket power, shader clock and power-limit residency of a loop of GPU
    calls, from read-only amdsmi queries on the device that cuda:0 is
    (matched by PCI bus).  Unavailable (every result None) when amdsmi cannot
    be used.  The firmware's accumulation counter ticks once per millisecond;
    its PPT residency counter ticks in the milliseconds during which the
    package-power limiter held the clock down."""

    THERMAL = ("socket_thm_residency_acc", "vr_thm_residency_acc", "hbm_thm_residency_acc", "prochot_residency_acc")

    def __init__(self):
        self.smi = self.h = None
        self.cap_w = None
        try:
            import amdsmi
            import torch
            amdsmi.amdsmi_init()
            bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
            for h in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                if bus is None or int(bdf.split(":")[1], 16) == bus:
                    self.smi, self.h = amdsmi, h
                    break
            if self.smi is not None:
                self.cap_w = self.smi.amdsmi_get_power_cap_info(self.h)["power_cap"] / 1e6
        except Exception:
            self.smi = self.h = None

    def _counters(self):
        m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
        return (m["accumulation_counter"], m["ppt_residency_acc"], sum(m[k] for k in self.THERMAL))

    def run(self, fn, seconds=1.0, per_sync=10, settle=0.3):
        """Run fn back to back for `seconds` (after `settle` seconds) while a
        thread samples the socket power and the shader clock every 20 ms."""
        if self.smi is None:
            return None
        import threading
        import torch
        warm(fn, settle)
        samples, stop = [], threading.Event()

        def sampler():
            while not stop.is_set():
                try:
                    m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
                    samples.append((m["current_socket_power"], m["current_gfxclk"]))
                except Exception:
                    pass
                time.sleep(0.02)

        th = threading.Thread(target=sampler, daemon=True)
        try:
            c0 = self._counters()
            th.start()
            t0, calls = time.perf_counter(), 0
            while time.perf_counter() - t0 < seconds:
                for _ in range(per_sync):
                    fn()
                torch.cuda.synchronize()
                calls += per_sync
            t1 = time.perf_counter()
            stop.set()
            th.join()
            c1 = self._counters()
        except Exception:
            stop.set()
            return None
        if not samples:
            return None
        n = len(samples)
        watts = sum(p for p, _ in samples) / n
        us = (t1 - t0) / calls * 1e6
        ticks = max(c1[0] - c0[0], 1)
        return {"socket_W": round(watts, 1), "gfxclk_MHz": round(sum(c for _, c in samples) / n),
                "ppt_limited": round((c1[1] - c0[1]) / ticks, 3), "thermal_limited": round((c1[2] - c0[2]) / ticks, 3),
                "mJ_per_call": round(watts * us * 1e-3, 3), "us_per_call": round(us, 2), "calls": calls,
                "samples": n}


def mfma_ceiling(log, ps, seconds=1.5):
    """The bf16 MFMA rate this board sustains: the calibration kernel
    (back-to-back MFMAs on register data, 8 waves per CU) run for `seconds`
    per shape, with power and clock sampled meanwhile."""
    import ctypes
    import torch
    from mla_latent_kv_attn_amd import build as _b
    if ps.smi is None or not os.path.exists(_b.CALIB_LIB):
        return None
    try:
        return _mfma_ceiling(log, ps, ctypes.CDLL(_b.CALIB_LIB), seconds)
    except Exception as e:  # the calibration is context only: never fail the benchmark on it
        log(f"bf16 MFMA ceiling not measured: {e}")
        return None


def _mfma_ceiling(log, ps, lib, seconds):
    import ctypes
    import torch
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.mla_calib_mfma_rate.argtypes = [vp, vp, i, i, i, vp]
    lib.mla_calib_mfma_rate.restype = i
    g = torch.Generator().manual_seed(11)
    tables = {"N(0,1)": torch.randn(65536 * 8, generator=g).to(torch.bfloat16).to("cuda:0"),
              "zero": torch.zeros(65536 * 8, dtype=torch.bfloat16, device="cuda:0")}
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    res = {}
    for shape, flop, iters, operands in ((16, 16384, 6000, "N(0,1)"), (32, 32768, 3000, "N(0,1)"),
                                         (16, 16384, 6000, "zero")):
        table = tables[operands]

        def fn():
            r = lib.mla_calib_mfma_rate(table.data_ptr(), out.data_ptr(), blocks, iters, shape, st)
            if r != 0:
                raise RuntimeError(f"calibration launch failed: hipError {r}")
        p = ps.run(fn, seconds=seconds, per_sync=2)
        if p is None:
            return None
        tf = blocks * 4 * iters * 64 * flop / (p["us_per_call"] * 1e-6) / 1e12
        name = f"{shape}x{shape}x{512 // shape}" + ("" if operands == "N(0,1)" else " zero operands")
        res[name] = dict(TFLOP_s=round(tf, 1), frac_of_peak=round(tf / BF16_PEAK_TFLOPS, 4), operands=operands, **p)
        log(f"bf16 MFMA ceiling ({shape}x{shape}x{512 // shape}, {operands} operands, 8 waves/CU): {tf:.0f} TFLOP/s at "
            f"{p['gfxclk_MHz']} MHz, {p['socket_W']} W, power-limited {p['ppt_limited']:.0%}")
    del tables, out
    return res


def bench_decode(args, log, ps=None):
    import torch
    from mla_latent_kv_attn_amd import binding, workloads
    dev = "cuda:0"
    w = workloads.mla_varlen_workload()
    lens = w["seqlens"].tolist()
    kv_bytes = sum(lens) * 576 * 2
    q_nope, w_uk = w["q_nope"].to(dev), w["w_uk"].to(dev)
    q_rope, cache, sl = w["q_rope"].to(dev), w["cache"].to(dev), w["seqlens"].to(dev)
    B, H = 256, 128
    ns = 32
    ws = binding.alloc_decode_workspace(B, H, ns, dev)
    q_lat = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    o = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)

    def absorb():
        binding.mla_absorb_q(q_nope, w_uk, q_lat=q_lat)

    def decode():
        binding.mla_decode_fwd(q_lat, q_rope, cache, sl, w["scale"], ns, workspace=ws, o=o, lse=lse)

    def step():
        absorb()
        decode()

    # Time-based warm-up to the steady state, then the --warmup steps.
    warm_calls, t_w = 0, time.perf_counter()
    while True:
        for _ in range(50):
            step()
        torch.cuda.synchronize()
        warm_calls += 50
        if time.perf_counter() - t_w >= args.warm_seconds:
            break
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_w
    warm_calls += args.warmup
    st = torch.cuda.current_stream()
    ev = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        a, m, b = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record(st)
        absorb()
        m.record(st)
        decode()
        b.record(st)
        ev.append((a, m, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    dec_ms = [m.elapsed_time(b) for a, m, b in ev]
    abs_ms = [a.elapsed_time(m) for a, m, b in ev]
    dec_avg = sum(dec_ms) / len(dec_ms)
    abs_avg = sum(abs_ms) / len(abs_ms)
    plan = binding.read_plan(ws, B)
    log(f"decode: {ms_step:.4f} ms/step wall, decode call {dec_avg*1e3:.1f} us, absorb {abs_avg*1e3:.1f} us, "
        f"parts_used={plan['parts_used']} t={plan['t']} max_nsplit={max(plan['nsplit'])}")
    absorb_bytes = (q_nope.numel() + w_uk.numel() + q_lat.numel()) * 2
    # The value up-projection (o_v = o W_UV[h], 512 -> 128) is the step after
    # the decode; it is timed outside the step, on its own and fused with the
    # decode's merge (mla_decode_fwd_v).
    w_uv = workloads.w_uv_weights(H=H).to(dev)
    o_v = torch.empty((B, H, 128), dtype=torch.bfloat16, device=dev)
    ws_v = binding.alloc_decode_v_workspace(B, H, ns, dev)
    up = lambda: binding.mla_up_proj_v(o, w_uv, o_v=o_v)
    dec_v = lambda: binding.mla_decode_fwd_v(q_lat, q_rope, cache, sl, w_uv, w["scale"], ns, workspace=ws_v,
                                             o_v=o_v, lse=lse)

    def unfused():
        decode()
        up()

    warm(dec_v, 0.3)
    warm(unfused, 0.3)
    up_ms = sorted(time_events(up, 50))[25]
    dv_ms = sorted(time_events(dec_v, 50))[25]
    uf_ms = sorted(time_events(unfused, 50))[25]
    up_bytes = (o.numel() + w_uv.numel() + o_v.numel()) * 2
    log(f"value up-projection: {up_ms*1e3:.1f} us ({up_bytes/(up_ms*1e-3)/1e9:.0f} GB/s); decode + W_UV fused "
        f"{dv_ms*1e3:.1f} us, unfused {uf_ms*1e3:.1f} us (medians)")
    dec_sorted = sorted(dec_ms)
    power = ps.run(decode) if ps else None
    return dict(power=power, workload=w, lens=lens, kv_bytes=kv_bytes, ms_step=ms_step, dec_ms=dec_avg, abs_ms=abs_avg,
                dec_median=dec_sorted[len(dec_sorted) // 2], dec_min=dec_sorted[0],
                absorb_bytes=absorb_bytes, plan=plan, up_ms=up_ms, up_bytes=up_bytes, dv_ms=dv_ms, uf_ms=uf_ms,
                warm_s=warm_s, warm_calls=warm_calls)


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max((p.get("num_threads", 1) for p in threadpool_info()), default=1))
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_prefill_oracle(log, q, k, v, scale, causal, what, budget_s=3.0):
    """Time the prefill oracle (as it stands) on whole (b, h) slices of the
    same CPU inputs, until about budget_s of CPU time; TFLOP/s counted with
    the same algorithmic FLOPs as the GPU line."""
    import numpy as np
    import oracle
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    flops, elapsed, done = 0.0, 0.0, 0
    for i in range(B * H):
        b, h = i % B, (i * 5) % H
        qs, ks, vs = (t[b:b + 1, h:h + 1].float().numpy().astype(np.float64) for t in (q, k, v))
        t0 = time.perf_counter()
        oracle.attn_ref(qs, ks, vs, scale, causal)
        elapsed += time.perf_counter() - t0
        flops += 4.0 * D * chunk_pairs(Nq, Nk, causal)
        done += 1
        if elapsed >= budget_s:
            break
    tf = flops / elapsed / 1e12
    log(f"cpu oracle {what}: {done} (b,h) slices in {elapsed:.2f} s -> {tf*1e3:.2f} GFLOP/s")
    return {"value": round(tf, 6), "unit": "TFLOP/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{done} whole (b,h) slices of {B * H} ({Nq} queries x {Nk} keys each), float64 numpy, "
                      f"{elapsed:.1f} s"}


def bench_prefill(log, name, causal, reps=None, cpu=False, ps=None):
    import torch
    from mla_latent_kv_attn_amd import binding, workloads
    dev = "cuda:0"
    w = workloads.attn_workload(name)
    q, k, v = w["q"].to(dev), w["k"].to(dev), w["v"].to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    fn = lambda: binding.attn_fwd(q, k, v, w["scale"], causal, o=o, lse=lse)
    ws, wc = warm(fn, 0.5)
    est = ws / wc
    ms = time_events(fn, reps or max(10, min(100, int(0.2 / est))))
    avg = sum(ms) / len(ms)
    med, mn = sorted(ms)[len(ms) // 2], min(ms)
    fl = attn_flops(w["B"], w["H"], w["N"], w["D"], causal)
    tf = fl / (avg * 1e-3) / 1e12
    peak = BF16_PEAK_TFLOPS if w["dtype"] == torch.bfloat16 else FP32_VALU_PEAK_TFLOPS
    log(f"prefill {name} causal={causal}: {avg:.3f} ms, {tf:.1f} TFLOP/s ({100*tf/peak:.1f}% of {peak})")
    line = {"workload": f"{name} B={w['B']} H={w['H']} N={w['N']} D={w['D']} causal={int(causal)}",
            "ms": round(avg, 4), "ms_median": round(med, 4), "ms_min": round(mn, 4), "tflops": round(tf, 2),
            "peak_tflops": peak, "frac": round(tf / peak, 4),
            "bound": "mfma" if w["dtype"] == torch.bfloat16 else "alu"}
    if ps:
        line["power"] = ps.run(fn)
    if cpu:
        del q, k, v, o, lse
        line["cpu_oracle"] = cpu_prefill_oracle(log, w["q"], w["k"], w["v"], w["scale"], causal,
                                                f"{name} causal={int(causal)}")
    return line


def bench_decode_fixed(log, copies=8, reps=200, ps=None):
    """MLA decode on the fixed-length batch (16 sequences x 4096 tokens, 128
    heads, num_splits 32).  Its 75.5 MB cache fits in the 256 MB Infinity
    Cache, so successive calls rotate over `copies` separate copies of the
    inputs (8 x 75.5 MB > 2 x 256 MB): every call reads its cache from HBM."""
    import torch
    from mla_latent_kv_attn_amd import binding, workloads
    dev = "cuda:0"
    w = workloads.mla_fixed_workload()
    B, H = w["B"], w["H"]
    kv_bytes = int(w["seqlens"].sum()) * 576 * 2
    sets = []
    for _ in range(copies):
        sets.append(dict(q_lat=w["q_lat"].to(dev), q_rope=w["q_rope"].to(dev), cache=w["cache"].to(dev),
                         sl=w["seqlens"].to(dev), ws=binding.alloc_decode_workspace(B, H, 32, dev),
                         o=torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev),
                         lse=torch.empty((B, H), dtype=torch.float32, device=dev)))

    def call(i):
        d = sets[i % copies]
        binding.mla_decode_fwd(d["q_lat"], d["q_rope"], d["cache"], d["sl"], w["scale"], 32, workspace=d["ws"],
                               o=d["o"], lse=d["lse"])

    ctr = [0]

    def rot():
        call(ctr[0])
        ctr[0] += 1

    warm(rot, 0.5, min_calls=100)
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record(st)
        call(i)
        b.record(st)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    avg = sum(ms) / len(ms)
    gbs = kv_bytes / (avg * 1e-3) / 1e9
    log(f"decode mla_fixed (16 x 4096, rotating {copies} input copies): {avg*1e3:.1f} us, {gbs:.0f} GB/s")
    power = ps.run(rot, per_sync=50) if ps else None
    return {"power": power, "workload": "mla_fixed: B=16, H=128, 4096 tokens each, num_splits<=32, "
                        f"{copies} rotating input copies (no Infinity Cache reuse)",
            "us": round(avg * 1e3, 2), "kv_bytes": kv_bytes, "GB_s": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm",
            "traffic": measured_traffic(log, PMC_SUMMARY_FIXED)}


def chunk_pairs(Nq, Nk, causal):
    """Visible (query, key) pairs of one (b, h) for a chunk: row i sees keys
    0..i + Nk - Nq when causal, all Nk otherwise."""
    if not causal:
        return Nq * Nk
    off = Nk - Nq
    return sum(max(0, min(i + off + 1, Nk)) for i in range(Nq))


def bench_prefill_chunk(log, B=4, H=16, Nq=1024, Nk=4096, D=128, seed=1007, cpu=False):
    """bf16 prefill of a chunk of Nq new queries over Nk keys (causal, bottom-right)."""
    import torch
    from mla_latent_kv_attn_amd import binding, workloads
    dev = "cuda:0"
    qc = workloads.attn_inputs(B, H, Nq, D, torch.bfloat16, seed=seed)[0]
    _, kc, vc = workloads.attn_inputs(B, H, Nk, D, torch.bfloat16, seed=seed + 1)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    fn = lambda: binding.attn_fwd_chunk(q, k, v, 1.0 / math.sqrt(D), True, o=o, lse=lse)
    ws, wc = warm(fn, 0.5)
    ms = time_events(fn, max(10, min(100, int(0.2 * wc / ws))))
    avg = sum(ms) / len(ms)
    tf = 4.0 * D * B * H * chunk_pairs(Nq, Nk, True) / (avg * 1e-3) / 1e12
    log(f"prefill chunk bf16 Nq={Nq} Nk={Nk}: {avg:.3f} ms, {tf:.1f} TFLOP/s ({100*tf/BF16_PEAK_TFLOPS:.1f}%)")
    line = {"workload": f"attn_fwd_chunk bf16 B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal=1 (bottom-right)",
            "ms": round(avg, 4), "tflops": round(tf, 2), "peak_tflops": BF16_PEAK_TFLOPS,
            "frac": round(tf / BF16_PEAK_TFLOPS, 4), "bound": "mfma"}
    if cpu:
        del q, k, v, o, lse
        line["cpu_oracle"] = cpu_prefill_oracle(log, qc, kc, vc, 1.0 / math.sqrt(D), True, "chunk")
    return line


# The decode kernels, their plan layout, and the host code that sets the plan
# constants (the split count, and with it the partial traffic, depends on them).
DECODE_SOURCES = ("mla_latent_kv_attn_amd/csrc/mla_decode.hip", "mla_latent_kv_attn_amd/csrc/mla_plan.h",
                  "mla_latent_kv_attn_amd/csrc/mla_merge.h", "mla_latent_kv_attn_amd/csrc/common.h",
                  "mla_latent_kv_attn_amd/csrc/api.hip")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "mla_decode_varlen_pmc.json")
PMC_SUMMARY_FIXED = os.path.join(ROOT, "profiles", "mla_decode_fixed_pmc.json")


def sources_sha():
    """SHA-256 over every library source (csrc/* and the C header), in name
    order; the kernel-stats summaries under profiles/ state the same hash."""
    import glob
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "mla_latent_kv_attn_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "mla_attn.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def decode_sources_sha():
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(log, path=PMC_SUMMARY):
    """HBM bytes per decode call from a committed counter summary, or None
    when it was taken on different kernel sources than the ones built here."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != decode_sources_sha():
        log("traffic: counter summary is stale (kernel sources changed); reporting null")
        return None
    return rec.get("hbm_bytes_per_call")


def plain_copy():
    import torch
    n = 256 << 20
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {n} bytes 3 times", file=sys.stderr, flush=True)


def copy_bandwidth(log, nbytes=1 << 30, reps=20, ps=None):
    """Attainable HBM rate of a plain device copy (context for the roofline):
    bytes read + bytes written per copy / time."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    ms = time_events(lambda: b.copy_(a), reps)
    avg = sum(ms) / len(ms)
    gbs = 2 * nbytes / (avg * 1e-3) / 1e9
    log(f"device copy of {nbytes >> 20} MiB: {avg*1e3:.1f} us, {gbs:.0f} GB/s (read + write)")
    power = ps.run(lambda: b.copy_(a), per_sync=4) if ps else None
    del a, b
    return round(gbs, 1), power


def cpu_baseline(d, log, budget_s=12.0):
    """Time the oracle (as it stands) on a bounded sample of the decode workload."""
    import numpy as np
    import oracle
    w = d["workload"]
    lens = d["lens"]
    w_uk64 = w["w_uk"].float().numpy().astype(np.float64)     # input conversion, outside the timing
    done, tbytes, elapsed = 0, 0, 0.0
    for b in range(len(lens)):
        L = lens[b]
        qn = w["q_nope"][b:b + 1].float().numpy()
        qr = w["q_rope"][b:b + 1].float().numpy()
        cb = w["cache"][b:b + 1, :L].float().numpy()
        t0 = time.perf_counter()
        ql64 = oracle.absorb_ref(qn, w_uk64)
        oracle.mla_decode_ref(ql64, qr, cb, [L], w["scale"])
        elapsed += time.perf_counter() - t0
        done += 1
        tbytes += L * 1152
        if elapsed >= budget_s:
            break
    cores = cpu_threads()
    gbs = tbytes / elapsed / 1e9
    log(f"cpu oracle: {done} sequences, {tbytes/1e6:.1f} MB of cache in {elapsed:.2f} s -> {gbs:.3f} GB/s")
    # The explicit-decompression check on a sample (4 sequences x 128 heads x
    # their first 256 tokens): decode through decompressed keys against the
    # absorbed decode, both in the oracle, timed separately.
    qn = w["q_nope"][:4].float().numpy()
    qr = w["q_rope"][:4].float().numpy()
    cb = w["cache"][:4, :256].float().numpy()
    sl = [min(256, lens[b]) for b in range(4)]
    t0 = time.perf_counter()
    o_exp, l_exp = oracle.mla_decode_explicit_ref(qn, qr, w_uk64, cb, sl, w["scale"])
    t_exp = time.perf_counter() - t0
    t0 = time.perf_counter()
    o_abs, l_abs = oracle.mla_decode_ref(oracle.absorb_ref(qn, w_uk64), qr, cb, sl, w["scale"])
    t_abs = time.perf_counter() - t0
    diff = float(np.abs(o_exp - o_abs).max())
    log(f"cpu oracle decompression check (4 seqs x 128 heads x 256 tokens): explicit {t_exp:.3f} s, "
        f"absorbed {t_abs:.3f} s, max |dO| {diff:.2e}")
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": model,
            "sample": f"first {done} of 256 sequences of the decode workload ({tbytes} cache bytes), "
                      f"absorption + decode in float64 numpy, {elapsed:.1f} s",
            "decompression_check": {"sample": "4 sequences x 128 heads x first 256 tokens",
                                    "explicit_s": round(t_exp, 4), "absorbed_s": round(t_abs, 4),
                                    "max_abs_diff_O": diff}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    log = lambda s: print(s, file=sys.stderr, flush=True)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.only == "copy":
        plain_copy()
        return
    if args.only == "prefill_bf16":
        bench_prefill(log, "attn_bf16", True, reps=args.steps)
        return
    if args.only == "prefill_chunk":
        bench_prefill_chunk(log)
        return
    if args.only == "decode_fixed":
        bench_decode_fixed(log)
        return
    if args.only == "prefill_fp32":
        bench_prefill(log, "attn_fp32", False, reps=args.steps)
        return
    ps = None if args.only == "decode" else PowerSampler()
    d = bench_decode(args, log, ps)
    if args.only == "decode":
        return
    decode_fixed = bench_decode_fixed(log, ps=ps)
    copy_gbs, copy_power = copy_bandwidth(log, ps=ps)
    prefill = {}
    if not args.no_prefill:
        cpu = not args.no_cpu
        prefill["bf16_causal"] = bench_prefill(log, "attn_bf16", True, cpu=cpu, ps=ps)
        prefill["fp32_noncausal"] = bench_prefill(log, "attn_fp32", False, reps=5, cpu=cpu)
        prefill["fp32_causal"] = bench_prefill(log, "attn_fp32", True, reps=5, cpu=cpu)
        prefill["bf16_chunk"] = bench_prefill_chunk(log, cpu=cpu)
    ceiling = mfma_ceiling(log, ps)
    if ceiling and "32x32x16" in ceiling:
        # The bf16 prefill kernels issue 32x32x16 MFMAs: their rate against what
        # the calibration loop of that shape sustains on this board.
        top = ceiling["32x32x16"]["TFLOP_s"]
        for key in ("bf16_causal", "bf16_chunk"):
            if key in prefill:
                prefill[key]["frac_of_mfma_loop"] = round(prefill[key]["tflops"] / top, 4)
    power = None
    if ps.smi is not None:
        power = {"cap_W": ps.cap_w, "decode": d["power"], "decode_fixed": decode_fixed.pop("power"),
                 "bf16_causal": prefill.get("bf16_causal", {}).pop("power", None), "copy": copy_power,
                 "mfma_bf16_ceiling": ceiling,
                 "note": "each leg re-run for ~1 s after its timed region; socket power and shader clock "
                         "sampled every 20 ms (amdsmi, read-only); ppt_limited = share of the firmware's 1 ms "
                         "ticks in which the package-power limiter was active; mJ_per_call = socket_W x "
                         "us_per_call"}
    else:
        decode_fixed.pop("power", None)
        prefill.get("bf16_causal", {}).pop("power", None)
    cpu = None if args.no_cpu else cpu_baseline(d, log)
    value = d["kv_bytes"] / (d["ms_step"] * 1e-3) / 1e9
    achieved = d["kv_bytes"] / (d["dec_ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mla_varlen: MLA absorbed decode, B=256, H=128, 1 query token, latent cache "
                               "576 bf16/token, lengths uniform [256,8192] (seed 1005), num_splits<=32, "
                               "step = absorption q_nope[256,128,128] @ W_UK[128,128,512] + decode",
                   "global_batch": 256, "seq_len": "256..8192 (sum %d)" % sum(d["lens"]),
                   "kv_bytes_per_step": d["kv_bytes"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "mla_decode_fwd (plan + split + combine kernels)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(log),
                     "decode_us": round(d["dec_ms"] * 1e3, 2), "decode_us_median": round(d["dec_median"] * 1e3, 2),
                     "decode_us_min": round(d["dec_min"] * 1e3, 2), "absorb_us": round(d["abs_ms"] * 1e3, 2),
                     "warmup_s": round(d["warm_s"], 2), "warmup_calls": d["warm_calls"],
                     "attainable_copy_GB_s": copy_gbs},
        "value_up_projection": {"workload": "o [256,128,512] @ W_UV [128,512,128] -> [256,128,128] bf16",
                                "us": round(d["up_ms"] * 1e3, 2),
                                "GB_s": round(d["up_bytes"] / (d["up_ms"] * 1e-3) / 1e9, 1),
                                "decode_v_fused_us": round(d["dv_ms"] * 1e3, 2),
                                "decode_then_up_proj_us": round(d["uf_ms"] * 1e3, 2),
                                "fused_GB_s": round(d["kv_bytes"] / (d["dv_ms"] * 1e-3) / 1e9, 1),
                                "note": "timed after the step (medians), not part of value; fused = "
                                        "mla_decode_fwd_v (merge + W_UV in one kernel)"},
        "sources_sha256": sources_sha(),
        "cpu_baseline": cpu,
        "decode_fixed": decode_fixed,
        "prefill": prefill,
        "power": power,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
