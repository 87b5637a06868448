"""Benchmark: W4/W2 GEMV effective HBM GB/s (% of peak) + M=2048 GEMM TFLOPS.

Headline workload (the `value`): one decode step of the four Llama-3-8B
linear shapes (N x K = 14336x4096 up/gate, 4096x14336 down, 4096x4096 q/o,
1024x4096 k/v), weights INT4 with groups of 128, M = 1 bf16 activation row.
A step is one grouped decode call (gq_linear_group) over the four linears;
value = algorithmic bytes of the step (packed codes + fp16 scales + uint8
zeros + x + y) / step time.  Weights are resident in HBM and 16 copies are
rotated (1.16 GB) so the 256 MB Infinity Cache cannot serve them.  Steps
run as replays of a captured HIP graph.

The same JSON line carries:
  roofline      the step's dominant launch (the grouped kernel over the
                three K = 4096 linears; the down projection's longer rows
                run in a second launch), bytes per launch / average launch
                time (HIP events around rotating graph replays on the
                launching stream), against 8 TB/s HBM; traffic from
                committed rocprofv3 PMC counters when they were taken on the
                current kernel source.
  cpu_baseline  the CPU oracle (the tests' reference implementation) timed on
                a bounded sample of the same workload on this host, BLAS on
                every core the process may use; plus a quantize+pack sample.
  secondary     the same step as four single-linear launches, the INT2 step,
                INT2 M=4/16, the 224-linear Layer-mix pass (one grouped call
                and a 224-launch graph), streaming ceilings of black-box torch
                kernels, the Channel-mix M=2048 GEMMs (TFLOPS vs 2.5 PFLOP/s
                bf16/fp16 dense), quantize+pack and fake quantization, dX,
                and KV-cache decode attention.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 / fp16
WARM_SECONDS = 0.1          # sustained replays before each secondary measurement
METRIC = "W4/W2 GEMV effective HBM GB/s (% of peak) + M=2048 GEMM TFLOPS"
PMC_FILE = os.path.join(ROOT, "profiles", "gemv_group_int4_decode_pmc.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=2048,
                    help="untimed steps first (2048 steps, ~40 ms: past the GPU's power ramp)")
    ap.add_argument("--copies", type=int, default=16, help="rotated weight copies (defeat MALL)")
    ap.add_argument("--bits", type=int, default=4, choices=(4, 2),
                    help="weight width of the headline decode step (4 is the headline; 2 runs the "
                         "INT2 g64 step alone, for counter runs)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--gemm-only", action="store_true",
                    help="only the Channel-mix M=2048 GEMM measurements (for counter runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=3)
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run a plain 256 MiB device copy (PMC byte-counter calibration)")
    return ap.parse_args()


def decode_bytes(N, K, bits, M):
    g = 128 if bits == 4 else 64
    return N * K * bits // 8 + (N * K // g) * 3 + 2 * M * K + 2 * M * N


def decode_step_bytes(bits, M=1):
    """Algorithmic bytes of the four-linear Llama-3-8B decode step."""
    import synth as S
    return sum(decode_bytes(N, K, bits, M) for (N, K) in S.LLAMA3_8B_SHAPE_LIST)


# ----------------------------------------------------------------- timing

class GraphTimer:
    """Capture a list of launches into one HIP graph and time replays with
    HIP events recorded on the stream the library launches on."""

    def __init__(self, torch, fn):
        self.torch = torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()                                    # warm: loads code objects
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            fn()
        torch.cuda.synchronize()

    def warm(self, seconds=None):
        """Replay for `seconds` of wall time.  Bandwidth-heavy work on this
        GPU runs up to 20% slower for its first 20-30 ms after an idle spell
        (the power state ramps with load), so each measurement starts from
        sustained load."""
        t = self.torch
        seconds = WARM_SECONDS if seconds is None else seconds
        w0 = time.perf_counter()
        while time.perf_counter() - w0 < seconds:
            self.g.replay()
            t.cuda.synchronize()

    def run(self, reps):
        t = self.torch
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record()
        for _ in range(reps):
            self.g.replay()
        e1.record()
        t.cuda.synchronize()
        wall = time.perf_counter() - w0
        return e0.elapsed_time(e1) / 1e3, wall


def rotated_copies(torch, gq, packed, copies):
    out = [packed]
    for _ in range(copies - 1):
        q = gq.Packed(packed.K, packed.N, packed.block_n, packed.bits, packed.codes.clone(),
                      packed.scales.clone(), packed.zeros.clone(), packed.flags.clone())
        out.append(q)
    return out


# ------------------------------------------------------------- workloads

def build_decode(torch, gq, S, bits, M, copies):
    """Packed Llama-3-8B decode linears (seeded), copies rotated."""
    sets, xs, ys, nbytes = [], [], [], 0
    for j, (N, K) in enumerate(S.LLAMA3_8B_SHAPE_LIST):
        W = torch.from_numpy(S.decode_weight(j)).cuda()
        p = gq.quantize_pack(W, bits)
        del W
        sets.append(rotated_copies(torch, gq, p, copies))
        x = torch.from_numpy(S.decode_x(j, M).view(np.int16)).cuda().view(torch.bfloat16)
        xs.append(x)
        ys.append(torch.empty((M, N), dtype=torch.bfloat16, device="cuda"))
        nbytes += decode_bytes(N, K, bits, M)
    torch.cuda.synchronize()
    return sets, xs, ys, nbytes


def decode_pass(gq, sets, xs, ys, c, shapes=None):
    for j in (range(len(sets)) if shapes is None else shapes):
        gq.linear(xs[j], sets[j][c], out=ys[j])


def group_plans(gq, sets, xs, ys, copies, shapes=(0, 1, 2, 3)):
    """One grouped-decode plan per rotated copy of the step's linears."""
    return [gq.group_plan([(xs[j], sets[j][c], ys[j]) for j in shapes]) for c in range(copies)]


def time_steps(torch, gq, sets, xs, ys, copies, steps, warmup, plans=None):
    """Time exactly `steps` decode steps (graph of `copies` steps + remainder);
    a step is one grouped call when plans are given, else one gq_linear per
    linear."""
    if plans is not None:
        step = lambda c: gq.linear_group(plans[c])
    else:
        step = lambda c: decode_pass(gq, sets, xs, ys, c)
    full = GraphTimer(torch, lambda: [step(c) for c in range(copies)])
    single = [GraphTimer(torch, lambda c=c: step(c)) for c in range(copies)]

    def run(n):
        t = torch
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record()
        for _ in range(n // copies):
            full.g.replay()
        for c in range(n % copies):
            single[c].g.replay()
        e1.record()
        t.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3, time.perf_counter() - w0

    run(warmup)
    return run(steps)


def kernel_avg(torch, gq, sets, xs, ys, j, copies, reps=40):
    """Average duration of one linear's launch (rotating copies)."""
    gt = GraphTimer(torch, lambda: [gq.linear(xs[j], sets[j][c], out=ys[j]) for c in range(copies)])
    gt.warm()
    t, _ = gt.run(reps)
    return t / (reps * copies)


def group_avg(torch, gq, plans, reps=40):
    """Average duration of one grouped call (rotating plans)."""
    gt = GraphTimer(torch, lambda: [gq.linear_group(p) for p in plans])
    gt.warm()
    t, _ = gt.run(reps)
    return t / (reps * len(plans))


def ceilings(torch):
    """Streaming rates of black-box torch kernels on this GPU, as context for
    the fractions of 8 TB/s: a float32 sum (reads the buffer once) and a
    device copy (reads and writes it), over 1 GB and over 30 MB buffers
    (the 30 MB case rotates 36 buffers, 1.08 GB, past the Infinity Cache)."""
    out = {}
    for label, nbytes, count in (("1GB", 1 << 30, 1), ("30MB", 30 << 20, 36)):
        bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda") for _ in range(count)]
        dsts = [torch.empty_like(b) for b in bufs]
        acc = torch.empty((), dtype=torch.float32, device="cuda")
        reps = 20 if count == 1 else 2
        st = GraphTimer(torch, lambda: [torch.sum(b, dim=0, out=acc) for b in bufs])
        st.warm()
        t, _ = st.run(reps)
        ct = GraphTimer(torch, lambda: [d.copy_(b) for b, d in zip(bufs, dsts)])
        ct.warm()
        tc, _ = ct.run(reps)
        n = reps * count
        out[f"torch_sum_read_{label}"] = {"GBps": round(nbytes * n / t / 1e9, 1),
                                          "frac_hbm": round(nbytes * n / t / 1e9 / HBM_PEAK_GBS, 3),
                                          "us_per_call": round(t / n * 1e6, 2)}
        out[f"torch_copy_read_write_{label}"] = {"GBps": round(2 * nbytes * n / tc / 1e9, 1),
                                                 "frac_hbm": round(2 * nbytes * n / tc / 1e9 / HBM_PEAK_GBS, 3),
                                                 "us_per_call": round(tc / n * 1e6, 2)}
        del bufs, dsts
        torch.cuda.empty_cache()
    return out


def read_ceiling(torch):
    """The plain streaming-read probe (libgq_probe.so: 128-bit nontemporal
    loads, one launch, no arithmetic) at the byte counts of the INT4 and INT2
    decode steps and at 1 GB: what one launch moving the same bytes gets
    from this GPU, ramp and drain included.  Buffers rotate past the
    Infinity Cache like the decode step's weight copies."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "quantized_gemm_groupwise_amd", "libgq_probe.so"))
    fn = lib.gqprobe_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    out = {}
    for label, nbytes, count in (("int4_decode_step_bytes", decode_step_bytes(4), 16),
                                 ("int2_decode_step_bytes", decode_step_bytes(2), 16),
                                 ("1GB", 1 << 30, 2)):
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(count)]

        def one():
            for b in bufs:
                st = fn(b.data_ptr(), nbytes, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
                if st != 0:
                    raise RuntimeError(f"gqprobe_stream_read: {st}")
        gt = GraphTimer(torch, one)
        gt.warm()
        reps = 50 if count > 2 else 20
        t, _ = gt.run(reps)
        n = reps * count
        out[label] = {"bytes": nbytes, "us": round(t / n * 1e6, 2), "GBps": round(nbytes * n / t / 1e9, 1),
                      "frac_hbm": round(nbytes * n / t / 1e9 / HBM_PEAK_GBS, 3)}
        del bufs
        torch.cuda.empty_cache()
    return out


def pmc_traffic():
    """Calibrated HBM bytes per launch from the committed PMC summary, if the
    kernel source it was taken on is the current one."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    from quantized_gemm_groupwise_amd.rocprof import source_digest
    if d.get("source_digest") != source_digest():
        return None
    return d.get("traffic_bytes_per_launch")


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        for lib in threadpool_info():
            if lib.get("user_api") == "blas":
                blas = f"{lib.get('internal_api')} {lib.get('version')} ({lib.get('threading_layer')})"
                break
    except ImportError:  # pragma: no cover
        pass
    return model, blas


def cpu_baseline(S, nsteps, gpu_value):
    """The oracle timed on this host: the decode step (unpack, fp64 dequant,
    fp64 matmul with BLAS on every core the process may use) and, apart, a
    sample of the Channel-mix quantize+pack (single-process numpy)."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    prep = []
    nbytes = 0
    for j, (N, K) in enumerate(S.LLAMA3_8B_SHAPE_LIST):
        p = O.quantize_pack(S.decode_weight(j), O.Layout(K, N, N, [4]))
        prep.append((S.decode_x(j, 1), p))
        nbytes += decode_bytes(N, K, 4, 1)
    ctx = threadpool_limits(cores) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        for _ in range(nsteps):
            for x, p in prep:
                O.linear(x, p)
        dt = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    value = nbytes * nsteps / dt / 1e9
    # quantize+pack: 1024 rows of the 28672 x 8192 Channel-mix matrix (8 blocks)
    W, bits = S.channel_mix_weight(0)
    rows = 1024
    Ws = np.ascontiguousarray(W[:rows])
    del W
    lay = O.Layout(Ws.shape[1], rows, 128, bits[: rows // 128])
    tq = time.perf_counter()
    qp = O.quantize_pack(Ws, lay)
    tq = time.perf_counter() - tq
    qbytes = Ws.nbytes + qp.codes.nbytes + qp.scales.nbytes + qp.zeros.nbytes
    model, blas = cpu_info()
    return {"value": round(value, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{nsteps} decode steps (4 INT4 g128 Llama-3-8B linears, M=1) through "
                      f"oracle.linear (unpack, fp64 dequant, fp64 matmul), {dt:.1f} s, BLAS on "
                      f"{cores} threads",
            "cpu_model": model, "blas": blas,
            "gpu_over_cpu": round(gpu_value / value, 1),
            "quantize_pack": {"GBps": round(qbytes / tq / 1e9, 4), "cores": 1, "seconds": round(tq, 2),
                              "sample": f"oracle.quantize_pack of {rows} x 8192 fp32 rows of the "
                                        "28672 x 8192 Channel-mix matrix (numpy, one process)"}}


def secondary(torch, gq, S, args):
    out = {}
    # INT2 decode step (M=1) and INT2 M=4/16 on up/gate
    copies2 = 32
    sets, xs, ys, nb = build_decode(torch, gq, S, 2, 1, copies2)
    plans = group_plans(gq, sets, xs, ys, copies2)
    t, _ = time_steps(torch, gq, sets, xs, ys, copies2, 256, 32, plans=plans)
    tl, _ = time_steps(torch, gq, sets, xs, ys, copies2, 256, 32)
    out["int2_decode_step_M1"] = {"GBps": round(nb * 256 / t / 1e9, 1),
                                  "frac_hbm": round(nb * 256 / t / 1e9 / HBM_PEAK_GBS, 3),
                                  "us_per_step": round(t / 256 * 1e6, 2), "bytes_per_step": nb,
                                  "launch": "one grouped call (gq_linear_group)"}
    out["int2_decode_step_M1_per_linear"] = {"GBps": round(nb * 256 / tl / 1e9, 1),
                                             "frac_hbm": round(nb * 256 / tl / 1e9 / HBM_PEAK_GBS, 3),
                                             "us_per_step": round(tl / 256 * 1e6, 2),
                                             "launch": "four gq_linear calls"}
    del plans
    per = {}
    for j, name in enumerate(("up_gate", "down", "q_o", "k_v")):
        N, K = S.LLAMA3_8B_SHAPE_LIST[j]
        avg = kernel_avg(torch, gq, sets, xs, ys, j, copies2, reps=10)
        per[name] = {"us": round(avg * 1e6, 2), "GBps": round(decode_bytes(N, K, 2, 1) / avg / 1e9, 1)}
    out["int2_M1_per_linear"] = per
    del sets, xs, ys
    for M in (4, 16):
        N, K = S.LLAMA3_8B_SHAPE_LIST[0]
        W = torch.from_numpy(S.decode_weight(0)).cuda()
        p = gq.quantize_pack(W, 2)
        del W
        cps = rotated_copies(torch, gq, p, copies2)
        x = torch.from_numpy(S.decode_x(0, M).view(np.int16)).cuda().view(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        avg = kernel_avg(torch, gq, [cps], [x], [y], 0, copies2, reps=10)
        b = decode_bytes(N, K, 2, M)
        out[f"int2_upgate_M{M}"] = {"us": round(avg * 1e6, 2), "GBps": round(b / avg / 1e9, 1),
                                    "frac_hbm": round(b / avg / 1e9 / HBM_PEAK_GBS, 3)}
        del cps, x, y
    torch.cuda.empty_cache()

    # Layer-mix pass: 224 linears, seeded per-linear INT4/INT2, M in {1, 8, 32}
    assign = S.layer_mix_assignment()
    packs, pbytes, n4 = [], 0, 0
    gen = torch.Generator(device="cuda")
    for (l, name, N, K, bits) in assign:
        gen.manual_seed(4000 + len(packs))
        W = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
        idx = torch.randperm(K, generator=gen, device="cuda")[: int(round(0.005 * K))]
        W[:, idx] *= 20.0
        p = gq.quantize_pack(W, bits)
        del W
        packs.append(p)
        pbytes += p.nbytes()
        n4 += bits == 4
    torch.cuda.synchronize()
    params = sum(N * K for (_, _, N, K, _) in assign)
    lm = {"linears": len(assign), "int4_linears": n4, "bpw": round(pbytes * 8 / params, 4),
          "packed_bytes": pbytes,
          "weights": "drawn on the GPU with torch's generator (normal, sigma 0.02, 0.5% of input "
                     "channels x20: the decode recipe's distribution, not its values; timing does "
                     "not depend on the values)"}
    lg = dict(lm)
    for M in (1, 2, 4):
        xs = {K: torch.from_numpy(S.layer_mix_x(K, M).view(np.int16)).cuda().view(torch.bfloat16)
              for K in (4096, 14336)}
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for (_, _, N, K, _) in assign]
        plan = gq.group_plan([(xs[p.K], p, y) for p, y in zip(packs, ys)])
        gt = GraphTimer(torch, lambda: gq.linear_group(plan))
        gt.warm()
        t, _ = gt.run(10)
        b = pbytes + sum(2 * M * K + 2 * M * N for (_, _, N, K, _) in assign)
        lg[f"M{M}"] = {"ms_per_pass": round(t / 10 * 1e3, 4), "GBps": round(b * 10 / t / 1e9, 1),
                       "frac_hbm": round(b * 10 / t / 1e9 / HBM_PEAK_GBS, 3)}
        del ys, xs, plan
    out["layer_mix_pass_grouped"] = lg
    for M in (1, 8, 32):
        xs = {K: torch.from_numpy(S.layer_mix_x(K, M).view(np.int16)).cuda().view(torch.bfloat16)
              for K in (4096, 14336)}
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for (_, _, N, K, _) in assign]
        ws = gq.workspace(max(gq.gq_linear_workspace_bytes(p.layout, M) for p in packs) + 256, "cuda")

        def one_pass():
            for p, y in zip(packs, ys):
                gq.linear(xs[p.K], p, out=y, ws=ws)
        gt = GraphTimer(torch, one_pass)
        gt.warm()
        t, _ = gt.run(10)
        b = pbytes + sum(2 * M * K + 2 * M * N for (_, _, N, K, _) in assign)
        lm[f"M{M}"] = {"ms_per_pass": round(t / 10 * 1e3, 4), "GBps": round(b * 10 / t / 1e9, 1),
                       "frac_hbm": round(b * 10 / t / 1e9 / HBM_PEAK_GBS, 3)}
        del ys, xs
    out["layer_mix_pass_graph"] = lm
    del packs
    torch.cuda.empty_cache()
    out["streaming_ceilings"] = ceilings(torch)
    out["read_ceiling"] = read_ceiling(torch)

    out.update(channel_mix(torch, gq, S))
    out.update(kv_decode(torch, gq))
    return out


def kv_decode(torch, gq):
    """One decode step of attention over a group-wise quantized KV cache:
    Llama-3-8B heads (32 query, 8 key/value, dim 128), the newest 128 tokens
    of a 32768-token context in a dense bf16 window and the rest packed INT4
    g128 or INT2 g64; and 32 sequences of 2048 tokens (64 in the window);
    and the 32768-token INT4 step with Llama-3-70B heads (64 query, 8
    key/value: 8 query heads per key/value head).
    Bytes: packed K and V (codes, scales, zeros), the window, q and out."""
    out = {}
    Hkv = 8
    for name, B, tp, tw, bits, Hq in [("kv_decode_32k_int4", 1, 32640, 128, 4, 32),
                                      ("kv_decode_32k_int2", 1, 32640, 128, 2, 32),
                                      ("kv_decode_b32_2k_int4", 32, 1984, 64, 4, 32),
                                      ("kv_decode_32k_int4_70b_heads", 1, 32640, 128, 4, 64)]:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(7000 + B + bits)
        k = torch.randn((B * tp, Hkv * 128), generator=gen, device="cuda")
        v = torch.randn((B * tp, Hkv * 128), generator=gen, device="cuda")
        kp, vp = gq.quantize_pack(k, bits), gq.quantize_pack(v, bits)
        del k, v
        kw = torch.randn((B, tw, Hkv, 128), generator=gen, device="cuda").to(torch.bfloat16)
        vw = torch.randn((B, tw, Hkv, 128), generator=gen, device="cuda").to(torch.bfloat16)
        q = torch.randn((B, Hq, 128), generator=gen, device="cuda").to(torch.bfloat16)
        o = torch.empty_like(q)
        cache = gq.kv_cache(B, Hq, Hkv, kp, vp, kw, vw)
        ws = gq.workspace(gq.gq_kv_attention_workspace_bytes(cache), "cuda")
        gt = GraphTimer(torch, lambda: gq.kv_attention(q, cache, out=o, ws=ws))
        gt.warm()
        t, _ = gt.run(50)
        nbytes = kp.nbytes() + vp.nbytes() + 2 * kw.numel() * 2 + 2 * q.numel() * 2
        out[name] = {"batch": B, "q_heads": Hq, "kv_heads": Hkv, "t_packed": tp, "t_window": tw, "bits": bits,
                     "us": round(t / 50 * 1e6, 1),
                     "GBps": round(nbytes * 50 / t / 1e9, 1),
                     "frac_hbm": round(nbytes * 50 / t / 1e9 / HBM_PEAK_GBS, 3), "bytes": nbytes}
        del kp, vp, kw, vw, q, o
        torch.cuda.empty_cache()
    return out


def channel_mix(torch, gq, S):
    """Channel-mix M=2048 GEMM on the 70B-class MLP, its data gradient dX,
    quantize/pack and fake quantization of its fp32 weights (and a dense fp16
    GEMM of the same shape for comparison)."""
    out = {}
    for j, (N, K) in enumerate(S.MLP70B_SHAPES):
        Wn, bits = S.channel_mix_weight(j)
        W = torch.from_numpy(Wn).cuda()
        del Wn
        p = gq.quantize_pack(W, bits, 128)
        torch.cuda.synchronize()
        qt = GraphTimer(torch, lambda: gq.gq_quantize_pack(
            p.layout, W.data_ptr(), p.codes.data_ptr(), p.scales.data_ptr(), p.zeros.data_ptr(),
            p.flags.data_ptr()))
        qt.warm()
        t, _ = qt.run(10)
        qb = N * K * 4 + p.nbytes()
        out[f"quantize_pack_mlp{j}"] = {"N": N, "K": K, "us": round(t / 10 * 1e6, 1),
                                        "GBps": round(qb * 10 / t / 1e9, 1),
                                        "frac_hbm": round(qb * 10 / t / 1e9 / HBM_PEAK_GBS, 3)}
        # fake quantization (quantize -> dequantize, bf16 out): the forward of
        # a FakeQuantize module; fp32 in, bf16 out
        wfq = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
        ft = GraphTimer(torch, lambda: gq.gq_fake_quant(p.layout, W.data_ptr(), gq.GQ_BF16,
                                                        wfq.data_ptr(), p.flags.data_ptr()))
        ft.warm()
        t, _ = ft.run(10)
        fb = N * K * (4 + 2)
        out[f"fake_quant_bf16_mlp{j}"] = {"N": N, "K": K, "us": round(t / 10 * 1e6, 1),
                                          "GBps": round(fb * 10 / t / 1e9, 1),
                                          "frac_hbm": round(fb * 10 / t / 1e9 / HBM_PEAK_GBS, 3)}
        del W, wfq
        torch.cuda.empty_cache()
        M = 2048
        x = torch.from_numpy(S.channel_mix_x(j).view(np.int16)).cuda().view(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ws = gq.workspace(gq.gq_linear_workspace_bytes(p.layout, M), "cuda")
        gt = GraphTimer(torch, lambda: gq.linear(x, p, out=y, ws=ws))
        gt.warm()
        t, _ = gt.run(20)
        fl = 2.0 * M * N * K
        tf = fl * 20 / t / 1e12
        # context: a dense fp16 GEMM of the same shape through torch.matmul
        # (hipBLASLt), i.e. what the MFMA units sustain here without any
        # dequantization
        xd = torch.randn((M, K), device="cuda", dtype=torch.float16)
        wd = torch.randn((K, N), device="cuda", dtype=torch.float16)   # W^T, contiguous
        yd = torch.empty((M, N), device="cuda", dtype=torch.float16)
        dt = GraphTimer(torch, lambda: torch.matmul(xd, wd, out=yd))
        dt.warm()
        td, _ = dt.run(20)
        tfd = fl * 20 / td / 1e12
        del xd, wd, yd
        out[f"gemm_channel_mix_M2048_mlp{j}"] = {
            "N": N, "K": K, "int4_blocks": int(sum(b == 4 for b in bits)), "blocks": len(bits),
            "ms": round(t / 20 * 1e3, 4), "TFLOPS": round(tf, 1),
            "frac_mfma": round(tf / MFMA_PEAK_TFLOPS, 3), "includes": "activation pre-pass + GEMM",
            "dense_fp16_torch_matmul_TFLOPS": round(tfd, 1),
            "frac_of_dense_fp16": round(tf / tfd, 3)}
        del x, y
        # backward data gradient dX = dY . W_hat through the same packed
        # weights, M = 2048 rows of output gradient (bf16)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(6000 + j)
        dy = (torch.randn((M, N), generator=gen, device="cuda") * 0.01).to(torch.bfloat16)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        wsd = gq.workspace(gq.gq_linear_dx_workspace_bytes(p.layout, M), "cuda")
        xt = GraphTimer(torch, lambda: gq.linear_dx(dy, p, out=dx, ws=wsd))
        xt.warm()
        t, _ = xt.run(20)
        tf = fl * 20 / t / 1e12
        out[f"dx_channel_mix_M2048_mlp{j}"] = {
            "N": N, "K": K, "ms": round(t / 20 * 1e3, 4), "TFLOPS": round(tf, 1),
            "frac_mfma": round(tf / MFMA_PEAK_TFLOPS, 3), "includes": "gradient pre-pass + dX GEMM"}
        del dy, dx, p
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_gemm_groupwise_amd as gq
    import synth as S

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gq.load_library()
    torch.cuda.set_device(0)
    if args.calibration_copy:
        # a plain copy of known size: 256 MiB read + 256 MiB written per launch
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.gemm_only:
        print(json.dumps({"metric": METRIC, "gemm_only": channel_mix(torch, gq, S)}), flush=True)
        return
    copies = args.copies
    steps = args.steps
    bits = args.bits
    log(f"bench: building INT{bits} decode weights ({copies} rotated copies)")
    sets, xs, ys, nbytes = build_decode(torch, gq, S, bits, 1, copies)
    plans = group_plans(gq, sets, xs, ys, copies)
    log("bench: timing decode steps (one grouped call per step)")
    t, wall = time_steps(torch, gq, sets, xs, ys, copies, steps, args.warmup, plans=plans)
    value = nbytes * steps / t / 1e9
    log(f"bench: {value:.1f} GB/s ({t / steps * 1e6:.2f} us/step, wall {wall / steps * 1e6:.2f} us/step)")
    tl, _ = time_steps(torch, gq, sets, xs, ys, copies, steps, args.warmup)
    per_linear_step = {"GBps": round(nbytes * steps / tl / 1e9, 1),
                       "frac_hbm": round(nbytes * steps / tl / 1e9 / HBM_PEAK_GBS, 4),
                       "us_per_step": round(tl / steps * 1e6, 2), "launch": "four gq_linear calls"}

    # roofline: the step is one launch (the grouped call's one-workgroup-per-
    # tile classes run in one grid: down's streamed tiles first, then the
    # K = 4096 linears' tiles), so the dominant kernel is that launch over
    # the step's bytes
    per_launch = nbytes
    avg = group_avg(torch, gq, plans)
    achieved = per_launch / avg / 1e9
    per_linear = {}
    for j, name in enumerate(("up_gate", "down", "q_o", "k_v")):
        Nj, Kj = S.LLAMA3_8B_SHAPE_LIST[j]
        a = kernel_avg(torch, gq, sets, xs, ys, j, copies, reps=20)
        per_linear[name] = {"us": round(a * 1e6, 2), "GBps": round(decode_bytes(Nj, Kj, bits, 1) / a / 1e9, 1)}
    log(f"bench: dominant launch {avg * 1e6:.2f} us -> {achieved:.1f} GB/s")
    tile = 8 if bits == 4 else 16
    down_tiles, short_tiles = 4096 // tile, 19456 // tile
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": pmc_traffic() if bits == 4 else None,
                "kernel": (f"gemv_group_fused_kernel<bf16, M=1, INT{bits}>, {down_tiles + short_tiles} "
                           f"workgroups of {tile} rows: down 4096x14336 ({down_tiles} streamed-row tiles), "
                           f"then up/gate 14336x4096 + q/o 4096x4096 + k/v 1024x4096 ({short_tiles} tiles "
                           "of one load group per row)"),
                "bytes_per_launch": per_launch, "avg_launch_us": round(avg * 1e6, 3)}
    del sets, xs, ys, plans
    torch.cuda.empty_cache()

    sec = None
    if not args.no_secondary:
        log("bench: secondary measurements")
        sec = secondary(torch, gq, S, args)
        sec["int4_decode_step_M1_per_linear"] = per_linear_step
        sec["int4_M1_per_linear"] = per_linear
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        cpu = cpu_baseline(S, args.cpu_steps, value)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(t / steps * 1e3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Llama-3-8B decode step: 4 linears (N x K = 14336x4096, 4096x14336, "
                               f"4096x4096, 1024x4096), INT{bits} g{128 if bits == 4 else 64} weights, "
                               "M=1 bf16 activations, one grouped decode call per step",
                   "bits": bits, "group": 128 if bits == 4 else 64, "M": 1, "bytes_per_step": nbytes,
                   "rotated_weight_copies": copies, "frac_hbm": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": sec,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
