"""Benchmark: Q2_K mmvq achieved HBM GB/s on one MI355X.

Workload: the large batched-verify matrix, Q2_K [32768, 7168] (28
super-blocks per row, 77 070 336 bytes), seeded synthetic weights and bf16
activations ~ N(0,1) with 5% +-20 outliers. One step is the whole decode hot
path for that matrix: q8_1 quantisation of the bf16 token(s), then the
Q2_K x q8_1 product, through q8_1_q2k_mmvq (one launch at m = 1: the
quantisation runs inside the product; the two-call step is timed beside
it). The headline runs m = 1; m = 8 is reported beside it. Further sections
time the other workloads (token groups past 8, grouped wo_a, engram step,
attention pair, routed-expert batch, single small product); --only picks
workloads for per-workload profiles.

Method:
* Inputs are resident in HBM before timing. The weights are replicated 16
  times (1.23 GB, over four times the 256 MB Infinity Cache) and step i reads
  copy i % 16, so every step streams its matrix from HBM.
* On the launching stream about 40 ms of untimed load (the m = 1 product
  over the copies) settles the clocks and covers the host's enqueueing,
  then the W warm-up steps, a start event, the K timed steps (copy i % 16)
  and an end event: the GPU is busy when the start event is reached and the
  events bracket exactly the K steps; ms_per_step = event time / K. Runs of
  up to 512 launches are launched directly (the host enqueues them while
  the load runs), longer ones as two uploaded HIP graphs (warm-up, timed):
  a graph launch adds ~10 us on the GPU, which 20 steps would feel. (After an idle GPU the shader clock runs at
  1.5-1.9 GHz for the first ~15 ms of streaming and at 2.0-2.25 GHz after.)
* Roofline of the dominant kernel (q2k_mmvq), timed first for each m:
  products alone, a graph of 128 launches replayed untimed for about 40 ms
  and then 5 times between HIP events, achieved = algorithmic bytes
  per launch / average launch time between the events (gaps between
  consecutive kernels included). Beside it, the per-dispatch average of the
  same kernel from the committed rocprofv3 kernel trace
  (profiles/mmvq_large_verify_rocprof.json), when that record was taken on
  the current kernel source.
* CPU baseline: the CPU oracle timed on a bounded sample of rows of the
  same matrix and token, on one thread and on one thread per available core
  (median of three runs each; about twenty seconds of host work).

Prints one JSON line.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q2_K mmvq achieved HBM GB/s (% of peak) at m=1 and m=8, 1x MI355X"
PEAK_GBS = 8000.0          # MI355X HBM3E
N, K = 32768, 7168
COPIES = 16
# Launches per captured HIP graph (copies rotate i % COPIES inside it). Each
# graph replay costs a few microseconds of its own; a decode step captured as
# a graph holds hundreds of kernels, so the graphs here hold 256 launches
# (with 16 the replay overhead added ~0.4 us to every 15 us launch).
GRAPH = 256
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mmvq_large_verify_traffic.json")
ROCPROF_FILE = os.path.join(ROOT, "profiles", "mmvq_large_verify_rocprof.json")
CSRC = os.path.join(ROOT, "q2_quantized_decode_amd", "csrc")
# The product kernel that runs at each m on this matrix, and its sources.
KERNELS = {1: ("mmvq_m1_kernel", ("mmvq.hip", "q2k_device.h")),
           8: ("mmvq_mfma_kernel", ("mmvq_mfma.hip", "q2k_device.h"))}
# The exact instantiation the product runs at each m on this matrix, as
# rocprofv3 names it in its kernel statistics.
KERNEL_INSTANCES = {1: "mmvq_m1_kernel<6, 4, 32, 0>", 8: "mmvq_mfma_kernel<28, 2, false>"}
COPY_BYTES = 256 << 20     # size of the calibration copy


def kernel_hash(m: int) -> str:
    h = hashlib.sha256()
    for f in KERNELS[m][1]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def mmvq_bytes(m: int) -> int:
    """Algorithmic bytes of one product launch: weights + q8_1 rows + f32 out."""
    return N * (K // 256) * 84 + m * K * 5 // 4 + 4 * m * N


def q8_bytes(m: int) -> int:
    """Algorithmic bytes of one q8_1 launch: bf16 in + q8_1 rows out."""
    return 2 * m * K + m * K * 5 // 4


def measured_traffic(m: int):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or
    None when absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(f"m{m}")
    if not r or r.get("kernel_hash") != kernel_hash(m):
        return None
    return float(r["bytes_per_launch"])


def measured_rocprof(m: int):
    """Per-dispatch average (us) of the product kernel at m from the committed
    rocprofv3 kernel statistics, or None when absent or taken on a different
    kernel source."""
    try:
        with open(ROCPROF_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    r = rec.get(f"m{m}")
    if not r or r.get("kernel_hash") != kernel_hash(m):
        return None
    return float(r["avg_us"])


def _oracle_rows(orc, case, xq, d8, r0: int, rows: int) -> int:
    w = case.w[r0:r0 + rows]
    orc.mmvq(w, xq, d8)
    return w.nbytes


def cpu_baseline(case, chunk: int = 2048, runs: int = 3, max_threads: int = 16):
    """The oracle's m = 1 product (the plain fp64 dense route) on row chunks
    of the matrix: one chunk on one thread, and one chunk per thread on one
    thread per core of this process's affinity mask (at most max_threads;
    numpy releases the GIL inside its array operations, and BLAS is held to
    one thread per call so the threads do not oversubscribe). Median of
    `runs` runs each; GB/s of weight bytes."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import q2k_oracle as orc

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:          # pragma: no cover - threadpoolctl ships with the image
        threadpool_limits = None
    affinity = len(os.sched_getaffinity(0))
    threads = max(1, min(affinity, max_threads))
    xq, d8, _ = orc.q8_1_from_bf16_bits(case.x_bits[:1])

    def timed(nthreads: int, run: int) -> float:
        starts = [((run * nthreads + i) * chunk) % N for i in range(nthreads)]
        t0 = time.perf_counter()
        if nthreads == 1:
            done = _oracle_rows(orc, case, xq, d8, starts[0], chunk)
        else:
            with ThreadPoolExecutor(max_workers=nthreads) as ex:
                done = sum(ex.map(lambda r0: _oracle_rows(orc, case, xq, d8, r0, chunk), starts))
        return done / (time.perf_counter() - t0) / 1e9

    def median_of(nthreads: int) -> float:
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                return float(np.median([timed(nthreads, r) for r in range(runs)]))
        return float(np.median([timed(nthreads, r) for r in range(runs)]))

    one = median_of(1)
    many = median_of(threads) if threads > 1 else one
    return {"value": round(many, 6), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "affinity_cores": affinity, "threads": threads, "value_1_thread": round(one, 6),
            "runs": runs,
            "sample": f"m=1 product of the [32768, 7168] Q2_K matrix on {chunk}-row chunks "
                      f"({chunk * (K // 256) * 84} weight bytes each): one chunk on 1 thread, and "
                      f"{threads} chunks on {threads} threads (one per core of the affinity "
                      f"mask, BLAS at one thread per call); median of {runs} runs each; "
                      "fp64 dense oracle"}


def graph_us(torch, fn, launches: int, reps: int = 20, chunk: int = GRAPH, info: dict = None) -> float:
    """Average time of fn(i), i = 0..launches-1, in microseconds: the calls
    are captured in HIP graphs of `chunk` calls each (after one eager pass),
    and HIP events on the capturing stream bracket `reps` replays of all of
    them."""
    stream = torch.cuda.Stream()
    graphs = []
    torch.cuda.synchronize()
    for c0 in range(0, launches, chunk):
        with torch.cuda.stream(stream):
            for i in range(c0, min(c0 + chunk, launches)):
                fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(c0, min(c0 + chunk, launches)):
                fn(i)
        graphs.append(g)
    def one_pass():
        for g in graphs:
            g.replay()

    n_settle = settle(torch, stream, one_pass)
    if info is not None:
        # passes over the launches ahead of the timed ones: eager, sizing, settle
        info["untimed_passes"] = 2 + n_settle
    with torch.cuda.stream(stream):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            one_pass()
        ev1.record(stream)
        ev1.synchronize()
    return ev0.elapsed_time(ev1) * 1e3 / (reps * launches)


# Untimed load ahead of every timed region, in milliseconds of GPU time.
# Measured with a copy of the m = 1 product kernel that reads the shader-clock
# and the constant 100 MHz counters at the start and end of each wave: after
# an idle GPU the clock runs at 1.5-1.9 GHz for the first ~15 ms of
# streaming, then at 2.0-2.25 GHz; the same launches take 14.8-18 us per
# launch in the first milliseconds and 13.9-14.5 us once settled.
SETTLE_MS = 40.0


def settle(torch, stream, replay) -> int:
    """Enqueues on `stream` untimed passes of `replay` (a callable that
    enqueues one pass of a workload) covering about SETTLE_MS of GPU time, so
    that the clocks have settled and the GPU is still busy when the caller
    records its start event. One pass is timed first to size the count.
    Returns the number of untimed passes enqueued after it."""
    with torch.cuda.stream(stream):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        replay()
        e1.record(stream)
    e1.synchronize()
    n = max(1, int(-(-SETTLE_MS // max(e0.elapsed_time(e1), 1e-3))))
    with torch.cuda.stream(stream):
        for _ in range(n):
            replay()
    return n


_HIP = None


def graph_upload(g, stream) -> None:
    """hipGraphUpload of a captured graph's executable on `stream`, so that its
    first replay costs the host no upload (torch does not expose the call)."""
    global _HIP
    import ctypes
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _HIP.hipGraphUpload.restype = ctypes.c_int
    rc = _HIP.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()),
                             ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"hipGraphUpload failed ({rc})")


def capture(torch, stream, fn, first: int, count: int):
    """fn(i), i = first .. first+count-1, captured into one uploaded HIP graph
    (None when count is 0)."""
    if count <= 0:
        return None
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(first, first + count):
            fn(i)
    graph_upload(g, stream)
    torch.cuda.synchronize()
    return g


# Step runs of at most this many launches (warm-up included) are launched
# directly on the busy stream instead of as graphs: the host enqueues them
# (~10 us per launch) while the settle load still runs, and no graph boundary
# falls inside the timed region. A graph launch adds ~10 us on the GPU (20
# steps measured 3-8 % slower as a graph than launched directly; 3200 steps
# agree within 0.2 %), while longer runs launched directly would outpace the
# host.
DIRECT_MAX_LAUNCHES = 512


def timed_steps(torch, stream, fn, warm: int, count: int, load, launches_per_step: int = 1):
    """Seconds per call of fn(i) over `count` calls i = warm .. warm+count-1,
    after `warm` untimed calls i = 0 .. warm-1, and how they were launched.
    On `stream` about SETTLE_MS of untimed load (passes of `load`, a callable
    enqueueing one pass of another workload) settles the clocks and covers
    the host's enqueueing; then the warm-up calls, the start event, the
    timed calls and the end event, so the events bracket exactly `count`
    calls with the GPU busy up to the start event. Short runs are launched
    directly (see DIRECT_MAX_LAUNCHES); longer ones are captured into two
    uploaded HIP graphs (warm-up and timed)."""
    if (warm + count) * launches_per_step <= DIRECT_MAX_LAUNCHES:
        settle(torch, stream, load)
        with torch.cuda.stream(stream):
            for i in range(warm):
                fn(i)
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for i in range(warm, warm + count):
                fn(i)
            ev1.record(stream)
        ev1.synchronize()
        return ev0.elapsed_time(ev1) / 1e3 / count, "direct"
    g_warm = capture(torch, stream, fn, 0, warm)
    g = capture(torch, stream, fn, warm, count)
    settle(torch, stream, load)
    with torch.cuda.stream(stream):
        if g_warm is not None:
            g_warm.replay()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        ev1.synchronize()
    del g, g_warm
    return ev0.elapsed_time(ev1) / 1e3 / count, "graph"


def replay_timed(torch, stream, fn, count: int, reps: int) -> float:
    """Seconds per call of fn(i), i = 0 .. count-1, captured into one HIP
    graph: untimed replays for about SETTLE_MS (they also keep the GPU busy
    while the host enqueues the rest), then `reps` replays between HIP
    events."""
    g = capture(torch, stream, fn, 0, count)
    settle(torch, stream, g.replay)
    with torch.cuda.stream(stream):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            g.replay()
        ev1.record(stream)
        ev1.synchronize()
    del g
    return ev0.elapsed_time(ev1) / 1e3 / (count * reps)


ROOF_GRAPH, ROOF_REPS = 128, 5


def product_roofline(torch, q2, stream, copies, x8, m: int, same_copy: bool = True):
    """Average time of one q2k_mmvq launch on the large verify matrix: a
    graph of 128 launches (copy i % 16), untimed replays for about SETTLE_MS
    (after an idle GPU the first ~15 ms of streaming run at lower clocks, up
    to ~18 us per launch), then 5 replays (640 launches) between HIP
    events; with same_copy also the same with one weight copy for every
    launch (cache-resident reference). Replaying one graph matters: a
    second graph of the same launches measured ~0.6 us per launch slower."""
    xq = q2.q8_1_rows(x8[:m].contiguous())
    y = torch.empty((m, N), dtype=torch.float32, device=x8.device)
    launch_s = replay_timed(torch, stream, lambda i: q2.q2k_mmvq(copies[i % COPIES], xq, N, K, m, out=y),
                            ROOF_GRAPH, ROOF_REPS)
    warm_s = None
    if same_copy:
        warm_s = replay_timed(torch, stream, lambda i: q2.q2k_mmvq(copies[0], xq, N, K, m, out=y), 128, 2)
    return launch_s, warm_s


def _roof(nbytes: int, us: float) -> dict:
    gbs = nbytes / us / 1e3
    return {"us_per_launch": round(us, 3), "bytes_per_launch": int(nbytes),
            "achieved": round(gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_GBS, 4)}


def bench_single(torch, q2, syn, dev, copies_n: int = 4096):
    """The single small product, Q2_K [256, 1024] at m = 1 (86 016 weight
    bytes): 4096 copies in one buffer (352 MB, past the Infinity Cache),
    launch i reads copy i."""
    case = syn.single_gemv_case()
    per = case.w.size
    buf = torch.from_numpy(case.w.reshape(-1)).to(dev).repeat(copies_n)
    x = syn.bf16_bits_to_tensor(case.x_bits).to(dev)
    xq = q2.q8_1_rows(x)
    y = torch.empty((1, case.n), dtype=torch.float32, device=dev)
    us = graph_us(torch, lambda i: q2.q2k_mmvq(buf[i * per:(i + 1) * per], xq, case.n, case.k, 1,
                                               out=y), copies_n, reps=5, chunk=256)
    from oracle import q2k_oracle as orc
    oq, od, _ = orc.q8_1_from_bf16_bits(case.x_bits)
    ref = orc.mmvq(case.w, oq, od)
    if not np.all(np.abs(y.cpu().numpy().astype(np.float64) - ref) <= 1e-4 + 2e-3 * np.abs(ref)):
        raise SystemExit("bench parity failed: single product")
    out = _roof(per + q2.q8_1_rows_bytes(1, case.k) + 4 * case.n, us)
    out["workload"] = (f"single Q2_K product [256, 1024], m = 1, {copies_n} copies in one "
                       "buffer; launch-bound (86 KB of weights)")
    return out


def bench_pair(torch, q2, syn, dev, copies_n: int = 512):
    """The attention input pair: q8_1 of x [m, 4096] once, then wq_a [1024,
    4096] and wkv [512, 4096] against it in one launch, m = 1, 4, 8; 512
    rotating copies of the two matrices (1.06 GB)."""
    from oracle import q2k_oracle as orc
    out = {}
    for m in (1, 4, 8):
        pc = syn.attention_pair_case(m)
        wa0 = torch.from_numpy(pc.wa.reshape(-1)).to(dev)
        wb0 = torch.from_numpy(pc.wb.reshape(-1)).to(dev)
        wa = wa0.repeat(copies_n)
        wb = wb0.repeat(copies_n)
        pa, pb = wa0.numel(), wb0.numel()
        x = syn.bf16_bits_to_tensor(pc.x_bits).to(dev)
        xq = torch.empty(q2.q8_1_rows_bytes(m, pc.k), dtype=torch.uint8, device=dev)
        ya = torch.empty((m, pc.na), dtype=torch.float32, device=dev)
        yb = torch.empty((m, pc.nb), dtype=torch.float32, device=dev)

        def prod(i):
            j = i % copies_n
            q2.q2k_mmvq_pair(wa[j * pa:(j + 1) * pa], pc.na, wb[j * pb:(j + 1) * pb], pc.nb, xq,
                             pc.k, m, ya=ya, yb=yb)

        def step(i):
            # q8_1 + pair in one call (two launches at these sizes)
            j = i % copies_n
            q2.q8_1_q2k_mmvq_pair(wa[j * pa:(j + 1) * pa], pc.na, wb[j * pb:(j + 1) * pb], pc.nb, x,
                                  pc.k, xq=xq, ya=ya, yb=yb)

        def step_two_calls(i):
            q2.q8_1_rows(x, out=xq)
            prod(i)

        us_step = graph_us(torch, step, copies_n, reps=10)
        us_step2 = graph_us(torch, step_two_calls, copies_n, reps=10)
        us_prod = graph_us(torch, prod, copies_n, reps=10)
        oq, od, _ = orc.q8_1_from_bf16_bits(pc.x_bits)
        ra, rb = orc.mmvq_pair(pc.wa, pc.wb, oq, od)
        for got, ref in ((ya, ra), (yb, rb)):
            if not np.all(np.abs(got.cpu().numpy().astype(np.float64) - ref)
                          <= 1e-4 + 2e-3 * np.abs(ref)):
                raise SystemExit(f"bench parity failed: attention pair m={m}")
        r = _roof(pa + pb + q2.q8_1_rows_bytes(m, pc.k) + 4 * m * (pc.na + pc.nb), us_prod)
        r["us_per_step"] = round(us_step, 3)
        r["us_per_step_two_calls"] = round(us_step2, 3)
        r["tokens_per_s"] = round(m / us_step * 1e6, 1)
        out[f"m{m}"] = r
    out["workload"] = ("attention input pair: x bf16 [m, 4096] -> q8_1 once -> wq_a Q2_K "
                       "[1024, 4096] and wkv Q2_K [512, 4096] in one launch; 512 rotating copies "
                       "(1.06 GB); step = q8_1 + pair (q8_1_q2k_mmvq_pair), product = the pair launch "
                       "alone")
    return out


def bench_experts(torch, q2, syn, dev, steps_n: int = 64):
    """The routed-expert decode batch: 256 resident experts of Q2_K gate and
    up [2048, 4096] and down [4096, 2048] (2.11 GB, all seeded), a fresh
    set of 8 ids per step (without replacement, seeded). Step: q8_1 of x
    [1, 4096], gate/up over the 8 ids (one launch), bf16 SwiGLU + q8_1 of
    the 8 rows, down with one input row per id -> f32 [8, 4096]."""
    from oracle import q2k_oracle as orc
    case = syn.expert_batch_case()
    dim, inter, ne = case.dim, case.inter, case.n_experts
    per_gu = inter * (dim // 256) * 84
    per_d = dim * (inter // 256) * 84
    sets = {}
    for kind, per in (("gate", per_gu), ("up", per_gu), ("down", per_d)):
        buf = torch.empty(ne * per, dtype=torch.uint8, device=dev)
        for e in range(ne):
            buf[e * per:(e + 1) * per] = torch.from_numpy(case.expert_matrix(e, kind).reshape(-1))
        sets[kind] = buf
    rng = syn.rng_for(case.seed, 1 << 20)
    ids_np = np.stack([rng.choice(ne, size=8, replace=False) for _ in range(steps_n)]).astype(np.int32)
    ids = torch.from_numpy(ids_np).to(dev)
    x = syn.bf16_bits_to_tensor(case.x_bits).to(dev)
    xq = torch.empty(q2.q8_1_rows_bytes(1, dim), dtype=torch.uint8, device=dev)
    gu = torch.empty((2, 8, 1, inter), dtype=torch.float32, device=dev)
    hq = torch.empty(q2.q8_1_rows_bytes(8, inter), dtype=torch.uint8, device=dev)
    yd = torch.empty((1, 8, 1, dim), dtype=torch.float32, device=dev)
    g, u = gu[0].view(8, inter), gu[1].view(8, inter)

    def gate_up(i):
        q2.q2k_mmvq_experts([sets["gate"], sets["up"]], per_gu, ne, ids[i % steps_n], xq, False,
                            inter, dim, 1, out=gu)

    def down(i):
        q2.q2k_mmvq_experts([sets["down"]], per_d, ne, ids[i % steps_n], hq, True, dim, inter, 1,
                            out=yd)

    def step(i):
        # q8_1 of x in the gate/up launch's prologue, the SwiGLU and its q8_1
        # in its epilogue, then the down launch: two launches for the token
        q2.q8_1_q2k_mmvq_experts_swiglu([sets["gate"], sets["up"]], per_gu, ne, ids[i % steps_n], x,
                                        inter, dim, xq=xq, out=gu, hq=hq)
        down(i)

    def step_swiglu_in_down(i):
        # q8_1 of x inside the gate/up launch, SwiGLU + q8_1 inside the down
        # launch: two launches for the token
        q2.q8_1_q2k_mmvq_experts([sets["gate"], sets["up"]], per_gu, ne, ids[i % steps_n], x, inter,
                                 dim, xq=xq, out=gu)
        q2.swiglu_q2k_mmvq_experts([sets["down"]], per_d, ne, ids[i % steps_n], g, u, dim, hq=hq,
                                   out=yd)

    def step_unfused(i):
        q2.q8_1_rows(x, out=xq)
        gate_up(i)
        q2.swiglu_q8_1_rows(g, u, hq=hq, want_h=False)
        down(i)

    us_step = graph_us(torch, step, steps_n)
    us_step_sw_down = graph_us(torch, step_swiglu_in_down, steps_n)
    us_step_unfused = graph_us(torch, step_unfused, steps_n)
    us_gu_sw = graph_us(torch, lambda i: q2.q8_1_q2k_mmvq_experts_swiglu(
        [sets["gate"], sets["up"]], per_gu, ne, ids[i % steps_n], x, inter, dim, xq=xq, out=gu, hq=hq),
        steps_n)
    us_down_fused = graph_us(torch, lambda i: q2.swiglu_q2k_mmvq_experts(
        [sets["down"]], per_d, ne, ids[i % steps_n], g, u, dim, hq=hq, out=yd), steps_n)
    us_gu = graph_us(torch, gate_up, steps_n)
    us_down = graph_us(torch, down, steps_n)
    us_q8 = graph_us(torch, lambda i: q2.q8_1_rows(x, out=xq), 16)
    us_sw = graph_us(torch, lambda i: q2.swiglu_q8_1_rows(g, u, hq=hq, want_h=False), 16)
    # parity of the last id set, stage by stage: gate/up against the oracle;
    # h within one bf16 step of the oracle's SwiGLU; then the down product
    # against the oracle on the oracle's q8_1 of that h
    i_last = steps_n - 1
    step(i_last)
    torch.cuda.synchronize()
    gu_fused, yd_fused = gu.clone(), yd.clone()
    for other in (step_swiglu_in_down, step_unfused):
        other(i_last)
        torch.cuda.synchronize()
        if not (torch.equal(gu_fused.view(torch.int32), gu.view(torch.int32))
                and torch.equal(yd_fused.view(torch.int32), yd.view(torch.int32))):
            raise SystemExit("bench parity failed: the two-launch step differs from "
                             f"{other.__name__}")
    h, hq_p = q2.swiglu_q8_1_rows(g, u)
    yp = q2.q2k_mmvq_experts([sets["down"]], per_d, ne, ids[i_last], hq_p, True, dim, inter, 1)
    torch.cuda.synchronize()
    sel = ids_np[i_last].tolist()
    oq, od, _ = orc.q8_1_from_bf16_bits(case.x_bits)
    gu_h = gu.cpu().numpy()
    for bi, kind in enumerate(("gate", "up")):
        ref = orc.mmvq_experts([case.expert_matrix(e, kind) for e in sel], oq, od, x_per_id=False)
        if not np.all(np.abs(gu_h[bi].astype(np.float64) - ref) <= 1e-4 + 2e-3 * np.abs(ref)):
            raise SystemExit(f"bench parity failed: experts {kind}")
    h_bits = h.view(torch.int16).cpu().numpy().view(np.uint16)
    h_ref = orc.swiglu_bf16_bits(gu_h[0].reshape(8, inter), gu_h[1].reshape(8, inter))

    def ordered(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)

    if np.abs(ordered(h_bits) - ordered(h_ref)).max() > 1:
        raise SystemExit("bench parity failed: SwiGLU more than one bf16 step off")
    hq_o, hd_o, _ = orc.q8_1_from_bf16_bits(h_bits)
    ref = orc.mmvq_experts([case.expert_matrix(e, "down") for e in sel], hq_o, hd_o, x_per_id=True)
    if not np.all(np.abs(yp.cpu().numpy()[0].astype(np.float64) - ref) <= 1e-4 + 2e-3 * np.abs(ref)):
        raise SystemExit("bench parity failed: experts down")
    b_gu = 16 * per_gu + q2.q8_1_rows_bytes(1, dim) + 4 * 16 * inter + 4 * 8
    b_d = 8 * per_d + q2.q8_1_rows_bytes(8, inter) + 4 * 8 * dim + 4 * 8
    step_bytes = b_gu + b_d + (2 * dim + q2.q8_1_rows_bytes(1, dim)) \
        + (8 * 16 * inter + q2.q8_1_rows_bytes(8, inter))
    return {"workload": "routed-expert decode batch, m = 1: 256 resident experts (Q2_K gate/up "
                        "[2048, 4096], down [4096, 2048]; 2.11 GB), 8 ids per step without "
                        "replacement, 64 id sets; step = gate/up with q8_1 of x in its prologue "
                        "and the bf16 SwiGLU + q8_1 of h in its epilogue (one launch, 16 "
                        "matrices) + down on those q8_1 rows (one launch, 8 matrices, one input "
                        "row per id)",
            "us_per_step": round(us_step, 3), "tokens_per_s": round(1e6 / us_step, 1),
            "us_per_step_swiglu_in_down": round(us_step_sw_down, 3),
            "us_per_step_four_launches": round(us_step_unfused, 3),
            "gate_up_swiglu_us": round(us_gu_sw, 3),
            "swiglu_down_fused_us": round(us_down_fused, 3),
            "step_gbs": round(step_bytes / us_step / 1e3, 1),
            "step_frac": round(step_bytes / us_step / 1e3 / PEAK_GBS, 4),
            "gate_up": _roof(b_gu, us_gu), "down": _roof(b_d, us_down),
            "q8_1_us": round(us_q8, 3), "swiglu_q8_1_us": round(us_sw, 3)}


def bench_mmq(torch, q2, syn, dev, copies, case):
    """The product past 8 tokens (q2k_mmq) on the large-verify matrix: m =
    16, 64, 256 tokens ~ N(0,1) with 5% +-20 outliers, over the same rotating
    copies; graphs of 16 launches, HIP events around the replays."""
    out = {}
    for m in (16, 64, 256):
        x = syn.bf16_bits_to_tensor(syn.bf16_normal(syn.rng_for(1004, m), (m, K), outlier_frac=0.05)).to(dev)
        xq = q2.q8_1_rows(x)
        y = torch.empty((m, N), dtype=torch.float32, device=dev)
        stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for i in range(COPIES):
                q2.q2k_mmq(copies[i], xq, N, K, m, out=y)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(COPIES):
                q2.q2k_mmq(copies[i], xq, N, K, m, out=y)
        reps = max(2, 64 // m)
        settle(torch, stream, g.replay)
        with torch.cuda.stream(stream):
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(reps):
                g.replay()
            ev1.record(stream)
            ev1.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / (reps * COPIES)
        nbytes = mmvq_bytes(m)
        int8_ops = 2.0 * N * K * m
        out[f"m{m}"] = {"us_per_launch": round(us, 2), "tokens_per_s": round(m / us * 1e6, 1),
                        "achieved_gbs": round(nbytes / us / 1e3, 1),
                        "frac_hbm": round(nbytes / us / 1e3 / PEAK_GBS, 4),
                        "tops": round(int8_ops / us / 1e6, 1)}
    out["workload"] = ("q2k_mmq on Q2_K [32768, 7168], m tokens (m = 16: the matrix-core kernel "
                       "on groups of 8; from 17: the tile kernel, 32 tokens x 64 rows per "
                       "workgroup), 16 rotating copies")
    return out


def bench_grouped(torch, q2, syn, dev, copies_n: int = 64):
    """The grouped-input product (wo_a shape: 8 groups x 1024 rows, 2048-wide
    slices of a 16384-wide input) at m = 1 and m = 8 over rotating weight
    copies, timed with HIP events around graph replays."""
    out = {}
    gc = syn.grouped_case(8)
    w0 = torch.from_numpy(gc.w.reshape(-1)).to(dev)
    wbytes = w0.numel()
    buf = w0.repeat(copies_n)            # one allocation, copy i at i * wbytes
    copies = [buf[i * wbytes:(i + 1) * wbytes] for i in range(copies_n)]
    x8 = syn.bf16_bits_to_tensor(gc.x_bits).to(dev)
    for m in (1, 8):
        xq = q2.q8_1_rows(x8[:m].contiguous())
        y = torch.empty((m, gc.groups * gc.rows), dtype=torch.float32, device=dev)
        us = graph_us(torch, lambda i: q2.q2k_mmvq_grouped(copies[i], xq, gc.groups, gc.rows, gc.k, m,
                                                           out=y), copies_n, reps=20)
        nbytes = wbytes + q2.q8_1_rows_bytes(m, gc.groups * gc.k) + 4 * m * gc.groups * gc.rows
        out[f"m{m}"] = {"us_per_launch": round(us, 3), "bytes_per_launch": nbytes,
                        "achieved": round(nbytes / us / 1e3, 1), "peak": PEAK_GBS, "unit": "GB/s",
                        "frac": round(nbytes / us / 1e3 / PEAK_GBS, 4)}
    out["workload"] = ("grouped-input wo_a product, Q2_K [8192, 2048] in 8 groups of 1024 rows "
                       f"over 2048-wide slices of x [m, 16384], {copies_n} rotating copies")
    return out


def bench_engram(torch, q2, syn, dev, copies_n: int = 80):
    """The engram step on the device, one token per step: n-gram hash (2
    hashed layers, 3-grams, 4 heads = 8 row ids), gather + dequantisation of
    8 table rows (500 000-row table) and q8_1 of the [1, 2048] row in one
    launch, the wkv product [20480, 2048] (80 rotating copies, 1.1 GB) and
    the gate on [1, 4, 4096]; HIP graphs of the steps, HIP events around the
    replays. The same step with the gather and the q8_1 as two launches, and
    the hash alone (one decode token, a 4096-token prefill), are timed the
    same way."""
    e = syn.engram_step_case()
    hc = syn.engram_hash_case(seqlen=4096)
    tm, mu, pr, of = (torch.from_numpy(a).to(dev) for a in
                      (hc.token_map, hc.multipliers, hc.primes, hc.offsets))
    cache = torch.zeros(8192, dtype=torch.int64, device=dev)
    toks = torch.from_numpy(hc.tokens).to(dev)
    table = torch.from_numpy(e.table.reshape(-1)).to(dev)
    w0 = torch.from_numpy(e.wkv.reshape(-1)).to(dev)
    copies = [w0] + [w0.clone() for _ in range(copies_n - 1)]
    h = torch.from_numpy(e.h).to(dev)
    qk = torch.from_numpy(e.qk).to(dev)
    ids = torch.empty((2, 1, 8), dtype=torch.int64, device=dev)
    rows = torch.empty((8, 256), dtype=torch.bfloat16, device=dev)
    xq = torch.empty(q2.q8_1_rows_bytes(1, 2048), dtype=torch.uint8, device=dev)
    n_out = e.dim * (e.hc + 1)
    kv = torch.empty((1, n_out), dtype=torch.float32, device=dev)
    # prefill positions 0..4095 once so the decode steps see a real look-back
    q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, toks, 0)

    ws = torch.empty(q2.engram_step_workspace_bytes(3, 4, e.hc, e.dim), dtype=torch.uint8, device=dev)

    def step(i):
        # one call: hash (hashed layer 1), gather, dequant and q8_1 in the wkv
        # product's prologue (one launch), then the gate
        q2.engram_step(tm, mu, pr, of, hc.pad_id, cache, toks[i % 64:i % 64 + 1], 4096 + (i % 64), 1,
                       table, 500000, copies[i % copies_n], qk, h, e.eps, workspace=ws)

    def step_rows_apart(i):
        # hash + gather + dequant + q8_1 in one launch of their own
        q2.engram_rows_q8_1(tm, mu, pr, of, hc.pad_id, cache, toks[i % 64:i % 64 + 1], 4096 + (i % 64), 1,
                            table, 500000, xq=xq)
        q2.q2k_mmvq(copies[i % copies_n], xq, n_out, 2048, 1, out=kv)
        q2.engram_gate(h, kv, qk, e.eps)

    def step_hash_apart(i):
        q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, toks[i % 64:i % 64 + 1], 4096 + (i % 64), out=ids)
        q2.q2k_dequant_rows_q8_1(table, 500000, ids[1].reshape(-1), 8, xq=xq)
        q2.q2k_mmvq(copies[i % copies_n], xq, n_out, 2048, 1, out=kv)
        q2.engram_gate(h, kv, qk, e.eps)

    def step_unfused(i):
        q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, toks[i % 64:i % 64 + 1], 4096 + (i % 64), out=ids)
        q2.q2k_dequant_rows(table, 500000, ids[1].reshape(-1), 8, out=rows)
        q2.q8_1_rows(rows.view(1, 2048), out=xq)
        q2.q2k_mmvq(copies[i % copies_n], xq, n_out, 2048, 1, out=kv)
        q2.engram_gate(h, kv, qk, e.eps)

    def timed(fn, launches, reps=20):
        return graph_us(torch, fn, launches, reps)

    def step_bf16(i):
        q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, toks[i % 64:i % 64 + 1], 4096 + (i % 64), out=ids)
        q2.q2k_dequant_rows(table, 500000, ids[1].reshape(-1), 8, out=rows)
        q2.q2k_gemv_bf16(copies[i % copies_n], rows.view(1, 2048), n_out, 2048, out=kv)
        q2.engram_gate(h, kv, qk, e.eps)

    us_step = timed(step, copies_n)
    us_step_rows_apart = timed(step_rows_apart, copies_n)
    us_step_hash_apart = timed(step_hash_apart, copies_n)
    us_step_unfused = timed(step_unfused, copies_n)
    us_step_bf16 = timed(step_bf16, copies_n)
    us_gemv = timed(lambda i: q2.q2k_gemv_bf16(copies[i % copies_n], rows.view(1, 2048), n_out, 2048,
                                               out=kv), copies_n)
    us_mmvq = timed(lambda i: q2.q2k_mmvq(copies[i % copies_n], xq, n_out, 2048, 1, out=kv), copies_n)
    us_hash1 = timed(lambda i: q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, toks[i % 64:i % 64 + 1],
                                              4096 + (i % 64), out=ids), 16)
    pre = torch.empty((2, 4096, 8), dtype=torch.int64, device=dev)
    us_pre = timed(lambda i: q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, toks, 0, out=pre), 16)
    wkv_bytes = w0.numel()
    return {"workload": "engram step, one token (engram_step): hash + 8-row gather + dequant + "
                        "q8_1 in the prologue of the wkv Q2_K [20480, 2048] product (one launch) -> "
                        "gate [1, 4, 4096]; 80 rotating wkv copies. rows_apart: hash, gather, "
                        "dequant and q8_1 as one launch of their own (engram_rows_q8_1); "
                        "hash_apart: the hash as its own launch as well; unfused: hash, gather and "
                        "q8_1 as three launches; the bf16 route skips q8_1: gathered bf16 rows "
                        "straight into the wkv product",
            "us_per_step": round(us_step, 3), "tokens_per_s": round(1e6 / us_step, 1),
            "us_per_step_rows_apart": round(us_step_rows_apart, 3),
            "us_per_step_hash_apart": round(us_step_hash_apart, 3),
            "us_per_step_unfused": round(us_step_unfused, 3),
            "us_per_step_bf16_route": round(us_step_bf16, 3),
            "wkv_bytes": wkv_bytes,
            "wkv_q8_1_product_us": round(us_mmvq, 3),
            "wkv_q8_1_product_gbs": round(wkv_bytes / us_mmvq / 1e3, 1),
            "wkv_bf16_product_us": round(us_gemv, 3),
            "wkv_bf16_product_gbs": round(wkv_bytes / us_gemv / 1e3, 1),
            "hash_decode_us": round(us_hash1, 3), "hash_prefill_4096_us": round(us_pre, 3)}


# Workloads in run order; "headline" is the large verify at m = 1 and 8.
# Single-matrix shapes of the workloads above (rows, k), for the product
# kernel sweep.
KERNEL_SWEEP_SHAPES = [(32768, 7168), (20480, 2048), (1024, 4096), (512, 4096), (2048, 4096),
                       (4096, 2048), (1024, 2048)]


def bench_kernels(torch, q2, syn, dev):
    """The two product kernels at m = 2..8 on each workload matrix shape:
    matrix cores (q2k_set_product_kernel(1)) and packed dots (2), same bits
    either way; each over rotating weight copies of >= 1 GiB, graphs of 16
    launches, HIP events around the replays. Reports both times and the
    kernel the default choice takes."""
    out = {}
    prev = q2.q2k_set_product_kernel(q2.KERNEL_AUTO)
    try:
        for (n, k) in KERNEL_SWEEP_SHAPES:
            w = syn.q2k_blocks(syn.rng_for(5, n, k), n, k // 256)
            per = w.size
            ncopy = max(2, min(1024, -(-(1 << 30) // per)))
            buf = torch.from_numpy(w.reshape(-1)).to(dev).repeat(ncopy)
            for m in range(2, 9):
                x = syn.bf16_bits_to_tensor(syn.bf16_normal(syn.rng_for(6, m), (m, k))).to(dev)
                xq = q2.q8_1_rows(x)
                y = torch.empty((m, n), dtype=torch.float32, device=dev)
                rec = {"auto": "mfma" if q2.q2k_product_kernel(n, k, m) == q2.KERNEL_MATRIX_CORES
                       else "dots"}
                for name, choice in (("mfma", q2.KERNEL_MATRIX_CORES), ("dots", q2.KERNEL_PACKED_DOTS)):
                    q2.q2k_set_product_kernel(choice)
                    launches = min(ncopy, 128)
                    info = {}
                    rec[name + "_us"] = round(graph_us(
                        torch, lambda i: q2.q2k_mmvq(buf[i * per:(i + 1) * per], xq, n, k, m, out=y),
                        launches, reps=max(2, 1024 // launches), chunk=16, info=info), 3)
                    rec[name + "_untimed_passes"] = info["untimed_passes"]
                    q2.q2k_set_product_kernel(q2.KERNEL_AUTO)
                rec["auto_is_faster"] = rec[rec["auto"] + "_us"] <= min(rec["mfma_us"], rec["dots_us"]) * 1.02
                out[f"{n}x{k}_m{m}"] = rec
            del buf
            torch.cuda.empty_cache()
    finally:
        q2.q2k_set_product_kernel(prev)
    out["workload"] = ("q2k_mmvq at m = 2..8 on the workloads' matrix shapes, both product "
                       "kernels (same bits), >= 1 GiB of rotating weight copies per shape")
    return out


SECTIONS = ["headline", "mmq", "grouped", "engram", "pair", "experts", "single", "kernels"]
ON_REQUEST = {"kernels"}     # run only when named in --only
SECTION_KEYS = {"mmq": "mmq", "grouped": "grouped", "engram": "engram_step",
                "pair": "attention_pair", "experts": "expert_batch", "single": "single",
                "kernels": "product_kernels"}
SECTION_FNS = {"grouped": bench_grouped, "engram": bench_engram, "pair": bench_pair,
               "experts": bench_experts, "single": bench_single, "kernels": bench_kernels}


def run(args):
    import torch

    import q2_quantized_decode_amd as q2
    from q2_quantized_decode_amd import synthetic as syn

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (HIP device)")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q2.lib()

    only = set(args.only.split(",")) if args.only else None
    if only is not None:
        unknown = only - set(SECTIONS)
        if unknown:
            raise SystemExit(f"--only: unknown sections {sorted(unknown)}; known: {SECTIONS}")
        if "headline" not in only:
            # profiling runs of single workloads: no headline, no contract line
            if "mmq" in only:
                raise SystemExit("--only: mmq reuses the headline's weights; add headline")
            line = {"sections": sorted(only)}
            for name in SECTIONS[2:]:
                if name in only:
                    line[SECTION_KEYS[name]] = SECTION_FNS[name](torch, q2, syn, dev)
                    torch.cuda.synchronize()
            print(json.dumps(line), flush=True)
            return

    case = syn.large_verify_case(m=8)
    w0 = torch.from_numpy(case.w.reshape(-1)).to(dev)
    copies = [w0] + [w0.clone() for _ in range(COPIES - 1)]
    x8 = syn.bf16_bits_to_tensor(case.x_bits).to(dev)
    if args.roofline_only:
        # only the product launches behind `roofline` (for kernel traces)
        stream = torch.cuda.Stream()
        out = {}
        for m in (1, 8):
            launch_s, _ = product_roofline(torch, q2, stream, copies, x8, m, same_copy=False)
            out[f"m{m}"] = {"us_per_launch": round(launch_s * 1e6, 3),
                            "achieved_gbs": round(mmvq_bytes(m) / launch_s / 1e9, 1),
                            "frac": round(mmvq_bytes(m) / launch_s / 1e9 / PEAK_GBS, 4)}
        print(json.dumps({"roofline_only": out}), flush=True)
        return

    results = {}
    stream = torch.cuda.Stream()
    # the untimed load ahead of each timed step run: the m = 1 product over
    # the rotating copies (see SETTLE_MS)
    xq_load = q2.q8_1_rows(x8[:1].contiguous())
    y_load = torch.empty((1, N), dtype=torch.float32, device=dev)
    g_load = capture(torch, stream, lambda i: q2.q2k_mmvq(copies[i % COPIES], xq_load, N, K, 1, out=y_load),
                     0, ROOF_GRAPH)
    warm, steps = args.warmup, args.steps
    roof_launches = ROOF_GRAPH * ROOF_REPS
    for m in (1, 8):
        x = x8[:m].contiguous()
        xq = torch.empty(q2.q8_1_rows_bytes(m, K), dtype=torch.uint8, device=dev)
        y = torch.empty((m, N), dtype=torch.float32, device=dev)

        def step(i):
            # q8_1 + product in one call (one launch at m = 1)
            q2.q8_1_q2k_mmvq(copies[i % COPIES], x, N, K, xq=xq, out=y)

        def step_two_calls(i):
            q2.q8_1_rows(x, out=xq)
            q2.q2k_mmvq(copies[i % COPIES], xq, N, K, m, out=y)

        # the dominant kernel alone first (its warm-up also brings the GPU to
        # its sustained clocks); the same-copy figure is cache-resident (the
        # 77 MB matrix fits the 256 MB Infinity Cache): reported beside, never
        # the roofline figure
        launch_s, warm_s = product_roofline(torch, q2, stream, copies, x8, m)
        step_s, launch_mode = timed_steps(torch, stream, step, warm, steps, g_load.replay,
                                          1 if m == 1 else 2)
        two_s, _ = timed_steps(torch, stream, step_two_calls, warm, steps, g_load.replay, 2)
        step(warm + steps - 1)               # y of the last timed step, for the parity check
        torch.cuda.synchronize()
        step_bytes = mmvq_bytes(m) + q8_bytes(m)
        y_host = y.cpu().numpy()
        results[m] = dict(step_s=step_s, launch_s=launch_s, warm_s=warm_s, steps=steps, y=y_host,
                          two_s=two_s, launch_mode=launch_mode,
                          step_gbs=step_bytes / step_s / 1e9,
                          achieved=mmvq_bytes(m) / launch_s / 1e9)

    # parity of the benchmarked output (the last step read copy 15 of the
    # same bytes) on sampled rows against the oracle
    from oracle import q2k_oracle as orc
    rows = np.sort(syn.rng_for(17).choice(N, 64, replace=False))
    for m in (1, 8):
        xq_o, d8_o, _ = orc.q8_1_from_bf16_bits(case.x_bits[:m])
        ref = orc.mmvq(case.w[rows], xq_o, d8_o)
        got = results[m]["y"][:, rows]
        if not np.all(np.abs(got.astype(np.float64) - ref) <= 1e-4 + 2e-3 * np.abs(ref)):
            raise SystemExit(f"bench parity failed at m={m}")
        if not np.array_equal(got.view(np.uint32), orc.mmvq_f32(case.w[rows], xq_o, d8_o).view(np.uint32)):
            raise SystemExit(f"bench parity failed at m={m}: not the fixed-order bits")

    r1, r8 = results[1], results[8]

    def roofline(m, r):
        out = {"bound": "hbm", "achieved": round(r["achieved"], 1), "peak": PEAK_GBS,
               "unit": "GB/s", "frac": round(r["achieved"] / PEAK_GBS, 4),
               "traffic": measured_traffic(m),
               "kernel": f"q2k_mmvq ({KERNEL_INSTANCES[m]})",
               "bytes_per_launch": mmvq_bytes(m),
               "us_per_launch": round(r["launch_s"] * 1e6, 3),
               "timing": f"HIP events around {roof_launches} back-to-back launches (5 replays "
                         "of a 128-launch graph after 4 untimed replays; gaps between kernels "
                         "included)"}
        rp = measured_rocprof(m)
        if rp is not None:
            gbs = mmvq_bytes(m) / rp / 1e3
            out["rocprof"] = {"us_per_launch": round(rp, 3), "achieved": round(gbs, 1),
                              "frac": round(gbs / PEAK_GBS, 4),
                              "source": "profiles/mmvq_large_verify_rocprof.json (kernel trace "
                                        "average on the current kernel source)"}
        return out

    line = {
        "metric": METRIC,
        "value": round(r1["step_gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": r1["steps"],
        "warmup": warm,
        "ms_per_step": round(r1["step_s"] * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "large batched verify, Q2_K [32768, 7168] x q8_1, m=1 "
                               "(step = q8_1 quantisation + product, q8_1_q2k_mmvq: one launch)",
                   "n": N, "k": K, "m": 1, "weight_copies": COPIES,
                   "pct_of_peak": round(100 * r1["step_gbs"] / PEAK_GBS, 2),
                   "tokens_per_s": round(1 / r1["step_s"], 1),
                   "ms_per_step_two_launches": round(r1["two_s"] * 1e3, 5)},
        "roofline": roofline(1, r1),
        "step_launches": ("direct (no graph boundary inside the timed region)"
                          if r1["launch_mode"] == "direct" else "one captured HIP graph of the timed steps"),
        "settle": {"ms": SETTLE_MS,
                   "note": "untimed load run before each timed region (the m = 1 product over the "
                           "rotating copies ahead of the warm-up steps; the region's own launches "
                           "elsewhere) so that the clocks have left their idle state"},
        "cache_resident_us_per_launch": {
            "m1": round(r1["warm_s"] * 1e6, 3), "m8": round(r8["warm_s"] * 1e6, 3),
            "note": "same weight copy every launch (fits the Infinity Cache); not a roofline figure"},
        "m8": {"value": round(r8["step_gbs"], 1), "unit": "GB/s",
               "ms_per_step": round(r8["step_s"] * 1e3, 5),
               "ms_per_step_two_calls": round(r8["two_s"] * 1e3, 5),
               "pct_of_peak": round(100 * r8["step_gbs"] / PEAK_GBS, 2),
               "tokens_per_s": round(8 / r8["step_s"], 1),
               "roofline": roofline(8, r8)},
    }
    if not args.headline_only and (only is None or "mmq" in only):
        line["mmq"] = bench_mmq(torch, q2, syn, dev, copies, case)
    del copies
    torch.cuda.synchronize()
    if not args.headline_only:
        for name in SECTIONS[2:]:
            if (only is None and name not in ON_REQUEST) or (only is not None and name in only):
                line[SECTION_KEYS[name]] = SECTION_FNS[name](torch, q2, syn, dev)
                torch.cuda.synchronize()
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(line), flush=True)


def pmc_calibration(args):
    """For counter runs: a plain device copy of known size, then a few
    products at m = 1 and m = 8 on distinct weight copies."""
    import torch

    import q2_quantized_decode_amd as q2
    from q2_quantized_decode_amd import synthetic as syn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = syn.large_verify_case(m=8)
    w0 = torch.from_numpy(case.w.reshape(-1)).to(dev)
    copies = [w0] + [w0.clone() for _ in range(7)]
    x8 = syn.bf16_bits_to_tensor(case.x_bits).to(dev)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    for m in (1, 8):
        x = x8[:m].contiguous()
        xq = q2.q8_1_rows(x)
        y = torch.empty((m, N), dtype=torch.float32, device=dev)
        for i in range(8):
            q2.q2k_mmvq(copies[i], xq, N, K, m, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 4, "mmvq_launches_per_m": 8}))


def _pmc_rows(path: str, counter: str):
    import csv
    with open(path, newline="") as f:
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(f)
                if r["Counter_Name"] == counter]


def traffic_from(fetch_csv: str, write_csv: str, out: str):
    """HBM bytes per product launch from two rocprofv3 --pmc runs of
    --pmc-calibration (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch). Each
    counter is scaled by the factor that makes it read COPY_BYTES for the
    calibration copies (read COPY_BYTES, write COPY_BYTES)."""
    rec = {"commands": [
        "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE -d <out>/pmc_fetch -o f "
        "--output-format csv -- python3 /root/repo/bench.py --pmc-calibration",
        "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE -d <out>/pmc_write -o w "
        "--output-format csv -- python3 /root/repo/bench.py --pmc-calibration",
        "python3 bench.py --traffic-from <out>/pmc_fetch/f_counter_collection.csv "
        "<out>/pmc_write/w_counter_collection.csv"],
        "calibration": f"four device copies of {COPY_BYTES} bytes (read {COPY_BYTES}, write "
                       f"{COPY_BYTES}); each counter is scaled by COPY_BYTES / its copy reading"}
    scaled = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _pmc_rows(path, counter)
        # the four COPY_BYTES copies are the largest copy dispatches
        copies = sorted(v for name, v in rows if "opy" in name)[-4:]
        if len(copies) < 4:
            raise SystemExit(f"{path}: calibration copies not found")
        factor = COPY_BYTES / (1024.0 * float(np.median(copies)))
        rec[f"{counter}_factor"] = round(factor, 4)
        for m, (kname, _) in KERNELS.items():
            vals = [v for name, v in rows if kname in name]
            if not vals:
                raise SystemExit(f"{path}: no {kname} dispatches")
            scaled.setdefault(m, {})[counter] = 1024.0 * factor * float(np.mean(vals))
    for m, (kname, _) in KERNELS.items():
        tot = scaled[m]["FETCH_SIZE"] + scaled[m]["WRITE_SIZE"]
        rec[f"m{m}"] = {"kernel": kname, "kernel_hash": kernel_hash(m),
                        "fetch_bytes": round(scaled[m]["FETCH_SIZE"]),
                        "write_bytes": round(scaled[m]["WRITE_SIZE"]),
                        "bytes_per_launch": round(tot),
                        "algorithmic_bytes": mmvq_bytes(m),
                        "ratio_to_algorithmic": round(tot / mmvq_bytes(m), 4)}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def rocprof_from(trace_csv: str, out: str):
    """The product kernel's average duration at m = 1 and m = 8 over exactly
    the dispatches the roofline's HIP events bracket (the last 640 of each
    instantiation in a rocprofv3 --kernel-trace run of --roofline-only),
    with the hash of each kernel's source, so that bench.py reports it only
    while the kernel is unchanged."""
    import csv
    with open(trace_csv, newline="") as f:
        rows = list(csv.DictReader(f))
    timed = ROOF_GRAPH * ROOF_REPS
    rec = {"command": ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d <out> -o prof "
                       "--output-format csv -- python3 /root/repo/bench.py --roofline-only; "
                       "python3 bench.py --rocprof-from <out>/prof_kernel_trace.csv"),
           "dispatches": f"per m: untimed replays for about {SETTLE_MS:g} ms, then {ROOF_REPS} timed "
                         f"replays of a {ROOF_GRAPH}-launch graph over 16 rotating weight copies; the "
                         f"average is "
                         f"over the {timed} timed dispatches (the last {timed} of the kernel)"}
    for m, inst in KERNEL_INSTANCES.items():
        hit = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
                     if inst in r["Kernel_Name"])
        if len(hit) < timed:
            raise SystemExit(f"{trace_csv}: {len(hit)} dispatches of {inst}, need {timed}")
        d = np.array([(e - s_) / 1e3 for s_, e in hit[-timed:]])
        avg_us = float(d.mean())
        span_us = (hit[-1][1] - hit[-timed][0]) / 1e3 / timed
        rec[f"m{m}"] = {"kernel": inst, "kernel_hash": kernel_hash(m), "dispatches": timed,
                        "avg_us": round(avg_us, 4), "median_us": round(float(np.median(d)), 3),
                        "p10_us": round(float(np.percentile(d, 10)), 3),
                        "p90_us": round(float(np.percentile(d, 90)), 3),
                        "span_per_dispatch_us": round(span_us, 4),
                        "algorithmic_bytes": mmvq_bytes(m),
                        "achieved_gbs": round(mmvq_bytes(m) / avg_us / 1e3, 1),
                        "frac": round(mmvq_bytes(m) / avg_us / 1e3 / PEAK_GBS, 4)}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def trace_summary(trace_csv: str) -> None:
    """Markdown table of this library's dispatches in a rocprofv3 kernel
    trace, grouped by kernel and workgroup count: dispatches, average and
    10th/50th/90th percentile durations (warm-up and capture included)."""
    import csv
    import re
    import statistics

    groups: dict = {}
    with open(trace_csv, newline="") as f:
        for r in csv.DictReader(f):
            if "q2k::" not in r["Kernel_Name"]:
                continue
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
            name = re.sub(r"\(.*", "", name).replace("void ", "")
            wgs = 1
            for ax in "XYZ":
                wgs *= int(r[f"Grid_Size_{ax}"]) // max(1, int(r[f"Workgroup_Size_{ax}"]))
            groups.setdefault((name, wgs), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| kernel | workgroups | dispatches | avg (us) | p10 | median | p90 |")
    print("|---|---|---|---|---|---|---|")
    for (name, wgs), d in sorted(groups.items(), key=lambda kv: -len(kv[1])):
        d.sort()
        def q(fr, d=d):
            return d[min(len(d) - 1, int(fr * len(d)))]
        print(f"| `{name}` | {wgs} | {len(d)} | {statistics.mean(d):.2f} | {q(0.1):.2f} | "
              f"{q(0.5):.2f} | {q(0.9):.2f} |")


def kernel_sweep_from(trace_csv: str, sweep_json: str) -> None:
    """Markdown table of a kernel trace of `--only kernels`, with the JSON
    line that same traced run printed: the product dispatches, in launch
    order, split per (shape, m, kernel) exactly as bench_kernels issues them
    (per configuration: the untimed passes the JSON records, then the timed
    replays of `launches` captured calls); the averages are over the timed
    replays only."""
    import csv
    import statistics

    rec = json.loads(open(sweep_json).read().strip().split("\n")[-1])["product_kernels"]
    with open(trace_csv, newline="") as f:
        rows = [r for r in csv.DictReader(f) if "mmvq_" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    i = 0
    print("| shape | m | matrix cores: kernel | avg (us) | packed dots: kernel | avg (us) "
          "| events: matrix cores / packed dots (us) | default choice |")
    print("|---|---|---|---|---|---|---|---|")
    for (n, k) in KERNEL_SWEEP_SHAPES:
        per = n * (k // 256) * 84
        ncopy = max(2, min(1024, -(-(1 << 30) // per)))
        launches = min(ncopy, 128)
        reps = max(2, 1024 // launches)
        for m in range(2, 9):
            cells = []
            r = rec[f"{n}x{k}_m{m}"]
            for name in ("mfma", "dots"):
                untimed = r[name + "_untimed_passes"]
                seg = rows[i:i + launches * (untimed + reps)]
                i += launches * (untimed + reps)
                names = sorted({x["Kernel_Name"].split("(")[0].replace("void ", "").replace("q2k::", "")
                                for x in seg})
                d = [(int(x["End_Timestamp"]) - int(x["Start_Timestamp"])) / 1e3
                     for x in seg[untimed * launches:]]
                cells.append((", ".join(names), statistics.mean(d)))
            print(f"| [{n}, {k}] | {m} | `{cells[0][0]}` | {cells[0][1]:.3f} | `{cells[1][0]}` | "
                  f"{cells[1][1]:.3f} | {r['mfma_us']} / {r['dots_us']} | "
                  f"{'matrix cores' if r['auto'] == 'mfma' else 'packed dots'} |")
    if i != len(rows):
        raise SystemExit(f"trace has {len(rows)} product dispatches, the sweep issues {i}")


def main():
    global SETTLE_MS
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3200)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--pmc-calibration", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed load ahead of every timed region, ms of GPU time")
    ap.add_argument("--only", default="",
                    help="comma list of workloads to run (" + ",".join(SECTIONS) + "); without "
                         "'headline' only their JSON is printed (profiling runs)")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the large-verify m = 1 and m = 8 steps (for kernel traces)")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the product launches the roofline figures time (for kernel traces)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic record from two counter runs and exit")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="print the per-kernel table of a rocprofv3 kernel trace and exit")
    ap.add_argument("--kernel-sweep-from", nargs=2, metavar=("KERNEL_TRACE_CSV", "SWEEP_JSON"),
                    help="print the per-configuration table of a kernel trace of --only kernels "
                         "and exit")
    ap.add_argument("--rocprof-from", metavar="KERNEL_TRACE_CSV",
                    help="write the product kernels' rocprofv3 averages from the kernel trace of "
                         "a --roofline-only run and exit")
    args = ap.parse_args()
    SETTLE_MS = args.settle_ms
    if args.traffic_from:
        traffic_from(*args.traffic_from, TRAFFIC_FILE)
        return
    if args.rocprof_from:
        rocprof_from(args.rocprof_from, ROCPROF_FILE)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.kernel_sweep_from:
        kernel_sweep_from(*args.kernel_sweep_from)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        raise SystemExit(2)
    if args.pmc_calibration:
        pmc_calibration(args)
    else:
        run(args)


if __name__ == "__main__":
    main()
