"""Benchmark of the Q4_0 x Q8_0 product on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c4]

A step is one whole operator call (activation quantization + product) on
inputs already resident in device memory.  The headline workload is the
Llama-3-8B vocabulary projection (128256 x 4096 Q4_0 weights, one token),
where the throughput metric is HBM bandwidth: value = algorithmic bytes per
step (Q4_0 weights + fp32 activations + fp32 output) / time per step.  The
line also carries the 512-token prefill (14336 x 4096) in int8 TOPS, the
roofline fraction of the dominant kernel (timed alone with HIP events on the
stream it runs on) and the CPU oracle timed on a bounded sample.

Weights rotate over enough copies (>= 1 GiB) that each step reads them from
HBM, not from the 256 MB last-level cache.  Before the warm-up steps the step
runs untimed for about a second so that the clocks have settled.  Prints ONE
JSON line on stdout.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 matrix peak (5.0 POP/s)
ROTATE_BYTES = 1 << 30

# HBM bytes per launch of the dominant kernels, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, each scaled by what the counter reads for the
# runtime's 512 MiB device copy in the same run); the summaries and commands
# are in profiles/.  They describe the kernels as profiled; re-profile after a
# kernel change.
TRAFFIC_BYTES = {
    ("llama3_8b_head", 1): 300577117,      # profiles/k_gemv_rows_fused_vocab_head_128256x4096_N1.md
    ("llama3_8b_head", 8): 300048329,      # profiles/k_gemv_mma_tile_vocab_head_128256x4096_N8.md (k_gemv_mma_tile)
    ("llama3_8b_prefill", 512): 98280177,   # profiles/k_prefill_14336x4096_N512.md
    ("llama3_8b_prefill_repacked", 512): 122577516,  # profiles/k_prefill_repacked_14336x4096_N512.md
    ("q8_0_weights_prefill", 512): 109794505,         # profiles/k_q8w_mm_q8_0_weights_prefill_14336x4096_N512.md
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c4", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--no-small", action="store_true", help="skip the other decode configurations (GPT-2, Llama layer, head at N=8)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of this many MiB, 5 times (a known-size kernel for "
                         "scaling HBM byte counters)")
    ap.add_argument("--profile-prefill", action="store_true",
                    help="only run the 512-token prefill (14336 x 4096) 30 times eagerly on the pages' blocks, then 30 "
                         "times on repacked weights, after a second of settling, for a profiler; prints no JSON line")
    ap.add_argument("--profile-decode", action="store_true",
                    help="only run the decode configurations (GPT-2 matrix and layer, Llama layer at N=1 and 4, the "
                         "vocabulary head at N=1 and 8) 30 steps each, eagerly, for a profiler; prints no JSON line")
    ap.add_argument("--profile-legs", action="store_true",
                    help="only run the other legs' kernels (Q8_0 weights on the head at N=1 and N=8, the fused "
                         "SwiGLU, get_rows) 20 times each, eagerly, for a profiler; prints no JSON line")
    return ap.parse_args()


def profile_legs(hip, torch):
    """Twenty eager calls of each of the bench's other legs, for rocprofv3
    (kernel trace and byte counters; the copy calibration runs first)."""
    import numpy as np
    from q4_block_quantized_amd import inputs
    dev = torch.device("cuda")
    rows, K = inputs.WORKLOADS[4].mats[0]
    Wt = torch.from_numpy(inputs.weights(4, 0, rows, K)).to(dev)
    Wq8 = hip.q8_0_quantize(Wt)
    T = hip.q4_0_quantize(Wt)
    del Wt
    for N in (1, 8):
        X = torch.from_numpy(inputs.activations(4, 0, N, K)).to(dev)
        Y = torch.empty(N, rows, device=dev)
        for _ in range(20):
            hip.mul_mat_q8_0_q8_0(Wq8, X, Y)
        torch.cuda.synchronize()
        log("Q8_0 weights %dx%d N=%d: 20 calls" % (rows, K, N))
    del Wq8
    torch.cuda.empty_cache()
    r3, K3 = inputs.WORKLOADS[3].mats[1]  # 14336 x 4096
    Wg = hip.q4_0_quantize(torch.from_numpy(inputs.weights(3, 1, r3, K3)).to(dev))
    Wu = hip.q4_0_quantize(torch.from_numpy(inputs.weights(3, 2, r3, K3)).to(dev))
    X = torch.from_numpy(inputs.activations(3, 1, 1, K3)).to(dev)
    gamma = torch.linspace(0.5, 1.5, K3, device=dev)
    beta = torch.linspace(-0.1, 0.1, K3, device=dev)
    H = torch.empty(1, r3, device=dev)
    ws = hip.fused_workspace(r3, K3, 1, device=dev)
    for _ in range(20):
        hip.mul_mat_q4_0_q8_0_swiglu(Wg, Wu, X, gamma, beta, 1e-5, H, ws)
    torch.cuda.synchronize()
    log("SwiGLU 2 x %dx%d N=1: 20 calls" % (r3, K3))
    del Wg, Wu
    ids = torch.from_numpy(np.random.default_rng(inputs.seed(4, 0, 9)).integers(0, rows, 512).astype(np.int32)).to(dev)
    out = torch.empty(512, K, device=dev)
    for _ in range(20):
        hip.q4_0_get_rows(T, K, ids, out)
    torch.cuda.synchronize()
    log("get_rows 512 ids of %dx%d: 20 calls" % (rows, K))


def profile_prefill(hip, torch):
    """Thirty eager prefill steps (activation records + k_prefill) on the
    pages' blocks, then thirty on repacked weights, for rocprofv3 (kernel
    trace and counters)."""
    for repack in (False, True):
        pm = Mats(hip, torch, 5, 512, repack=repack)
        settle(torch, lambda i: pm.step(hip, i))
        for i in range(30):
            pm.step(hip, i)
        torch.cuda.synchronize()
        log("prefill 14336x4096 N=512%s: 30 steps" % (" (repacked weights)" if repack else ""))
        del pm
        torch.cuda.empty_cache()


def profile_decode(hip, torch):
    """Thirty eager steps of each decode configuration (weights rotating over
    >= 1 GiB of copies), for rocprofv3: kernel durations without the launch
    gaps that the graph-timed figures include."""
    from q4_block_quantized_amd import inputs
    for cid, N in ((1, 1), (2, 1), (3, 1), (3, 4), (4, 1), (4, 8)):
        mats = Mats(hip, torch, cid, N)
        # several products of one token: the one-launch set as well
        fns = [mats.step] + ([mats.step_set] if N == 1 and len(mats.items) > 1 else [])
        for fn in fns:
            settle(torch, lambda i: fn(hip, i), 0.3)
            for i in range(30):
                fn(hip, i)
            torch.cuda.synchronize()
            log("%s N=%d: 30 steps%s" % (inputs.WORKLOADS[cid].name, N, " (one launch)" if fn == mats.step_set else ""))
        del mats
        torch.cuda.empty_cache()


def q4_bytes(rows, K):
    return rows * (K // 32) * 18


def step_bytes(rows, K, N):
    """Algorithmic bytes of one operator call: weights + fp32 X + fp32 Y."""
    return q4_bytes(rows, K) + N * K * 4 + N * rows * 4


def kernel_bytes(rows, K, N):
    """Algorithmic bytes of the product kernel alone: weights + the quantized
    activations it reads (32 int8 + 8-byte scale record per block) + fp32 Y."""
    return q4_bytes(rows, K) + N * (K // 32) * 40 + N * rows * 4


class Mats:
    """Device copies of one workload's weights (rotated) and activations."""

    def __init__(self, hip, torch, cid, N, repack=False):
        from q4_block_quantized_amd import inputs
        wl = inputs.WORKLOADS[cid]
        self.wl, self.N = wl, N
        self.items = []
        for m, (rows, K) in enumerate(wl.mats):
            W = torch.from_numpy(inputs.weights(cid, m, rows, K, outliers=wl.outliers)).cuda()
            Wq = hip.q4_0_quantize(W)
            del W
            if repack:  # the optional one-time repack (nibble stream + scale stream)
                Wq = hip.q4_0_repack(Wq, K)
            X = torch.from_numpy(inputs.activations(cid, m, max(wl.ns), K)[:N].copy()).cuda()
            Y = torch.empty((N, rows), dtype=torch.float32, device="cuda")
            ws = hip.workspace(rows, K, N)
            self.items.append([rows, K, [Wq], X, Y, ws])
        total = sum(q4_bytes(r, k) for r, k, *_ in self.items)
        copies = max(1, -(-ROTATE_BYTES // total))
        for it in self.items:
            it[2] += [it[2][0].clone() for _ in range(copies - 1)]
        self.copies = copies
        self.repack = repack
        torch.cuda.synchronize()

    def step(self, hip, i):
        f = hip.mul_mat_q4_0r_q8_0_ex if self.repack else hip.mul_mat_q4_0_q8_0_ex
        for rows, K, Wqs, X, Y, ws in self.items:
            f(Wqs[i % self.copies], X, ws, Y)

    def step_set(self, hip, i):
        """One token per product, every product of the workload in one launch."""
        hip.mul_mat_q4_0_q8_0_set([Wqs[i % self.copies] for rows, K, Wqs, X, Y, ws in self.items],
                                  [X for rows, K, Wqs, X, Y, ws in self.items],
                                  [Y for rows, K, Wqs, X, Y, ws in self.items])

    def kernel_only(self, hip, i):
        for rows, K, Wqs, X, Y, ws in self.items:
            hip.mul_mat_q4_0_q8_0_prepared(Wqs[i % self.copies], ws, self.N, K, Y)

    def prepare(self, hip):
        for rows, K, Wqs, X, Y, ws in self.items:
            hip.q4bq_quantize_activations(X, ws)

    def bytes_step(self):
        return sum(step_bytes(r, k, self.N) for r, k, *_ in self.items)

    def bytes_kernel(self):
        return sum(kernel_bytes(r, k, self.N) for r, k, *_ in self.items)

    def ops(self):
        return sum(2 * r * k * self.N for r, k, *_ in self.items)


def fused_step(N):
    """The operator runs as one kernel (activation quantizer fused) for one token."""
    return N == 1


def decode_kernel(K, N):
    """Name of the decode kernel the library picks: whole waves per row for one
    token on long rows (an even block count whose pairs fill at least three
    quarters of 64, 128 or 256 lanes), the task kernel otherwise."""
    nb = K // 32
    P = nb // 2
    if N == 1 and nb % 2 == 0:
        for ppl in (1, 2, 4):
            if P <= 64 * ppl:
                return "k_gemv_rows" if 4 * P >= 3 * 64 * ppl else "k_gemv"
    return "k_gemv"


def settle(torch, fn, seconds=1.0):
    """Run the step, untimed, for about a second before any measurement: an
    idle GPU ramps its clocks up over the first tenths of a second of work,
    and a measurement taken during the ramp reads several percent slow."""
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            fn(i)
            i += 1
        torch.cuda.synchronize()


REPS = 7            # timed repetitions per measurement
MIN_LOOP_MS = 20.0  # each repetition times a loop of at least this long


def timed(torch, fn, steps, warmup):
    """The timing protocol: `warmup` untimed steps, then REPS repetitions of a
    loop of L >= `steps` steps lasting at least MIN_LOOP_MS, each bracketed by
    HIP events on the current stream (the one the library launches on).
    Returns {"median", "min"} in ms per step, the per-repetition figures and
    L."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def loop(n, first):
        start.record()
        for i in range(n):
            fn(first + i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    est = loop(steps, warmup) / steps
    L = max(steps, int(np.ceil(MIN_LOOP_MS / max(est, 1e-6))))
    reps = [loop(L, warmup + steps + r * L) / L for r in range(REPS)]
    return {"median": float(np.median(reps)), "min": float(np.min(reps)), "reps_ms": [round(x, 6) for x in reps],
            "steps_per_rep": L}


def proto(t):
    """The timing record as it goes into the JSON line (microseconds)."""
    return {"median_us": round(t["median"] * 1e3, 3), "min_us": round(t["min"] * 1e3, 3), "reps": REPS,
            "steps_per_rep": t["steps_per_rep"], "loop_ms_min": round(t["min"] * t["steps_per_rep"], 2)}


def multi_matrix(hip, torch, args):
    from q4_block_quantized_amd import inputs
    wl = inputs.WORKLOADS[3]
    mats = [(m, rk) for m, rk in enumerate(wl.mats) if rk[1] == 4096]
    base = [hip.q4_0_quantize(torch.from_numpy(inputs.weights(3, m, r, k, outliers=wl.outliers)).cuda())
            for m, (r, k) in mats]
    total = sum(q4_bytes(r, k) for _, (r, k) in mats)
    copies = max(1, -(-ROTATE_BYTES // total))
    sets = [base] + [[w.clone() for w in base] for _ in range(copies - 1)]
    X = torch.from_numpy(inputs.activations(3, 0, max(wl.ns), 4096)[:1].copy()).cuda()
    Ys = [torch.empty((1, r), dtype=torch.float32, device="cuda") for _, (r, _k) in mats]
    ws = hip.workspace(max(r for _, (r, _k) in mats), 4096, 1)
    ms_one = timed(torch, lambda i: hip.mul_mat_q4_0_q8_0_multi(sets[i % copies], X, Ys), args.steps,
                   args.warmup)["median"]
    def sep(i):
        for w, y in zip(sets[i % copies], Ys):
            hip.mul_mat_q4_0_q8_0_ex(w, X, ws, y)
    ms_sep = timed(torch, sep, args.steps, args.warmup)["median"]
    nbytes = sum(step_bytes(r, k, 1) for _, (r, k) in mats)
    log("multi-matrix decode (%s): one launch %.2f us, one call per matrix %.2f us"
        % (" + ".join("%dx%d" % rk for _, rk in mats), ms_one * 1e3, ms_sep * 1e3))
    del sets, base
    torch.cuda.empty_cache()
    return {"workload": "llama3_8b_decode matrices with K=4096: " + ", ".join("%dx%d" % rk for _, rk in mats),
            "N": 1, "one_launch_us": round(ms_one * 1e3, 3), "per_matrix_calls_us": round(ms_sep * 1e3, 3),
            "one_launch_GB/s": round(nbytes / (ms_one * 1e-3) / 1e9, 1)}


def graph_timed(torch, fn, n_steps, replays):
    """Per-step time of n_steps consecutive steps captured in one HIP graph and
    replayed: the device time of back-to-back operator calls, without the
    host's per-call cost."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_steps):
            fn(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (replays * n_steps), g


def decode_configs(hip, torch):
    """The other decode configurations (GPT-2 matrices, the Llama layer's three
    matrices at one and four tokens, the vocabulary head at eight tokens),
    whose steps run from a HIP graph so that the host's per-call cost of the
    short ones is not counted.  Every replay's output is checked against an
    eager call."""
    from q4_block_quantized_amd import inputs
    res = []
    for cid, N in ((1, 1), (2, 1), (3, 1), (3, 4), (4, 8)):
        wl = inputs.WORKLOADS[cid]
        mats = Mats(hip, torch, cid, N)
        # several products of one token: one launch for all of them
        # (mul_mat_q4_0_q8_0_set), the separate calls timed beside it
        paths = [("separate", mats.step)]
        if N == 1 and len(mats.items) > 1:
            paths.insert(0, ("set", mats.step_set))
        timed_paths = {}
        for pname, fn in paths:
            fn(hip, 0)
            torch.cuda.synchronize()
            ref = [it[4].clone() for it in mats.items]
            settle(torch, lambda i: fn(hip, i), 0.3)
            n_steps = mats.copies
            replays = max(3, int(0.05 / max(n_steps * len(mats.items) * 4e-6, 1e-9)))
            ms, g = graph_timed(torch, lambda i: fn(hip, i), n_steps, replays)
            same = all(torch.equal(it[4], r) for it, r in zip(mats.items, ref))
            if not same:
                raise RuntimeError("graph replay of %s N=%d (%s) differs from the eager call" % (wl.name, N, pname))
            timed_paths[pname] = (ms, ref)
            del g
        if "set" in timed_paths and not all(torch.equal(a, b) for a, b in zip(timed_paths["set"][1],
                                                                             timed_paths["separate"][1])):
            raise RuntimeError("%s: the one-launch set differs from the separate calls" % wl.name)
        # the step: the faster of the library's two forms (both are reported)
        pname = min(timed_paths, key=lambda k: timed_paths[k][0])
        ms = timed_paths[pname][0]
        gbs = mats.bytes_step() / (ms * 1e-3) / 1e9
        log("%s N=%d: %.2f us per step (%s, HIP graph) -> %.1f GB/s"
            % (wl.name, N, ms * 1e3, "one launch" if pname == "set" else "%d launches" % len(mats.items), gbs))
        res.append({"workload": wl.name, "N": N, "matrices": [list(m) for m in wl.mats],
                    "us_per_step": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
                    "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                    "form": "mul_mat_q4_0_q8_0_set (one launch)" if pname == "set" else "one call per matrix"})
        if "set" in timed_paths:
            res[-1]["set_us_per_step"] = round(timed_paths["set"][0] * 1e3, 3)
            res[-1]["separate_calls_us_per_step"] = round(timed_paths["separate"][0] * 1e3, 3)
            log("   one launch: %.2f us, separate calls: %.2f us per step"
                % (timed_paths["set"][0] * 1e3, timed_paths["separate"][0] * 1e3))
        if N > 1 and (wl.name, N) in TRAFFIC_BYTES:  # the product kernel's counted HBM bytes per launch
            res[-1]["traffic_product_kernel"] = TRAFFIC_BYTES[(wl.name, N)]
        del mats
        torch.cuda.empty_cache()
    return res


def get_rows_leg(hip, torch):
    """Q4_0 get_rows (decoded embedding rows) on the Llama-3-8B-shaped token
    table (128256 x 4096), for a 512-token batch and one token; device time
    from HIP graphs, each replay's output checked against an eager call.
    Algorithmic bytes: the selected Q4_0 rows, the int32 ids and the fp32
    output (7x the rows read)."""
    from q4_block_quantized_amd import inputs
    rows, K = 128256, 4096
    W = torch.from_numpy(inputs.weights(4, 0, rows, K)).cuda()
    Wq = hip.q4_0_quantize(W)
    del W
    res = []
    for n in (512, 1):
        ids = torch.from_numpy(np.random.default_rng(11 + n).integers(0, rows, n).astype(np.int32)).cuda()
        out = torch.empty((n, K), dtype=torch.float32, device="cuda")
        fn = lambda i: hip.q4_0_get_rows(Wq, K, ids, out)
        fn(0)
        torch.cuda.synchronize()
        ref = out.clone()
        ms, g = graph_timed(torch, fn, 20, 50)
        if not torch.equal(out, ref):
            raise RuntimeError("graph replay of get_rows n=%d differs from the eager call" % n)
        nbytes = n * (K // 32 * 18 + 4 + K * 4)
        gbs = nbytes / (ms * 1e-3) / 1e9
        log("get_rows 128256x4096 table, %d ids: %.2f us -> %.1f GB/s" % (n, ms * 1e3, gbs))
        res.append({"table": [rows, K], "n": n, "us_per_call": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
                    "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
        del g
    del Wq
    torch.cuda.empty_cache()
    return res


def q8w_leg(hip, torch):
    """Q8_0 weights (Q8_0 blocks of 34 bytes from the same Q8_0 rule as the
    activations) at N = 1 and N = 8 on the vocabulary head (128256 x 4096) and
    the Llama MLP matrix (14336 x 4096); weights rotate over >= 1 GiB of copies
    so every step reads HBM; device time from HIP graphs, each replay checked
    against an eager call.  Algorithmic bytes: Q8_0 weights + fp32 X + fp32 Y."""
    from q4_block_quantized_amd import inputs
    res = []
    for cid, rows, K in ((4, 128256, 4096), (5, 14336, 4096)):
        Wq8 = hip.q8_0_quantize(torch.from_numpy(inputs.weights(cid, 0, rows, K)).cuda())
        wbytes = rows * (K // 32) * 34
        copies = max(2, -(-ROTATE_BYTES // wbytes))
        Ws = [Wq8] + [Wq8.clone() for _ in range(copies - 1)]
        for N in (1, 8):
            X = torch.from_numpy(inputs.activations(cid, 0, N, K).copy()).cuda()
            Y = torch.empty((N, rows), dtype=torch.float32, device="cuda")
            fn = lambda i: hip.mul_mat_q8_0_q8_0(Ws[i % copies], X, Y)
            fn(0)
            torch.cuda.synchronize()
            ref = Y.clone()
            settle(torch, fn, 0.3)
            ms, g = graph_timed(torch, fn, copies, max(3, int(0.05 / (copies * wbytes / 6e12))))
            if not torch.equal(Y, ref):
                raise RuntimeError("graph replay of the Q8_0-weight product differs from the eager call")
            nbytes = wbytes + N * K * 4 + N * rows * 4
            gbs = nbytes / (ms * 1e-3) / 1e9
            log("Q8_0 weights %dx%d N=%d: %.2f us -> %.1f GB/s" % (rows, K, N, ms * 1e3, gbs))
            res.append({"matrix": [rows, K], "N": N, "us_per_call": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
                        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
            del g
        del Ws, Wq8
        torch.cuda.empty_cache()
    return res


def q8w_prefill_leg(hip, torch, args, peaks):
    """Q8_0 weights against 512 tokens (14336 x 4096, the prefill shape) on the
    int8 matrix-core kernel: the whole call (activation records + product),
    timed by the protocol; weights rotate over >= 1 GiB.  Throughput in
    int8-equivalent TOPS (2 rows K N), against the int8 MFMA peak."""
    from q4_block_quantized_amd import inputs
    rows, K, N = 14336, 4096, 512
    Wq8 = hip.q8_0_quantize(torch.from_numpy(inputs.weights(5, 0, rows, K)).cuda())
    copies = max(2, -(-ROTATE_BYTES // (rows * (K // 32) * 34)))
    Ws = [Wq8] + [Wq8.clone() for _ in range(copies - 1)]
    X = torch.from_numpy(inputs.activations(5, 0, N, K)).cuda()
    Y = torch.empty((N, rows), dtype=torch.float32, device="cuda")
    fn = lambda i: hip.mul_mat_q8_0_q8_0(Ws[i % copies], X, Y)
    settle(torch, fn, 0.3)
    t = timed(torch, fn, max(10, args.steps // 4), max(3, args.warmup // 4))
    tops = 2 * rows * K * N / (t["median"] * 1e-3) / 1e12
    log("Q8_0 weights prefill %dx%d N=%d: %.2f us -> %.1f TOPS" % (rows, K, N, t["median"] * 1e3, tops))
    del Ws, Wq8
    torch.cuda.empty_cache()
    return {"matrix": [rows, K], "N": N, "kernel": "k_act8_from_f32 + k_q8w_mm (int8 MFMA)",
            "us_per_call": round(t["median"] * 1e3, 3), "TOPS": round(tops, 1), "timing": proto(t),
            "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
            "frac_of_measured_int8_peak": round(tops / peaks["mfma_int8_TOPS"], 4),
            "traffic_k_q8w_mm": TRAFFIC_BYTES.get(("q8_0_weights_prefill", N))}


def fused_leg(hip, torch):
    """The steps around the product, fused (HIP graphs, each replay checked
    against an eager call; weights rotate over >= 1 GiB):
      * Llama-3-8B feed-forward first half at one token: LayerNorm, the gate
        and up products (14336 x 4096 each) and SiLU(gate) * up in
        mul_mat_q4_0_q8_0_swiglu, against the two bare products;
      * GPT-2's c_mlp_fc (3072 x 768) at one token with LayerNorm, bias and
        GELU (mul_mat_q4_0_q8_0_fused), against the bare product.
    Bytes: the Q4_0 weights + fp32 X + fp32 outputs of the fused call."""
    from q4_block_quantized_amd import inputs
    res = []
    # Llama SwiGLU
    rows, K = 14336, 4096
    Wg = hip.q4_0_quantize(torch.from_numpy(inputs.weights(3, 1, rows, K, outliers=True)).cuda())
    Wu = hip.q4_0_quantize(torch.from_numpy(inputs.weights(3, 4, rows, K, outliers=True)).cuda())
    wbytes = 2 * q4_bytes(rows, K)
    copies = max(1, -(-ROTATE_BYTES // wbytes))
    sets = [(Wg, Wu)] + [(Wg.clone(), Wu.clone()) for _ in range(copies - 1)]
    X = torch.from_numpy(inputs.activations(3, 0, 1, K).copy()).cuda()
    g = torch.from_numpy(inputs.random_matrix(5500, 1, K, 0.5)[0] + 1.0).cuda()
    b = torch.from_numpy(inputs.random_matrix(5501, 1, K, 0.1)[0]).cuda()
    H = torch.empty((1, rows), dtype=torch.float32, device="cuda")
    Y2 = torch.empty((2, 1, rows), dtype=torch.float32, device="cuda")
    ws = hip.fused_workspace(rows, K, 1)
    fused = lambda i: hip.mul_mat_q4_0_q8_0_swiglu(sets[i % copies][0], sets[i % copies][1], X, g, b, 1e-5, H, ws)
    def bare(i):
        hip.mul_mat_q4_0_q8_0(sets[i % copies][0], X, Y2[0])
        hip.mul_mat_q4_0_q8_0(sets[i % copies][1], X, Y2[1])
    for name, fn, out in (("swiglu", fused, H), ("bare", bare, Y2)):
        fn(0)
        torch.cuda.synchronize()
        ref = out.clone()
        settle(torch, fn, 0.3)
        ms, gr = graph_timed(torch, fn, copies, 40)
        if not torch.equal(out, ref):
            raise RuntimeError("graph replay of the %s leg differs from the eager call" % name)
        del gr
        if name == "swiglu":
            ms_fused = ms
        else:
            ms_bare = ms
    nbytes = wbytes + K * 4 + rows * 4
    log("Llama SwiGLU (LayerNorm + gate + up + SiLU*up), N=1: %.2f us (bare products %.2f us) -> %.1f GB/s"
        % (ms_fused * 1e3, ms_bare * 1e3, nbytes / (ms_fused * 1e-3) / 1e9))
    res.append({"workload": "llama3_8b ffn gate+up 2 x 14336x4096, LayerNorm, SiLU(gate)*up", "N": 1,
                "fused_us": round(ms_fused * 1e3, 3), "bare_products_us": round(ms_bare * 1e3, 3),
                "GB/s": round(nbytes / (ms_fused * 1e-3) / 1e9, 1)})
    del sets, Wg, Wu
    torch.cuda.empty_cache()
    # GPT-2 c_mlp_fc with LayerNorm, bias, GELU
    rows, K = 3072, 768
    W = hip.q4_0_quantize(torch.from_numpy(inputs.weights(2, 2, rows, K)).cuda())
    copies = max(1, -(-ROTATE_BYTES // q4_bytes(rows, K)))
    Ws = [W] + [W.clone() for _ in range(copies - 1)]
    X = torch.from_numpy(inputs.activations(2, 2, 1, K).copy()).cuda()
    g = torch.from_numpy(inputs.random_matrix(5600, 1, K, 0.5)[0] + 1.0).cuda()
    b = torch.from_numpy(inputs.random_matrix(5601, 1, K, 0.1)[0]).cuda()
    bias = torch.from_numpy(inputs.random_matrix(5602, 1, rows, 0.1)[0]).cuda()
    Y = torch.empty((1, rows), dtype=torch.float32, device="cuda")
    ws = hip.fused_workspace(rows, K, 1)
    fused = lambda i: hip.mul_mat_q4_0_q8_0_fused(Ws[i % copies], X, g, b, 1e-5, bias, hip.ACT_GELU, None, Y, ws)
    bare = lambda i: hip.mul_mat_q4_0_q8_0(Ws[i % copies], X, Y)
    out = {}
    for name, fn in (("fused", fused), ("bare", bare)):
        fn(0)
        torch.cuda.synchronize()
        ref = Y.clone()
        settle(torch, fn, 0.3)
        ms, gr = graph_timed(torch, fn, min(copies, 64), 40)
        if not torch.equal(Y, ref):
            raise RuntimeError("graph replay of the GPT-2 %s leg differs from the eager call" % name)
        del gr
        out[name] = ms
    log("GPT-2 c_mlp_fc (LayerNorm + product + bias + GELU), N=1: %.2f us (bare product %.2f us)"
        % (out["fused"] * 1e3, out["bare"] * 1e3))
    res.append({"workload": "gpt2 c_mlp_fc 3072x768, LayerNorm, bias, GELU", "N": 1,
                "fused_us": round(out["fused"] * 1e3, 3), "bare_product_us": round(out["bare"] * 1e3, 3)})
    del Ws, W
    torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(fn, seconds):
    """Runs fn until `seconds` have passed (at least once); seconds per run."""
    runs, t0 = 0, time.perf_counter()
    while True:
        fn()
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return el / runs, runs, el


def cpu_baseline(N_decode, seconds=3.0):
    """The oracle as it stands (plain C loops, fp64 accumulation, threads over
    rows) on bounded samples of the headline decode workload and of the
    512-token prefill, each on one thread and on all the cores this process
    may use (capped at 16: the share of a one-GPU job on a shared host).
    Rates are scaled to the metrics' units: GB/s of the operator's
    algorithmic bytes for the decode, int8-equivalent TOPS for the prefill."""
    import oracle
    from q4_block_quantized_amd import inputs
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    allc = max(1, min(avail, 16))
    # decode: the first 16384 rows of the 128256 x 4096 head, one token
    wl = inputs.WORKLOADS[4]
    rows, K = wl.mats[0]
    take = 16384
    Wq = oracle.q4_0_quantize(inputs.weights(4, 0, rows, K, outliers=wl.outliers, row_slice=slice(0, take)))
    X = inputs.activations(4, 0, max(wl.ns), K)[:N_decode].copy()
    dec = {}
    for label, th in (("one_thread", 1), ("all_cores", allc)):
        per, runs, el = _oracle_rate(lambda: oracle.mul_mat(Wq, X, nthreads=th), seconds)
        dec[label] = {"GB/s": round(step_bytes(take, K, N_decode) / per / 1e9, 3), "threads": th,
                      "ms_per_run": round(per * 1e3, 2), "runs": runs}
    # prefill: 112 rows of the 14336 x 4096 matrix against all 512 tokens
    wl5 = inputs.WORKLOADS[5]
    r5, K5 = wl5.mats[0]
    t5 = 112
    Wq5 = oracle.q4_0_quantize(inputs.weights(5, 0, r5, K5, outliers=wl5.outliers, row_slice=slice(0, t5)))
    X5 = inputs.activations(5, 0, 512, K5)
    pre = {}
    for label, th in (("one_thread", 1), ("all_cores", allc)):
        per, runs, el = _oracle_rate(lambda: oracle.mul_mat(Wq5, X5, nthreads=th), seconds)
        pre[label] = {"TOPS": round(2 * t5 * K5 * 512 / per / 1e12, 5), "threads": th,
                      "ms_per_run": round(per * 1e3, 1), "runs": runs}
    return {"value": dec["all_cores"]["GB/s"], "unit": "GB/s", "cores": allc, "kind": "oracle",
            "sample": "decode: rows 0..%d of the %dx%d head, N=%d (per leg >= %.0f s of runs); the whole operator "
                      "(Q8_0 quantization of X, int32 block dots, fp64 accumulation)" % (take - 1, rows, K, N_decode,
                                                                                      seconds),
            "decode": dec,
            "prefill": {"sample": "rows 0..%d of the %dx%d matrix x 512 tokens" % (t5 - 1, r5, K5), **pre},
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(), "cores_available": avail}


def measured_peaks(torch):
    """Peak rates of this GPU for the instructions the kernels use (the probe
    library), each the best of three launches timed with HIP events."""
    import ctypes
    from q4_block_quantized_amd import build as qb
    L = ctypes.CDLL(qb.PROBE_LIB)
    L.q4bq_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.q4bq_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.q4bq_probe_ops.restype = ctypes.c_double
    L.q4bq_probe_ops.argtypes = [ctypes.c_int, ctypes.c_int64]
    out = torch.empty(L.q4bq_probe_threads(), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(launch, count):
        t = []
        for _ in range(4):
            ev0.record()
            if launch() != 0:
                raise RuntimeError("probe launch failed")
            ev1.record()
            torch.cuda.synchronize()
            t.append(ev0.elapsed_time(ev1) * 1e-3)
        return count / min(t[1:])

    res = {}
    for kind, name, iters in ((0, "mfma_int8_TOPS", 4000), (1, "mfma_fp6_TFLOPS", 4000),
                              (2, "mfma_f16_32x32x8_TFLOPS", 4000), (3, "valu_fp32_fma_TFLOPS", 20000)):
        ops = L.q4bq_probe_ops(kind, iters)
        res[name] = round(best(lambda: L.q4bq_probe_mfma(kind, iters, out.data_ptr(), stream.cuda_stream), ops)
                          / 1e12, 1)
    buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    res["stream_read_GB/s"] = round(best(lambda: L.q4bq_probe_read(buf.data_ptr(), buf.numel(), out.data_ptr(),
                                                                    stream.cuda_stream), buf.numel()) / 1e9, 1)
    # the same probe over the vocabulary head's weight bytes (ramp and tail
    # weigh as much as in the decode launch), three buffers rotated
    head = (q4_bytes(128256, 4096) + 15) // 16 * 16
    ptrs = [buf.data_ptr() + i * ((head + 4095) // 4096 * 4096) for i in range(3)]
    cnt = [0]

    def rot():
        cnt[0] += 1
        return L.q4bq_probe_read(ptrs[cnt[0] % 3], head, out.data_ptr(), stream.cuda_stream)
    res["stream_read_head_bytes_GB/s"] = round(best(rot, head) / 1e9, 1)
    del buf
    torch.cuda.empty_cache()
    return res


def prefill_ceiling(rows, K, N, peaks):
    """Lower bounds on the prefill kernel's time from its work at the measured
    peak rates: per 32-token x 32-row tile and 32-value block one fp6 MFMA
    (32x32x64: the block dot, exact), one f16 MFMA (32x32x8: the 1024 scale
    products) and 1024 fp32 FMAs on the vector ALU.  'overlapped' assumes the
    matrix cores and the vector ALU run side by side, 'serial' one after the
    other."""
    tiles = (rows / 32) * (N / 32) * (K / 32)
    t_fp6 = tiles * 2 * 32 * 32 * 64 / (peaks["mfma_fp6_TFLOPS"] * 1e12)
    t_f16 = tiles * 2 * 32 * 32 * 8 / (peaks["mfma_f16_32x32x8_TFLOPS"] * 1e12)
    t_valu = tiles * 1024 * 2 / (peaks["valu_fp32_fma_TFLOPS"] * 1e12)
    ops = 2 * rows * K * N
    over = max(t_fp6 + t_f16, t_valu)
    return {"mfma_us": round((t_fp6 + t_f16) * 1e6, 2), "valu_us": round(t_valu * 1e6, 2),
            "overlapped_us": round(over * 1e6, 2), "serial_us": round((t_fp6 + t_f16 + t_valu) * 1e6, 2),
            "overlapped_TOPS": round(ops / over / 1e12, 1),
            "overlapped_frac_of_int8_peak": round(ops / over / 1e12 / INT8_PEAK_TOPS, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    from q4_block_quantized_amd import binding as hip
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(2)
    hip.lib()
    if args.copy_calib:
        n = args.copy_calib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 5 x %d bytes" % n)
        del src, dst
    if args.profile_legs:
        profile_legs(hip, torch)
        return
    if args.profile_decode:
        profile_decode(hip, torch)
        return
    if args.profile_prefill:
        profile_prefill(hip, torch)
        return
    cid = int(args.workload[1])
    from q4_block_quantized_amd import inputs
    wl = inputs.WORKLOADS[cid]
    N = wl.ns[0]

    peaks = measured_peaks(torch)
    log("measured peaks: %s" % json.dumps(peaks))

    log("workload %s N=%d: preparing" % (wl.name, N))
    mats = Mats(hip, torch, cid, N)
    n_launch = len(mats.items)
    settle(torch, lambda i: mats.step(hip, i))
    t_step = timed(torch, lambda i: mats.step(hip, i), args.steps, args.warmup)
    ms_step = t_step["median"]
    gbs = mats.bytes_step() / (ms_step * 1e-3) / 1e9
    # two-phase form: activation quantizer once, then the product kernel alone
    mats.prepare(hip)
    t_kernel = timed(torch, lambda i: mats.kernel_only(hip, i), args.steps, args.warmup)
    ms_kernel = t_kernel["median"]
    kern_gbs = mats.bytes_kernel() / (ms_kernel * 1e-3) / 1e9
    log("step %.2f us (min %.2f) -> %.1f GB/s; two-phase product kernel %.2f us/launch -> %.1f GB/s"
        % (ms_step * 1e3, t_step["min"] * 1e3, gbs, ms_kernel * 1e3 / n_launch, kern_gbs))
    if fused_step(N):
        # one kernel per matrix: the step is the dominant kernel
        roof = {"kernel": decode_kernel(mats.items[0][1], N) + " (fused activation quantizer)", "achieved": gbs,
                "ms": ms_step, "t": t_step,
                "bytes": mats.bytes_step() // n_launch}
    else:
        roof = {"kernel": decode_kernel(mats.items[0][1], N) + " (product kernel alone)", "achieved": kern_gbs,
                "ms": ms_kernel, "t": t_kernel,
                "bytes": mats.bytes_kernel() // n_launch}
    del mats
    torch.cuda.empty_cache()
    # the same step on repacked weights (q4_0_repack, done once, outside the timed region)
    rmats = Mats(hip, torch, cid, N, repack=True)
    t_r = timed(torch, lambda i: rmats.step(hip, i), args.steps, args.warmup)
    rgbs = rmats.bytes_step() / (t_r["median"] * 1e-3) / 1e9
    log("repacked weights: step %.2f us -> %.1f GB/s" % (t_r["median"] * 1e3, rgbs))
    repacked = {"decode": {"ms_per_step": round(t_r["median"], 5), "GB/s": round(rgbs, 1), "timing": proto(t_r)}}
    del rmats
    torch.cuda.empty_cache()

    # several matrices sharing one token (the Llama decode set's two K = 4096
    # matrices): one launch against one call per matrix
    multi = multi_matrix(hip, torch, args)

    # the other decode configurations, device time from HIP graphs
    small = None if args.no_small else decode_configs(hip, torch)
    rows_lookup = None if args.no_small else get_rows_leg(hip, torch)
    q8_weights = None if args.no_small else q8w_leg(hip, torch)
    fusion = None if args.no_small else fused_leg(hip, torch)
    q8w_prefill = None if args.no_prefill else q8w_prefill_leg(hip, torch, args, peaks)

    prefill = None
    if not args.no_prefill:
        log("prefill: preparing")
        pm = Mats(hip, torch, 5, 512)
        settle(torch, lambda i: pm.step(hip, i))  # clocks settle again under the matrix-core load
        t_p = timed(torch, lambda i: pm.step(hip, i), max(10, args.steps // 4), max(3, args.warmup // 4))
        pm.prepare(hip)
        t_pk = timed(torch, lambda i: pm.kernel_only(hip, i), max(10, args.steps // 4), max(3, args.warmup // 4))
        ms_p, ms_pk = t_p["median"], t_pk["median"]
        tops = pm.ops() / (ms_p * 1e-3) / 1e12
        ktops = pm.ops() / (ms_pk * 1e-3) / 1e12
        log("prefill step %.2f us -> %.1f TOPS; kernel %.2f us -> %.1f TOPS" % (ms_p * 1e3, tops, ms_pk * 1e3, ktops))
        ceil = prefill_ceiling(14336, 4096, 512, peaks)
        prefill = {"workload": "llama3_8b_prefill", "rows": 14336, "K": 4096, "N": 512,
                   "ms_per_step": round(ms_p, 5), "value": round(tops, 2), "unit": "TOPS (int8)",
                   "timing": proto(t_p),
                   "roofline": {"bound": "mfma", "achieved": round(ktops, 2), "peak": INT8_PEAK_TOPS,
                                "unit": "TOPS", "frac": round(ktops / INT8_PEAK_TOPS, 4),
                                "traffic": TRAFFIC_BYTES.get(("llama3_8b_prefill", 512)),
                                "kernel": "k_prefill", "us_per_launch": round(ms_pk * 1e3, 3),
                                "timing": proto(t_pk),
                                "frac_of_measured_int8_peak": round(ktops / peaks["mfma_int8_TOPS"], 4),
                                "ceiling_mfma_plus_valu": ceil,
                                "frac_of_overlapped_ceiling": round(ktops / ceil["overlapped_TOPS"], 4)}}
        del pm
        torch.cuda.empty_cache()
        rpm = Mats(hip, torch, 5, 512, repack=True)
        settle(torch, lambda i: rpm.step(hip, i), 0.3)
        t_rp = timed(torch, lambda i: rpm.step(hip, i), max(10, args.steps // 4), max(3, args.warmup // 4))
        rtops = rpm.ops() / (t_rp["median"] * 1e-3) / 1e12
        log("repacked weights: prefill step %.2f us -> %.1f TOPS" % (t_rp["median"] * 1e3, rtops))
        repacked["prefill"] = {"ms_per_step": round(t_rp["median"], 5), "TOPS": round(rtops, 2),
                               "timing": proto(t_rp),
                               "traffic_k_prefill": TRAFFIC_BYTES.get(("llama3_8b_prefill_repacked", 512))}
        del rpm
        torch.cuda.empty_cache()

    cpu = None if args.no_cpu else cpu_baseline(N)

    out = {
        "metric": "Q4_0xQ8_0 mul_mat HBM bandwidth (GB/s, N=1 decode)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4xint8->int32, fp32 scale/accumulate", "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations)",
        "config": {"workload": wl.name, "matrices": [list(m) for m in wl.mats], "N": N,
                   "weights_cold": "rotating copies >= 1 GiB"},
        "timing": dict(proto(t_step), note="value and ms_per_step are the median of %d repetitions" % REPS),
        "roofline": {"bound": "hbm", "achieved": round(roof["achieved"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(roof["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": TRAFFIC_BYTES.get((wl.name, N)) if fused_step(N) else None,
                     "kernel": roof["kernel"], "bytes_per_launch": roof["bytes"],
                     "us_per_launch": round(roof["ms"] * 1e3 / n_launch, 3),
                     "us_per_launch_min": round(roof["t"]["min"] * 1e3 / n_launch, 3),
                     "frac_of_measured_stream_read": round(roof["achieved"] / peaks["stream_read_head_bytes_GB/s"], 4)},
        "two_phase_product_kernel": {"us_per_launch": round(ms_kernel * 1e3 / n_launch, 3),
                                     "GB/s": round(kern_gbs, 1), "timing": proto(t_kernel)},
        "measured_peaks": peaks,
        "prefill": prefill,
        "repacked_weights": repacked,
        "multi_matrix_decode": multi,
        "decode_configs_graph": small,
        "get_rows_graph": rows_lookup,
        "q8_0_weights_graph": q8_weights,
        "q8_0_weights_prefill": q8w_prefill,
        "fused_graph": fusion,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
