"""Benchmark: full exact solve of the n = 1024, c = 1, 24-bit system on one MI355X.

A step is one full solve through the C ABI (es_solve_device): inputs already
resident in HBM, output as host limbs (numerators and denominators in lowest
terms) -- the checks, residues, batched Gauss-Jordan inverse, the lift, the
digit copy and the host reconstruction.  W warm-up steps, then K timed steps
bracketed by device synchronisation.  One JSON line goes to stdout.

Extra passes (outside the timed region): one profiled solve with HIP events
around every hot-kernel launch gives each kernel's average launch duration,
from which the roofline fractions are computed; the benched output is checked
against the oracle's stored digest; and the CPU oracle (plain-C Bareiss) is
timed on a bounded sample of the same workload (its first elimination steps)
and projected to a full solve.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, TOP/s
# VALU rates from the unit counts: 256 CUs x 4 SIMDs x 16 lanes at 2.4 GHz for a
# full-rate 32-bit operation; a 64-bit integer multiply-add (v_mad_u64_u32) issues
# at a quarter of that
INT32_VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12          # 39.3
INT64_MAD_PEAK_TOPS = INT32_VALU_PEAK_TOPS / 4               # 9.83
PAGES_MS_C4 = {"rtx_pro_6000": 2411.0, "h200": 2235.0}   # card, "Measured" table, n=1024 c=1


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="c4_n1024_int24")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0,
                    help="approximate seconds for the oracle's measured first steps")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--sweep", action="store_true", help="time every workload and print a table")
    ap.add_argument("--no-multi-column", dest="multi_column", action="store_false",
                    help="skip the short n = 2048, c = 16 block")
    return ap.parse_args()


MULTI_COLUMN = "c5_n2048_c16_int24"


def digest(pairs):
    def h(v):
        return ("-" + format(-v, "x")) if v < 0 else format(v, "x")
    return hashlib.sha256("".join(f"{h(p)} {h(q)}\n" for row in pairs for (p, q) in row).encode()).hexdigest()


class Solver:
    """Raw C-ABI solves on torch-allocated device memory and the current stream.

    Holds several inputs of one shape, all resident in HBM: input 0 is the
    workload's canonical draw, the others are its seeded redraws, so that
    consecutive solves never see the same system."""

    def __init__(self, inputs):
        import torch
        import dixon_adic_lifting_amd as es
        from dixon_adic_lifting_amd import _lib
        self.torch, self.es, self._lib = torch, es, _lib
        self.lib = _lib.load()
        self.dev = torch.device("cuda", 0)
        self.inputs = [(torch.as_tensor(A, device=self.dev).contiguous(), torch.as_tensor(b, device=self.dev).contiguous())
                       for (A, b) in inputs]
        self.n, self.c = self.inputs[0][0].shape[0], self.inputs[0][1].shape[1]
        self.ws = torch.empty(es.workspace_bytes(self.n, self.c), dtype=torch.uint8, device=self.dev)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream(self.dev).cuda_stream)

    def solve(self, idx=0, keep=False):
        A, b = self.inputs[idx % len(self.inputs)]
        sol = ctypes.c_void_p()
        st = self.lib.es_solve_device(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                      self.n, self.c, ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel(),
                                      self.stream, ctypes.byref(sol))
        if st != 0:
            raise RuntimeError(f"solve failed: {self._lib.strerror(st)}")
        if keep:
            return sol
        self.lib.es_solution_free(sol)
        return None

    def sync(self):
        self.torch.cuda.synchronize(self.dev)


MAX_DISTINCT_INPUTS = 32


def workload_inputs(name, count):
    """The workload's canonical draw and count - 1 seeded redraws (at most
    MAX_DISTINCT_INPUTS in all; a longer run cycles through them)."""
    from dixon_adic_lifting_amd import workloads as W
    return [W.generate(name, attempt=k) for k in range(max(1, min(count, MAX_DISTINCT_INPUTS)))]


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_solves(S, steps, warmup):
    """W warm-up solves on redraws 1..W, then K timed solves: the canonical
    draw, then redraws W+1, W+2, ... (each input once while there are enough)."""
    for w in range(warmup):
        t1 = time.perf_counter()
        S.solve(1 + w)
        progress(f"warmup {w + 1}/{warmup}: {1e3 * (time.perf_counter() - t1):.1f} ms")
    S.sync()
    per = []
    stage_runs = []
    order = [0] + [warmup + k for k in range(1, steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        t1 = time.perf_counter()
        S.solve(order[k])
        per.append(time.perf_counter() - t1)
        stage_runs.append(S._lib.last_timings())
        progress(f"step {k + 1}/{steps}: {1e3 * per[-1]:.1f} ms")
    S.sync()
    total = time.perf_counter() - t0
    # host-clock stage times of the timed (unprofiled) solves, median per stage
    stages = {key: sorted(r[key] for r in stage_runs)[len(stage_runs) // 2] for key in stage_runs[0]} if stage_runs else {}
    return total, per, stages


def profiled_pass(S):
    _lib = S._lib
    _lib.set_profiling(True)
    sol = S.solve(keep=True)
    S.sync()
    _lib.set_profiling(False)
    prof = _lib.kernel_profile()
    info = _lib.solution_info(sol)
    stages = _lib.last_timings()
    pairs = _lib.read_solution(sol)
    S.lib.es_solution_free(sol)
    return prof, info, stages, pairs


MOD_PRIMES = [1048573, 1048571, 1048559]   # primes below 2^20: int64 products stay exact


def verify_mod_primes(A, b, pairs):
    """A x == b modulo a few 20-bit primes for every component (a property
    that holds only for the true solution, up to a 2^-60 chance), plus lowest
    terms and positive denominators on a sample."""
    import numpy as np
    for p in MOD_PRIMES:
        try:
            xm = np.array([[(num % p) * pow(den % p, -1, p) % p for (num, den) in row] for row in pairs],
                          dtype=np.int64)
        except ValueError:
            return False
        if not np.array_equal((np.mod(A, p).astype(np.int64) @ xm) % p, np.mod(b, p)):
            return False
    for row in pairs[:: max(1, len(pairs) // 16)]:
        for (num, den) in row:
            if den <= 0 or math.gcd(num, den) != 1:
                return False
    return True


def kernel_sources_sha256():
    """SHA-256 over the HIP kernel sources (kernels.hip, recon.hip), in that order."""
    h = hashlib.sha256()
    for f in ("kernels.hip", "recon.hip"):
        with open(os.path.join(ROOT, "dixon_adic_lifting_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(workload):
    """Per-launch HBM bytes from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs (profiles/pmc_traffic_<workload>.json), or None when absent or when
    the kernel sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_{workload}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        data = json.load(f)
    if data.get("kernel_sources_sha256") != kernel_sources_sha256():
        return {}
    out = {}
    for name, v in data["kernels"].items():
        if "gj_step_kernel" in name and "true>" not in name:
            out["gj_step"] = v["traffic_bytes"]
        elif "gj_update_kernel" in name:
            out["gj_update"] = v["traffic_bytes"]
        elif "lift_gemv" in name or "lift_mfma_kernel" in name:
            out["lift_contract"] = v["traffic_bytes"]
        elif "recon_gemm_kernel" in name:
            out["recon_gemm"] = v["traffic_bytes"]
        elif "residual1_kernel" in name or "residual_mfma_kernel" in name:
            out["residual"] = v["traffic_bytes"]
        elif "residue_kernel" in name:
            out["residues"] = v["traffic_bytes"]
        elif "gcd_kernel" in name:
            out["recon_gcd"] = v["traffic_bytes"]
    return out


def mfma_counters(workload):
    """Int8 MFMA counters per kernel class from the committed rocprofv3 run
    (profiles/pmc_mfma_<workload>.json: SQ_INSTS_VALU_MFMA_MOPS_I8 as int8
    operations per dispatch and SQ_VALU_MFMA_BUSY_CYCLES as the share of
    SIMD cycles), or {} when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"pmc_mfma_{workload}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        data = json.load(f)
    if data.get("kernel_sources_sha256") != kernel_sources_sha256():
        return {}
    names = {"lift_mfma_kernel": "lift_contract", "residual_mfma_kernel": "residual", "gj_update_kernel": "gj_update",
             "recon_gemm_kernel": "recon_gemm"}
    out = {}
    for name, v in data["kernels"].items():
        for key, cls in names.items():
            if key in name:
                out[cls] = {"int8_ops_per_launch": v["int8_ops_per_dispatch"], "mfma_busy": round(v["mfma_busy"], 5)}
    return out


def rooflines(prof, info, n, c, traffic=None):
    traffic = traffic or {}
    pitch = 64
    while pitch < n and n <= 1024:
        pitch <<= 1
    if n > 1024:
        pitch = -(-n // 64) * 64
    E = info["live_primes"]
    out = {}
    ms, cnt = prof.get("gj_step", (0.0, 0))
    if cnt:
        # each launch reads and writes every live prime's n x pitch u8 working matrix
        bytes_per = 2.0 * E * n * pitch
        avg_s = ms / cnt / 1e3
        gbs = bytes_per / avg_s / 1e9
        out["gj_step"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic.get("gj_step"),
                          "avg_launch_us": round(avg_s * 1e6, 2), "launches": cnt,
                          "algorithmic_bytes_per_launch": int(bytes_per)}
    ms, cnt = prof.get("gj_update", (0.0, 0))
    if cnt:
        # blocked elimination update: every live prime's n x pitch matrix read and written once,
        # the transposed old pivot rows (32 bytes per column) read; ops of the rank-32 product
        bytes_per = 2.0 * E * n * pitch + E * pitch * 32
        ops_per = 2.0 * E * n * pitch * 32
        avg_s = ms / cnt / 1e3
        gbs = bytes_per / avg_s / 1e9
        out["gj_update"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic.get("gj_update"),
                            "avg_launch_us": round(avg_s * 1e6, 2), "launches": cnt,
                            "algorithmic_bytes_per_launch": int(bytes_per),
                            "int8_tops": round(ops_per / avg_s / 1e12, 2)}
    ms, cnt = prof.get("gj_panel", (0.0, 0))
    if cnt:
        # 32 elimination steps on each live prime's n x 32 panel (the rows that can still pivot,
        # in registers), one 1024-thread block per prime (latency-bound: 53 of 256 CUs)
        out["gj_panel"] = {"avg_launch_us": round(ms / cnt * 1e3, 2), "launches": cnt, "total_ms": round(ms, 3),
                           "element_updates_per_launch": int(32 * E * n * 32)}
    ms, cnt = prof["lift_contract"]
    if cnt:
        # B_j (int8, n x pitch) once per step, plus the residue vector in and the residues out;
        # with one right-hand side and rows of 1 KB or more the step's share of the CRT runs
        # in the same kernel, which writes per component a record of the E balanced residues
        # and k (E + 1 bytes) and x mod 2^64 (8 bytes) instead; the digits are formed from
        # the records by a later launch per run of steps
        fused = c == 1 and pitch >= 1024 and 53 * n * pitch <= 0x7fffffff
        bytes_per = E * n * pitch + E * c * pitch + ((E + 9) * n if fused else E * n * c)
        ops_per = 2.0 * E * n * n * c
        avg_s = ms / cnt / 1e3
        gbs = bytes_per / avg_s / 1e9
        out["lift_contract"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic.get("lift_contract"),
                                "avg_launch_us": round(avg_s * 1e6, 2), "launches": cnt,
                                "algorithmic_bytes_per_launch": int(bytes_per),
                                "int8_tops": round(ops_per / avg_s / 1e12, 3),
                                "int8_frac_of_peak": round(ops_per / avg_s / 1e12 / INT8_PEAK_TOPS, 5)}
    ms, cnt = prof.get("recon_gemm", (0.0, 0))
    if cnt:
        # one launch per chunk of components: the modular multiply of every component's
        # digit bytes (42 m of them) by the weight rows (4 NW bytes wide, NW = words of M)
        NC = n * c
        nw_m = (info["modulus_bits"] + 31) // 32
        ops = 2.0 * NC * (42 * info["m"]) * (4 * nw_m)
        s = ms / 1e3
        out["recon_gemm"] = {"bound": "mfma", "achieved": round(ops / s / 1e12, 2), "peak": INT8_PEAK_TOPS,
                             "unit": "TOP/s", "frac": round(ops / s / 1e12 / INT8_PEAK_TOPS, 4),
                             "traffic": traffic.get("recon_gemm"),
                             "avg_launch_us": round(s / cnt * 1e6, 2), "launches": cnt,
                             "algorithmic_ops_total": ops}
    for k in ("crt", "residual", "residues", "recon_other", "recon_gcd"):
        ms, cnt = prof.get(k, (0.0, 0))
        if cnt:
            out[k] = {"avg_launch_us": round(ms / cnt * 1e3, 2), "launches": cnt, "total_ms": round(ms, 3)}
    if c == 1 and "residual" in out:
        # one right-hand side: A as int32 once per step, r in and out, the next residues out
        bytes_per = 4.0 * n * n + 16.0 * n + E * pitch
        gbs = bytes_per / (out["residual"]["avg_launch_us"] / 1e6) / 1e9
        out["residual"].update({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic.get("residual"),
                                "algorithmic_bytes_per_launch": int(bytes_per)})
    if "residues" in out:
        # A (int64) read once; every prime's residue matrix and the int32 copy of A written
        bytes_per = 8.0 * n * n + 53.0 * n * pitch + 4.0 * n * n
        gbs = bytes_per / (out["residues"]["avg_launch_us"] / 1e6) / 1e9
        out["residues"].update({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic.get("residues"),
                                "algorithmic_bytes_per_launch": int(bytes_per)})
    if "gj_panel" in out:
        # the panel's element updates, four 32-bit integer operations each (multiply-add,
        # reduction), against the chip's 32-bit integer VALU rate
        ops = 4.0 * out["gj_panel"]["element_updates_per_launch"]
        r = ops / (out["gj_panel"]["avg_launch_us"] / 1e6) / 1e12
        out["gj_panel"].update({"bound": "alu", "achieved": round(r, 3), "peak": INT32_VALU_PEAK_TOPS,
                                "unit": "TOP/s", "frac": round(r / INT32_VALU_PEAK_TOPS, 5), "traffic": None})
    if "recon_gcd" in out and info.get("gcd_bits"):
        # Lehmer gcd of every component's numerator and d: rounds of about 28 quotient bits,
        # each applying a 2 x 2 matrix to both numbers' live 30-bit limbs (4 multiply-adds a
        # limb), so about B^2 / 420 64-bit multiply-adds for B-bit operands
        B = info["gcd_bits"]
        ops = n * c * B * B / 420.0
        r = ops / (out["recon_gcd"]["total_ms"] / 1e3) / 1e12
        out["recon_gcd"].update({"bound": "alu", "achieved": round(r, 3), "peak": INT64_MAD_PEAK_TOPS,
                                 "unit": "T mul-add/s", "frac": round(r / INT64_MAD_PEAK_TOPS, 4),
                                 "traffic": traffic.get("recon_gcd"),
                                 "algorithmic_mul_adds_total": ops})
    if c > 1 and info.get("entry_bits", 64) <= 30 and "residual" in out:
        # several right-hand sides: A x mod 2^64 as int8 MFMA products of 4 byte planes of A
        # and 8 of x (the 26 plane pairs below 2^64), 2 n^2 c ops each
        ops_per = 26 * 2.0 * n * n * c
        s_per = out["residual"]["avg_launch_us"] / 1e6
        out["residual"].update({"bound": "mfma", "int8_tops": round(ops_per / s_per / 1e12, 2),
                                "int8_frac_of_peak": round(ops_per / s_per / 1e12 / INT8_PEAK_TOPS, 5),
                                "algorithmic_ops_per_launch": ops_per})
    return out


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _minor_limbs(k, log2_sigma):
    """64-bit limbs of a (k + 1)-minor of a matrix with i.i.d. entries of RMS
    2^log2_sigma: log2 |det| is about (k + 1) log2 sigma + log2 sqrt((k + 1)!)."""
    bits = (k + 1) * log2_sigma + 0.5 * math.lgamma(k + 2) / math.log(2.0)
    return max(1.0, bits / 64.0 + 1.0)


def _entry_cost_table(threads, max_limbs):
    """Seconds per elimination entry update of the C oracle at operand sizes
    on a geometric grid up to max_limbs, every thread running at once."""
    from oracle import cbareiss
    grid, L = [], 1.0
    while L < 1.15 * max_limbs:
        grid.append(int(round(L)))
        L *= 1.35
    grid.append(int(math.ceil(1.15 * max_limbs)))
    table = []
    for L in sorted(set(grid)):
        reps = max(3, int(0.02 / (1e-7 + 4e-9 * L * L)))
        table.append((L, cbareiss.entry_update_seconds(L, max(1, L - 1), reps, threads)))
    return table


def _cost(table, L):
    """log-log interpolation in the measured table"""
    if L <= table[0][0]:
        return table[0][1]
    for (L0, t0), (L1, t1) in zip(table, table[1:]):
        if L <= L1:
            w = math.log(L / L0) / math.log(L1 / L0)
            return math.exp((1 - w) * math.log(t0) + w * math.log(t1))
    return table[-1][1] * (L / table[-1][0]) ** 2


def _project(A, c, threads, table, gcd_s, steps=None, first=0):
    """Projected wall time of the oracle (oracle/bareiss.c) on an n x n system
    with entries like A's, from elimination step `first` on (the steps before
    it are timed by running them): per elimination step, each thread updates
    ceil((n - k - 1) / T) rows of n + c - k - 1 entries at the measured cost
    for the step's operand size; back substitution takes per row the row's
    share of products of an L_i-limb by an L_n-limb number (a third of an
    entry update at their geometric mean size); lowest terms take one binary
    gcd of L_n-limb numbers per component.  With `steps`, only elimination
    steps [first, steps) are projected."""
    import numpy as np
    n = A.shape[0]
    log2_sigma = 0.5 * math.log2(max(1.0, float(np.mean(A.astype(np.float64) ** 2))))
    K = n if steps is None else steps
    elim = 0.0
    for k in range(first, K):
        rows = -(-(n - k - 1) // threads)
        elim += rows * (n + c - k - 1) * _cost(table, _minor_limbs(k, log2_sigma))
    if steps is not None:
        return elim
    Ln = _minor_limbs(n - 1, log2_sigma)
    back = 0.0
    for i in range(n):
        Li = _minor_limbs(i, log2_sigma)
        back += (-(-(n - i - 1) // threads) + 2) * _cost(table, math.sqrt(Li * Ln)) / 3.0
    back *= c
    lowest = -(-(n * c) // threads) * gcd_s
    return elim + back + lowest


def _gcd_seconds(limbs):
    """Seconds per binary gcd of two limbs-limb numbers in the C oracle."""
    import random
    from oracle import cbareiss
    rng = random.Random(7)
    a, b = rng.getrandbits(64 * limbs) | 1, rng.getrandbits(64 * limbs) | 1
    t0 = time.perf_counter()
    for _ in range(3):
        cbareiss.gcd_magnitudes(a, b)
    return (time.perf_counter() - t0) / 3


def cpu_baseline(A, b, budget_s):
    """The CPU oracle on the host cores for a full solve of this system: its
    first elimination steps actually run and timed (a bounded sample of the
    workload, sized to the budget), the remaining steps projected from the
    oracle's measured cost per entry update at each step's operand size
    (small entries carry memory and allocation costs that the measured first
    steps include; large ones are bound by the limb arithmetic that the
    per-entry timing captures).

    Checked in the same run the same way on the n = 256 workload: its first
    steps timed, the rest projected, against a full timed oracle run."""
    import numpy as np
    from dixon_adic_lifting_amd import workloads as W
    from oracle import cbareiss
    n, c = A.shape[0], b.shape[1]
    threads = cbareiss.default_threads()
    t_start = time.perf_counter()
    log2_sigma = 0.5 * math.log2(max(1.0, float(np.mean(A.astype(np.float64) ** 2))))
    table = _entry_cost_table(threads, _minor_limbs(n - 1, log2_sigma))
    gcd_s = _gcd_seconds(int(_minor_limbs(n - 1, log2_sigma)))

    def prefix_and_rest(A_, b_, budget, gcd_):
        n_, c_ = A_.shape[0], b_.shape[1]
        K = min(n_, 16)
        while K < n_ and _project(A_, c_, threads, table, gcd_, steps=2 * K) < 0.6 * budget:
            K *= 2
        t0 = time.perf_counter()
        cbareiss.run(A_, b_, threads=threads, max_steps=K)
        measured = time.perf_counter() - t0
        rest = _project(A_, c_, threads, table, gcd_, first=K)
        return K, measured, rest

    K, measured, rest = prefix_and_rest(A, b, budget_s, gcd_s)
    est = measured + rest
    A3, b3 = W.generate("c3_n256_int24")
    gcd3 = _gcd_seconds(int(_minor_limbs(255, log2_sigma)))
    K3, m3, r3 = prefix_and_rest(A3, b3, 1.0, gcd3)
    t0 = time.perf_counter()
    cbareiss.run(A3, b3, threads=threads)
    full3 = time.perf_counter() - t0
    est3 = m3 + r3
    spent = time.perf_counter() - t_start
    return {"value": round(est * 1e3, 1), "unit": "ms per full solve (first steps timed, rest projected)",
            "cores": threads, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": (f"plain-C Bareiss oracle (oracle/bareiss.c), {threads} threads, on this {n}x{n}, c={c} "
                       f"system: its first {K} of {n} elimination steps run and timed ({measured:.2f} s); the other "
                       f"steps, back substitution and lowest terms projected ({rest:.1f} s) from the oracle's entry "
                       f"update (two products, difference, exact division) timed at {len(table)} operand sizes up "
                       f"to {table[-1][0]} limbs with every thread busy, over each step's exact entry count"),
            "sample_steps": K, "sample_seconds": round(measured, 3), "projected_seconds": round(rest, 2),
            "cpu_seconds_spent": round(spent, 2),
            "check_full_n256": {"measured_s": round(full3, 3), "projected_s": round(est3, 3),
                                "relative_error": round((est3 - full3) / full3, 4), "timed_steps": K3,
                                "workload": "c3_n256_int24"}}


def copy_calibration(mb):
    import torch
    x = torch.empty(mb << 20, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    return {"copy_bytes_each_way": mb << 20, "copies": 3}


def analyse(S, name, traffic=None):
    """Profiled pass on the canonical draw: per-kernel rooflines, the output
    checks, and the dominant kernel (largest total event time, any class)."""
    import numpy as np
    from dixon_adic_lifting_amd import workloads as W
    A, b = W.generate(name)
    prof, info, stages_prof, pairs = profiled_pass(S)
    info = dict(info, entry_bits=int(np.abs(A).max()).bit_length(),
                gcd_bits=max(q.bit_length() for row in pairs for (_, q) in row))
    rf = rooflines(prof, info, S.n, S.c, traffic)
    timed = {k: v for k, v in rf.items() if "bound" in v}
    dominant = max(timed, key=lambda k: prof[k][0]) if timed else None
    return {"prof": prof, "info": info, "stages_prof": stages_prof, "pairs": pairs, "rf": rf,
            "dominant": dominant, "A": A, "b": b}


def multi_column_block(name, warmup, steps):
    """A short run of the multi-column workload for the same JSON line: ms per
    solve over distinct inputs, stage split, per-kernel rooflines (the lift's
    int8 MFMA rate among them) and the mod-prime output check."""
    S = Solver(workload_inputs(name, warmup + steps))
    total, per, stages = time_solves(S, steps, warmup)
    an = analyse(S, name, counter_traffic(name))
    ok = verify_mod_primes(an["A"], an["b"], an["pairs"])
    progress(f"{name}: {1e3 * total / steps:.1f} ms per solve, A x = b mod primes {ok}")
    rf = an["rf"]
    out = {"workload": name, "ms_per_solve": round(1e3 * total / steps, 2), "steps": steps, "warmup": warmup,
           "ms_each": [round(1e3 * t, 2) for t in per], "solves_per_s": round(steps / total, 3),
           "m": an["info"]["m"], "live_primes": an["info"]["live_primes"],
           "stages_ms": {k: round(v, 2) for k, v in stages.items()},
           "output_check_Ax_eq_b_mod_primes": ok, "dominant_kernel": an["dominant"], "kernels": rf}
    if "lift_contract" in rf:
        out["lift_int8_mfma_frac_of_peak"] = rf["lift_contract"].get("int8_frac_of_peak")
    # the committed counter run's int8 operations per launch, against the
    # algorithmic count the fractions above use, and its MFMA busy share
    cnt = mfma_counters(name)
    if cnt:
        E, n, c = an["info"]["live_primes"], S.n, S.c
        algo = {"lift_contract": 2.0 * E * n * n * c, "residual": 26 * 2.0 * n * n * c}
        for cls, v in cnt.items():
            if cls in algo:
                v["algorithmic_ops_per_launch"] = algo[cls]
                v["counter_over_algorithmic"] = round(v["int8_ops_per_launch"] / algo[cls], 4)
        out["mfma_counters"] = cnt
    del S
    return out


def sweep(args):
    from dixon_adic_lifting_amd import workloads as W
    rows = []
    for name in list(W.WORKLOADS):
        A, _ = W.generate(name)
        steps = 3 if A.shape[0] >= 2048 else 5
        S = Solver(workload_inputs(name, steps + 1))
        total, per, stages = time_solves(S, steps, 1)
        an = analyse(S, name)
        rows.append({"workload": name, "ms_median": round(1e3 * sorted(per)[len(per) // 2], 2),
                     "ms_min": round(1e3 * min(per), 2), "stages_ms": {k: round(v, 2) for k, v in stages.items()},
                     "m": an["info"]["m"], "live": an["info"]["live_primes"], "dominant": an["dominant"],
                     "roofline": an["rf"]})
        print(json.dumps(rows[-1]), flush=True)
    for (n, c) in W.CARD_SHAPES:
        S = Solver([W.uniform_system(n, c, 24, 1000 + n + c + 100000 * k) for k in range(6)])
        total, per, stages = time_solves(S, 5, 1)
        print(json.dumps({"workload": f"card_n{n}_c{c}_int24", "ms_median": round(1e3 * sorted(per)[len(per) // 2], 2),
                          "ms_min": round(1e3 * min(per), 2), "stages_ms": {k: round(v, 2) for k, v in stages.items()}}),
              flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this solver has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.sweep:
        sweep(args)
        return
    from dixon_adic_lifting_amd import workloads as W
    S = Solver(workload_inputs(args.workload, args.warmup + args.steps))
    total, per, stages = time_solves(S, args.steps, args.warmup)
    ms_per = total / args.steps * 1e3
    an = analyse(S, args.workload, counter_traffic(args.workload))
    progress(f"profiled pass done: stages {an['stages_prof']}")
    A, b, pairs, info, rf, dominant = an["A"], an["b"], an["pairs"], an["info"], an["rf"], an["dominant"]
    # parity of the benched output: the oracle's stored digest
    gold = None
    gpath = os.path.join(ROOT, "tests", "golden", "oracle_digests.json")
    if os.path.exists(gpath):
        with open(gpath) as f:
            gold = json.load(f).get(args.workload)
    parity = None if gold is None else (digest(pairs) == gold["sha256"])
    identity_ok = verify_mod_primes(A, b, pairs)
    progress(f"output checks done: digest match {parity}, A x = b mod primes {identity_ok}")
    max_bits = max(max(abs(p).bit_length(), q.bit_length()) for row in pairs for (p, q) in row)
    if args.copy_calib_mb:
        copy_calibration(args.copy_calib_mb)
    del S
    multi = None
    if args.multi_column and args.workload != MULTI_COLUMN:
        multi = multi_column_block(MULTI_COLUMN, 1, 2)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(A, b, args.cpu_budget_s)
    wl = W.WORKLOADS[args.workload]
    line = {
        "metric": f"full exact-solve ms at n={wl.n} c={wl.c} int24" if wl.name.endswith("int24") else
                  f"full exact-solve ms for {wl.name}",
        "value": round(ms_per, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per, 3),
        "solves_per_s": round(1e3 / ms_per, 3),
        "ms_min": round(1e3 * min(per), 3),
        "ms_median": round(1e3 * sorted(per)[len(per) // 2], 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round(ms_per / PAGES_MS_C4["h200"], 5) if wl.name == "c4_n1024_int24" else None,
        "dtype": "int8/int32/int64 (exact)",
        "data": "synthetic (seeded, i.i.d. uniform 24-bit entries; every solve a distinct draw)",
        "config": {"workload": wl.name, "n": wl.n, "c": wl.c, "entries": "uniform [-2^23, 2^23)",
                   "seed": wl.seed, "distinct_inputs": min(args.warmup + args.steps, MAX_DISTINCT_INPUTS),
                   "m": info["m"], "live_primes": info["live_primes"]},
        "parity_vs_oracle_digest": parity,
        "output_check_Ax_eq_b_mod_primes": identity_ok,
        "output_max_bits": max_bits,
        "stages_ms": {k: round(v, 3) for k, v in stages.items()},
        "stages_ms_profiled": {k: round(v, 3) for k, v in an["stages_prof"].items()},
        "roofline": {**{k: rf[dominant][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
                     "kernel": dominant} if dominant else None,
        "kernels": rf,
        "multi_column": multi,
        "pages_context_ms": PAGES_MS_C4,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
