"""HBM traffic and matrix-core work of the kernels from rocprofv3 counters.

    python -m gated_delta_rule_amd.traffic collect [--out DIR]

runs, for each target below, two rocprofv3 counter passes (FETCH_SIZE, then
WRITE_SIZE; one pass per counter, each under its own time limit) as child
processes, and writes `profiles/<kernel>_<workload>_traffic.json` with the
bytes per launch.  The counters read KiB per dispatch; they are scaled by
what the same counters read for a plain elementwise copy (y = 1 * x over
1 GiB of fp32, so 1 GiB read and 1 GiB written) measured in the same way.

    python -m gated_delta_rule_amd.traffic target {copy,prefill,decode}

is the profiled program: it prepares the resident inputs of one workload
and launches its kernel a few times.  The orchestrating process never
touches the GPU itself.

    python -m gated_delta_rule_amd.traffic phases [--out DIR]

builds the contraction-phase probe (csrc/kda_phase_probe.hip, into its own
libkda_probe.so), times it with HIP events and runs one rocprofv3 pass per
matrix-core counter over it, and writes
`profiles/contraction_phases_probe.json`: for the K+ S / Q+ S phase, the
state-update phase and both, the matrix-core flops per launch, the rate
against the 2.5 PFLOP/s 16-bit peak, the busy fraction of the matrix cores
(SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) and the
share of LDS active cycles lost to bank conflicts (SQ_LDS_BANK_CONFLICT over
SQ_LDS_IDX_ACTIVE), with one wave per SIMD and nothing else on the compute
units.

    python -m gated_delta_rule_amd.traffic ceiling

times the stream probe (csrc/kda_phase_probe.hip: x <- a x in place over the
decode state's 1.61 GB with nontemporal 16-byte accesses, the decode step's
access pattern without its arithmetic) over several grid sizes and writes
`profiles/hbm_stream_ceiling.json`: the read+write rate one such pass reaches,
the practical ceiling for the decode step.

    python -m gated_delta_rule_amd.traffic bwd [--out DIR]

does the same for the backward pass (`kda_chunk_bwd` at B=1, T=8192, H=96,
bf16, with a one-window workspace): one FETCH_SIZE and one WRITE_SIZE pass
over its four kernels, scaled by the copy, into
`profiles/chunk_bwd_workload1_traffic.json` (bytes per launch of each
kernel).

    python -m gated_delta_rule_amd.traffic mfma [--out DIR]

runs one rocprofv3 pass per counter (MFMA operations per data type, MFMA
busy cycles, SQ busy cycles, GPU active cycles, VALU / MFMA / LDS
instructions issued, LDS bank-conflict and LDS active cycles) over the
prefill target and writes `profiles/chunk_fwd_workload1_mfma.json`: the
counters per launch, the hardware flops they imply (each MOPS count stands
for 512 flops) and the flops the kernel's instruction mix implies
(`prefill_mfma_flops`).

The JSON records a hash of the kernel's sources; the benchmark reports the
counters only while that hash matches the sources it runs.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")

COPY_ELEMS = 1 << 28          # 1 GiB of fp32
LAUNCHES = {"copy": 6, "prefill": 6, "decode": 8, "backward": 3}

# Kernel symbol fragment, profile name, sources the kernel is built from.
TARGETS = {
    "prefill": ("chunk_fwd_pipe_kernel", "chunk_fwd_workload1",
                ("kda_prefill_pipe.hip", "kda_prefill.hip", "kda_chunk.h", "kda_device.h", "kda_launch.h",
                 "kda_abi.hip")),
    "decode": ("recurrent_kernel", "decode_step_workload4",
               ("kda_recurrent.hip", "kda_device.h", "kda_launch.h", "kda_abi.hip")),
    "backward": ("bwd_", "chunk_bwd_workload1",
                 ("kda_backward.hip", "kda_prefill_pipe.hip", "kda_chunk.h", "kda_device.h", "kda_launch.h",
                  "kda_abi.hip")),
}
# the backward's kernels, in launch order (symbol fragment, what it is)
BWD_KERNELS = (("chunk_fwd_pipe_kernel<4, true", "forward keeping chunk states, V - K+S and U"),
               ("bwd_tmp_kernel", "chunk matrices"),
               ("bwd_scan_kernel", "state-gradient walk"),
               ("bwd_grad_kernel", "per-chunk gradients"))


PROBE_SRC = "kda_phase_probe.hip"
PROBE_LIB = os.path.join(PKG, "libkda_probe.so")
PROBE_MODES = {0: "K+S/Q+S", 1: "state update", 2: "K+S/Q+S then state update"}
PROBE_WG, PROBE_ITERS, PROBE_LAUNCHES = 256, 2048, 6
PEAK_16BIT_TFLOPS = 2500.0


def build_probe(verbose=False):
    """Compile the contraction-phase probe into libkda_probe.so (hipcc, gfx950)."""
    from gated_delta_rule_amd import build as B
    tmp = PROBE_LIB + ".tmp"
    cmd = [B.hipcc(), *B.FLAGS, f"-I{os.path.join(ROOT, 'include')}", "-o", tmp,
           os.path.join(CSRC, PROBE_SRC)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def run_probe_target():
    """The profiled program of `phases`: PROBE_LAUNCHES launches of each mode
    (the first untimed), timed with HIP events; prints one JSON line."""
    import ctypes
    import torch
    lib = ctypes.CDLL(PROBE_LIB)
    lib.kda_probe_contraction.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.kda_probe_contraction.restype = ctypes.c_int
    lib.kda_probe_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.kda_probe_flops.restype = ctypes.c_double
    dev = torch.device("cuda:0")
    out = torch.empty(PROBE_WG * 256 * 48, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for mode in PROBE_MODES:
        def launch():
            rc = lib.kda_probe_contraction(ctypes.c_void_p(out.data_ptr()), PROBE_WG, PROBE_ITERS, mode,
                                           ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"probe launch failed: {rc}")
        launch()
        torch.cuda.synchronize()
        ms = []
        for _ in range(PROBE_LAUNCHES - 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        ms.sort()
        flops = lib.kda_probe_flops(PROBE_WG, PROBE_ITERS, mode)
        med = ms[len(ms) // 2]
        res[mode] = {"ms_median": med, "flops_per_launch": flops,
                     "tflops": flops / (med * 1e-3) / 1e12}
    print("PROBE " + json.dumps(res), flush=True)


STREAM_FLOATS = 256 * 96 * 128 * 128   # the decode workload's fp32 state, 1.61 GB
STREAM_GRIDS = (256, 512, 1024, 2048, 4096, 8192)


STREAM_MODES = {0: ("in place x <- a x", 2), 1: ("copy y <- a x", 2), 2: ("read only", 1)}


def collect_ceiling(profiles_dir):
    """Time the stream probe (csrc/kda_phase_probe.hip) over the decode
    state's 1.61 GB of fp32, nontemporal 16-byte accesses, after a clock
    settle: in place (the decode step's read-then-write pattern without its
    arithmetic), as a copy to a second buffer, and read only, each over
    several grid sizes.  Writes profiles/hbm_stream_ceiling.json with the
    best rate of each (bytes moved / time)."""
    import ctypes
    import time
    import torch
    build_probe(verbose=True)
    lib = ctypes.CDLL(PROBE_LIB)
    lib.kda_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.kda_probe_stream.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    x = torch.ones(STREAM_FLOATS, dtype=torch.float32, device=dev)
    y = torch.empty(STREAM_FLOATS, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch(n_wg, mode):
        rc = lib.kda_probe_stream(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                  STREAM_FLOATS, 1.0, n_wg, mode, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"stream probe launch failed: {rc}")
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.5:   # clock settle
        launch(2048, 0)
        torch.cuda.synchronize()
    modes = {}
    for mode, (name, passes) in STREAM_MODES.items():
        nbytes = passes * STREAM_FLOATS * 4
        rows = []
        for n_wg in STREAM_GRIDS:
            launch(n_wg, mode)
            ms = []
            for _ in range(10):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                launch(n_wg, mode)
                e1.record(stream)
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1))
            ms.sort()
            med = ms[len(ms) // 2]
            rows.append({"workgroups": n_wg, "ms_median": med, "ms_min": ms[0],
                         "gbps_median": nbytes / (med * 1e-3) / 1e9})
            print(f"stream probe {name}, {n_wg} workgroups: {med:.4f} ms, "
                  f"{rows[-1]['gbps_median']:.0f} GB/s", flush=True)
        best = max(rows, key=lambda r: r["gbps_median"])
        modes[name] = {"bytes_per_launch": nbytes, "grids": rows, "best_gbps": best["gbps_median"],
                       "best_frac_of_8tbps": best["gbps_median"] / 8000.0}
    doc = {
        "probe": "csrc/kda_phase_probe.hip stream_probe_kernel over 1.61 GB of fp32 (the decode "
                 "state's size): 1024-thread workgroups, 16-byte nontemporal loads and stores, 1 KB "
                 "per wave instruction, 8 loads in flight per lane",
        "command": "python -m gated_delta_rule_amd.traffic ceiling",
        "modes": modes,
        "probe_source_sha256_16": probe_hash(),
    }
    path = os.path.join(profiles_dir, "hbm_stream_ceiling.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print("stream ceilings: " + ", ".join(f"{k} {v['best_gbps']:.0f} GB/s" for k, v in modes.items())
          + f" -> {path}", flush=True)


def probe_hash():
    h = hashlib.sha256()
    for name in (PROBE_SRC, "kda_chunk.h", "kda_device.h"):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def collect_phases(out, profiles_dir, run=True):
    os.makedirs(out, exist_ok=True)
    os.makedirs(profiles_dir, exist_ok=True)
    if run:
        build_probe(verbose=True)
    env = dict(os.environ, TMPDIR="/tmp", PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    if run:
        r = subprocess.run(["timeout", "-s", "KILL", "120", sys.executable, "-u", "-m",
                            "gated_delta_rule_amd.traffic", "target", "probe"],
                           cwd="/tmp", env=env, capture_output=True, text=True)
        if r.returncode != 0:
            raise SystemExit(f"probe timing run failed ({r.returncode}): {r.stderr[-2000:]}")
        timing = None
        for line in r.stdout.splitlines():
            if line.startswith("PROBE "):
                timing = json.loads(line[6:])
        with open(os.path.join(out, "probe_timing.json"), "w") as f:
            json.dump(timing, f)
    with open(os.path.join(out, "probe_timing.json")) as f:
        timing = json.load(f)
    counters = {}
    for counter in ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                    "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"):
        per = counter_pass("probe", counter, out, run)
        disp = sorted((int(k[0]), v) for k, v in per.items() if "contraction_probe" in k[1])
        if len(disp) != PROBE_LAUNCHES * len(PROBE_MODES):
            raise SystemExit(f"{counter}: {len(disp)} probe dispatches, expected "
                             f"{PROBE_LAUNCHES * len(PROBE_MODES)}")
        for i, mode in enumerate(PROBE_MODES):
            vals = [v for _, v in disp[i * PROBE_LAUNCHES + 1:(i + 1) * PROBE_LAUNCHES]]
            counters.setdefault(str(mode), {})[counter] = sum(vals) / len(vals)
    modes = {}
    for mode, name in PROBE_MODES.items():
        c = counters[str(mode)]
        t = timing[str(mode)]
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / 8 * 1024)
        hw = (c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + c["SQ_INSTS_VALU_MFMA_MOPS_F16"]) * MOPS_FLOPS
        modes[name] = {"counters_per_launch": c, "ms_median": t["ms_median"],
                       "flops_per_launch_instruction_mix": t["flops_per_launch"],
                       "flops_per_launch_counters": hw,
                       "tflops": t["tflops"], "frac_of_16bit_peak": t["tflops"] / PEAK_16BIT_TFLOPS,
                       "mfma_busy_frac": busy,
                       "lds_bank_conflict_frac": c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]}
        print(f"{name}: {t['tflops']:.0f} TFLOP/s = {t['tflops'] / PEAK_16BIT_TFLOPS:.3f} of peak, "
              f"matrix cores busy {busy:.3f}, LDS bank conflicts "
              f"{modes[name]['lds_bank_conflict_frac']:.3f} of LDS active cycles", flush=True)
    doc = {
        "probe": "csrc/kda_phase_probe.hip: the prefill consumer's K+S/Q+S and state-update instruction "
                 "sequences on LDS-resident operands, one wave per SIMD, 256 workgroups x "
                 f"{PROBE_ITERS} iterations, nothing else on the compute units",
        "command": "python -m gated_delta_rule_amd.traffic phases (timing: python -u -m "
                   "gated_delta_rule_amd.traffic target probe; per counter: rocprofv3 --pmc <counter> -d "
                   "<dir> -o run --output-format csv -- python -u -m gated_delta_rule_amd.traffic target probe)",
        "peak_tflops_16bit": PEAK_16BIT_TFLOPS,
        "modes": modes,
        "probe_source_sha256_16": probe_hash(),
    }
    path = os.path.join(profiles_dir, "contraction_phases_probe.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"contraction phases -> {path}", flush=True)


def code_only(text):
    """C/C++ source without its comments, indentation or blank lines, so that
    a record stays valid while only the comments around a kernel change.
    String and character literals are kept as written."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (" ".join(line.split()) for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line)


def sources_hash(kind):
    """Hash of the code (comments and blank space removed) of the sources a
    profiled kernel is built from."""
    h = hashlib.sha256()
    for name in TARGETS[kind][2]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + code_only(f.read()).encode())
    return h.hexdigest()[:16]


def profile_path(kind, profiles_dir=None):
    return os.path.join(profiles_dir or os.path.join(ROOT, "profiles"), TARGETS[kind][1] + "_traffic.json")


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES",
                 "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
                 "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE")
MOPS_FLOPS = 512              # flops per count of an SQ_INSTS_VALU_MFMA_MOPS_* counter


def prefill_mfma_flops(T=8192, H=96, chunk=32, slices=2):
    """Matrix-core flops one launch of the pipelined bf16 prefill kernel issues,
    counted from its instruction mix (16x16x32 = 16,384 flops, 16x16x16 = 8,192).

    Per chunk and workgroup (64 value columns of one head):
      consumer wave x4: K+S 8 bf16 and Q+S 8 fp16 16x16x32; block substitution
        3 x (hi, lo) 16x16x16 bf16; O = M U 2 x 3 16x16x32; state update
        8 x 3 16x16x32;
      tile waves: L00 and L11 4 each, -L10 4, M00 12, M10 and M11 24 (16x16x32).
    """
    k32, k16 = 16384, 8192
    consumer_bf16 = 8 * k32 + 6 * k16 + 6 * k32 + 24 * k32
    consumer_f16 = 8 * k32
    tiles_bf16 = (4 + 4 + 4 + 12 + 24) * k32
    units = (T // chunk) * H * slices
    return {"bf16": units * (4 * consumer_bf16 + tiles_bf16), "f16": units * 4 * consumer_f16}


def mfma_profile_path(profiles_dir=None):
    return os.path.join(profiles_dir or os.path.join(ROOT, "profiles"), "chunk_fwd_workload1_mfma.json")


def measured_mfma():
    """The prefill kernel's stored matrix-core counters, or None when they were
    taken on other sources (or never)."""
    try:
        with open(mfma_profile_path()) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_sha256_16") != sources_hash("prefill"):
        return None
    return rec


def measured_phases(profiles_dir=None):
    """The contraction-phase probe's stored results, or None when they were
    taken on other probe sources (or never)."""
    path = os.path.join(profiles_dir or os.path.join(ROOT, "profiles"), "contraction_phases_probe.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("probe_source_sha256_16") != probe_hash():
        return None
    return rec


def measured(kind):
    """Bytes per launch from the stored counters, or None when they were taken
    on other sources (or never)."""
    try:
        with open(profile_path(kind)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_sha256_16") != sources_hash(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ targets
def run_target(kind):
    if kind == "probe":
        run_probe_target()
        return
    import torch
    import gated_delta_rule_amd as kda
    from gated_delta_rule_amd import workloads as W

    dev = torch.device("cuda:0")
    n = LAUNCHES[kind]
    if kind == "copy":
        x = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(n):
            torch.mul(x, 1.0, out=y)
    elif kind == "prefill":
        w = W.workload(1)
        a = W.prefill_inputs(w)
        shp = (w.B, w.T, w.H, 128)
        d = {k: torch.from_numpy(a[k]).to(dev, torch.bfloat16).view(shp) for k in ("q", "k", "v")}
        la = torch.from_numpy(a["log_alpha"]).to(dev).view(shp)
        b = torch.from_numpy(a["beta"]).to(dev).view(w.B, w.T, w.H)
        o = torch.empty(shp, dtype=torch.float32, device=dev)
        st = torch.empty((w.B, w.H, 128, 128), dtype=torch.float32, device=dev)
        for _ in range(n):
            kda.chunk_fwd(d["q"], d["k"], d["v"], la, b, None, None, o=o, S_T=st)
    elif kind == "backward":
        # the benchmark's backward inputs: B=1, T=8192, H=96, drawn on the device
        T, H = 8192, 96
        g = torch.Generator(device=dev).manual_seed(13)
        shp = (1, T, H, 128)
        nrm = torch.nn.functional.normalize
        q = nrm(torch.randn(shp, device=dev, generator=g), dim=-1).to(torch.bfloat16)
        k = nrm(torch.randn(shp, device=dev, generator=g), dim=-1).to(torch.bfloat16)
        v = torch.randn(shp, device=dev, generator=g).to(torch.bfloat16)
        la = -5.0 * torch.sigmoid(torch.randn(shp, device=dev, generator=g))
        beta = torch.sigmoid(torch.randn((1, T, H), device=dev, generator=g))
        go = torch.randn(shp, device=dev, generator=g)
        gst = torch.randn((1, H, 128, 128), device=dev, generator=g)
        ws = torch.empty(kda.chunk_bwd_workspace_bytes(1, T, H, window_tokens=T), dtype=torch.uint8,
                         device=dev)
        for _ in range(n):
            kda.chunk_bwd(q, k, v, la, beta, None, go, gst, workspace=ws)
    else:
        w = W.workload(4)
        S = torch.from_numpy(W.decode_state(w)).to(dev)
        x = W.decode_inputs(w, 0)
        e = {k: torch.from_numpy(x[k]).to(dev, torch.bfloat16) for k in ("q", "k", "v")}
        la = torch.from_numpy(x["log_alpha"]).to(dev)
        b = torch.from_numpy(x["beta"]).to(dev)
        o = torch.empty((w.B, w.H, 128), dtype=torch.float32, device=dev)
        for _ in range(n):
            kda.decode_step(e["q"], e["k"], e["v"], la, b, S, o=o)
    torch.cuda.synchronize()
    print(f"target {kind}: {n} launches done", flush=True)


# ------------------------------------------------------------ orchestration
def counter_pass(kind, counter, out, run=True):
    """One rocprofv3 pass of `counter` over the target (skipped with run=False,
    which re-reads a previous pass's output); returns its value per
    (dispatch, kernel)."""
    d = os.path.join(out, f"{kind}_{counter}")
    cmd = ["timeout", "-s", "KILL", "120", "rocprofv3", "--pmc", counter, "-d", d, "-o", "run",
           "--output-format", "csv", "--", sys.executable, "-u", "-m", "gated_delta_rule_amd.traffic",
           "target", kind]
    env = dict(os.environ, TMPDIR="/tmp", PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    if run:
        print("running:", " ".join(cmd), flush=True)
        r = subprocess.run(cmd, cwd="/tmp", env=env)
        if r.returncode != 0:
            raise SystemExit(f"rocprofv3 pass {kind}/{counter} failed with status {r.returncode}")
    files = []
    for dp, _, fs in os.walk(d):
        files += [os.path.join(dp, f) for f in fs if f.endswith("counter_collection.csv")]
    if not files:
        raise SystemExit(f"no counter output under {d}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                key = (row["Dispatch_Id"], row["Kernel_Name"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    return per


def kib_per_dispatch(per, fragment):
    vals = [v for (_, name), v in per.items() if fragment in name]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {fragment!r}")
    vals = vals[1:] if len(vals) > 2 else vals      # drop the first (cold) launch
    return sum(vals) / len(vals), len(vals)


def calibrate(out, run=True):
    """FETCH_SIZE and WRITE_SIZE of the plain copy, as counter KiB per byte moved."""
    copy_bytes = COPY_ELEMS * 4
    cal = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        per = counter_pass("copy", counter, out, run)
        # the copy kernel is the one launched most often in its process
        names = [name for (_, name) in per]
        big = max(set(names), key=names.count)
        kib, n = kib_per_dispatch(per, big)
        cal[counter] = {"kib_per_dispatch": kib, "dispatches": n, "kernel": big,
                        "scale": kib * 1024.0 / copy_bytes}
        print(f"copy {counter}: {kib:.0f} KiB per dispatch, scale {cal[counter]['scale']:.4f}", flush=True)
    return cal


def calibration_doc(cal):
    return {"kernel": "torch elementwise y = 1 * x, 1 GiB fp32 read + 1 GiB written",
            **{k: {kk: vv for kk, vv in v.items() if kk != "kernel"} for k, v in cal.items()}}


def collect_bwd(out, profiles_dir, run=True):
    os.makedirs(out, exist_ok=True)
    os.makedirs(profiles_dir, exist_ok=True)
    cal = calibrate(out, run)
    passes = {c: counter_pass("backward", c, out, run) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    kernels = []
    for frag, what in BWD_KERNELS:
        rec = {"kernel": frag, "pass": what}
        for counter, per in passes.items():
            kib, n = kib_per_dispatch(per, frag)
            rec[counter] = {"kib_per_dispatch": kib, "dispatches": n,
                            "bytes_scaled": kib * 1024.0 / cal[counter]["scale"]}
        rec["hbm_bytes_per_launch"] = rec["FETCH_SIZE"]["bytes_scaled"] + rec["WRITE_SIZE"]["bytes_scaled"]
        kernels.append(rec)
        print(f"{frag}: read {rec['FETCH_SIZE']['bytes_scaled'] / 1e9:.3f} GB, "
              f"written {rec['WRITE_SIZE']['bytes_scaled'] / 1e9:.3f} GB per launch", flush=True)
    doc = {
        "workload": "kda_chunk_bwd B=1 T=8192 H=96 d=128, bf16 q/k/v, fp32 gates, dL/do and dL/dS_T given, "
                    "one-window workspace (every chunk's values kept)",
        "command": "python -m gated_delta_rule_amd.traffic bwd (per pass: rocprofv3 --pmc "
                   "<FETCH_SIZE|WRITE_SIZE> -d <dir> -o run --output-format csv -- python -u -m "
                   "gated_delta_rule_amd.traffic target backward)",
        "kernels": kernels,
        "copy_calibration": calibration_doc(cal),
        "kernel_sources_sha256_16": sources_hash("backward"),
    }
    path = profile_path("backward", profiles_dir)
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"backward -> {path}", flush=True)


def collect(out, profiles_dir):
    os.makedirs(out, exist_ok=True)
    os.makedirs(profiles_dir, exist_ok=True)
    cal = calibrate(out)
    for kind in ("prefill", "decode"):
        frag = TARGETS[kind][0]
        rec = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            kib, n = kib_per_dispatch(counter_pass(kind, counter, out), frag)
            rec[counter] = {"kib_per_dispatch": kib, "dispatches": n,
                            "bytes_scaled": kib * 1024.0 / cal[counter]["scale"]}
        total = rec["FETCH_SIZE"]["bytes_scaled"] + rec["WRITE_SIZE"]["bytes_scaled"]
        doc = {
            "kernel": frag,
            "workload": ("prefill B=1 T=8192 H=96 d=128 bf16, S0=0, o and S_T fp32" if kind == "prefill"
                         else "decode B=256 H=96 d=128 bf16 inputs, fp32 state in place"),
            "command": "python -m gated_delta_rule_amd.traffic collect (per pass: rocprofv3 --pmc "
                       "<FETCH_SIZE|WRITE_SIZE> -d <dir> -o run --output-format csv -- python -u -m "
                       f"gated_delta_rule_amd.traffic target {kind})",
            "counters": rec,
            "copy_calibration": calibration_doc(cal),
            "hbm_bytes_per_launch": total,
            "kernel_sources_sha256_16": sources_hash(kind),
        }
        path = profile_path(kind, profiles_dir)
        with open(path, "w") as f:
            json.dump(doc, f, indent=1)
            f.write("\n")
        print(f"{kind}: {total / 1e9:.4f} GB per launch -> {path}", flush=True)


def collect_mfma(out, profiles_dir, run=True):
    os.makedirs(out, exist_ok=True)
    os.makedirs(profiles_dir, exist_ok=True)
    frag = TARGETS["prefill"][0]
    rec = {}
    for counter in MFMA_COUNTERS:
        val, n = kib_per_dispatch(counter_pass("prefill", counter, out, run), frag)
        rec[counter] = {"per_dispatch": val, "dispatches": n}
        print(f"prefill {counter}: {val:.6g} per dispatch", flush=True)
    hw = {t: rec[f"SQ_INSTS_VALU_MFMA_MOPS_{t.upper()}"]["per_dispatch"] * MOPS_FLOPS
          for t in ("bf16", "f16", "f32")}
    doc = {
        "kernel": frag,
        "workload": "prefill B=1 T=8192 H=96 d=128 bf16, S0=0, o and S_T fp32",
        "command": "python -m gated_delta_rule_amd.traffic mfma (per pass: rocprofv3 --pmc <counter> "
                   "-d <dir> -o run --output-format csv -- python -u -m gated_delta_rule_amd.traffic "
                   "target prefill)",
        "counters": rec,
        "hw_flops_per_launch_from_counters": hw,
        "hw_flops_per_launch_from_instruction_mix": prefill_mfma_flops(),
        "lds_bank_conflict_frac": rec["SQ_LDS_BANK_CONFLICT"]["per_dispatch"]
        / rec["SQ_LDS_IDX_ACTIVE"]["per_dispatch"],
        "kernel_sources_sha256_16": sources_hash("prefill"),
    }
    path = mfma_profile_path(profiles_dir)
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"prefill matrix-core counters -> {path}", flush=True)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("target")
    t.add_argument("kind", choices=["copy", "prefill", "decode", "backward", "probe"])
    bw = sub.add_parser("bwd")
    bw.add_argument("--out", default=os.path.join(ROOT, "counters_out", "bwd"))
    bw.add_argument("--profiles-dir", default=os.path.join(ROOT, "profiles"))
    bw.add_argument("--parse-only", action="store_true",
                    help="summarise the counter output already under --out")
    c = sub.add_parser("collect")
    c.add_argument("--out", default=os.path.join(ROOT, "counters_out", "traffic"),
                   help="directory for the raw counter output")
    c.add_argument("--profiles-dir", default=os.path.join(ROOT, "profiles"),
                   help="where the per-kernel JSON summaries go")
    m = sub.add_parser("mfma")
    m.add_argument("--out", default=os.path.join(ROOT, "counters_out", "mfma"))
    m.add_argument("--profiles-dir", default=os.path.join(ROOT, "profiles"))
    m.add_argument("--parse-only", action="store_true",
                   help="summarise the counter output already under --out")
    ph = sub.add_parser("phases")
    ph.add_argument("--out", default=os.path.join(ROOT, "counters_out", "phases"))
    ph.add_argument("--profiles-dir", default=os.path.join(ROOT, "profiles"))
    ph.add_argument("--parse-only", action="store_true")
    ce = sub.add_parser("ceiling")
    ce.add_argument("--profiles-dir", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()
    if args.cmd == "ceiling":
        collect_ceiling(os.path.abspath(args.profiles_dir))
        return
    if args.cmd == "phases":
        collect_phases(os.path.abspath(args.out), os.path.abspath(args.profiles_dir), not args.parse_only)
        return
    if args.cmd == "bwd":
        collect_bwd(os.path.abspath(args.out), os.path.abspath(args.profiles_dir), not args.parse_only)
        return
    if args.cmd == "target":
        run_target(args.kind)
    elif args.cmd == "mfma":
        collect_mfma(os.path.abspath(args.out), os.path.abspath(args.profiles_dir), not args.parse_only)
    else:
        collect(os.path.abspath(args.out), os.path.abspath(args.profiles_dir))


if __name__ == "__main__":
    main()
