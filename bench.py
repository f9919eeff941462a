"""Benchmark of the DSpark Markov head on one MI355X.

One step = one greedy left-to-right draft of 64 sequences x 5 positions at
vocabulary 129280, rank 256, bf16 (sample_block_tokens with the corrected
logits returned): every step of the head's hot path (predecessor select,
W1 gather, low-rank projection, streaming add, argmax, chain).

The timed region starts with all inputs resident in HBM.  Successive steps
rotate over several input sets whose total exceeds the 256 MB Infinity
Cache, so every step streams its logits and weights from HBM.

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, vendor figure
WORKLOAD = "greedy_draft_64x5"
DOMINANT_KERNEL = "markov_chain_greedy_bf16<8, false>"   # the whole sample call is this one launch
KERNEL_SOURCES = [os.path.join(ROOT, "rank_markov_draft_amd", "csrc", name)
                  for name in ("markov_chain.hip", "chain_common.h", "device_common.h", "markov_chain.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
VALU_FILE = os.path.join(ROOT, "profiles", "valu.json")
VALU_KERNEL = "markov_chain_sample_bf16<8, false, false>"   # persistent temperature chain at rank 256
VALU_SOURCES = [os.path.join(ROOT, "rank_markov_draft_amd", "csrc", name)
                for name in ("markov_chain_sample.hip", "chain_common.h", "device_common.h", "markov_chain.h")]
# Issue cost (SIMD cycles) of a wave64 instruction, measured with a
# throughput microbenchmark at the measured shader clock: plain VALU 4 (16
# lanes per cycle), v_mad_u64_u32 (the Philox multiply) 4.5, v_log_f32 9.6.
VALU_COST, INT64_COST, TRANS_COST = 4.0, 4.5, 9.6
# Vector issue: 256 CUs x 4 SIMDs at 2.4 GHz, each SIMD issuing one cycle's
# worth of the costs above per cycle (a plain wave64 VALU instruction holds
# it for 4 cycles: 16 lanes per cycle, the non-packed rate).
SIMD_CYCLES_PEAK_G = 256 * 4 * 2.4
EXTRA_WORKLOADS = ("teacher_forced_320", "teacher_forced_2560_zipf", "temperature_draft_256x8",
                   "teacher_forced_320_f32logits", "greedy_draft_64x5_f32logits",
                   "temperature_draft_256x8_f32logits", "greedy_draft_64x5_fp32", "gated_teacher_forced_320",
                   "gated_greedy_draft_64x5", "teacher_forced_320_backward", "lm_head_teacher_forced_320")


def source_hash(paths) -> str:
    """Hash of the code of the dominant kernel's sources with comments and
    whitespace removed, so that documentation edits keep the counters valid
    while any code change invalidates them."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in paths:
        with open(path, "r", encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    runs (profiles/traffic.json), or None once the kernel source changed."""
    import json as _json
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = _json.load(f)
    if t.get("kernel_source_sha256_16") != source_hash(KERNEL_SOURCES):
        return None
    return t.get("hbm_bytes_per_launch")


def calibrate_copy(torch):
    """A plain device copy of known size for scaling the byte counters:
    256 MiB read + 256 MiB written per launch, 3 launches."""
    src = torch.empty(128 * 1024 * 1024, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"calibration copy: {src.numel() * 2} bytes read and written per launch, 3 launches",
          file=sys.stderr)


def copy_ceiling(torch, np, bw):
    """The practical HBM ceilings, from the bandwidth probes of
    libdspark_bandwidth.so (streaming policy, not steps of the head), each
    timed with events on the current stream (3 warm-up and 10 timed runs,
    median): a 1 GiB copy (read and written, 1 : 1), and a read-mix pass that
    reads 1.8 bytes per byte written, the head's own mix (base logits and W2
    read, corrected logits written); torch's copy_ of the 1 GiB buffers
    beside them."""
    import ctypes
    src = torch.empty(512 * 1024 * 1024, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    size = src.numel() * 2
    nbytes = 2 * size
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sp, dp = ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr())

    def stream_copy(i):
        st = bw.dspark_bandwidth_copy(dp, sp, size, stream)
        if st != 0:
            raise RuntimeError(f"dspark_bandwidth_copy: status {st}")

    _, per = time_calls(stream_copy, 1, 10, 3, torch)
    ms = float(np.median(per))
    _, per_t = time_calls(lambda i: dst.copy_(src), 1, 10, 3, torch)
    ms_t = float(np.median(per_t))
    if not torch.equal(dst, src):
        raise RuntimeError("the reference copy is wrong")
    wbytes = (int(size / 1.8) // 16) * 16          # written; reads all `size` source bytes

    def read_mix(i):
        st = bw.dspark_bandwidth_read_mix(dp, wbytes, sp, size, stream)
        if st != 0:
            raise RuntimeError(f"dspark_bandwidth_read_mix: status {st}")

    _, per_m = time_calls(read_mix, 1, 10, 3, torch)
    ms_m = float(np.median(per_m))
    del src, dst
    torch.cuda.empty_cache()
    gbs = nbytes / (ms * 1e-3) / 1e9
    gbs_m = (size + wbytes) / (ms_m * 1e-3) / 1e9
    return {"GBps": gbs, "bytes_per_copy": nbytes, "ms_per_copy": ms, "frac_of_peak": gbs / HBM_PEAK_GBS,
            "kind": "streaming-policy device copy (dspark_bandwidth_copy, libdspark_bandwidth.so)",
            "read_mix_GBps": gbs_m, "read_mix_read_per_write": size / wbytes,
            "read_mix_frac_of_peak": gbs_m / HBM_PEAK_GBS,
            "torch_copy_GBps": nbytes / (ms_t * 1e-3) / 1e9}


def mfma_ceiling(torch, np, bw, iters=4000):
    """The matrix-core throughput each bf16 product form reaches on this
    device, from libdspark_bandwidth.so's probe (eight independent
    accumulators per wave, 16 waves per CU on every CU; 2 warm-up and 5
    timed launches, median): the kernels here use the 16 x 16 x 32 form."""
    import ctypes
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    waves = 16
    out = torch.empty(cus * waves * 64, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for form, name, flops in ((0, "v_mfma_f32_16x16x32_bf16", 16384), (1, "v_mfma_f32_32x32x16_bf16", 32768)):
        def run(i):
            st = bw.dspark_bandwidth_mfma(ctypes.c_void_p(out.data_ptr()), out.numel() * 4, form, waves, iters, stream)
            if st != 0:
                raise RuntimeError(f"dspark_bandwidth_mfma: status {st}")
        _, per = time_calls(run, 1, 5, 2, torch)
        ms = float(np.median(per))
        res[name] = cus * waves * iters * 8 * flops / (ms * 1e-3) / 1e12
    return {"unit": "TFLOP/s", "kind": "bf16 product throughput per instruction form (dspark_bandwidth_mfma)",
            **res, "frac_of_peak_16x16x32": res["v_mfma_f32_16x16x32_bf16"] / BF16_MFMA_PEAK_TFLOPS,
            "frac_of_peak_32x32x16": res["v_mfma_f32_32x32x16_bf16"] / BF16_MFMA_PEAK_TFLOPS}


def same_size_ceiling(torch, np, bw, read_bytes, write_bytes, steps=200, warmup=100):
    """The read-mix probe at one launch's own bytes (read_bytes read,
    write_bytes written), timed like the kernel: back to back, one event pair
    around `steps` launches, over four rotating buffer sets (so the 256 MB
    Infinity Cache serves none of them).  A copy this size carries the same
    launch ramp-up and drain as the kernel, which a 2 GiB copy hides."""
    import ctypes
    read_bytes, write_bytes = (read_bytes // 16) * 16, (write_bytes // 16) * 16
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    srcs = [torch.empty(read_bytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0) for _ in range(4)]
    dsts = [torch.empty(write_bytes // 2, dtype=torch.bfloat16, device="cuda") for _ in range(4)]

    def launch(i):
        st = bw.dspark_bandwidth_read_mix(ctypes.c_void_p(dsts[i].data_ptr()), write_bytes,
                                          ctypes.c_void_p(srcs[i].data_ptr()), read_bytes, stream)
        if st != 0:
            raise RuntimeError(f"dspark_bandwidth_read_mix: status {st}")

    _, ms = time_region(launch, 4, steps, warmup, torch)
    del srcs, dsts
    torch.cuda.empty_cache()
    return {"read_bytes": read_bytes, "write_bytes": write_bytes, "us_per_launch": ms * 1e3,
            "GBps": (read_bytes + write_bytes) / (ms * 1e-3) / 1e9}


def write_traffic(fetch_csv: str, write_csv: str) -> dict:
    """Turn two rocprofv3 counter runs of `bench.py --calibrate-copy` (one with
    FETCH_SIZE, one with WRITE_SIZE, KiB per dispatch) into HBM bytes per
    launch of the dominant kernel.  Each counter is scaled by what it reads
    for the calibration copy (the first three copy dispatches of the run, of
    known size) and the result goes to profiles/traffic.json, tagged with a
    hash of the kernel source so a later kernel change voids it."""
    import csv
    known_kib = 128 * 1024 * 1024 * 2 / 1024.0
    out = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]][:3]
        kern = [float(r["Counter_Value"]) for r in rows if DOMINANT_KERNEL in r["Kernel_Name"]]
        if len(copies) < 3 or not kern:
            raise SystemExit(f"{path}: calibration copies or {DOMINANT_KERNEL} dispatches missing")
        scale = known_kib / (sum(copies) / len(copies))
        out[counter] = {"kib_per_dispatch": sum(kern) / len(kern), "dispatches": len(kern),
                        "copy_kib_per_dispatch": sum(copies) / len(copies), "scale": scale,
                        "bytes_per_launch": sum(kern) / len(kern) * 1024.0 * scale}
    t = {"kernel": DOMINANT_KERNEL, "workload": WORKLOAD,
         "kernel_source_sha256_16": source_hash(KERNEL_SOURCES),
         "hbm_read_bytes_per_launch": out["FETCH_SIZE"]["bytes_per_launch"],
         "hbm_write_bytes_per_launch": out["WRITE_SIZE"]["bytes_per_launch"],
         "hbm_bytes_per_launch": out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"],
         "counters": out}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    return t


def write_valu(csv_path: str) -> dict:
    """profiles/valu.json from one SQ_INSTS_VALU / SQ_INSTS_VALU_TRANS_F32 /
    SQ_INSTS_VALU_MFMA_BF16 / SQ_INSTS_VALU_INT64 counter run: the temperature
    chain's vector issue cycles per dispatch at the measured instruction
    costs (MFMA instructions run on the matrix cores beside the VALU)."""
    import collections
    import csv
    import json as _json
    acc = collections.defaultdict(list)
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if VALU_KERNEL in row["Kernel_Name"]:
                acc[row["Counter_Name"]].append(float(row["Counter_Value"]))
    avg = {k: sum(v) / len(v) for k, v in acc.items()}
    valu, trans, mfma = avg["SQ_INSTS_VALU"], avg["SQ_INSTS_VALU_TRANS_F32"], avg["SQ_INSTS_VALU_MFMA_BF16"]
    int64 = avg["SQ_INSTS_VALU_INT64"]
    t = {"kernel": VALU_KERNEL, "workload": "temperature_draft_256x8",
         "kernel_source_sha256_16": source_hash(VALU_SOURCES),
         "dispatches": len(acc["SQ_INSTS_VALU"]),
         "valu_wave_insts": valu, "trans_wave_insts": trans, "mfma_wave_insts": mfma, "int64_wave_insts": int64,
         "cost_cycles": {"valu": VALU_COST, "int64": INT64_COST, "trans": TRANS_COST},
         "simd_issue_cycles": (valu - mfma - trans - int64) * VALU_COST + int64 * INT64_COST + trans * TRANS_COST}
    with open(VALU_FILE, "w") as f:
        _json.dump(t, f, indent=1)
        f.write("\n")
    return t


def measured_valu():
    """Vector issue cycles per temperature-chain dispatch (profiles/valu.json),
    or None once the kernel's source changed."""
    import json as _json
    if not os.path.exists(VALU_FILE):
        return None
    with open(VALU_FILE) as f:
        t = _json.load(f)
    if t.get("kernel_source_sha256_16") != source_hash(VALU_SOURCES):
        return None
    return t.get("simd_issue_cycles")


def algorithmic_bytes_sample(w, return_logits=True) -> int:
    """Bytes one sample call must move at least: base logits read, corrected
    logits written, W2 read once, the gathered W1 rows, tokens and ids."""
    lb = 2 if w.ldtype == 1 else 4
    wb = 2 if w.dtype == 1 else 4
    elems = w.B * w.M * w.V
    b = elems * lb * (2 if return_logits else 1)
    b += w.V * w.r * wb                 # W2 once
    b += w.B * w.M * w.r * wb           # gathered W1 rows
    b += w.B * w.M * 8 + w.B * 8        # tokens out, first_prev in
    return b


def algorithmic_bytes_apply(w) -> int:
    lb = 2 if w.ldtype == 1 else 4   # logits
    wb = 2 if w.dtype == 1 else 4    # weights
    return w.B * w.M * w.V * lb * 2 + w.V * w.r * wb + w.B * w.M * (w.r * wb + 8)


def algorithmic_bytes_backward(w) -> int:
    """Bytes the backward must move at least: the gradient of the logits
    read, W2 read, the gathered W1 rows, dW2 and the dense dW1 written."""
    lb = 2 if w.ldtype == 1 else 4
    wb = 2 if w.dtype == 1 else 4
    return w.B * w.M * w.V * lb + 3 * w.V * w.r * wb + w.B * w.M * (w.r * wb + 8)


def algorithmic_bytes_gate(w) -> int:
    """Extra bytes of the gated head: hidden states read, gate_proj weight and
    bias read once (the latent rows stay in cache-sized scratch)."""
    if not w.hidden:
        return 0
    wb = 2 if w.dtype == 1 else 4
    return w.B * w.M * w.hidden * wb + w.r * (w.hidden + w.r) * wb + w.r * wb


def algorithmic_bytes_lm_head(w) -> int:
    """Bytes the fused head must move at least: the head's weight and W2 read
    once, the hidden states and gathered W1 rows, ids, and the fp32 corrected
    logits written (the base logits never exist)."""
    rows = w.B * w.M
    return w.V * w.lm_head * 2 + rows * w.lm_head * 2 + w.V * w.r * 2 + rows * (w.r * 2 + 8) + rows * w.V * 4


def to_dev(a, torch, np):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def time_calls(fn, n_sets, steps, warmup, torch, min_warm_s=0.0):
    """Warm up (`warmup` calls, and at least `min_warm_s` seconds of calls),
    then time exactly `steps` calls (rotating over input sets) with events on
    the current stream; returns (wall seconds, per-call ms)."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < min_warm_s:
        fn(i % n_sets)
        i += 1
        if min_warm_s > 0 and i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn(i % n_sets)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall, per


def time_region(fn, n_sets, steps, warmup, torch, min_warm_s=0.0):
    """Warm up as time_calls does, then time exactly `steps` calls issued
    back to back, with one event pair around the whole timed region on the
    current stream (events between the calls would add gaps of their own);
    returns (wall seconds, event ms per call)."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < min_warm_s:
        fn(i % n_sets)
        i += 1
        if min_warm_s > 0 and i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        fn(i % n_sets)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / steps


def cpu_baseline(w, inp, np):
    """The oracle as it stands, on the host cores: the same workload, timed
    over a few whole calls (a bounded sample of seconds of CPU work)."""
    from oracle import oracle as orc
    cores = len(os.sched_getaffinity(0))
    reps = 3
    orc.lib()
    t0 = time.perf_counter()
    for _ in range(reps):
        orc.sample_block(inp["base"], inp["first_prev"], inp["w1"], inp["w2"], temperature=0.0,
                         n_threads=cores)
    dt = (time.perf_counter() - t0) / reps
    elems = w.B * w.M * w.V
    return {"value": elems / dt, "unit": "corrected-logit elems/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole workload ({w.B} chains x {w.M} positions, V={w.V}, r={w.r}, greedy), "
                      f"{reps} calls, {dt:.2f} s wall each", "tokens_per_s": w.B * w.M / dt}


def measure_extra(name, rmd, wl, torch, np, steps=50, warmup=3):
    """Time one other workload (a parity case, reported beside the main line)."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    distinct = len(np.unique(inp["token_ids"]))
    lbytes = 2 if w.ldtype == 1 else 4
    wbytes = 2 if w.dtype == 1 else 4
    per_set = 2 * w.B * w.M * w.V * lbytes + 2 * w.V * w.r * wbytes
    n_sets = max(2, int(np.ceil(600e6 / per_set)))
    sets = []
    for i in range(n_sets):
        keys = ("base", "first_prev", "token_ids", "w1", "w2") + (("hidden", "gate_w", "gate_b") if w.hidden else ()) \
            + (("grad",) if w.mode == "backward" else ()) + (("lm_hidden", "lm_head") if w.lm_head else ())
        d = {k: to_dev(inp[k], torch, np) for k in keys}
        d["out"] = torch.empty_like(d["base"]) if (w.mode == "apply" or w.return_logits) else None
        if w.lm_head:
            d["out"] = torch.empty(d["base"].shape, dtype=torch.float32, device="cuda")
        d["tok"] = torch.empty((w.B, w.M), dtype=torch.int64, device="cuda")
        d["ws"] = rmd.Workspace(w.B, w.M, w.V, w.r, sample=(w.mode not in ("apply", "backward")),
                                hidden=w.hidden or None, backward=(w.mode == "backward"))
        sets.append(d)
    del inp

    def call(i):
        d = sets[i]
        if w.lm_head:
            rmd.apply_block_logits_lm_head(d["lm_hidden"], d["lm_head"], d["token_ids"], d["w1"], d["w2"],
                                           out=d["out"], workspace=d["ws"])
        elif w.mode == "backward":
            rmd.apply_block_logits_backward(d["grad"], d["token_ids"], d["w1"], d["w2"], workspace=d["ws"])
        elif w.hidden and w.mode == "apply":
            rmd.apply_block_logits_gated(d["base"], d["token_ids"], d["w1"], d["w2"], d["gate_w"], d["gate_b"],
                                         d["hidden"], out=d["out"], workspace=d["ws"])
        elif w.hidden:
            rmd.sample_block_tokens_gated(d["base"], d["first_prev"], d["w1"], d["w2"], d["gate_w"], d["gate_b"],
                                          d["hidden"], w.temperature, seed=w.gumbel_seed,
                                          return_logits=w.return_logits, workspace=d["ws"])
        elif w.mode == "apply":
            rmd.apply_block_logits(d["base"], d["token_ids"], d["w1"], d["w2"], out=d["out"], workspace=d["ws"])
        else:
            rmd.sample_block_tokens(d["base"], d["first_prev"], d["w1"], d["w2"], w.temperature,
                                    seed=w.gumbel_seed, return_logits=w.return_logits, tokens_out=d["tok"],
                                    logits_out=d["out"], workspace=d["ws"])

    # steady state: the first calls after a workload change run slower
    # (measured up to 10% on the apply kernels), so the warm-up runs for a
    # quarter second of calls
    wall, ms = time_region(call, n_sets, steps, warmup, torch, min_warm_s=0.25)
    if w.lm_head:
        alg = algorithmic_bytes_lm_head(w)
    elif w.mode == "backward":
        alg = algorithmic_bytes_backward(w)
    elif w.mode == "apply":
        alg = algorithmic_bytes_apply(w)
    else:
        alg = algorithmic_bytes_sample(w, w.return_logits)
    alg += algorithmic_bytes_gate(w)
    res = {"ms_per_call": ms, "elems_per_s": w.B * w.M * w.V / (ms * 1e-3),
           "algorithmic_GBps": alg / (ms * 1e-3) / 1e9,
           "hbm_frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": alg}
    if w.mode not in ("apply", "backward"):
        res["tokens_per_s"] = w.B * w.M / (ms * 1e-3)
    if w.lm_head:
        # both products on the matrix cores: bf16 dense peak
        flops = 2.0 * w.B * w.M * w.V * (w.lm_head + w.r)
        res["roofline"] = {"bound": "mfma", "kernel": "markov_lm_head_bf16", "achieved": flops / (ms * 1e-3) / 1e12,
                           "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, "flops_per_call": flops}
    cycles = measured_valu() if name == "temperature_draft_256x8" else None
    if cycles:
        # vector-issue roofline of the whole call (one persistent launch;
        # its prologue, exchange waits and launch gap count against it)
        achieved = cycles / (ms * 1e-3) / 1e9
        res["roofline"] = {"bound": "alu", "kernel": VALU_KERNEL, "achieved": achieved,
                           "peak": SIMD_CYCLES_PEAK_G, "unit": "G SIMD issue cycles/s",
                           "frac": achieved / SIMD_CYCLES_PEAK_G,
                           "cost_cycles": {"valu": VALU_COST, "int64": INT64_COST, "trans": TRANS_COST}}
    if w.mode == "apply" and not w.lm_head and not w.hidden:
        # the bias products on the matrix cores: 2 U V r flops, U the rows'
        # distinct predecessors where the grouped kernel plans (>= 1024 rows),
        # else every row
        U = distinct if w.B * w.M >= 1024 else w.B * w.M
        flops = 2.0 * U * w.V * w.r
        res["mfma"] = {"flops_per_call": flops, "distinct_rows": U,
                       "achieved": flops / (ms * 1e-3) / 1e12, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}
    del sets
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads' timings")
    ap.add_argument("--extra", default=",".join(EXTRA_WORKLOADS),
                    help="comma-separated other workloads to time (default: all)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain copy of known size (for scaling byte counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two counter runs and exit (no GPU)")
    ap.add_argument("--write-valu", metavar="VALU_CSV",
                    help="write profiles/valu.json from a vector-instruction counter run and exit (no GPU)")
    args = ap.parse_args()
    if args.write_traffic:
        print(json.dumps(write_traffic(*args.write_traffic)))
        return
    if args.write_valu:
        print(json.dumps(write_valu(args.write_valu)))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the head's sharding is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rank_markov_draft_amd as rmd
    from rank_markov_draft_amd import _lib
    from rank_markov_draft_amd import workloads as wl

    if not os.path.exists(_lib.LIB_PATH):
        _lib.build()
    _lib.load()
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        calibrate_copy(torch)

    w = wl.WORKLOADS[WORKLOAD]
    inp = wl.make_inputs(w)
    n_sets = 4   # 4 x (82.7 + 82.7 + 66.2 + 66.2) MB > 256 MB cache
    sets = []
    for i in range(n_sets):
        d = {k: to_dev(inp[k], torch, np) for k in ("base", "first_prev", "w1", "w2")}
        if i > 0:
            d = {k: v.clone() for k, v in d.items()}
        d["tok"] = torch.empty((w.B, w.M), dtype=torch.int64, device="cuda")
        d["corr"] = torch.empty_like(d["base"])
        d["ws"] = rmd.Workspace(w.B, w.M, w.V, w.r, sample=True)
        sets.append(d)

    def step(i):
        d = sets[i]
        rmd.sample_block_tokens(d["base"], d["first_prev"], d["w1"], d["w2"], 0.0, tokens_out=d["tok"],
                                logits_out=d["corr"], workspace=d["ws"])

    wall, call_ms = time_region(step, n_sets, args.steps, args.warmup, torch)
    ms = wall * 1e3 / args.steps
    elems = w.B * w.M * w.V
    alg = algorithmic_bytes_sample(w)
    achieved = alg / (call_ms * 1e-3) / 1e9

    result = {
        "metric": "corrected-logit elems/s + draft tokens/s at V=129280; % HBM roofline",
        "value": elems / (ms * 1e-3),
        "unit": "corrected-logit elems/s",
        "draft_tokens_per_s": w.B * w.M / (ms * 1e-3),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: greedy left-to-right draft, batch {w.B}, block {w.M}, "
                               f"V={w.V}, r={w.r}, bf16 logits and weights, corrected logits returned",
                   "global_batch": w.B, "block": w.M, "vocab": w.V, "rank": w.r},
        "roofline": {"bound": "hbm", "kernel": DOMINANT_KERNEL,
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "algorithmic_bytes_per_launch": alg, "launch_ms": call_ms},
    }
    del sets
    torch.cuda.empty_cache()
    ceiling = copy_ceiling(torch, np, _lib.load_bandwidth())
    result["copy_ceiling"] = ceiling
    result["roofline"]["frac_of_copy_ceiling"] = achieved / ceiling["GBps"]
    result["roofline"]["frac_of_read_mix_ceiling"] = achieved / ceiling["read_mix_GBps"]
    written = w.B * w.M * w.V * 2
    same = same_size_ceiling(torch, np, _lib.load_bandwidth(), alg - written, written)
    result["copy_ceiling"]["same_size"] = same
    result["roofline"]["frac_of_same_size_copy"] = achieved / same["GBps"]
    if not args.no_extra:
        names = [n for n in args.extra.split(",") if n]
        unknown = [n for n in names if n not in wl.WORKLOADS]
        if unknown:
            raise SystemExit(f"unknown workloads: {unknown}")
        result["other_workloads"] = {n: measure_extra(n, rmd, wl, torch, np) for n in names}
        # matrix-core fractions also against what their instruction form
        # reaches here (every bf16 product kernel uses 16 x 16 x 32)
        mc = mfma_ceiling(torch, np, _lib.load_bandwidth())
        result["mfma_ceiling"] = mc
        for res in result["other_workloads"].values():
            for key in ("mfma", "roofline"):
                if key in res and res[key].get("unit") == "TFLOP/s":
                    res[key]["frac_of_instruction_ceiling"] = res[key]["achieved"] / mc["v_mfma_f32_16x16x32_bf16"]
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp, np)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
