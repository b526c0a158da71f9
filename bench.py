"""Benchmark of the gated-delta-rule hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 20] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of synthetic inputs,
already resident in HBM:

  prefill  gdr_chunk_fwd     8 ragged sequences, 32768 tokens, 32 heads, K=V=128, bf16,
                             fp32 initial and final state          (chunked GDN prefill)
  decode   gdr_decode_paged  256 sequences x 1 token, 16/32 heads, fp32 pool [1024, 32, 128, 128],
                             26 padded slots, commit               (paged decode)
  verify   gdr_decode_paged  64 sequences x 12 tokens, bf16 pool, bf16 per-token states
                             [1025, 12, 32, 128, 128], no commit  (speculative verify)

After the step, legs outside it are timed the same way: the decode and verify launches with the
gating front fused into the token loop (raw q, k, a, b in; gdr_decode_paged_gated), the gating
pass followed by the plain verify launch (gdr_gating_prepass + gdr_decode_paged), the
per-channel-gate (KDA) chunked forward over one sequence of 65573 tokens with 16 heads, 4 x 16384
GDN tokens with 16 heads on the segmented and the single-pass route, and the fused KDA decode
front (gdr_kda_decode_fused) at 1, 16 and 64 sequences x 1 token with 32 heads.

The JSON line reports prefill tokens/s as ``value`` and the decode state GB/s beside it,
each leg's time from HIP events recorded on the stream the library launches on (torch's
current stream, passed explicitly to every call), every launch starting from a clean cache (a
512 MiB read outside the event window evicts L2 and the MALL and leaves no dirty lines), the roofline of the step's dominant kernel
(the longest leg; each leg's own roofline beside it), HBM traffic per launch where the
rocprofv3 counter passes recorded under profiles/ match the current kernel sources, and the
CPU oracle timed on a bounded sample of the prefill workload. Beside the nominal peaks it reports a
measured dense bf16 MFMA rate (a probe kernel) and the HBM rates of the runtime's copy kernel and
torch's fill.

Profiling passes: ``--legs prefill`` runs only that leg, ``--calib-copy-mib N`` first runs one
device copy of N MiB (known traffic, to scale FETCH_SIZE / WRITE_SIZE); both print a short
JSON line instead of the full report.

Summaries (host only, no GPU): ``--summarize-counters FETCH_DIR WRITE_DIR`` turns the two counter
passes' CSV output into profiles/hbm_traffic.md (bytes per launch per leg, and the records this
script reads back), ``--summarize-trace TRACE_DIR PROFILED_LOG PLAIN_LOG`` turns a kernel trace of a
bench run into profiles/bench_kernel_trace.md.

Clock counters (GPU): ``--flow-stamps [SEQ HEAD]`` runs the prefill workload on libgdr_stamps.so (the
flow kernel with shader-clock counters compiled in) and writes profiles/prefill_flow_stamps.md: the
cycles of each phase of the two wave roles per chunk, for the workgroup of sequence SEQ and head HEAD
(default 0 0: the longest sequence), and every workgroup's cycles and clock from entry to its last
chunk.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK = 8.0e12          # B/s
BF16_MFMA_PEAK = 2.5e15    # dense flop/s
FP32_VALU_PEAK = 157.3e12  # flop/s, fp32 vector


def _alg_bytes_prefill(p, with_cu: bool = True):
    """q, k, v, o (io dtype) + g fp32 (per key channel for the per-K gate) + beta (io dtype) per
    token-head, initial (if given) + final state, cu_seqlens (when the call passes them)."""
    io = 2 if p.io_dtype == "bf16" else 4
    gate = p.HV * p.K * 4 if p.per_k_gate else p.HV * 4
    per_tok = p.HK * p.K * io * 2 + p.HV * p.V * io * 2 + gate + p.HV * io
    states = (2 if p.initial_state is not None else 1) * p.N * p.HV * p.V * p.K * 4
    return p.T * per_tok + states + (4 * (p.N + 1) if with_cu else 0)


def _alg_flops_prefill(p, full_tile=False):
    """Chunk-algorithm flops per 64-token chunk-head, counted per token (x T x HV / 64).
    Triangle-exact: K K^T strictly lower, (I+L)^-1 (C^3/3), A.(beta V) and A.(beta e^g K) over the
    strictly lower part, W.h, (K*)^T v_new, Q.h, Q K^T and P v_new over the lower triangle incl.
    the diagonal.  Full-tile: every MFMA tile counted whole."""
    C, K, V = 64, p.K, p.V
    if full_tile:
        per_chunk = 2 * C * C * K * 2 + 2 * C * C * (K + V) + 2 * C * K * V * 3 + 2 * C * C * V
    else:
        tri_strict = C * (C - 1) // 2
        tri_incl = C * (C + 1) // 2
        per_chunk = (2 * tri_strict * K + C ** 3 // 3 + 2 * tri_strict * V + 2 * tri_strict * K
                     + 2 * C * K * V * 3 + 2 * tri_incl * K + 2 * tri_incl * V)
    return per_chunk * p.T * p.HV // C


def _alg_bytes_paged(p, with_ibuf: bool, gated: bool = False):
    """Per active sequence: state read (+ write on commit) per value head, q/k/v/o/g/beta per token
    (gated: the raw a, b in the io dtype instead of g, beta, plus A_log and dt_bias once),
    per-token intermediate states; 4 bytes (the index) per padded sequence."""
    io = 2 if p.io_dtype == "bf16" else 4
    st = 4 if p.pool_dtype == "f32" else 2
    lens = p.lengths
    gate_bytes = p.HV * io * 2 if gated else p.HV * 4 + p.HV * io
    total = p.HV * 8 if gated else 0
    for b in range(p.N):
        if p.state_indices[b] < 0:
            total += 4
            continue
        L = int(lens[b])
        total += 4 + p.HV * p.V * p.K * st * (2 if p.commit else 1)
        total += L * (2 * p.HK * p.K * io + 2 * p.HV * p.V * io + gate_bytes)
        if with_ibuf:
            ib = 2 if p.inter_dtype == "bf16" else 4
            total += L * p.HV * p.V * p.K * ib + 4
    if getattr(p, "_use_cu", True):
        total += 4 * (p.N + 1)
    return total


def _alg_bytes_prepass(p):
    """Gating pass: q, k read and written, a and b read, g (fp32) and beta written, A_log and dt_bias."""
    io = 2 if p.io_dtype == "bf16" else 4
    return p.T * (4 * p.HK * p.K * io + 3 * p.HV * io + p.HV * 4) + p.HV * 8


def _alg_bytes_kda_front(p):
    """Fused KDA decode front, per call: for each active sequence the state read and written once per
    head (commit), the convolution windows read and written, and per token the raw q, k, v, the gate
    input, b, the epilogue gate (when on) and o; once per call the convolution taps and bias, the gate
    projection, A_log, dt_bias and the norm weight; 4 bytes of index per sequence and the cu_seqlens."""
    io = 2 if p.io_dtype == "bf16" else 4
    st = 4 if p.pool_dtype == "f32" else 2
    C = 2 * p.H * p.K + p.H * p.V
    epi = p.norm_weight is not None
    once = C * p.W * io + (C * io if p.conv_bias is not None else 0) + p.H * p.K * p.R * io + p.H * 4 \
        + p.H * p.K * 4 + (p.V * io if epi else 0) + 4 * (p.N + 1)
    per_tok = C * io + p.R * io + p.H * io + p.H * p.V * io * (2 if epi else 1)
    per_seq = 2 * p.H * p.V * p.K * st + 2 * C * (p.W - 1) * io
    lens = np.diff(p.cu_seqlens.astype(np.int64))
    total = once + 4 * p.N
    for n in range(p.N):
        if p.state_indices[n] >= 0:
            total += per_seq + int(lens[n]) * per_tok
    return total


_HERE = os.path.dirname(os.path.abspath(__file__))
_CSRC = os.path.join(_HERE, "gated_delta_rule_63_amd", "csrc")
_TRAFFIC = os.path.join(_HERE, "profiles", "hbm_traffic.md")


def _code_only(text: str) -> str:
    """C/C++ source with comments and all whitespace removed: edits to comments or layout leave it
    unchanged, any change to the code changes it."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return "".join(text.split())


def _source_digest(names):
    """sha256 over the code (comments and whitespace stripped) of the kernel sources a leg runs, so
    measured traffic is dropped once the code changes.  Never edited by hand: a changed digest means
    the counters are taken again."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(_CSRC, n), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def _measured_traffic():
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE passes recorded in
    profiles/hbm_traffic.md (one JSON object per leg on lines starting with '{')."""
    out = {}
    if not os.path.exists(_TRAFFIC):
        return out
    with open(_TRAFFIC) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                rec = json.loads(line)
                out[rec["leg"]] = rec
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(p, pass_s: float = 4.0):
    """The fp64 oracle on the host cores, on the first heads of the prefill workload: the first pass
    picks as many whole heads as fit about ``pass_s`` seconds, then the same heads run twice more;
    the median of the three passes is reported."""
    import oracle  # test infrastructure: only this leg of the benchmark loads it
    from gated_delta_rule_63_amd import inputs

    threads = oracle.default_threads()
    w = [inputs.widen(x) for x in (p.q, p.k, p.v, p.g, p.beta)]

    def run_head(h):
        sel = lambda x: np.ascontiguousarray(x[:, h:h + 1])
        hk = h // (p.HV // p.HK)
        t0 = time.perf_counter()
        oracle.recurrent(np.ascontiguousarray(w[0][:, hk:hk + 1]), np.ascontiguousarray(w[1][:, hk:hk + 1]),
                         sel(w[2]), sel(w[3]), sel(w[4]), p.cu_seqlens, p.scale,
                         None if p.initial_state is None else np.ascontiguousarray(p.initial_state[:, h:h + 1]),
                         threads=threads)
        return time.perf_counter() - t0

    first, heads = 0.0, 0
    while first < pass_s and heads < p.HV:
        first += run_head(heads)
        heads += 1
    passes = [first] + [sum(run_head(h) for h in range(heads)) for _ in range(2)]
    secs = float(np.median(passes))
    tok_per_s = p.T * heads / p.HV / secs
    return {"value": tok_per_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(), "passes_s": passes,
            "sample": f"prefill workload, all {p.T} tokens of {heads} of {p.HV} value heads per pass, "
                      f"median of 3 passes ({secs:.2f} s), scaled to whole-problem tokens/s"}


def _provenance():
    """git commit (where the tree carries .git), a digest of the library sources (always), ROCm and
    torch versions."""
    import hashlib
    import subprocess
    sha = None
    try:
        sha = subprocess.run(["git", "-C", _HERE, "rev-parse", "HEAD"], capture_output=True, text=True,
                             timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        sha = None
    h = hashlib.sha256()
    for root in (_CSRC, os.path.join(_HERE, "include")):
        for dp, _, fs in sorted(os.walk(root)):
            for fn in sorted(fs):
                if fn.endswith((".hip", ".h")):
                    with open(os.path.join(dp, fn), "rb") as f:
                        h.update(f.read())
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    import torch
    return {"git_sha": sha, "source_sha256": h.hexdigest(), "rocm": rocm, "torch": torch.__version__,
            "torch_hip": getattr(torch.version, "hip", None)}


def _measured_mfma_peak(dev):
    """Dense bf16 MFMA rate measured on this GPU by the probe kernel (back-to-back 16x16x32 products,
    8 independent accumulators per wave, 16 waves per CU), best of 5 launches after 2 warm-up launches,
    for low-toggle operands (mode 0, the peak) and random-looking operands (mode 1, closer to real
    data); None when the probe library is missing."""
    import ctypes
    import torch
    path = os.path.join(_HERE, "gated_delta_rule_63_amd", "libgdr_probe.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.gdr_probe_mfma_bf16.restype = ctypes.c_int
    L.gdr_probe_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]
    L.gdr_probe_mfma_bf16_flops.restype = ctypes.c_double
    L.gdr_probe_mfma_bf16_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    blocks, iters = 4096, 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    fl = L.gdr_probe_mfma_bf16_flops(blocks, iters)
    res = {}
    for mode, name in ((0, "tflops"), (1, "tflops_random_operands")):
        ts = []
        for i in range(7):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = L.gdr_probe_mfma_bf16(blocks, iters, mode, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream))
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                return None
            if i >= 2:
                ts.append(e0.elapsed_time(e1) / 1e3)
        res[name] = fl / float(np.min(ts)) / 1e12
    res["kernel"] = (f"v_mfma_f32_16x16x32_bf16, 8 chains per wave, {blocks} x 256 threads x {iters} iterations; "
                     "best of 5 launches")
    return res


def _measured_hbm_rates(dev):
    """HBM rates of the runtime's own streaming kernels on 1 GiB buffers (far past L2 and the MALL),
    best of 5 launches after 2 warm-up launches: a device-to-device copy (torch's copy_, which the HIP
    runtime serves with its copy kernel; 1 GiB read and 1 GiB written) and torch's fill (1 GiB
    written).  Context beside the nominal 8 TB/s: what a plain streaming kernel reaches here."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty(n, dtype=torch.float32, device=dev)
    res = {}
    for name, fn, nbytes in (("runtime_copy_GBps", lambda: dst.copy_(src), 2 * 4 * n),
                             ("torch_fill_GBps", lambda: dst.fill_(2.0), 4 * n)):
        ts = []
        for i in range(7):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1) / 1e3)
        res[name] = nbytes / float(np.min(ts)) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    res["buffers"] = "1 GiB fp32; the copy counts read + write bytes; best of 5 launches"
    return res


def _stats(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"median": float(np.median(a)), "p90": float(np.percentile(a, 90)), "mean": float(np.mean(a)),
            "min": float(np.min(a)), "n": int(a.size)}


# Kernels each leg launches per call: (name fragment, grid size in work-items or None, dispatches per
# call).  A leg's dispatches are told apart from another leg's launches of the same kernel by the
# grid; a spec without a grid takes every dispatch of that name that no gridded spec claimed (two
# such specs share them: the segment-setup kernel has one block in both segmented legs).
_VERIFY_K = "recurrent_kernel<128, gdr::bf16_t, gdr::bf16_t, gdr::bf16_t, gdr::bf16_t, false, 4, true, 0>"


def _leg_kernel_specs():
    from gated_delta_rule_63_amd import inputs
    pp, pk, pc = inputs.prefill(), inputs.kda(), inputs.long_batch()
    flow = "chunk_flow_kernel<gdr::bf16_t>"
    specs = {
        "prefill": [(flow, 512 * pp.HV * pp.N, 1)],
        "decode": [("recurrent_kernel<128, gdr::bf16_t, float, float, void, false, 4, false, 0>", None, 1)],
        "verify": [(_VERIFY_K, None, 1)],
        "decode_gated": [("recurrent_kernel<128, gdr::bf16_t, float, float, void, false, 4, false, 2>", None, 1)],
        "verify_gated": [("recurrent_kernel<128, gdr::bf16_t, gdr::bf16_t, gdr::bf16_t, gdr::bf16_t, false, 4, true, 2>",
                          None, 1)],
        "verify_prepass": [("gating_prepass_kernel<128, gdr::bf16_t>", None, 1), (_VERIFY_K, None, 1)],
        "kda": [("chunk_fused_kernel<128, 128, gdr::bf16_t, gdr::bf16_t, true, true>", None, 1),
                ("chunk_fused_kernel<128, 128, gdr::bf16_t, gdr::bf16_t, true, false>", None, 1),
                ("cp_scan_kernel<128>", 256 * (pk.V // 16) * pk.HV * pk.N, 1), ("cp_setup_kernel", None, 1),
                ("cp_final_kernel", 256 * 256 * pk.N, 1)],
        "cp_segmented": [("chunk_fused_kernel<128, 128, gdr::bf16_t, gdr::bf16_t, false, true>", None, 1),
                         (flow, None, 1), ("cp_scan_kernel<128>", None, 1), ("cp_setup_kernel", None, 1),
                         ("cp_final_kernel", None, 1)],
        "cp_direct": [(flow, 512 * pc.HV * pc.N, 1)],
    }
    for nb in (1, 16, 64):
        specs[f"kda_front_b{nb}"] = [("kda_decode_kernel", 512 * 32 * nb, 1)]
    return specs


def _leg_sources():
    chunk = ["gdr_chunk.hip", "gdr_device.h"]
    cp = ["gdr_chunk.hip", "gdr_device.h", "gdr_cp.hip", "gdr_api.hip"]
    rec = ["gdr_recurrent.hip", "gdr_device.h"]
    out = {"prefill": chunk, "decode": rec, "verify": rec, "decode_gated": rec, "verify_gated": rec,
           "verify_prepass": ["gdr_gating.hip"] + rec, "kda": cp, "cp_segmented": cp, "cp_direct": cp}
    for nb in (1, 16, 64):
        out[f"kda_front_b{nb}"] = ["gdr_kda.hip", "gdr_device.h"]
    return out


def _assign_dispatches(dispatches, specs):
    """dispatches: list of (kernel name, grid, value).  Returns {leg: [(fragment, count, values)]}."""
    claimed = set()
    out = {leg: [None] * len(sp) for leg, sp in specs.items()}
    for leg, sp in specs.items():
        for j, (frag, grid, cnt) in enumerate(sp):
            if grid is not None:
                idx = [i for i, (nm, g, _) in enumerate(dispatches) if frag in nm and g == grid]
                claimed.update(idx)
                out[leg][j] = (frag, cnt, [dispatches[i][2] for i in idx])
    for leg, sp in specs.items():
        for j, (frag, grid, cnt) in enumerate(sp):
            if grid is None:
                idx = [i for i, (nm, g, _) in enumerate(dispatches) if frag in nm and i not in claimed]
                out[leg][j] = (frag, cnt, [dispatches[i][2] for i in idx])
    return out


def _summarize_counters(fetch_dir, write_dir):
    """profiles/hbm_traffic.md from the FETCH_SIZE and WRITE_SIZE passes (rocprofv3 csv output)."""
    import csv
    import glob
    from gated_delta_rule_63_amd import inputs

    def load(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        per = {}
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                key = (r["Dispatch_Id"], r["Kernel_Name"], int(r["Grid_Size"]))
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        return [(nm, g, v) for (_, nm, g), v in sorted(per.items(), key=lambda kv: int(kv[0][0]))]

    fe, wr = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    cf = max(v for nm, _, v in fe if "copyBuffer" in nm)
    cw = max(v for nm, _, v in wr if "copyBuffer" in nm)
    copy_kib = 1024 * 1024  # the --calib-copy-mib 1024 copy reads and writes 1 GiB
    ff, wf = copy_kib / cf, copy_kib / cw
    specs = _leg_kernel_specs()
    af, aw = _assign_dispatches(fe, specs), _assign_dispatches(wr, specs)
    pp, pd, pv, pk, pc = inputs.prefill(), inputs.decode(), inputs.verify(), inputs.kda(), inputs.long_batch()
    alg = {"prefill": _alg_bytes_prefill(pp), "decode": _alg_bytes_paged(pd, with_ibuf=False),
           "verify": _alg_bytes_paged(pv, with_ibuf=True),
           "decode_gated": _alg_bytes_paged(pd, with_ibuf=False, gated=True),
           "verify_gated": _alg_bytes_paged(pv, with_ibuf=True, gated=True),
           "verify_prepass": _alg_bytes_prepass(pv) + _alg_bytes_paged(pv, with_ibuf=True),
           "kda": _alg_bytes_prefill(pk, with_cu=False), "cp_segmented": _alg_bytes_prefill(pc),
           "cp_direct": _alg_bytes_prefill(pc)}
    for nb in (1, 16, 64):
        alg[f"kda_front_b{nb}"] = _alg_bytes_kda_front(
            inputs.kda_front_problem(560 + nb, B=nb, q_len=1, H=32, R=128, num_slots=max(2 * nb, 8)))
    srcs = _leg_sources()
    rows, recs = [], []
    for leg in specs:
        fk = wk = 0.0
        parts, ok = [], True
        for (frag, cnt, fv), (_, _, wv) in zip(af[leg], aw[leg]):
            if not fv or not wv:
                ok = False
                break
            fk += cnt * sum(fv) / len(fv)
            wk += cnt * sum(wv) / len(wv)
            parts.append(f"`{frag}` x{cnt} ({len(fv)})")
        if not ok:
            continue
        b = (fk * ff + wk * wf) * 1024
        rows.append(f"| {leg} | {', '.join(parts)} | {fk:.1f} | {wk:.1f} | {b:.4e} | {alg[leg]:.4e} | "
                    f"{b / alg[leg]:.3f} |")
        recs.append(json.dumps({"leg": leg, "kernels": [f for f, _, _ in specs[leg]],
                                "source_sha256": _source_digest(srcs[leg]), "fetch_kib_raw": fk, "write_kib_raw": wk,
                                "fetch_factor": ff, "write_factor": wf, "bytes_per_launch": b,
                                "alg_bytes_per_launch": alg[leg]}))
    cmd = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 240 rocprofv3 --pmc {c} --output-format csv -d "
           "/root/repo/gpurun_out/prof_{d} -o run -- python3 /root/repo/bench.py --steps 2 --warmup 1 "
           "--no-cpu-baseline --calib-copy-mib 1024")
    out = f"""# HBM traffic per call (rocprofv3 FETCH_SIZE / WRITE_SIZE), MI355X

Two counter passes, each in a run of its own, then this summary (host only):

```
{cmd.format(c='FETCH_SIZE', d='fetch')}
{cmd.format(c='WRITE_SIZE', d='write')}
python3 bench.py --summarize-counters gpurun_out/prof_fetch gpurun_out/prof_write
```

Scaling: the run first copies 1 GiB device-to-device (`__amd_rocclr_copyBuffer`, reads and writes 1048576 KiB). FETCH_SIZE reads {cf:.1f} KiB and WRITE_SIZE {cw:.1f} KiB for it, so the factors are {ff:.4f} (fetch) and {wf:.4f} (write).

Each leg sums, per call, the kernels it launches (the count after each kernel is the dispatches per call; the number in parentheses, the dispatches averaged). Launches of one kernel by two legs are told apart by their grids.

| leg | kernels per call | FETCH_SIZE KiB (raw) | WRITE_SIZE KiB (raw) | scaled bytes/call | algorithmic bytes | ratio |
|---|---|---|---|---|---|---|
""" + "\n".join(rows) + """

Records read by bench.py (`traffic` is reported only while the sha256 of the leg's kernel sources still matches):

""" + "\n".join(recs) + "\n"
    with open(_TRAFFIC, "w") as f:
        f.write(out)
    print(out)


def _flow_stamps(seq: int, head: int, reps: int = 6):
    """Clock counters of chunk_flow_kernel on the prefill workload (measurement build); writes
    profiles/prefill_flow_stamps.md."""
    import ctypes
    import torch
    from gated_delta_rule_63_amd import gdr, inputs

    gdr.use_library(os.path.join(_HERE, "gated_delta_rule_63_amd", "libgdr_stamps.so"))
    L = gdr.lib()
    L.gdr_dbg_flow_target.restype = ctypes.c_int
    L.gdr_dbg_flow_target.argtypes = [ctypes.c_int, ctypes.c_int]
    L.gdr_dbg_flow_stamps.restype = ctypes.c_int
    L.gdr_dbg_flow_stamps.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")

    def to_dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    pp = inputs.prefill()
    if not (0 <= seq < pp.N and 0 <= head < pp.HV):
        raise SystemExit(f"--flow-stamps: SEQ in 0..{pp.N - 1}, HEAD in 0..{pp.HV - 1}")
    P = {k: to_dev(getattr(pp, k)) for k in ("q", "k", "v", "g", "beta")}
    cu, h0 = to_dev(pp.cu_seqlens.astype(np.int32)), to_dev(pp.initial_state)
    o = torch.empty((pp.T, pp.HV, pp.V), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((pp.N, pp.HV, pp.V, pp.K), dtype=torch.float32, device=dev)
    flush = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)
    assert L.gdr_dbg_flow_target(seq, head) == 0
    st = np.zeros((2, 128, 8), dtype=np.uint64)
    wg = np.zeros((8, 32, 4), dtype=np.uint64)
    ms = []
    for _ in range(reps):  # the last launch is read; each starts from a clean cache, as in the bench
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gdr.gdr_chunk_fwd(P["q"], P["k"], P["v"], P["g"], P["beta"], cu, pp.scale, h0, o=o, final_state=ht)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    assert L.gdr_dbg_flow_stamps(ctypes.c_void_p(st.ctypes.data), ctypes.c_void_p(wg.ctypes.data)) == 0
    s, w = st.astype(np.int64), wg.astype(np.int64)
    lens = [int(x) for x in pp.lengths]
    nc = (lens[seq] + 63) // 64
    it = np.arange(1, nc + 1)
    sl = it[(it >= 5) & (it <= nc - 5)]  # steady state: away from the first and last chunks
    med = lambda x: float(np.median(x))
    a, b = s[0], s[1]
    rows = [
        ("iteration", med(a[sl, 3] - a[sl - 1, 3]), med(b[sl, 3] - b[sl - 1, 3])),
        ("phase X: work", med(a[sl, 0] - a[sl - 1, 3]), med(b[sl, 0] - b[sl - 1, 3])),
        ("phase X: barrier wait", med(a[sl, 1] - a[sl, 0]), med(b[sl, 1] - b[sl, 0])),
        ("phase Y: work", med(a[sl, 2] - a[sl, 1]), med(b[sl, 2] - b[sl, 1])),
        ("phase Y: barrier wait", med(a[sl, 3] - a[sl, 2]), med(b[sl, 3] - b[sl, 2])),
    ]
    state_x = [("K S^T and S Q^T products", med(a[sl, 5] - a[sl - 1, 3])), ("R and the block solve", med(a[sl, 6] - a[sl, 5])),
               ("output scaling, the state update", med(a[sl, 0] - a[sl, 6]))]
    state_y = [("P v_new part of the output, its stores", med(a[sl, 4] - a[sl, 1])),
               ("the off-diagonal P tiles", med(a[sl, 2] - a[sl, 4]))]
    prep_x = [("q and k load issue", med(b[sl, 6] - b[sl, 5])),
              ("L tiles, diagonal inverses, diagonal P tiles", med(b[sl, 4] - b[sl, 6])),
              ("v, g, beta load issue", med(b[sl, 7] - b[sl, 4])), ("L stores, remaining L tiles, P stores", med(b[sl, 0] - b[sl, 7]))]
    cyc = w[:, :, 2] - w[:, :, 0]
    ns = (w[:, :, 3] - w[:, :, 1]) * 10.0  # the real-time clock counts at 100 MHz
    t0 = w[:, :, 1].min()
    end_us = (w[:, :, 3] - t0) * 10.0 / 1e3
    cmd = "python3 bench.py --flow-stamps" + ("" if (seq, head) == (0, 0) else f" {seq} {head}")
    out = ["# Clock counters of `chunk_flow_kernel<bf16>`, prefill workload, MI355X", "",
           "```", cmd, "```", "",
           f"The measurement build `libgdr_stamps.so` (the flow kernel compiled with `GDR_FLOW_STAMPS`: "
           f"shader-clock reads at the phase boundaries and inside the phases, and each workgroup's entry "
           f"and exit) runs the prefill workload {reps} times, each launch after a 512 MiB cache-flush "
           f"read; the last launch is read. Launch times (HIP events): "
           + ", ".join(f"{x:.3f}" for x in ms) + " ms.", "",
           f"## Per chunk, workgroup of sequence {seq} ({lens[seq]} tokens, {nc} chunks), head {head}", "",
           f"Medians over chunks 5 .. {nc - 5}, in shader-clock cycles. Waves 0 and 4 share a SIMD.", "",
           "| | state waves (wave 0) | prep waves (wave 4) |", "|---|---|---|"]
    out += [f"| {nm} | {x:.0f} | {y:.0f} |" for nm, x, y in rows]
    out += ["", "Inside the phases:", "", "| role, phase | part | cycles |", "|---|---|---|"]
    out += [f"| state, X | {nm} | {x:.0f} |" for nm, x in state_x]
    out += [f"| state, Y | {nm} | {x:.0f} |" for nm, x in state_y]
    out += [f"| prep, X | {nm} | {x:.0f} |" for nm, x in prep_x]
    out += ["", "## Every workgroup: entry to the end of its last chunk", "",
            "Cycles (shader clock), clock (cycles over the 100 MHz real-time clock) and end time after the "
            "first workgroup's entry, over the heads of each sequence.", "",
            "| sequence | tokens | chunks | cycles: min / median / max | clock GHz: median | end µs: median / max |",
            "|---|---|---|---|---|---|"]
    for n in range(min(pp.N, 8)):
        c, g, e = cyc[n, :pp.HV], cyc[n, :pp.HV] / np.maximum(ns[n, :pp.HV], 1), end_us[n, :pp.HV]
        out.append(f"| {n} | {lens[n]} | {(lens[n] + 63) // 64} | {c.min()} / {int(np.median(c))} / {c.max()} | "
                   f"{np.median(g):.2f} | {np.median(e):.1f} / {e.max():.1f} |")
    text = "\n".join(out) + "\n"
    path = os.path.join(_HERE, "profiles", "prefill_flow_stamps.md")
    with open(path, "w") as f:
        f.write(text)
    print(text)


def _summarize_trace(trace_dir, profiled_log, plain_log):
    """profiles/bench_kernel_trace.md from a kernel trace of a bench run and two bench JSON lines."""
    import csv
    import glob

    def jl(p):
        with open(p) as f:
            for line in f:
                if line.startswith("{") and '"metric"' in line:
                    return json.loads(line)
        raise SystemExit(f"no bench line in {p}")
    stats = list(csv.DictReader(open(glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)[0])))
    trace = list(csv.DictReader(open(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)[0])))
    disp = [(r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
             (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in trace]
    specs = _leg_kernel_specs()
    per_leg = _assign_dispatches(disp, specs)
    pr, un = jl(profiled_log), jl(plain_log)
    nm = lambda x: x if len(x) <= 110 else x[:107] + "..."
    t = "\n".join(f"| `{nm(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                  f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}% |" for r in stats)
    legs = {**{k: v for k, v in pr["leg_ms"].items()}, **{k: v["ms"] for k, v in pr["extra_legs"].items()}}
    plain = {**{k: v for k, v in un["leg_ms"].items()}, **{k: v["ms"] for k, v in un["extra_legs"].items()}}
    lines = []
    for leg, parts in per_leg.items():
        if leg not in legs:
            continue
        # the timed calls come after the warm-up ones: keep each kernel's last steps x count dispatches
        parts = [(frag, cnt, v[-pr["steps"] * cnt:]) for frag, cnt, v in parts]
        us = [f"`{frag}` x{cnt}: {sum(v) / len(v):.1f} us over {len(v)}" for frag, cnt, v in parts if v]
        tot = sum(cnt * sum(v) / len(v) for frag, cnt, v in parts if v)
        lines.append(f"| {leg} | {'; '.join(us)} | {tot / 1e3:.4f} | {legs[leg]:.4f} | {plain.get(leg, float('nan')):.4f} |")
    cmd = (f"cd /tmp && export TMPDIR=/tmp && timeout -k 10 600 rocprofv3 --kernel-trace --stats --output-format csv -d "
           f"/root/repo/gpurun_out/prof_trace -o run -- python3 /root/repo/bench.py --no-cpu-baseline "
           f"--steps {pr['steps']} --warmup {pr['warmup']}")
    out = f"""# Kernel trace of a bench run, MI355X

```
{cmd}
python3 bench.py --summarize-trace gpurun_out/prof_trace PROFILED_LOG PLAIN_LOG
```

PROFILED_LOG is the bench line the profiled run printed, PLAIN_LOG the line of an unprofiled
`python3 bench.py` on the same box.  `run_kernel_stats.csv` ({pr['warmup']} warm-up and {pr['steps']} timed calls per leg; `reduce_kernel` is torch's sum that cleans the cache before each timed launch):

| kernel | calls | avg us | min us | max us | share |
|---|---|---|---|---|---|
{t}

Per leg, from `run_kernel_trace.csv` (each kernel's mean over the leg's timed dispatches, the last ones of the run; a leg's launches of a kernel are told apart from another leg's by the grid), against the HIP-event times (ms, mean over the timed calls) of the profiled and the unprofiled run:

| leg | kernels per call | kernel sum ms | HIP events, profiled | HIP events, plain |
|---|---|---|---|---|
""" + "\n".join(lines) + "\n"
    path = os.path.join(_HERE, "profiles", "bench_kernel_trace.md")
    with open(path, "w") as f:
        f.write(out)
    print(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the first steps after process start run several percent slower (clocks and caches settle):
    # the default warm-up lets the timed steps see the steady state
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", default="prefill,decode,verify",
                    help="comma-separated subset of legs to run (profiling passes); the JSON line needs all three")
    ap.add_argument("--extra-legs", default="decode_gated,verify_gated,verify_prepass,kda,cp_segmented,cp_direct,"
                                            "kda_front_b1,kda_front_b16,kda_front_b64",
                    help="legs outside the step, timed after it: the gating front fused into the decode and verify "
                         "launches, the gating pass followed by the plain verify launch, the per-channel-gate "
                         "(KDA) chunked forward over one 65573-token sequence, and 4 x 16384-token GDN sequences "
                         "with 16 heads on the segmented and the single-pass route, and the fused KDA decode front at "
                         "1, 16 and 64 sequences x 1 token with 32 heads ('' for none)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before the legs, run one device-to-device copy of this many MiB (a plain copy kernel of "
                         "known size, used to scale the HBM byte counters of a profiling pass) and stop after the legs")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="host only: write profiles/hbm_traffic.md from the two counter passes and stop")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_DIR", "PROFILED_LOG", "PLAIN_LOG"),
                    help="host only: write profiles/bench_kernel_trace.md from a kernel trace of a bench run and stop")
    ap.add_argument("--flow-stamps", nargs="*", type=int, metavar="SEQ_HEAD",
                    help="GPU: per-phase clock counters of the prefill flow kernel (measurement build) into "
                         "profiles/prefill_flow_stamps.md, for the workgroup of sequence SEQ and head HEAD "
                         "(default 0 0), and stop")
    args = ap.parse_args()
    if args.flow_stamps is not None:
        if len(args.flow_stamps) not in (0, 2):
            ap.error("--flow-stamps takes no value or SEQ HEAD")
        _flow_stamps(*(args.flow_stamps or [0, 0]))
        return
    if args.summarize_counters:
        _summarize_counters(*args.summarize_counters)
        return
    if args.summarize_trace:
        _summarize_trace(*args.summarize_trace)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the gated-delta-rule path here is built and timed on a single "
              "MI355X (every (sequence, head) state is independent; sharding is described, not run). "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_63_amd import gdr, inputs

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    print("bench: generating inputs", file=sys.stderr, flush=True)
    pp = inputs.prefill()
    pd = inputs.decode()
    pv = inputs.verify()

    P = {k: to_dev(getattr(pp, k)) for k in ("q", "k", "v", "g", "beta")}
    P["cu"] = to_dev(pp.cu_seqlens.astype(np.int32))
    P["h0"] = to_dev(pp.initial_state)
    P["o"] = torch.empty((pp.T, pp.HV, pp.V), dtype=torch.bfloat16, device=dev)
    P["ht"] = torch.empty((pp.N, pp.HV, pp.V, pp.K), dtype=torch.float32, device=dev)
    ws_bytes = gdr.gdr_chunk_workspace_size(P["q"], P["v"], P["g"], pp.N)
    P["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    D = {k: to_dev(getattr(pd, k)) for k in ("q", "k", "v", "g", "beta")}
    D["pool"] = to_dev(pd.pool)
    D["idx"] = to_dev(pd.state_indices)
    D["o"] = torch.empty((pd.T, pd.HV, pd.V), dtype=torch.bfloat16, device=dev)

    V_ = {k: to_dev(getattr(pv, k)) for k in ("q", "k", "v", "g", "beta")}
    V_["cu"] = to_dev(pv.cu_seqlens.astype(np.int32))
    V_["pool"] = to_dev(pv.pool)
    V_["idx"] = to_dev(pv.state_indices)
    V_["ibi"] = to_dev(pv.inter_state_indices)
    V_["ib"] = torch.zeros((pv.num_cache_slots, pv.cache_steps, pv.HV, pv.V, pv.K), dtype=torch.bfloat16, device=dev)
    V_["o"] = torch.empty((pv.T, pv.HV, pv.V), dtype=torch.bfloat16, device=dev)

    # gating front: raw q, k, a, b (same shapes as the step's decode / verify inputs)
    rd = inputs.raw_gating(12, pd.T, pd.HK, pd.HV, pd.K)
    rv = inputs.raw_gating(13, pv.T, pv.HK, pv.HV, pv.K)
    DG = {k: to_dev(getattr(rd, k)) for k in ("q", "k", "a", "b", "A_log", "dt_bias")}
    VG = {k: to_dev(getattr(rv, k)) for k in ("q", "k", "a", "b", "A_log", "dt_bias")}
    VP = {"q": torch.empty_like(VG["q"]), "k": torch.empty_like(VG["k"]),
          "g": torch.empty((pv.T, pv.HV), dtype=torch.float32, device=dev),
          "beta": torch.empty((pv.T, pv.HV), dtype=torch.bfloat16, device=dev)}

    C_ = None
    if {"cp_segmented", "cp_direct"} & set(args.extra_legs.split(",")):
        pc = inputs.long_batch()
        C_ = {k: to_dev(getattr(pc, k)) for k in ("q", "k", "v", "g", "beta")}
        C_["cu"] = to_dev(pc.cu_seqlens.astype(np.int32))
        C_["h0"] = to_dev(pc.initial_state)
        C_["o"] = torch.empty((pc.T, pc.HV, pc.V), dtype=torch.bfloat16, device=dev)
        C_["ht"] = torch.empty((pc.N, pc.HV, pc.V, pc.K), dtype=torch.float32, device=dev)
        C_["ws"] = torch.empty(max(256, gdr.gdr_chunk_workspace_size(C_["q"], C_["v"], C_["g"], pc.N)),
                               dtype=torch.uint8, device=dev)

    def cp_segmented():
        gdr.gdr_chunk_fwd(C_["q"], C_["k"], C_["v"], C_["g"], C_["beta"], C_["cu"], pc.scale, C_["h0"], o=C_["o"],
                          final_state=C_["ht"], workspace=C_["ws"])

    def cp_direct():
        gdr.gdr_chunk_fwd(C_["q"], C_["k"], C_["v"], C_["g"], C_["beta"], C_["cu"], pc.scale, C_["h0"], o=C_["o"],
                          final_state=C_["ht"], segmented=False)

    # fused KDA decode front at decode shapes: 1, 16 and 64 sequences x 1 token, 32 heads, K=V=128,
    # gate rank 128, convolution width 4, epilogue on, fp32 pool, commit
    KF = {}
    for nb in (1, 16, 64):
        if f"kda_front_b{nb}" not in args.extra_legs.split(","):
            continue
        pf = inputs.kda_front_problem(560 + nb, B=nb, q_len=1, H=32, R=128, num_slots=max(2 * nb, 8))
        dd = {n: to_dev(getattr(pf, n)) for n in ("q", "k", "v", "conv_weight", "conv_bias", "conv_state", "gate_in",
                                                 "gate_weight", "A_log", "dt_bias", "b", "norm_weight", "norm_gate",
                                                 "pool", "state_indices")}
        dd["o"] = torch.empty((pf.T, pf.H, pf.V), dtype=torch.bfloat16, device=dev)
        KF[nb] = (pf, dd)

    def kda_front(nb):
        pf, dd = KF[nb]
        gdr.gdr_kda_decode_fused(dd["q"], dd["k"], dd["v"], dd["conv_weight"], dd["conv_state"], dd["gate_in"],
                                 dd["gate_weight"], dd["A_log"], dd["dt_bias"], dd["b"], dd["pool"], dd["state_indices"],
                                 max_q_len=1, commit=True, scale=pf.scale, conv_bias=dd["conv_bias"],
                                 l2norm_eps=pf.l2_eps, norm_weight=dd["norm_weight"], norm_gate=dd["norm_gate"],
                                 norm_eps=pf.norm_eps, o=dd["o"])

    K_ = None
    if "kda" in args.extra_legs.split(","):
        pk = inputs.kda()
        K_ = {k: to_dev(getattr(pk, k)) for k in ("q", "k", "v", "g", "beta")}
        K_["o"] = torch.empty((pk.T, pk.HV, pk.V), dtype=torch.bfloat16, device=dev)
        K_["ht"] = torch.empty((pk.N, pk.HV, pk.V, pk.K), dtype=torch.float32, device=dev)
        K_["ws"] = torch.empty(max(256, gdr.gdr_chunk_workspace_size(K_["q"], K_["v"], K_["g"], pk.N)),
                               dtype=torch.uint8, device=dev)

    def kda():
        gdr.gdr_chunk_fwd(K_["q"], K_["k"], K_["v"], K_["g"], K_["beta"], None, pk.scale, None, o=K_["o"],
                          final_state=K_["ht"], workspace=K_["ws"])

    def prefill():
        gdr.gdr_chunk_fwd(P["q"], P["k"], P["v"], P["g"], P["beta"], P["cu"], pp.scale, P["h0"], o=P["o"],
                          final_state=P["ht"], workspace=P["ws"])

    def decode():
        gdr.gdr_decode_paged(D["q"], D["k"], D["v"], D["g"], D["beta"], D["pool"], D["idx"], cu_seqlens=None,
                             max_q_len=1, commit=True, scale=pd.scale, o=D["o"])

    def verify():
        gdr.gdr_decode_paged(V_["q"], V_["k"], V_["v"], V_["g"], V_["beta"], V_["pool"], V_["idx"],
                             cu_seqlens=V_["cu"], max_q_len=12, commit=False, inter_states=V_["ib"],
                             inter_state_indices=V_["ibi"], scale=pv.scale, o=V_["o"])

    def decode_gated():
        gdr.gdr_decode_paged_gated(DG["q"], DG["k"], D["v"], DG["a"], DG["b"], DG["A_log"], DG["dt_bias"], D["pool"],
                                   D["idx"], cu_seqlens=None, max_q_len=1, commit=True, scale=pd.scale,
                                   l2norm_eps=rd.eps, o=D["o"])

    def verify_gated():
        gdr.gdr_decode_paged_gated(VG["q"], VG["k"], V_["v"], VG["a"], VG["b"], VG["A_log"], VG["dt_bias"],
                                   V_["pool"], V_["idx"], cu_seqlens=V_["cu"], max_q_len=12, commit=False,
                                   inter_states=V_["ib"], inter_state_indices=V_["ibi"], scale=pv.scale,
                                   l2norm_eps=rv.eps, o=V_["o"])

    def verify_prepass():
        gdr.gdr_gating_prepass(VG["q"], VG["k"], VG["a"], VG["b"], VG["A_log"], VG["dt_bias"], l2norm_eps=rv.eps,
                               q_out=VP["q"], k_out=VP["k"], g_out=VP["g"], beta_out=VP["beta"])
        gdr.gdr_decode_paged(VP["q"], VP["k"], V_["v"], VP["g"], VP["beta"], V_["pool"], V_["idx"],
                             cu_seqlens=V_["cu"], max_q_len=12, commit=False, inter_states=V_["ib"],
                             inter_state_indices=V_["ibi"], scale=pv.scale, o=V_["o"])

    legs = [(n, f) for n, f in (("prefill", prefill), ("decode", decode), ("verify", verify))
            if n in args.legs.split(",")]
    extra = [(n, f) for n, f in (("decode_gated", decode_gated), ("verify_gated", verify_gated),
                                 ("verify_prepass", verify_prepass), ("kda", kda), ("cp_segmented", cp_segmented),
                                 ("cp_direct", cp_direct), ("kda_front_b1", lambda: kda_front(1)),
                                 ("kda_front_b16", lambda: kda_front(16)), ("kda_front_b64", lambda: kda_front(64)))
             if n in args.extra_legs.split(",")]
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # Each timed launch starts from a clean cache: a 512 MiB read outside the event window evicts
    # L2 and the 256 MB MALL, and, being a read, leaves no dirty lines behind (a leg that follows a
    # write-heavy leg would otherwise pay for writing back the previous leg's output).
    flush_buf = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)

    def clean_cache():
        flush_buf.sum()

    print("bench: warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for _, fn in legs:
            fn()
    torch.cuda.synchronize()

    K = args.steps
    ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
          for name, _ in legs}
    print(f"bench: timing {K} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        for name, fn in legs:
            clean_cache()
            ev[name][i][0].record()
            fn()
            ev[name][i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # legs outside the step, timed the same way after it
    extra_ms, extra_stats = {}, {}
    if extra and len(legs) == 3:  # (also in a counter pass, so its kernels are sampled)
        print("bench: timing the gated legs", file=sys.stderr, flush=True)
        for _ in range(args.warmup):
            for _, fn in extra:
                fn()
        xev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(K)] for name, _ in extra}
        for i in range(K):
            for name, fn in extra:
                clean_cache()
                xev[name][i][0].record()
                fn()
                xev[name][i][1].record()
        torch.cuda.synchronize()
        extra_stats = {name: _stats([a.elapsed_time(b) for a, b in xev[name]]) for name, _ in extra}
        extra_ms = {name: st["mean"] for name, st in extra_stats.items()}
    if len(legs) < 3 or args.calib_copy_mib:
        print(json.dumps({"profiling_pass": [n for n, _ in legs], "steps": K}))
        return
    # every figure below uses the mean launch time (what rocprofv3's average duration reports);
    # median, p90 and min sit beside it in leg_stats_ms
    leg_stats = {name: _stats([a.elapsed_time(b) for a, b in ev[name]]) for name, _ in legs}
    leg_ms = {name: st["mean"] for name, st in leg_stats.items()}

    b_pre = _alg_bytes_prefill(pp)
    f_pre = _alg_flops_prefill(pp)
    f_pre_full = _alg_flops_prefill(pp, full_tile=True)
    b_dec = _alg_bytes_paged(pd, with_ibuf=False)
    b_ver = _alg_bytes_paged(pv, with_ibuf=True)
    s_pre, s_dec, s_ver = leg_ms["prefill"] / 1e3, leg_ms["decode"] / 1e3, leg_ms["verify"] / 1e3
    state_bytes_dec = int(sum(1 for s in pd.state_indices if s >= 0)) * pd.HV * pd.V * pd.K * 4 * 2

    prefill_tps = pp.T / s_pre
    leg_info = {
        "prefill": {"kernel": "chunk_flow_kernel<bf16> (one launch per call)", "bytes": b_pre,
                    "flops": f_pre, "secs": s_pre, "sources": ["gdr_chunk.hip", "gdr_device.h"]},
        "decode": {"kernel": "recurrent_kernel (256 x 1 token, fp32 pool, commit)", "bytes": b_dec, "flops": None,
                   "secs": s_dec, "sources": ["gdr_recurrent.hip", "gdr_device.h"]},
        "verify": {"kernel": "recurrent_kernel (64 x 12 tokens, bf16 pool, bf16 per-token states)", "bytes": b_ver,
                   "flops": None, "secs": s_ver, "sources": ["gdr_recurrent.hip", "gdr_device.h"]},
    }
    gated_sources = ["gdr_recurrent.hip", "gdr_device.h"]
    if "decode_gated" in extra_ms:
        leg_info["decode_gated"] = {"kernel": "recurrent_kernel, gating front in the token loop (decode shape)",
                                    "bytes": _alg_bytes_paged(pd, with_ibuf=False, gated=True), "flops": None,
                                    "secs": extra_ms["decode_gated"] / 1e3, "sources": gated_sources}
    if "verify_gated" in extra_ms:
        leg_info["verify_gated"] = {"kernel": "recurrent_kernel, gating front in the token loop (verify shape)",
                                    "bytes": _alg_bytes_paged(pv, with_ibuf=True, gated=True), "flops": None,
                                    "secs": extra_ms["verify_gated"] / 1e3, "sources": gated_sources}
    if "verify_prepass" in extra_ms:
        leg_info["verify_prepass"] = {"kernel": "gating_prepass_kernel then recurrent_kernel (verify shape)",
                                      "bytes": _alg_bytes_prepass(pv) + b_ver, "flops": None,
                                      "secs": extra_ms["verify_prepass"] / 1e3,
                                      "sources": ["gdr_gating.hip"] + gated_sources}
    if "kda" in extra_ms:
        leg_info["kda"] = {"kernel": "segmented route: setup, paired offset/map run and outputs run of "
                                     "chunk_fused_kernel<128,128,bf16,per-K gate>, scan, final-state copy "
                                     "(1 x 65573 tokens, 16 heads; bytes, time and traffic per call)",
                           "bytes": _alg_bytes_prefill(pk, with_cu=False), "flops": None, "secs": extra_ms["kda"] / 1e3,
                           "sources": ["gdr_chunk.hip", "gdr_device.h", "gdr_cp.hip", "gdr_api.hip"]}
    for leg, route in (("cp_segmented", "segmented route: setup, paired offset/map run (chunk_fused_kernel), scan, "
                                         "outputs run (chunk_flow_kernel), final-state copy"),
                       ("cp_direct", "single pass: one chunk_flow_kernel launch, one workgroup per (sequence, head)")):
        if leg in extra_ms:
            leg_info[leg] = {"kernel": f"{route} (4 x 16384 tokens, 16 heads, K=V=128, bf16; per call)",
                             "bytes": _alg_bytes_prefill(pc), "flops": _alg_flops_prefill(pc),
                             "secs": extra_ms[leg] / 1e3,
                             "sources": ["gdr_chunk.hip", "gdr_device.h", "gdr_cp.hip", "gdr_api.hip"]}
    for nb in (1, 16, 64):
        leg = f"kda_front_b{nb}"
        if leg in extra_ms:
            leg_info[leg] = {"kernel": f"kda_decode_kernel (fused KDA decode front: {nb} x 1 token, 32 heads, K=V=128, "
                                       "gate rank 128, width 4, epilogue, fp32 pool, commit)",
                             "bytes": _alg_bytes_kda_front(KF[nb][0]), "flops": None, "secs": extra_ms[leg] / 1e3,
                             "sources": ["gdr_kda.hip", "gdr_device.h"]}
    traffic = _measured_traffic()

    def roofline(leg):
        li = leg_info[leg]
        t_hbm = li["bytes"] / HBM_PEAK
        t_mfma = li["flops"] / BF16_MFMA_PEAK if li["flops"] else 0.0
        tr = traffic.get(leg)
        tr_ok = tr is not None and tr.get("source_sha256") == _source_digest(li["sources"])
        if t_mfma > t_hbm:
            r = {"bound": "mfma", "achieved": li["flops"] / li["secs"] / 1e12, "peak": BF16_MFMA_PEAK / 1e12,
                 "unit": "TFLOP/s", "frac": li["flops"] / li["secs"] / BF16_MFMA_PEAK}
        else:
            r = {"bound": "hbm", "achieved": li["bytes"] / li["secs"] / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                 "frac": li["bytes"] / li["secs"] / HBM_PEAK}
        r["traffic"] = tr["bytes_per_launch"] if tr_ok else None
        r["kernel"] = li["kernel"]
        r["alg_bytes_per_launch"] = li["bytes"]
        r["avg_launch_ms"] = li["secs"] * 1e3
        if li["flops"]:
            r["alg_flops_per_launch"] = li["flops"]
            r["frac_bf16_mfma"] = li["flops"] / li["secs"] / BF16_MFMA_PEAK
            r["frac_hbm"] = li["bytes"] / li["secs"] / HBM_PEAK
        return r

    step_legs = ("prefill", "decode", "verify")
    dominant = max(step_legs, key=lambda n: leg_info[n]["secs"])
    roof = roofline(dominant)
    roof_legs = {n: roofline(n) for n in step_legs}
    extra_legs = {n: {"ms": extra_ms[n], "stats_ms": extra_stats[n], "roofline": roofline(n)} for n in extra_ms}
    if "kda" in extra_legs:
        extra_legs["kda"]["tokens_per_s"] = pk.T / (extra_ms["kda"] / 1e3)
    for leg in ("cp_segmented", "cp_direct"):
        if leg in extra_legs:
            extra_legs[leg]["tokens_per_s"] = pc.T / (extra_ms[leg] / 1e3)
    roof_legs["prefill"]["frac_bf16_mfma_full_tile"] = f_pre_full / s_pre / BF16_MFMA_PEAK
    roof_legs["prefill"]["alg_flops_full_tile"] = f_pre_full
    roof_legs["decode"]["state_GBps"] = state_bytes_dec / s_dec / 1e9
    # the token loop is fp32 vector arithmetic (7 V K flops per token and value head): its share of the
    # fp32 VALU peak shows how far the decode and verify launches are from an ALU bound
    for leg, pr, secs in (("decode", pd, s_dec), ("verify", pv, s_ver)):
        active = int(sum(n for n, slot in zip(pr.lengths, pr.state_indices) if slot >= 0))  # padded: no work
        fl = 7.0 * pr.V * pr.K * pr.HV * active
        roof_legs[leg]["alg_valu_flops_per_launch"] = fl
        roof_legs[leg]["frac_fp32_valu"] = fl / secs / FP32_VALU_PEAK
    out = {
        "metric": "GDN prefill tokens/s + decode state GB/s (fraction of HBM/MFMA peak), 1 GPU",
        "value": prefill_tps,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill: chunked GDN, 8 ragged sequences (incl. 64 and 65) summing to 32768 tokens, "
                               "32 heads, K=V=128, bf16, fp32 h0/final; decode: 256 seqs x 1 token, HK=16/HV=32, "
                               "fp32 pool [1024,32,128,128], 26 padded, commit; verify: 64 seqs x 12 tokens, "
                               "bf16 pool, bf16 per-token states [1025,12,32,128,128], no commit",
                   "global_batch": pp.N, "seq_len": pp.T, "parallelism": "none (1 GPU)"},
        "decode_state_GBps": state_bytes_dec / s_dec / 1e9,
        "ms_per_step_note": "host wall time per step: the three legs' launches plus, outside their event "
                            "windows, three 512 MiB cache-flush reads and Python launch overhead; the legs' own "
                            "HIP-event times are in leg_ms",
        "leg_ms": leg_ms,
        "leg_stats_ms": leg_stats,
        "roofline": roof,
        "roofline_legs": roof_legs,
        "extra_legs": extra_legs,
    }
    mp = _measured_mfma_peak(dev)
    if mp is not None:
        mp["prefill_frac"] = f_pre / s_pre / (mp["tflops"] * 1e12)
        mp["prefill_frac_full_tile"] = f_pre_full / s_pre / (mp["tflops"] * 1e12)
        roof_legs["prefill"]["frac_measured_mfma"] = mp["prefill_frac"]
    out["measured_bf16_mfma_peak"] = mp
    hb = _measured_hbm_rates(dev)
    for leg in ("decode", "verify", "prefill"):
        hb[f"{leg}_vs_runtime_copy"] = leg_info[leg]["bytes"] / leg_info[leg]["secs"] / 1e9 / hb["runtime_copy_GBps"]
    out["measured_hbm"] = hb
    out["provenance"] = _provenance()
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = _cpu_baseline(pp)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
