"""Benchmark of the hot path on one MI355X.

One step = one pass of every entry point over its full-size synthetic
workload, inputs already resident in HBM:
  * mqa_prefill          causal MQA, B=2, Hq=16, Hkv=1, T=4096, d=512
  * mqa_decode           MQA, batch 64, Hq=16, Hkv=1, d=512, cache 8192
  * mqa_prefill          causal GQA, B=1, Hq=64, Hkv=8, T=8192, d=128
  * mqa_decode           GQA, batch 128, Hq=64, Hkv=8, d=128, cache
                         lengths uniform in [1024, 16384]
  * mla_decode_absorbed  batch 32, H=128, latent 576 (V = first 512), ctx 32768
  * mqa_prefill_ex       expanded MLA prefill, causal, B=1, H=128 (MHA),
                         T=8192, q/k 192 wide, v 128 wide
  * mqa_prefill_ex       chunked causal MQA prefill, B=2, Hq=16, Hkv=1,
                         d=512, 1024 new tokens after 7168 (bottom-right)
  * mla_decode_sparse    batch 32, H=128, cache 32768, 2048 selected rows
  * mla_absorb_query + mla_cache_append + mla_output_project
                         the steps around the absorbed decode, batch 32,
                         H=128 (weights W_UK, W_UV read once per call)
  * mqa_prefill          the first workload with fp16 inputs and output
  * mqa_prefill          causal MQA in fp32 end to end, B=1, Hq=16, Hkv=1,
                         T=128, d=512 (a latency-sized call on the fp32
                         MFMA kernel; its roofline is the fp32 MFMA rate)
bf16 in (but the fp16 and fp32 ones), fp32 accumulation, 16-bit out.

W untimed warm-up steps run first, extended (at most 400 steps) until they
have kept the GPU busy for 1 s: a fresh device runs its first ~25 calls
20-25 % slower while its clocks settle.  Then exactly K steps are timed.
Every call is bracketed with HIP events on the stream it is launched on.
The headline `value` is the causal MQA prefill TFLOP/s (visible query/key
pairs only, 2 (d_qk + d_v) flops per pair); the other workloads sit beside it, each
with its roofline.  `roofline.traffic` is the HBM traffic per call measured
with rocprofv3 counters (profiles/traffic.json), reported only while the
kernel sources still hash to the value recorded with the counters.
`cpu_baseline` times the fp64 numpy oracle on a bounded sample on the host
cores.  `attainable_peaks` are measured on the device by the probes of
libmqa_peaks.so (bf16 MFMA loop at one and two waves per SIMD with the
clock it ran at, HBM streaming read and copy, LDS reads); every roofline
also carries `frac_attainable` against the matching measured ceiling.
`host` records the ROCm, hipcc, torch and numpy versions, the GPU, the CPU
model, its core count, this process's affinity and the BLAS threads.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--only name,name] [--no-peaks] [--copy-calibration MIB]
       python bench.py --counters-summary DIR [DIR ...]   (rocprofv3 --pmc output)
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

METRIC = "causal prefill TFLOP/s + decode KV-read GB/s, MQA Hq=16 d=512 bf16"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

# name -> role in the record; shapes come from synthetic.WORKLOADS
ORDER = (
    ("mqa_prefill_bf16_b2_t4096", "headline"),
    ("mqa_decode_bf16_b64_l8192", "decode_kv_read"),
    ("gqa_prefill_bf16_b1_t8192", "gqa_prefill"),
    ("gqa_decode_bf16_b128_l1024to16384", "gqa_decode"),
    ("mla_decode_bf16_b32_l32768", "mla_decode"),
    ("mla_prefill_bf16_b1_h128_t8192", "mla_prefill"),
    ("mqa_chunk_prefill_bf16_b2_q1024_kv8192", "chunk_prefill"),
    ("mla_sparse_decode_bf16_b32_l32768_k2048", "mla_sparse_decode"),
    ("mla_step_proj_bf16_b32_h128", "mla_step_proj"),
    ("mqa_prefill_f16_b2_t4096", "f16_prefill"),
    ("mqa_prefill_f32_b1_t128", "f32_prefill"),
)

PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 MFMA

# waves per SIMD of each prefill kernel (the matching measured MFMA ceiling)
PREFILL_WAVES_PER_SIMD = {512: 1, 128: 2, 192: 2}


def prefill_flops(B, Hq, T, D, causal=True, T_kv=None, DV=None, **_):
    """Visible (query, key) pairs x 2 (d_qk + d_v).  Causal with T queries
    after T_kv - T earlier tokens: query i sees T_kv - T + i + 1 keys."""
    T_kv = T if T_kv is None else T_kv
    DV = D if DV is None else DV
    pairs = T * (T_kv - T) + T * (T + 1) // 2 if causal else T * T_kv
    return B * Hq * pairs * 2 * (D + DV)


def prefill_bytes(B, Hq, Hkv, T, D, T_kv=None, DV=None, **_):
    T_kv = T if T_kv is None else T_kv
    DV = D if DV is None else DV
    return (B * Hq * T * (D + DV) + B * Hkv * T_kv * (D + DV)) * 2      # q, out, k, v (bf16)


def decode_bytes(B, Hq, Hkv, D, seq_lens, **_):
    kv = int(np.sum(seq_lens)) * Hkv * 2 * D * 2
    return kv + B * Hq * D * 2 * 2          # + q and out (bf16)


def decode_flops(Hq, D, seq_lens, **_):
    return int(np.sum(seq_lens)) * Hq * 2 * (D + D)


def mla_bytes(B, H, D, seq_lens, DV=512, **_):
    return int(np.sum(seq_lens)) * D * 2 + B * H * D * 2 + B * H * DV * 2


def mla_flops(H, D, seq_lens, DV=512, **_):
    return int(np.sum(seq_lens)) * H * 2 * (D + DV)


def source_hash():
    """sha256 over the kernel sources and the ABI header (what the counters
    were taken on)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_mqa_gqa_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".hpp")))
    files.append(os.path.join(ROOT, "include", "mqa_attn.h"))
    files.append(os.path.join(ROOT, "attention_mqa_gqa_amd", "build.py"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def load_traffic():
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return {}
    if t.get("source_sha256") != source_hash():
        return {}
    return t.get("per_call_bytes", {})


def roofline(bound, achieved, peak, unit, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info()]
        return max(n) if n else 1
    except Exception:
        return 1


def cpu_baseline(q, k, v, scale, shape, min_seconds=10.0):
    """fp64 oracle on a bounded sample: all heads of batch 0 of the MQA
    prefill workload (full causal rows), repeated until at least
    `min_seconds` of host time have been spent (and at least once)."""
    import oracle
    q0, k0, v0 = q.f32()[0:1], k.f32()[0:1], v.f32()[0:1]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.prefill_ref(q0, k0, v0, scale, True)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    fl = prefill_flops(1, shape["Hq"], shape["T"], shape["D"]) * reps
    threads = blas_threads()
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"causal MQA prefill, batch 0 of {shape['B']} ({shape['Hq']} heads x T={shape['T']} "
                      f"x d={shape['D']}), fp64 numpy, {reps} passes in {dt:.1f} s",
            "threads_note": f"numpy's BLAS ran on {threads} threads; the host has {os.cpu_count()} logical CPUs, "
                            f"{len(os.sched_getaffinity(0)) if hasattr(os, 'sched_getaffinity') else '?'} "
                            f"in this process's affinity"}


def host_record():
    """Versions and host facts for the record: ROCm, hipcc, torch (and its HIP),
    the host's CPU model, core count, affinity and BLAS threads."""
    import platform
    import subprocess
    rec = {"python": platform.python_version()}
    try:
        with open("/opt/rocm/.info/version") as fh:
            rec["rocm"] = fh.read().strip()
    except OSError:
        rec["rocm"] = None
    try:
        out = subprocess.run(["hipcc", "--version"], capture_output=True, text=True, timeout=30).stdout
        rec["hipcc"] = " | ".join(l.strip() for l in out.splitlines() if "version" in l.lower())[:200]
    except Exception:
        rec["hipcc"] = None
    try:
        import torch
        rec["torch"] = torch.__version__
        rec["torch_hip"] = getattr(torch.version, "hip", None)
        if torch.cuda.is_available():
            pr = torch.cuda.get_device_properties(0)
            rec["gpu"] = f"{pr.name} ({getattr(pr, 'gcnArchName', '')}, {pr.multi_processor_count} CUs)"
    except Exception:
        pass
    rec["numpy"] = np.__version__
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rec["cpu_model"] = model
    rec["cpu_count"] = os.cpu_count()
    rec["cpu_affinity"] = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    rec["blas_threads"] = blas_threads()
    return rec


def counters_summary(dirs, num_xcd=8, num_cu=256, simds_per_cu=4):
    """Summarise rocprofv3 --pmc runs (counter_collection CSVs under `dirs`)
    per kernel: the mean of every counter per dispatch and derived rates.

    Normalisation (one dispatch): GRBM_GUI_ACTIVE is summed over the XCDs,
    so cycles = GRBM_GUI_ACTIVE / XCDs and clock = cycles / duration;
    SQ_VALU_MFMA_BUSY_CYCLES is summed over all SIMDs (MFMA busy = it /
    (SIMDs x cycles)); SQ_*_CYCLES / SQ_ACTIVE_* / SQ_WAIT_* count in units
    of 4 cycles summed over waves (per-wave share = 4 x value / waves /
    wave lifetime); LDS counters are summed over CUs."""
    import csv
    import glob
    per = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    k = r["Kernel_Name"]
                    c = per.setdefault(k, {})
                    c.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                    if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                        c.setdefault("_dur_ns", []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = []
    for k in sorted(per):
        c = {n: float(np.mean(v)) for n, v in per[k].items()}
        if "GRBM_GUI_ACTIVE" not in c or c.get("SQ_WAVES", 1) < 64:
            continue
        short = k.split("(")[0][:110]
        cyc = c["GRBM_GUI_ACTIVE"] / num_xcd
        dur = c["_dur_ns"] * 1e-9
        simd_cycles = cyc * num_cu * simds_per_cu
        cu_cycles = cyc * num_cu
        lines.append(f"kernel {short}")
        # (the clock is meaningful only for long dispatches: GRBM_GUI_ACTIVE
        # also counts the dispatch's start-up and drain)
        clock = f" -> clock {cyc / dur / 1e9:.3f} GHz" if dur > 50e-6 else ""
        lines.append(f"  dispatches {len(per[k]['GRBM_GUI_ACTIVE'])}, mean duration {dur * 1e6:.1f} us, "
                     f"GPU cycles {cyc:.0f}{clock}")
        der = []
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            der.append(("MFMA busy (of SIMD cycles)", c["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles))
        waves = c.get("SQ_WAVES")
        if waves and "SQ_WAVE_CYCLES" in c:
            life = 4 * c["SQ_WAVE_CYCLES"] / waves
            der.append(("wave lifetime (cycles)", life))
            for n in ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_MISC",
                      "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS"):
                if n in c:
                    der.append((f"{n} (share of wave time)", 4 * c[n] / waves / life))
        if "SQ_LDS_IDX_ACTIVE" in c:
            der.append(("LDS active (of CU cycles)", c["SQ_LDS_IDX_ACTIVE"] / cu_cycles))
        if "SQ_LDS_BANK_CONFLICT" in c:
            der.append(("LDS bank-conflict cycles (of CU cycles)", c["SQ_LDS_BANK_CONFLICT"] / cu_cycles))
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in c:
            der.append(("VALU issued beside an MFMA (of SIMD cycles)", c["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd_cycles))
        if waves:
            for n in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM", "SQ_INSTS_SALU"):
                if n in c:
                    der.append((f"{n} per wave", c[n] / waves))
        for name, val in der:
            lines.append(f"  {name:48s} {val:12.3f}")
        raw = ", ".join(f"{n}={v:.4g}" for n, v in sorted(c.items()) if not n.startswith("_"))
        lines.append(f"  raw means per dispatch: {raw}")
    return "\n".join(lines)


# The kernels each entry-point call dispatches, in order (substrings of the
# demangled names in rocprofv3 output); used to assign profiled dispatches to
# workloads by their order within a step.
CALL_KERNELS = {
    "mqa_prefill_bf16_b2_t4096": ("kv_pack_kernel<512", "prefill_bf16_kernel<512"),
    "mqa_decode_bf16_b64_l8192": ("decode_split_kernel<512", "lse_merge_kernel<512"),
    "gqa_prefill_bf16_b1_t8192": ("kv_pack_kernel<128", "prefill_bf16_kernel<128"),
    "gqa_decode_bf16_b128_l1024to16384": ("decode_split_kernel<128", "lse_merge_kernel<128"),
    "mla_decode_bf16_b32_l32768": ("mla_decode_kernel<false", "mla_merge_kernel"),
    "mla_prefill_bf16_b1_h128_t8192": ("kv_pack_kernel<192", "prefill_bf16_kernel<192"),
    "mqa_chunk_prefill_bf16_b2_q1024_kv8192": ("kv_pack_kernel<512", "prefill_bf16_kernel<512"),
    "mla_sparse_decode_bf16_b32_l32768_k2048": ("mla_decode_kernel<true", "mla_merge_kernel"),
    "mla_step_proj_bf16_b32_h128": ("mla_absorb_kernel", "mla_cache_append_kernel", "mla_out_proj_kernel"),
    "mqa_prefill_f16_b2_t4096": ("kv_pack_kernel<512", "prefill_bf16_kernel<512"),
    "mqa_prefill_f32_b1_t128": ("prefill_f32_kernel<512",),
}


def _read_csvs(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def assign_dispatches(kernel_names, names=None):
    """Assign an ordered list of dispatched kernel names to (workload, kernel
    slot) by walking the per-step kernel sequence of the bench (dispatches
    that do not fit the sequence, e.g. set-up calls, are skipped).  Returns a
    list of (workload, slot) or None per dispatch."""
    names = [n for n, _ in ORDER if names is None or n in names]
    seq = [(n, i, pat) for n in names for i, pat in enumerate(CALL_KERNELS[n])]
    out, p = [], 0
    for k in kernel_names:
        if "mqa::" in k and seq[p][2] in k:
            out.append((seq[p][0], seq[p][1]))
            p = (p + 1) % len(seq)
        else:
            out.append(None)
    return out


def kernel_trace_summary(d):
    """Per-workload, per-kernel durations from a rocprofv3 --kernel-trace run
    of bench.py (all steps, warm-up included)."""
    rows = _read_csvs(d, "kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    names = [r["Kernel_Name"] for r in rows]
    asg = assign_dispatches(names)
    per = {}
    for r, a in zip(rows, asg):
        if a is None:
            continue
        per.setdefault(a, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    lines = [f"{'workload':40s} {'kernel':84s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s}"]
    for n, _ in ORDER:
        for i, pat in enumerate(CALL_KERNELS[n]):
            v = per.get((n, i))
            if not v:
                continue
            kname = next(k for k, a in zip(names, asg) if a == (n, i)).split("(")[0].replace("void ", "").replace("mqa::", "")
            lines.append(f"{n:40s} {kname[:84]:84s} {len(v):6d} {np.mean(v):9.1f} {np.min(v):9.1f} {np.max(v):9.1f}")
    stray = sum(1 for k, a in zip(names, asg) if a is None and "mqa::" in k)
    lines.append(f"library dispatches outside the step sequence (set-up calls): {stray}")
    return "\n".join(lines), per


def traffic_summary(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, cal_bytes):
    """HBM bytes per entry-point call from rocprofv3 FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch, one counter per run), each scaled by what the same
    counter reads for a plain device copy of `cal_bytes` (read factor =
    cal_bytes / (1024 x FETCH_SIZE of the copy), write factor likewise)."""
    def per_dispatch(d, counter):
        rows = [r for r in _read_csvs(d, "counter_collection.csv") if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows]

    def cal_factor(d, counter):
        vals = [v for k, v in per_dispatch(d, counter)]
        big = max(vals)
        return cal_bytes / (1024.0 * big)

    rf, wf = cal_factor(cal_fetch_dir, "FETCH_SIZE"), cal_factor(cal_write_dir, "WRITE_SIZE")
    calls = {}
    for d, counter, f in ((fetch_dir, "FETCH_SIZE", rf), (write_dir, "WRITE_SIZE", wf)):
        disp = per_dispatch(d, counter)
        asg = assign_dispatches([k for k, _ in disp])
        acc = {}
        for (k, v), a in zip(disp, asg):
            if a is not None:
                acc.setdefault(a, []).append(v * 1024.0 * f)
        for (n, i), v in acc.items():
            calls.setdefault(n, {}).setdefault(counter, {})[i] = float(np.mean(v))
    per_call = {n: int(round(sum(c.get("FETCH_SIZE", {}).values()) + sum(c.get("WRITE_SIZE", {}).values())))
                for n, c in calls.items()}
    lines = [f"{'workload':40s} {'kernel':26s} {'read MB':>9s} {'write MB':>9s}"]
    for n, _ in ORDER:
        for i, pat in enumerate(CALL_KERNELS[n]):
            c = calls.get(n, {})
            if i in c.get("FETCH_SIZE", {}):
                kname = pat.split("<")[0]
                lines.append(f"{n:40s} {kname:26s} {c['FETCH_SIZE'].get(i, 0) / 1e6:9.1f} "
                             f"{c.get('WRITE_SIZE', {}).get(i, 0) / 1e6:9.1f}")
    return {"source_sha256": source_hash(), "read_factor": round(rf, 4), "write_factor": round(wf, 4),
            "per_call_bytes": per_call, "table": "\n".join(lines),
            "per_call_detail": {n: {k: {str(i): round(x) for i, x in v.items()} for k, v in c.items()}
                                for n, c in calls.items()}}


def copy_calibration(mib, reps):
    """A plain device copy of known size (for scaling the HBM counters)."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_call": n, "bytes_written_per_call": n, "calls": reps}}))
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma-separated workload names (default: all)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the attainable-peak probes")
    ap.add_argument("--counters-summary", nargs="+", default=None, metavar="DIR",
                    help="only summarise rocprofv3 --pmc output directories (no GPU needed)")
    ap.add_argument("--trace-summary", default=None, metavar="DIR",
                    help="only summarise a rocprofv3 --kernel-trace run of this bench per workload")
    ap.add_argument("--traffic-summary", nargs=5, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR", "CAL_MIB"),
                    help="only compute per-call HBM bytes from FETCH_SIZE / WRITE_SIZE runs and a copy "
                         "calibration, and write profiles/traffic.json")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: every kernel here runs on a single MI355X "
              "(sharding across GPUs is a design note, not built). Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.counters_summary:
        print(counters_summary(args.counters_summary))
        return 0
    if args.trace_summary:
        print(kernel_trace_summary(args.trace_summary)[0])
        return 0
    if args.traffic_summary:
        fd, wd, cfd, cwd, mib = args.traffic_summary
        t = traffic_summary(fd, wd, cfd, cwd, int(mib) << 20)
        t["note"] = ("HBM bytes per entry-point call (all its kernels) from rocprofv3 FETCH_SIZE / WRITE_SIZE, "
                     "scaled by the factors a plain device copy gives; bench.py reports them only while the "
                     "kernel sources hash to source_sha256")
        table = t.pop("table")
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(t, fh, indent=1)
        print(f"read factor {t['read_factor']}, write factor {t['write_factor']}, "
              f"sources sha256 {t['source_sha256']}")
        print(table)
        return 0
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration, max(args.steps, 1))

    import torch
    import attention_mqa_gqa_amd as mqa
    from synthetic import WORKLOADS, decode_inputs, draw_topk, mla_inputs, mla_step_inputs, prefill_inputs, rope_tables

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    only = [s for s in args.only.split(",") if s]
    names = [n for n, _ in ORDER if not only or n in only]

    def to_dev(t):
        if t.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(t.data)).to(dev)

    calls, work, host, graphs = {}, {}, {}, []
    t_gen = time.perf_counter()
    for name in names:
        wl = WORKLOADS[name]
        s = dict(wl.shape)
        if wl.kind == "prefill":
            T_kv, DV = s.get("T_kv", s["T"]), s.get("DV", s["D"])
            q, k, v = prefill_inputs(s["B"], s["Hq"], s["Hkv"], s["T"], s["D"], wl.dtype, seed=0, d_v=DV, T_kv=T_kv)
            dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
            out = torch.empty((s["B"], s["Hq"], s["T"], DV), dtype=dq.dtype, device=dev)
            in_code = mqa.DTYPE_F32 if wl.dtype == "f32" else mqa.DTYPE_BF16
            ws = torch.empty(max(1, mqa.mqa_prefill_ex_workspace_size(s["B"], s["Hq"], s["Hkv"], s["T"], T_kv, s["D"],
                                                                      DV, in_code)),
                             dtype=torch.uint8, device=dev)
            sc = s["D"] ** -0.5
            if T_kv == s["T"] and DV == s["D"]:
                calls[name] = (lambda dq=dq, dk=dk, dv=dv, out=out, ws=ws, sc=sc:
                               mqa.mqa_prefill(dq, dk, dv, causal=True, scale=sc, out=out, workspace=ws))
            else:
                calls[name] = (lambda dq=dq, dk=dk, dv=dv, out=out, ws=ws, sc=sc:
                               mqa.mqa_prefill_ex(dq, dk, dv, causal=True, scale=sc, out=out, workspace=ws))
            if wl.dtype == "f32":
                work[name] = dict(flops=prefill_flops(**s), bytes=prefill_bytes(**s) * 2, bound="mfma_f32", shape=s)
            else:
                work[name] = dict(flops=prefill_flops(**s), bytes=prefill_bytes(**s), bound="mfma", shape=s,
                                  waves_per_simd=PREFILL_WAVES_PER_SIMD.get(s["D"], 1))
            if name == ORDER[0][0]:
                host[name] = (q, k, v, sc, s)
        elif wl.kind == "decode":
            q, k, v, sl = decode_inputs(s["B"], s["Hq"], s["Hkv"], s["L"], s["D"], "bf16", seed=0,
                                        lengths=s.get("lengths"))
            dq, dk, dv, dsl = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(sl).to(dev)
            del k, v
            out = torch.empty((s["B"], s["Hq"], s["D"]), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(mqa.mqa_decode_workspace_size(s["B"], s["Hq"], s["Hkv"], s["L"], s["D"]),
                             dtype=torch.uint8, device=dev)
            sc = s["D"] ** -0.5
            calls[name] = (lambda dq=dq, dk=dk, dv=dv, dsl=dsl, out=out, ws=ws, sc=sc:
                           mqa.mqa_decode(dq, dk, dv, dsl, scale=sc, out=out, workspace=ws))
            work[name] = dict(flops=decode_flops(s["Hq"], s["D"], sl),
                              bytes=decode_bytes(s["B"], s["Hq"], s["Hkv"], s["D"], sl), bound="hbm", shape=s,
                              mean_len=float(np.mean(sl)))
        elif wl.kind == "mla_step":
            B, H, L = s["B"], s["H"], s["L"]
            qn, qr, ck, kp, wuk, wuv = (to_dev(t) for t in mla_step_inputs(B, H, seed=0))
            pos = np.arange(B, dtype=np.int32) * 997 % L
            cs, sn = (torch.from_numpy(t).to(dev) for t in rope_tables(pos))
            dpos = torch.from_numpy(pos).to(dev)
            cache = torch.zeros((B, L, 576), dtype=torch.bfloat16, device=dev)
            q_abs = torch.empty((B, H, 576), dtype=torch.bfloat16, device=dev)
            o_lat = to_dev(mla_inputs(B, H, 1, 512, "bf16", seed=1)[0])
            out = torch.empty((B, H, 128), dtype=torch.bfloat16, device=dev)

            def step_call(qn=qn, qr=qr, ck=ck, kp=kp, wuk=wuk, wuv=wuv, cs=cs, sn=sn, dpos=dpos, cache=cache,
                          q_abs=q_abs, o_lat=o_lat, out=out):
                mqa.mla_absorb_query(qn, qr, wuk, cs, sn, out=q_abs)
                mqa.mla_cache_append(cache, ck, kp, cs, sn, dpos)
                mqa.mla_output_project(o_lat, wuv, out=out)
            # three short kernels: captured once in a HIP graph and replayed,
            # as a serving loop runs its decode steps, so the figure does not
            # depend on the host's launch rate (about 7 us of Python and
            # launch per eager call); the dependent dispatches still sit
            # 4-7 us apart on the device
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(side):
                step_call()
            torch.cuda.current_stream(dev).wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step_call()
            calls[name] = graph.replay
            graphs.append(graph)
            gemm = B * H * 512 * 128
            work[name] = dict(flops=2 * 2 * gemm,
                              bytes=2 * (2 * H * 512 * 128 + B * H * (128 + 64 + 576 + 512 + 128) + B * (512 + 64 + 576))
                              + 4 * B * (64 + 64 + 1),
                              bound="hbm", shape=s)
        elif wl.kind == "mla_sparse":
            q, kv, sl = mla_inputs(s["B"], s["H"], s["L"], s["D"], "bf16", seed=0)
            idx = draw_topk(s["B"], sl, s["topk"], seed=0)
            dq, dkv, didx = to_dev(q), to_dev(kv), torch.from_numpy(idx).to(dev)
            del kv
            out = torch.empty((s["B"], s["H"], 512), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(mqa.mla_decode_sparse_workspace_size(s["B"], s["H"], s["topk"]), dtype=torch.uint8,
                             device=dev)
            sc = 192 ** -0.5
            calls[name] = (lambda dq=dq, dkv=dkv, didx=didx, out=out, ws=ws, sc=sc:
                           mqa.mla_decode_sparse(dq, dkv, didx, scale=sc, out=out, workspace=ws))
            n_sel = (idx >= 0).sum(axis=1)              # rows read per sequence
            work[name] = dict(flops=mla_flops(s["H"], s["D"], n_sel),
                              bytes=mla_bytes(s["B"], s["H"], s["D"], n_sel) + idx.size * 4,
                              bound="hbm", shape=s)
        else:
            q, kv, sl = mla_inputs(s["B"], s["H"], s["L"], s["D"], "bf16", seed=0)
            dq, dkv, dsl = to_dev(q), to_dev(kv), torch.from_numpy(sl).to(dev)
            del kv
            out = torch.empty((s["B"], s["H"], 512), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(mqa.mla_decode_workspace_size(s["B"], s["H"], s["L"]), dtype=torch.uint8, device=dev)
            sc = 192 ** -0.5
            calls[name] = (lambda dq=dq, dkv=dkv, dsl=dsl, out=out, ws=ws, sc=sc:
                           mqa.mla_decode_absorbed(dq, dkv, dsl, scale=sc, out=out, workspace=ws))
            work[name] = dict(flops=mla_flops(s["H"], s["D"], sl), bytes=mla_bytes(s["B"], s["H"], s["D"], sl),
                              bound="hbm", shape=s)
        print(f"[bench] {name} ready ({time.perf_counter() - t_gen:.1f} s)", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        for name in names:
            if events is not None:
                events[name][0].record(stream)
            calls[name]()
            if events is not None:
                events[name][1].record(stream)

    t_w = time.perf_counter()
    n_w = 0
    while n_w < args.warmup or (time.perf_counter() - t_w < 1.0 and n_w < 400):
        step()
        n_w += 1
        if n_w >= args.warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    peaks = {}
    if not args.no_peaks:
        from attention_mqa_gqa_amd import peaks as peak_probes
        print("[bench] measuring attainable peaks ...", file=sys.stderr, flush=True)
        peaks = peak_probes.measure()

    def _attainable(roof, peak):
        # the same achieved figure against the ceiling measured on this device
        roof["attainable_peak"] = peak
        roof["frac_attainable"] = round(roof["achieved"] / peak, 4) if peak else None

    traffic = load_traffic()
    sub = {}
    for name in names:
        w = work[name]
        ms = np.array([e[name][0].elapsed_time(e[name][1]) for e in evs])
        mean = float(ms.mean())
        tflops = w["flops"] / (mean * 1e-3) / 1e12
        gbs = w["bytes"] / (mean * 1e-3) / 1e9
        tr = traffic.get(name)
        r = {"workload": name, "dtype": WORKLOADS[name].dtype, "shape": {k: v for k, v in w["shape"].items()},
             "ms": {"mean": round(mean, 4), "median": round(float(np.median(ms)), 4), "min": round(float(ms.min()), 4)},
             "algorithmic_flops": w["flops"], "algorithmic_bytes": w["bytes"],
             "tflops": round(tflops, 2), "gbs": round(gbs, 1)}
        if w["bound"] == "mfma":
            r["roofline"] = roofline("mfma", tflops, PEAK_BF16_TFLOPS, "TFLOP/s", tr)
            _attainable(r["roofline"], peaks.get(f"mfma_bf16_tflops_{w.get('waves_per_simd', 1)}wave"))
        elif w["bound"] == "mfma_f32":
            # the fp32 MFMA; no probe measures its attainable rate
            r["roofline"] = roofline("mfma", tflops, PEAK_FP32_MFMA_TFLOPS, "TFLOP/s", tr)
        else:
            r["roofline"] = roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", tr)
            _attainable(r["roofline"], peaks.get("hbm_read_gbs"))
            if name.startswith("mla"):
                r["roofline_mfma"] = roofline("mfma", tflops, PEAK_BF16_TFLOPS, "TFLOP/s", tr)
                _attainable(r["roofline_mfma"], peaks.get("mfma_bf16_tflops_1wave"))
        if "mean_len" in w:
            r["mean_seq_len"] = w["mean_len"]
        if r["shape"].get("lengths") is not None:
            r["shape"]["lengths"] = list(r["shape"]["lengths"])
        sub[name] = r

    head = ORDER[0][0]
    rec = {
        "metric": METRIC,
        "value": sub[head]["tflops"] if head in sub else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": n_w,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1), bf16-rounded)",
        "config": {
            "workload": "mqa_prefill causal B=2 Hq=16 Hkv=1 T=4096 d=512 bf16",
            "global_batch": 2,
            "seq_len": 4096,
            "heads": "Hq=16 Hkv=1",
            "head_dim": 512,
            "step": " + ".join(names),
        },
        "roofline": sub[head]["roofline"] if head in sub else None,
    }
    for name, role in ORDER:
        if name in sub and role != "headline":
            rec[role] = sub[name]
    if head in sub:
        rec["prefill"] = sub[head]
    rec["attainable_peaks"] = peaks or None
    rec["host"] = host_record()
    rec["cpu_baseline"] = None
    if not args.no_cpu_baseline and head in host:
        print("[bench] timing the fp64 oracle on a sample ...", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(*host[head])
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
