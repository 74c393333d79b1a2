"""Benchmark of the PaTH attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu] [--cpu-heads N] [--traffic FILE]
                    [--no-decode] [--decode-steps N] [--no-backward] [--backward-steps N]
                    [--no-partial] [--no-varlen] [--no-producer]

One step = one call of path_attn_fwd (gate prefix when present, chunk
preparation and the streaming scan) over the whole workload, inputs already
resident in HBM and the workspace preallocated.  W untimed warm-up steps, then
K steps timed with HIP events on the launch stream, bracketed by device
synchronisation (mean, plus median and min of the per-step times from events
recorded between steps).  Prints one JSON line.

The default workload is bf16 B=2, H=16, T=16384, d=64 (synthetic inputs,
seeded).  value = tokens/s = B*T / (time per step).  The roofline object is
for the dominant kernel, the streaming scan: its algorithmic flops
B*H*T^2*(2d + d^2/64) divided by its own average duration, timed with HIP
events over K launches of path_attn_stream alone on the same stream, against
the bf16 dense matrix-core peak of 2.5 PFLOP/s (with the forget gate, the scan
with every key block computed, PATH_ATTN_NO_SKIP, so that the rate counts
executed work; the exact skip's effective rate is reported in fox_skip).
cpu_baseline times the fp64
CPU oracle on a bounded sample (N whole heads) with all host threads and
scales the rate to the full workload.  The decode object times decoding
with in-place key refinement after the workload's prompt (prefill alignment of
a float32 key cache, then decode steps), bound by HBM.  The producer object
times the w / beta producer (path_attn_wbeta: low-rank projection, width-3
convolution, per-head L2 norm; beta = 2 sigmoid) from hidden states of size
H d, bound by HBM.  The backward object
times path_attn_bwd (all gradients, from the forward's out and lse and seeded
cotangents dout, dlse) on the same workload: algorithmic flops
B*H*T^2*(5d + 3d^2/64) (the causal products S, dP, dV, dQ, dK of 2d each per
query-key pair, plus three d x d chunk-transition products per pair of 64-token
chunks: key levels, the key-gradient transition and dM), without the
recomputation the kernels do.
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

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 matrix-core peak
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The GPU clock settles over the first tens of steps (kernel durations drift
    # by up to 20 % meanwhile); 50 untimed steps reach the steady state.
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="bf16_b2h16t16384d64")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decoding measurement")
    ap.add_argument("--decode-steps", type=int, default=20,
                    help="timed decode steps after the prompt (decoding measurement)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--backward-steps", type=int, default=5)
    ap.add_argument("--no-partial", action="store_true",
                    help="skip the partial-PaTH (d_path = d / 2) measurement")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the strided / packed forward measurement")
    ap.add_argument("--no-producer", action="store_true",
                    help="skip the w / beta producer measurement")
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="whole (b, h) heads the CPU oracle runs for its baseline")
    ap.add_argument("--counters", default=os.path.join(ROOT, "profiles", "counters.json"),
                    help="JSON of per-launch hardware-counter figures (HBM bytes, matrix-core "
                         "use) of the stream kernel, written by --pmc-report")
    ap.add_argument("--pmc-report", nargs="+", metavar="DIR", default=None,
                    help="do not run: summarise the rocprofv3 --pmc output directories given "
                         "(run_counter_collection.csv below each) per kernel, write the "
                         "markdown summary (--pmc-md) and this workload's record in --counters")
    ap.add_argument("--trace-report", metavar="DIR", default=None,
                    help="do not run: summarise a rocprofv3 --kernel-trace --stats output "
                         "directory (run_kernel_stats.csv) into --pmc-md (default "
                         "profiles/kernel_trace_<workload>.md), with the stream kernel's "
                         "F_path rate at its average duration")
    ap.add_argument("--pmc-md", default=None,
                    help="markdown file of --pmc-report (default profiles/counters_<workload>.md)")
    ap.add_argument("--pmc-command", action="append", default=[],
                    help="command line that produced a --pmc-report input (repeatable; "
                         "quoted in the summary)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (reference "
                         "kernel for scaling HBM traffic counters) and report its GB/s")
    return ap.parse_args()


def stream_kernel_name(wl) -> str:
    """The streaming-scan kernel that path_attn_stream launches for this shape."""
    wide = wl.dtype == "bf16" and wl.d == 64
    return ("stream_wide_kernel" if wide else "stream_kernel") + \
        f"<{wl.dtype}, d={wl.d}, {'gate' if wl.fox else 'no gate'}>"


def cpu_threads() -> int:
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(wl, inp, n_heads: int, out=None, lse=None):
    """fp64 oracle on n_heads whole (b, h) heads spread over the flat head
    index, all rows; the rate is scaled to the whole workload (every head
    costs the same).  With the GPU's out and lse of the same inputs, also the
    max-abs errors of every row of those heads against the oracle."""
    import numpy as np
    import oracle
    BH = wl.B * wl.H
    n_heads = max(1, min(n_heads, BH))
    heads = np.unique(np.linspace(0, BH - 1, n_heads).round().astype(np.int64))
    n_heads = len(heads)
    flat = lambda x: x.reshape(BH, wl.T, -1)[heads].astype(np.float64)
    q, k, v, w = (flat(inp[n]) for n in ("q", "k", "v", "w"))
    beta = inp["beta"].reshape(BH, wl.T)[heads].astype(np.float64)
    logf = None if inp["logf"] is None else inp["logf"].reshape(BH, wl.T)[heads].astype(np.float64)
    rows = np.stack(np.meshgrid(np.arange(n_heads), np.arange(wl.T), indexing="ij"), -1).reshape(-1, 2)
    threads = cpu_threads()
    t0 = time.perf_counter()
    o_ref, l_ref = oracle.path_attn_rows(q, k, v, w, beta, logf, 1.0 / np.sqrt(wl.d), rows,
                                         n_threads=threads)
    dt = time.perf_counter() - t0
    full_s = dt * BH / n_heads
    res = {"value": wl.B * wl.T / full_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{n_heads} of {BH} (b,h) heads (flat indices {heads.tolist()}), all {wl.T} "
                     f"query rows each ({n_heads * wl.T * (wl.T + 1) // 2:.3g} causal pairs) in "
                     f"{dt:.2f} s; rate scaled by {BH / n_heads:g} to the whole workload",
           "seconds_sample": dt}
    parity = None
    if out is not None:
        got_o = out.reshape(BH, wl.T, wl.d)[heads.tolist()].float().cpu().numpy().astype(np.float64)
        got_l = lse.reshape(BH, wl.T)[heads.tolist()].cpu().numpy().astype(np.float64)
        tol_o, tol_l = (2e-2, 1e-2) if wl.dtype == "bf16" else (1e-4, 1e-4)
        eo = float(np.max(np.abs(got_o.reshape(-1, wl.d) - o_ref)))
        el = float(np.max(np.abs(got_l.reshape(-1) - l_ref)))
        parity = {"max_abs_err_o": eo, "max_abs_err_lse": el, "tol_o": tol_o, "tol_lse": tol_l,
                  "within_tol": eo <= tol_o and el <= tol_l, "rows": int(n_heads * wl.T),
                  "heads_flat": heads.tolist(),
                  "what": "GPU out/lse of the timed steps against the fp64 oracle, every row of "
                          "the oracle's heads"}
    return res, parity


def bench_decode(wl, q, k, v, w, beta, logf, args, timed):
    """Decoding with in-place key refinement after the workload's prompt:
    align the prompt's key cache (float32 cache), then time decode steps at
    positions T, T+1, ...  Each step reads and writes every cached key and
    reads every cached value, so it is bound by HBM: algorithmic bytes per
    step = B*H*t*(2*4*d + e*d) (+ 8 per key for the float64 gate prefix),
    e = value bytes."""
    import torch
    import householder_position_encoding_amd as pa
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    n_steps = max(2, args.decode_steps)
    T_cap = T + 2 * n_steps + 8
    cache = pa.DecodeCache(B, H, T_cap, d, q.dtype, kc_dtype=torch.float32, fox=logf is not None)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pre_ws = torch.empty(max(256, pa.load_library().path_attn_prefill_workspace_bytes(B, H, T, d)),
                         dtype=torch.uint8, device=q.device)
    pa.path_attn_prefill_cache(cache, k, v, w, beta, logf, workspace=pre_ws)   # warm-up
    torch.cuda.synchronize()
    a.record(stream)
    pa.path_attn_prefill_cache(cache, k, v, w, beta, logf, workspace=pre_ws)
    b.record(stream)
    torch.cuda.synchronize()
    ms_prefill = a.elapsed_time(b)
    del pre_ws
    # decode tokens: the last prompt token's vectors again (any values will do)
    at = lambda x: None if x is None else x[:, :, T - 1].contiguous()
    qt, kt, vt, wt, bt, ft = at(q), at(k), at(v), at(w), at(beta), at(logf)
    out = torch.empty_like(qt)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    for _ in range(2):   # warm-up steps
        pa.path_attn_decode_step(cache, qt, kt, vt, wt, bt, ft, out=out, lse=lse)
    torch.cuda.synchronize()
    t0 = cache.length
    a.record(stream)
    for _ in range(n_steps):
        pa.path_attn_decode_step(cache, qt, kt, vt, wt, bt, ft, out=out, lse=lse)
    b.record(stream)
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / n_steps
    t_mean = t0 + (n_steps - 1) / 2.0
    e = 2 if wl.dtype == "bf16" else 4
    per_key = 2 * 4 * d + e * d + (8 if logf is not None else 0)
    nbytes = B * H * t_mean * per_key
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    return {"context": int(t_mean), "key_cache": "f32", "ms_per_step": ms_step,
            "tokens_per_s": B / (ms_step * 1e-3), "ms_prefill_align": ms_prefill,
            "roofline": {"kernel": "decode step (split-key refinement kernel, then the merge kernel)", "bound": "hbm",
                         "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "bytes_per_step": nbytes}}


def bench_backward(wl, q, k, v, w, beta, logf, out, lse, args):
    """path_attn_bwd over the whole workload (inputs, forward outputs and
    cotangents resident in HBM, workspace preallocated): with the smallest
    workspace (the default: the sweep in windows of 16 query chunks past 33
    chunks) and, in "one_window", with the workspace of a single window
    (every key level stored; faster, T^2 memory)."""
    import torch
    import householder_position_encoding_amd as pa
    import workloads
    cot = workloads.cotangents(wl.dtype, wl.B, wl.H, wl.T, wl.d, seed=1000 + wl.seed)
    dout = torch.from_numpy(cot["dout"]).to(q.device, q.dtype)
    dlse = torch.from_numpy(cot["dlse"]).to(q.device)
    dt_code = pa.BF16 if wl.dtype == "bf16" else pa.F32
    flops = float(wl.B * wl.H) * wl.T * wl.T * (5 * wl.d + 3 * wl.d * wl.d / 64.0)
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    stream = torch.cuda.current_stream()
    n = max(1, args.backward_steps)

    def run(nbytes):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        fn = lambda: pa.path_attn_bwd(q, k, v, w, beta, logf, out, lse, dout, dlse, workspace=ws)
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        del ws
        torch.cuda.empty_cache()
        return a.elapsed_time(b) / n

    small = pa.path_attn_bwd_workspace_bytes(wl.B, wl.H, wl.T, wl.d, dt_code)
    ms = run(small)
    tf = flops / (ms * 1e-3) / 1e12
    res = {"ms": ms, "steps": n, "tokens_per_s": wl.n_tokens / (ms * 1e-3),
           "workspace_gib": small / 2**30,
           "roofline": {"kernel": "path_attn_bwd (whole call)", "bound": "mfma", "achieved": tf,
                        "peak": peak, "unit": "TFLOP/s", "frac": tf / peak,
                        "flops_per_call": flops}}
    big = pa.path_attn_bwd_workspace_bytes_window(wl.B, wl.H, wl.T, wl.d, dt_code, 0)
    if big > small:
        free, _ = torch.cuda.mem_get_info()
        if big < 0.8 * free:
            ms1 = run(big)
            res["one_window"] = {"ms": ms1, "workspace_gib": big / 2**30,
                                 "frac": flops / (ms1 * 1e-3) / 1e12 / peak}
    return res


def bench_partial(wl, q, k, v, w, beta, logf, args, timed, ms_full):
    """Partial PaTH (path_attn_fwd_partial) with the factors on the leading
    d / 2 coordinates, on the same inputs and workspace size: the time of the
    whole call against the full forward's step.  Its algorithmic flops are
    B*H*T^2*(2d + (d/2)^2/64): the transition product shrinks to (d/2)^2."""
    import torch
    import householder_position_encoding_amd as pa
    dp = wl.d // 2
    out = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.T), dtype=torch.float32, device=q.device)
    dt_code = pa.BF16 if wl.dtype == "bf16" else pa.F32
    ws = torch.empty(pa.path_attn_workspace_bytes(wl.B, wl.H, wl.T, wl.d, dt_code),
                     dtype=torch.uint8, device=q.device)
    ms = timed(lambda: pa.path_attn_fwd_partial(q, k, v, w, beta, logf, d_path=dp, out=out,
                                                lse=lse, workspace=ws), args.steps)
    flops = float(wl.B * wl.H) * wl.T * wl.T * (2 * wl.d + dp * dp / 64.0)
    return {"d_path": dp, "ms": ms, "ms_full_path": ms_full, "speedup": ms_full / ms,
            "tokens_per_s": wl.n_tokens / (ms * 1e-3),
            "tflops_path_partial": flops / (ms * 1e-3) / 1e12}


def bench_producer(wl, args, timed):
    """The w / beta producer (path_attn_wbeta) for the workload's B, T, H, d
    from hidden states of size Dm = H d through a rank R = 64 projection
    (seeded synthetic bf16 weights): HBM-bound; algorithmic bytes per call
    B T (2 Dm + 2 H d + 4 H) (read x, write w and beta) plus the weights
    2 (R Dm + H d R + H Dm) + 12 H d + 4 H."""
    import torch
    import householder_position_encoding_amd as pa
    B, T, H, d = wl.B, wl.T, wl.H, wl.d
    Dm, R = H * d, 64
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(11)
    rn = lambda *shape: torch.randn(*shape, generator=g, device=dev)
    x = rn(B, T, Dm).to(torch.bfloat16)
    wd = (rn(R, Dm) / Dm ** 0.5).to(torch.bfloat16)
    wu = (rn(H * d, R) / R ** 0.5).to(torch.bfloat16)
    u = (rn(H, Dm) / Dm ** 0.5).to(torch.bfloat16)
    cw = rn(H * d, 3) / 3 ** 0.5
    ub = rn(H)
    wo = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev)
    bo = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    ms = timed(lambda: pa.path_attn_wbeta(x, wd, wu, cw, u, ub, H, d, w=wo, beta=bo), args.steps)
    nbytes = B * T * (2 * Dm + 2 * H * d + 4 * H) + 2 * (R * Dm + H * d * R + H * Dm) + 12 * H * d + 4 * H
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"Dm": Dm, "R": R, "ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "roofline": {"kernel": "wbeta_kernel", "bound": "hbm", "achieved": gbs, "peak": 8000.0,
                         "unit": "GB/s", "frac": gbs / 8000.0, "bytes_per_call": nbytes}}


def bench_varlen(wl, q, k, v, w, beta, logf, args, timed, ms_dense):
    """The forward (and backward) on views of the same workload: q, k, v, w as
    slices of one fused token-major [B, T, 4, H, d] projection buffer, beta
    and log f of a [B, T, H, 2] buffer, out and lse into [B, T, H, ...]
    buffers (strided); and the same tokens packed as [B*T, H, d] sequences
    with cu_seqlens (packed).  Views are gathered into zero-padded staging and
    the outputs scattered back, so the difference to the dense call is the
    staging traffic: per (token, head) every input and output row is read
    and written once more."""
    import torch
    import householder_position_encoding_amd as pa
    B, H, T, d = wl.B, wl.H, wl.T, wl.d
    dev, tdt = q.device, q.dtype
    fused = torch.empty(B, T, 4, H, d, dtype=tdt, device=dev)
    for i, x in enumerate((q, k, v, w)):
        fused[:, :, i] = x.permute(0, 2, 1, 3)
    sc = torch.zeros(B, T, H, 2, dtype=torch.float32, device=dev)
    sc[..., 0] = beta.permute(0, 2, 1)
    if logf is not None:
        sc[..., 1] = logf.permute(0, 2, 1)
    views = [fused[:, :, i].permute(0, 2, 1, 3) for i in range(4)]
    vb = sc[..., 0].permute(0, 2, 1)
    vl = None if logf is None else sc[..., 1].permute(0, 2, 1)
    out_b = torch.empty(B, T, H, d, dtype=tdt, device=dev)
    lse_b = torch.empty(B, T, H, dtype=torch.float32, device=dev)
    dt_code = pa.BF16 if wl.dtype == "bf16" else pa.F32
    ws = torch.empty(pa.path_attn_varlen_workspace_bytes(B, H, T, d, dt_code),
                     dtype=torch.uint8, device=dev)
    n = max(1, args.steps // 2)
    ms_strided = timed(lambda: pa.path_attn_fwd_varlen(
        *views, vb, vl, out=out_b.permute(0, 2, 1, 3), lse=lse_b.permute(0, 2, 1),
        workspace=ws), n)
    # packed: the same tokens as B sequences of T tokens, token-major
    flat = fused.view(B * T, 4, H, d)
    pv = [flat[:, i] for i in range(4)]
    scf = sc.view(B * T, H, 2)
    pb, pl = scf[..., 0], (None if logf is None else scf[..., 1])
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device=dev)
    out_p = torch.empty(B * T, H, d, dtype=tdt, device=dev)
    lse_p = torch.empty(B * T, H, dtype=torch.float32, device=dev)
    ms_packed = timed(lambda: pa.path_attn_fwd_varlen(
        *pv, pb, pl, cu_seqlens=cu, max_seqlen=T, out=out_p, lse=lse_p, workspace=ws), n)
    e = 2 if wl.dtype == "bf16" else 4
    # The strided views are read and written in place (bf16, whole chunks,
    # 16-byte rows); the packed batch is staged.  Staging bytes: 4 input
    # vectors + beta (+ log f) gathered (read + write), out and lse scattered
    # (read + write).
    per_row = 2 * (5 * d * e + 4 + (4 if logf is not None else 0) + 4)
    nbytes = B * H * T * per_row
    over = ms_packed - ms_dense
    gbs = nbytes / (over * 1e-3) / 1e9 if over > 0 else None
    return {"ms_dense": ms_dense, "ms_strided_fwd": ms_strided, "ms_packed_fwd": ms_packed,
            "tokens_per_s_strided_fwd": wl.n_tokens / (ms_strided * 1e-3),
            "strided_in_place": wl.dtype == "bf16" and T % 64 == 0,
            "strided_overhead_ms": ms_strided - ms_dense,
            "staging_bytes": nbytes, "staging_ms": over,
            "staging_gbs": gbs, "staging_frac_hbm": None if gbs is None else gbs / PEAK_HBM_GBS}


# ---------------------------------------------------------------- counters

def _short_kernel_name(mangled: str) -> str:
    """Readable name of a library kernel from its mangled name: the function
    name and its template arguments (integers, bools, float / bf16 types)."""
    import re
    m = re.search(r"_GLOBAL__N_1(\d+)", mangled) or re.search(r"N8pathattn(\d+)", mangled)
    if not m:
        return mangled
    n = int(m.group(1))
    name = mangled[m.end():m.end() + n]
    rest = mangled[m.end() + n:]
    args = []
    if rest.startswith("I"):
        rest = rest[1:]
        while rest and not rest.startswith("E"):
            t = re.match(r"L(i|j|b)(\d+)E|DF16b|f|d", rest)
            if not t:
                break
            tok = t.group(0)
            if tok.startswith("Lb"):
                args.append("true" if t.group(2) == "1" else "false")
            elif tok.startswith("L"):
                args.append(t.group(2))
            else:
                args.append({"DF16b": "bf16", "f": "float", "d": "double"}[tok])
            rest = rest[len(tok):]
    return name + (f"<{', '.join(args)}>" if args else "")


def read_counter_dirs(dirs):
    """Per kernel (mangled name) and counter: the list of per-dispatch values,
    the per-dispatch durations (ns) seen with each counter, and the agent's
    SIMD count, XCD count and peak engine clock (MHz) from run_agent_info.csv."""
    import csv
    import glob
    vals, durs = {}, {}
    agent = {"simd": 1024, "xcc": 8, "mhz": 2400}
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    key = (r["Kernel_Name"], r["Counter_Name"])
                    vals.setdefault(key, []).append(float(r["Counter_Value"]))
                    durs.setdefault(r["Kernel_Name"], []).append(
                        int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            info = os.path.join(os.path.dirname(f), os.path.basename(f).replace(
                "counter_collection", "agent_info"))
            if os.path.exists(info):
                with open(info) as fh:
                    for r in csv.DictReader(fh):
                        if r.get("Agent_Type") == "GPU":
                            agent = {"simd": int(r["Simd_Count"]), "xcc": int(r["Num_Xcc"]),
                                     "mhz": int(r["Max_Engine_Clk_Fcompute"])}
    return vals, durs, agent


def summarise_counters(vals, durs, agent, copy_bytes=0):
    """Figures per kernel from the raw counters, means over its dispatches.

    Matrix cores: executed flop = 512 * SQ_INSTS_VALU_MFMA_MOPS_{BF16,F32}
    (the counters count flop / 512); busy = SQ_VALU_MFMA_BUSY_CYCLES (summed
    over SIMDs) over the SIMD-cycles of the dispatch, GRBM_GUI_ACTIVE / XCDs
    * SIMDs (GRBM_GUI_ACTIVE is summed over the XCDs), as rocprofv3's
    MfmaUtil; co-execution likewise from SQ_VALU_MFMA_COEXEC_CYCLES.  HBM:
    FETCH_SIZE and WRITE_SIZE (KiB) scaled by what they read for the plain
    device copy of copy_bytes (torch copy_, a "copyBuffer" kernel)."""
    import statistics
    mean = lambda k, c: statistics.mean(vals[(k, c)]) if (k, c) in vals else None
    kernels = sorted({k for k, _ in vals})
    scale_f = scale_w = None
    if copy_bytes:
        copies = [k for k in kernels if "copyBuffer" in k or "copy" in k.lower()]
        cf = max((v for k in copies for v in vals.get((k, "FETCH_SIZE"), [])), default=None)
        cw = max((v for k in copies for v in vals.get((k, "WRITE_SIZE"), [])), default=None)
        scale_f = copy_bytes / 1024 / cf if cf else None
        scale_w = copy_bytes / 1024 / cw if cw else None
    out = {}
    for k in kernels:
        dur = statistics.mean(durs[k]) * 1e-9
        rec = {"name": _short_kernel_name(k), "dispatches": len(vals.get((k, next(
            c for kk, c in vals if kk == k)), [])), "mean_duration_ms": dur * 1e3}
        gui = mean(k, "GRBM_GUI_ACTIVE")
        busy = mean(k, "SQ_VALU_MFMA_BUSY_CYCLES")
        mops = [mean(k, "SQ_INSTS_VALU_MFMA_MOPS_" + t) for t in ("BF16", "F32")]
        if any(m is not None for m in mops):
            flop = 512.0 * sum(m for m in mops if m is not None)
            rec["mfma_flop"] = flop
            rec["mfma_flop_bf16"] = None if mops[0] is None else 512.0 * mops[0]
            rec["mfma_tflops"] = flop / dur / 1e12
        if mean(k, "SQ_INSTS_MFMA") is not None:
            rec["mfma_insts"] = mean(k, "SQ_INSTS_MFMA")
        if gui is not None:
            simd_cycles = gui / agent["xcc"] * agent["simd"]
            rec["clock_mhz"] = gui / agent["xcc"] / dur / 1e6
            if busy is not None:
                rec["mfma_busy_frac"] = busy / simd_cycles
            co = mean(k, "SQ_VALU_MFMA_COEXEC_CYCLES")
            if co is not None:
                rec["mfma_valu_coexec_frac"] = co / simd_cycles
        if busy is not None:
            rec["mfma_busy_frac_at_peak_clock"] = busy / (dur * agent["mhz"] * 1e6 * agent["simd"])
        fetch, write = mean(k, "FETCH_SIZE"), mean(k, "WRITE_SIZE")
        if fetch is not None:
            rec["fetch_kib_raw"] = fetch
        if write is not None:
            rec["write_kib_raw"] = write
        if fetch is not None and write is not None and scale_f and scale_w:
            rec["hbm_bytes"] = (fetch * scale_f + write * scale_w) * 1024
            rec["hbm_gbs"] = rec["hbm_bytes"] / dur / 1e9
            rec["hbm_frac"] = rec["hbm_gbs"] / PEAK_HBM_GBS
        out[k] = rec
    return out, {"fetch_scale": scale_f, "write_scale": scale_w}


def pmc_report(args):
    """--pmc-report: summarise rocprofv3 counter runs (markdown + JSON)."""
    import hashlib
    import workloads
    wl = workloads.BY_NAME[args.workload]
    vals, durs, agent = read_counter_dirs(args.pmc_report)
    copy_bytes = args.calib_copy_mb << 20
    per, scales = summarise_counters(vals, durs, agent, copy_bytes)
    flops = wl.flops_path()
    want = stream_kernel_name(wl).split("<")[0]
    stream_k = [k for k in per if want in k and ("Lb1E" in k) == wl.fox]
    src = os.path.join(ROOT, "householder_position_encoding_amd", "csrc", "stream.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    md = os.path.join(ROOT, "profiles", f"counters_{wl.name}.md") if args.pmc_md is None else args.pmc_md
    lines = [f"# Hardware counters: {wl.name} (B={wl.B} H={wl.H} T={wl.T} d={wl.d}, {wl.dtype}"
             f"{', gate' if wl.fox else ''})", "",
             "Made by `python bench.py --pmc-report <dirs> --workload " + wl.name +
             (f" --calib-copy-mb {args.calib_copy_mb}" if args.calib_copy_mb else "") +
             "` from these rocprofv3 runs (each its own process, after `cd /tmp && export "
             "TMPDIR=/tmp`):", ""]
    lines += [f"    {c}" for c in args.pmc_command] + [""]
    lines += [f"GPU: {agent['simd']} SIMDs, {agent['xcc']} XCDs, peak engine clock {agent['mhz']} MHz.",
              "Matrix-core busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x SIMDs) "
              "(rocprofv3's MfmaUtil); executed flop = 512 x SQ_INSTS_VALU_MFMA_MOPS_*.", ""]
    if scales["fetch_scale"]:
        lines += [f"HBM bytes = FETCH_SIZE x {scales['fetch_scale']:.3f} + WRITE_SIZE x "
                  f"{scales['write_scale']:.3f} (KiB): the factors make the counters read "
                  f"{copy_bytes} bytes each way for the bench's plain device copy of that size.", ""]
    lines += ["| kernel | dispatches | mean ms (profiled) | clock MHz | MFMA flop | MFMA busy | "
              "MFMA+VALU co-exec | HBM bytes | HBM GB/s |", "|---|---|---|---|---|---|---|---|---|"]
    f = lambda x, fmt: "" if x is None else format(x, fmt)
    for k, r in sorted(per.items(), key=lambda kv: -kv[1]["mean_duration_ms"] * kv[1]["dispatches"]):
        if "copy" in k.lower() and "pathattn" not in k:
            continue
        lines.append(f"| {r['name'][:70]} | {r['dispatches']} | {r['mean_duration_ms']:.3f} | "
                     f"{f(r.get('clock_mhz'), '.0f')} | {f(r.get('mfma_flop'), '.4g')} | "
                     f"{f(r.get('mfma_busy_frac'), '.3f')} | {f(r.get('mfma_valu_coexec_frac'), '.3f')} | "
                     f"{f(r.get('hbm_bytes'), '.4g')} | {f(r.get('hbm_gbs'), '.0f')} |")
    rec = None
    if stream_k:
        r = per[stream_k[0]]
        rec = {"kernel": stream_k[0], "stream_hip_sha256_16": sha,
               "flops_path": flops,
               "mfma_flop_per_launch": r.get("mfma_flop"),
               "mfma_flop_over_flops_path": None if r.get("mfma_flop") is None else r["mfma_flop"] / flops,
               "mfma_busy_frac": r.get("mfma_busy_frac"),
               "mfma_busy_frac_at_peak_clock": r.get("mfma_busy_frac_at_peak_clock"),
               "mfma_valu_coexec_frac": r.get("mfma_valu_coexec_frac"),
               "clock_mhz_profiled": r.get("clock_mhz"),
               "hbm_bytes_per_launch": r.get("hbm_bytes"),
               "hbm_gbs_profiled": r.get("hbm_gbs"),
               "mean_duration_ms_profiled": r["mean_duration_ms"]}
        lines += ["", f"Stream kernel `{r['name']}`: F_path = B*H*T^2*(2d + d^2/64) = {flops:.4g} flop per "
                  "launch" + ("" if rec["mfma_flop_over_flops_path"] is None else
                              f"; executed matrix-core flop / F_path = {rec['mfma_flop_over_flops_path']:.4f}") + ".",
                  f"stream.hip sha256[:16] at measurement: {sha}"]
        db = json.load(open(args.counters)) if os.path.exists(args.counters) else {}
        old = db.get(wl.name, {})
        if old.get("stream_hip_sha256_16") == sha:   # merge passes of the same kernel
            rec = {k: (v if v is not None else old.get(k)) for k, v in rec.items()}
        db[wl.name] = rec
        with open(args.counters, "w") as fh:
            json.dump(db, fh, indent=1)
    with open(md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return rec


def trace_report(args):
    """--trace-report: per-kernel durations from rocprofv3 --stats (markdown)."""
    import csv
    import glob
    import workloads
    wl = workloads.BY_NAME[args.workload]
    files = glob.glob(os.path.join(args.trace_report, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv below {args.trace_report}")
    rows = list(csv.DictReader(open(files[0])))
    flops = wl.flops_path()
    want = stream_kernel_name(wl).split("<")[0]
    md = (os.path.join(ROOT, "profiles", f"kernel_trace_{wl.name}.md") if args.pmc_md is None
          else args.pmc_md)
    lines = [f"# Kernel trace: {wl.name} (B={wl.B} H={wl.H} T={wl.T} d={wl.d}, {wl.dtype}"
             f"{', gate' if wl.fox else ''})", "",
             "Made by `python bench.py --trace-report <dir> --workload " + wl.name +
             "` from this rocprofv3 run (after `cd /tmp && export TMPDIR=/tmp`):", ""]
    lines += [f"    {c}" for c in args.pmc_command] + [""]
    lines += ["| kernel | calls | average us | min us | max us | share of GPU time |",
              "|---|---|---|---|---|---|"]
    stream = None
    for r in rows:
        name = _short_kernel_name(r["Name"])
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} % |")
        if stream is None and want in r["Name"] and ("Lb1E" in r["Name"]) == wl.fox:
            stream = r
    if stream is not None:
        avg, mn = float(stream["AverageNs"]) * 1e-9, float(stream["MinNs"]) * 1e-9
        peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
        lines += ["", f"Stream kernel `{_short_kernel_name(stream['Name'])}`: F_path = "
                  f"{flops:.4g} flop per launch; at the average duration {avg * 1e3:.4f} ms that "
                  f"is {flops / avg / 1e12:.0f} TFLOP/s = {flops / avg / 1e12 / peak:.3f} of the "
                  f"{peak:.0f} TFLOP/s peak (at the minimum, {flops / mn / 1e12 / peak:.3f})."]
        if wl.fox:
            lines += ["With the forget gate the bench launches the scan both with the exact block "
                      "skip and with every block computed (PATH_ATTN_NO_SKIP), so these durations "
                      "mix the two and the rate above is partly effective; the bench line's "
                      "roofline takes the no-skip calls alone."]
    with open(md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counters_record(path, wl):
    """This workload's counter record if it was taken on the current
    stream.hip (else None: the kernel changed since)."""
    import hashlib
    try:
        rec = json.load(open(path)).get(wl.name)
        src = os.path.join(ROOT, "householder_position_encoding_amd", "csrc", "stream.hip")
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except (OSError, ValueError):
        return None
    return rec if rec is not None and rec.get("stream_hip_sha256_16") == sha else None


def main():
    args = parse()
    if args.pmc_report:
        pmc_report(args)
        return
    if args.trace_report:
        trace_report(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch
    import householder_position_encoding_amd as pa
    import workloads

    wl = workloads.BY_NAME[args.workload]
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    inp = workloads.generate(wl)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q, k, v, w = (torch.from_numpy(inp[n]).to(dev, tdt) for n in ("q", "k", "v", "w"))
    beta = torch.from_numpy(inp["beta"]).to(dev)
    logf = None if inp["logf"] is None else torch.from_numpy(inp["logf"]).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.T), dtype=torch.float32, device=dev)
    dt_code = pa.BF16 if wl.dtype == "bf16" else pa.F32
    ws = torch.empty(pa.path_attn_workspace_bytes(wl.B, wl.H, wl.T, wl.d, dt_code),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        pa.path_attn_fwd(q, k, v, w, beta, logf, out=out, lse=lse, workspace=ws)

    # ---- whole path ----
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # an event between consecutive steps gives per-step times as well
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))

    # ---- the two phases on their own (same stream, same workspace) ----
    def timed(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    ms_prep = timed(lambda: pa.path_attn_prepare(q, k, v, w, beta, logf, workspace=ws), args.steps)
    ms_stream = timed(lambda: pa.path_attn_stream(ws, logf is not None, out, lse), args.steps)

    fox_skip = None
    if logf is not None:
        # exact forget-gate block skip: share of cross steps it left out, and
        # the scan's time with every block computed
        cnt = torch.zeros(1, dtype=torch.int64, device=dev)
        pa.path_attn_stream(ws, True, out, lse, skipped=cnt)
        torch.cuda.synchronize()
        N = wl.T // 64
        waves_per_chunk = 1 if (wl.dtype == "bf16" and wl.d == 64) else 2
        cross_steps = wl.B * wl.H * N * (N - 1) // 2 * waves_per_chunk
        ms_noskip = timed(lambda: pa.path_attn_stream(ws, True, out, lse, flags=pa.NO_SKIP),
                          args.steps)
        fox_skip = {"skipped_steps": int(cnt.item()), "cross_steps": cross_steps,
                    "skipped_frac": int(cnt.item()) / max(1, cross_steps),
                    "ms_stream_no_skip": ms_noskip}

    flops = wl.flops_path()
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    # with the gate the roofline takes the scan with every block computed
    # (the work F_path counts); the skip's effective rate is in fox_skip
    ms_roof = ms_stream if fox_skip is None else fox_skip["ms_stream_no_skip"]
    stream_tflops = flops / (ms_roof * 1e-3) / 1e12
    if fox_skip is not None:
        fox_skip["effective_tflops_path"] = flops / (ms_stream * 1e-3) / 1e12
        fox_skip["effective_frac"] = fox_skip["effective_tflops_path"] / peak
    # per-launch figures of the stream kernel from rocprofv3 counters (valid
    # only for the kernel source they were measured on)
    crec = counters_record(args.counters, wl)
    traffic = None if crec is None else crec.get("hbm_bytes_per_launch")
    mfma_util = None
    if crec is not None and crec.get("mfma_busy_frac") is not None:
        mfma_util = {"kernel": stream_kernel_name(wl), "busy_frac": crec["mfma_busy_frac"],
                     "busy_frac_at_peak_clock": crec.get("mfma_busy_frac_at_peak_clock"),
                     "valu_coexec_frac": crec.get("mfma_valu_coexec_frac"),
                     "executed_flop_per_launch": crec.get("mfma_flop_per_launch"),
                     "executed_over_flops_path": crec.get("mfma_flop_over_flops_path"),
                     "source": os.path.relpath(args.counters, ROOT) + " (rocprofv3 --pmc; "
                               f"profiles/counters_{wl.name}.md)"}
    res = {
        "metric": "PaTH attn fwd tokens/s + TFLOP/s (% bf16 MFMA peak), B2 T16384 d64, 1 GPU",
        "value": wl.n_tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_median": per_step[len(per_step) // 2],
        "ms_min": per_step[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "d": wl.d,
                   "fox": wl.fox, "global_batch": wl.B, "seq_len": wl.T,
                   "parallelism": "single GPU"},
        "tflops_path": tflops,
        "tflops_attn": wl.flops_attn() / (ms * 1e-3) / 1e12,
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "ms_prep": ms_prep,
        "ms_stream": ms_stream,
        "roofline": {"kernel": stream_kernel_name(wl) + ("" if fox_skip is None else
                                                           ", every block computed"),
                     "bound": "mfma", "achieved": stream_tflops,
                     "peak": peak, "unit": "TFLOP/s", "frac": stream_tflops / peak,
                     "traffic": traffic,
                     "flops_per_launch": flops},
        "mfma_util": mfma_util,
    }
    if fox_skip is not None:
        res["fox_skip"] = fox_skip
    if args.calib_copy_mb > 0:
        nbytes = args.calib_copy_mb << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        ms_copy = timed(lambda: dst.copy_(src), 5)
        res["copy_calibration"] = {"bytes_read": nbytes, "bytes_written": nbytes,
                                   "ms": ms_copy, "gbs": 2 * nbytes / (ms_copy * 1e-3) / 1e9}
    if not args.no_partial:
        res["partial"] = bench_partial(wl, q, k, v, w, beta, logf, args, timed, ms)
        torch.cuda.empty_cache()
    if not args.no_varlen:
        res["varlen"] = bench_varlen(wl, q, k, v, w, beta, logf, args, timed, ms)
        torch.cuda.empty_cache()
    if not args.no_producer and wl.dtype == "bf16":
        res["producer"] = bench_producer(wl, args, timed)
        torch.cuda.empty_cache()
    if not args.no_decode:
        res["decode"] = bench_decode(wl, q, k, v, w, beta, logf, args, timed)
    if not args.no_backward:
        step()
        torch.cuda.synchronize()
        res["backward"] = bench_backward(wl, q, k, v, w, beta, logf, out, lse, args)
    if not args.no_cpu:
        step()
        torch.cuda.synchronize()
        res["cpu_baseline"], res["parity"] = cpu_baseline(wl, inp, args.cpu_heads, out, lse)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
