"""Helpers for the GPU parity tests: move workload arrays to the GPU, call the
HIP path through the C ABI binding, and call the oracle on the same values."""
from __future__ import annotations

import json
import os

import numpy as np

import oracle

# Tolerances (max-abs over every compared element, GPU value upcast to fp64):
# float32 inputs 1e-4 on o and lse; bf16 inputs 2e-2 on o and 1e-2 on lse.
TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-2)}


def to_device(inputs: dict, dtype: str, device="cuda"):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = {}
    for name in ("q", "k", "v", "w"):
        dev[name] = torch.from_numpy(inputs[name]).to(device=device, dtype=tdt).contiguous()
    dev["beta"] = torch.from_numpy(inputs["beta"]).to(device).contiguous()
    dev["logf"] = None if inputs["logf"] is None else torch.from_numpy(inputs["logf"]).to(device).contiguous()
    return dev


def run_hip(dev: dict, workspace=None):
    """path_attn_fwd on device tensors; returns fp64 numpy (out, lse)."""
    import torch
    import householder_position_encoding_amd as pa
    out, lse = pa.path_attn_fwd(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"],
                                dev["logf"], workspace=workspace)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle_full(inputs: dict):
    """Oracle outputs of every row (small sizes only)."""
    return oracle.path_attn(inputs["q"], inputs["k"], inputs["v"], inputs["w"],
                            inputs["beta"], inputs["logf"])


def oracle_rows(inputs: dict, heads, rows_per_head):
    """Oracle outputs of selected rows of selected (b, h) heads.

    heads: list of (b, h); rows_per_head: list of int arrays (query indices).
    Returns (out [R, d], lse [R]) with rows in the order given."""
    q = inputs["q"]
    d = q.shape[-1]
    sel = lambda x: np.stack([x[b, h] for b, h in heads]).astype(np.float64)
    logf = inputs["logf"]
    rows = np.concatenate([np.stack([np.full(len(r), n), r], 1)
                           for n, r in enumerate(rows_per_head)])
    return oracle.path_attn_rows(sel(q), sel(inputs["k"]), sel(inputs["v"]), sel(inputs["w"]),
                                 sel(inputs["beta"]), None if logf is None else sel(logf),
                                 1.0 / np.sqrt(d), rows)


def sample_rows(T: int, rng, n_random=96):
    """Deterministic stratified row sample: the first rows, chunk-boundary
    rows, the whole last chunk (longest walks), and random rows."""
    fixed = [0, 1, 2, 31, 32, 63, 64, 65, 127, 128]
    fixed = [i for i in fixed if i < T]
    last = list(range(max(0, T - 64), T))
    rand = rng.choice(T, size=min(T, n_random), replace=False).tolist()
    return np.array(sorted(set(fixed + last + rand)), dtype=np.int64)


def record(name: str, **values):
    """Print measured errors of a case; with the environment variable
    PATH_ATTN_ERROR_LOG set, also append them as one JSON line to that file
    (the measured errors of a test run, kept beside its log)."""
    msg = " ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}" for k, v in values.items())
    print(f"{name}: {msg}", flush=True)
    path = os.environ.get("PATH_ATTN_ERROR_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": name, **{k: (float(v) if isinstance(v, (float, np.floating)) else v)
                                                 for k, v in values.items()}}) + "\n")


def spread_heads(B: int, H: int):
    """Heads (b, h) to compare at full size: eight spread over the flat head
    index b*H + h, one in each residue class mod 8 when B*H >= 8 (the scan
    places the blocks of head bh at block index group*B*H + bh), plus the
    last head."""
    BH = B * H
    flat = sorted({(i * BH // 8 + i) % BH for i in range(8)} | {BH - 1})
    return [(bh // H, bh % H) for bh in flat]
