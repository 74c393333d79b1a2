"""GPU parity of decoding with in-place key refinement (prefill alignment of
the key cache, then decode steps) against the fp64 oracle.

PaTH slides, frame "Decoding updates historical keys in place" (Sec. 3.4,
Eq. 1).  The output of the decode step at position t is row t of the
attention over tokens 0..t, so it is compared with the forward oracle's row
t; the key cache after the step at t is compared with the oracle's keys
aligned to t (oracle/decode.py).  Bars: outputs as in the forward parity
tests (float32 inputs 1e-4; bf16 inputs 2e-2 on o, 1e-2 on lse), where a
bf16 key cache counts as bf16 (the logits use the stored keys); keys of a
float32 cache 1e-4 max-abs.  A bf16 key cache is rounded again at every step
(at most half an ulp, 2^-9 relative, each time), and reflections do not grow
errors, so after a prefill and n steps its keys are within
(n + 1) * 2^-9 * max|k| of the exact ones (worst case, linear accumulation).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from oracle import decode as odec
from tests.gpu_util import TOL

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _tensors(inp, dtype):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = {n: torch.from_numpy(inp[n]).to("cuda", tdt).contiguous() for n in ("q", "k", "v", "w")}
    dev["beta"] = torch.from_numpy(inp["beta"]).to("cuda").contiguous()
    dev["logf"] = None if inp["logf"] is None else torch.from_numpy(inp["logf"]).to("cuda").contiguous()
    return dev


def _run(inp, dtype, kc, L, n_dec, T_cap):
    """Prefill the first L tokens, then decode tokens L .. L+n_dec-1.
    Returns (outputs [n_dec, B, H, d], lse [n_dec, B, H], the cache)."""
    import torch
    import householder_position_encoding_amd as pa
    dev = _tensors(inp, dtype)
    B, H, T, d = inp["q"].shape
    fox = inp["logf"] is not None
    cache = pa.DecodeCache(B, H, T_cap, d, dev["q"].dtype,
                           kc_dtype=torch.bfloat16 if kc == "bf16" else torch.float32, fox=fox)
    if L > 0:
        pre = lambda x: x[:, :, :L].contiguous()
        pa.path_attn_prefill_cache(cache, pre(dev["k"]), pre(dev["v"]), pre(dev["w"]),
                                   pre(dev["beta"]), None if not fox else pre(dev["logf"]))
    outs, lses = [], []
    for t in range(L, L + n_dec):
        at = lambda x: x[:, :, t].contiguous()
        o, l = pa.path_attn_decode_step(cache, at(dev["q"]), at(dev["k"]), at(dev["v"]),
                                        at(dev["w"]), at(dev["beta"]),
                                        None if not fox else at(dev["logf"]))
        outs.append(o.float())
        lses.append(l)
    torch.cuda.synchronize()
    assert cache.length == L + n_dec
    return (torch.stack(outs).cpu().numpy().astype(np.float64),
            torch.stack(lses).cpu().numpy().astype(np.float64), cache)


def _oracle_rows(inp, b, h, rows):
    d = inp["q"].shape[-1]
    one = lambda x: x[b, h][None].astype(np.float64)
    logf = inp["logf"]
    r = np.stack([np.zeros(len(rows), dtype=np.int64), np.asarray(rows)], 1)
    return oracle.path_attn_rows(one(inp["q"]), one(inp["k"]), one(inp["v"]), one(inp["w"]),
                                 one(inp["beta"]), None if logf is None else one(logf),
                                 1.0 / np.sqrt(d), r)


CASES = [
    # dtype, kc, d, fox, B, H, L, n_dec
    ("f32", "f32", 64, False, 1, 2, 192, 70),
    ("f32", "f32", 128, True, 1, 2, 128, 40),
    ("bf16", "f32", 64, True, 2, 2, 128, 40),
    ("bf16", "f32", 128, False, 1, 2, 64, 33),
    ("bf16", "bf16", 64, False, 1, 2, 64, 32),
    ("f32", "bf16", 128, True, 1, 1, 64, 16),
    ("f32", "f32", 64, False, 1, 2, 0, 80),        # decode from an empty cache
    ("f32", "f32", 128, True, 1, 1, 576, 6),       # two key splits per step
    ("bf16", "f32", 64, False, 1, 1, 1024, 3),     # three key splits per step
]


@pytest.mark.parametrize("dtype,kc,d,fox,B,H,L,n_dec", CASES,
                         ids=lambda v: str(v))
def test_decode_matches_oracle(dtype, kc, d, fox, B, H, L, n_dec):
    T = L + n_dec
    inp = workloads.small(dtype, B, H, T, d, seed=31 + L + d, fox=fox)
    T_cap = T + 5
    _log(f"decode case dtype={dtype} kc={kc} d={d} fox={fox} B={B} H={H} L={L} n_dec={n_dec}")
    outs, lses, cache = _run(inp, dtype, kc, L, n_dec, T_cap)
    tol_o, tol_l = TOL["bf16" if kc == "bf16" else dtype]
    kc_np = cache.kcache.float().cpu().numpy().astype(np.float64)
    eo = el = ek = 0.0
    for b in range(B):
        for h in range(H):
            o_ref, l_ref = _oracle_rows(inp, b, h, list(range(L, T)))
            eo = max(eo, float(np.max(np.abs(outs[:, b, h] - o_ref))))
            el = max(el, float(np.max(np.abs(lses[:, b, h] - l_ref))))
            k_ref = odec.refined_keys(inp["k"][b, h], inp["w"][b, h], inp["beta"][b, h], T - 1)
            ek = max(ek, float(np.max(np.abs(kc_np[b, h, :T] - k_ref))))
    tol_k = 1e-4 if kc == "f32" else (n_dec + 1) * 2.0 ** -9 * float(np.max(np.abs(inp["k"][:, :, :T])))
    _log(f"  max|do|={eo:.3g} (tol {tol_o}) max|dlse|={el:.3g} (tol {tol_l}) "
         f"max|dk|={ek:.3g} (tol {tol_k})")
    assert np.all(np.isfinite(outs)) and np.all(np.isfinite(lses))
    assert eo <= tol_o and el <= tol_l and ek <= tol_k


def test_prefill_alignment_only():
    """Aligned keys of a prompt of several chunks, no decode step: every row
    j equals H_{L-1} ... H_{j+1} k_j; values are copied; positions beyond L
    are untouched."""
    import torch
    import householder_position_encoding_amd as pa
    for dtype, d in (("f32", 64), ("bf16", 128)):
        B, H, L = 1, 2, 256
        inp = workloads.small(dtype, B, H, L, d, seed=77, beta_sigma=1.5, near2_frac=0.1, fox=True)
        dev = _tensors(inp, dtype)
        cache = pa.DecodeCache(B, H, L + 64, d, dev["q"].dtype, fox=True)
        cache.kcache.fill_(7.0)
        pa.path_attn_prefill_cache(cache, dev["k"], dev["v"], dev["w"], dev["beta"], dev["logf"])
        torch.cuda.synchronize()
        kc_np = cache.kcache.cpu().numpy().astype(np.float64)
        err = 0.0
        for h in range(H):
            k_ref = odec.refined_keys(inp["k"][0, h], inp["w"][0, h], inp["beta"][0, h], L - 1)
            err = max(err, float(np.max(np.abs(kc_np[0, h, :L] - k_ref))))
        lam = odec.gate_prefix(inp["logf"].astype(np.float64))
        eg = float(np.max(np.abs(cache.gcache.cpu().numpy()[..., :L] - lam)))
        ev = float(np.max(np.abs(cache.vcache[:, :, :L].float().cpu().numpy() - inp["v"])))
        _log(f"prefill {dtype} d={d}: max|dk|={err:.3g} max|dgate|={eg:.3g} max|dv|={ev:.3g}")
        assert err <= 1e-4 and eg <= 1e-9 and ev == 0.0
        assert np.all(kc_np[:, :, L:] == 7.0)


def test_decode_beta0_is_causal_attention():
    """beta = 0: the cache is never changed and each step is ordinary causal
    softmax attention (PaTH with H_t = I)."""
    import torch
    dtype, d, L, n_dec = "f32", 64, 64, 8
    inp = workloads.small(dtype, 1, 2, L + n_dec, d, seed=91, beta_const=0.0)
    outs, lses, cache = _run(inp, dtype, "f32", L, n_dec, L + n_dec)
    kc_np = cache.kcache.cpu().numpy()
    assert np.array_equal(kc_np, inp["k"]), "beta = 0 must leave the keys bitwise unchanged"
    scale = 1.0 / np.sqrt(d)
    for h in range(2):
        for n, t in enumerate(range(L, L + n_dec)):
            s = inp["k"][0, h, :t + 1].astype(np.float64) @ inp["q"][0, h, t].astype(np.float64) * scale
            p = np.exp(s - s.max())
            o = p @ inp["v"][0, h, :t + 1] / p.sum()
            assert np.max(np.abs(outs[n, 0, h] - o)) <= 1e-4
            assert abs(lses[n, 0, h] - (s.max() + np.log(p.sum()))) <= 1e-4


def test_decode_full_context_sampled():
    """Long context at the benchmark's head count: B=2, H=16, a 16384-token
    prompt (bf16, float32 key cache), then two decode steps; outputs of every
    head against the oracle's rows, and sampled cache rows against the
    per-row alignment."""
    dtype, d, B, H, L, n_dec = "bf16", 64, 2, 16, 16384, 2
    wl = workloads.BY_NAME["bf16_b2h16t16384d64"]
    inp = workloads.generate(wl)
    # the decoded tokens are drawn separately with the same recipe
    tail = workloads.small(dtype, B, H, 64, d, seed=1234)
    full = {n: np.concatenate([inp[n], tail[n][:, :, :n_dec]], axis=2) for n in ("q", "k", "v", "w", "beta")}
    full["logf"] = None
    _log("decode full context: prefill 16384 + 2 steps")
    outs, lses, cache = _run(full, dtype, "f32", L, n_dec, L + n_dec)
    tol_o, tol_l = TOL[dtype]
    eo = el = 0.0
    for b in range(B):
        for h in range(H):
            o_ref, l_ref = _oracle_rows(full, b, h, [L, L + 1])
            eo = max(eo, float(np.max(np.abs(outs[:, b, h] - o_ref))))
            el = max(el, float(np.max(np.abs(lses[:, b, h] - l_ref))))
    kc_np = cache.kcache.cpu().numpy()
    ek = 0.0
    rows = [0, 1, 63, 64, 8191, 16383, 16384, 16385]
    for b, h in ((0, 0), (1, 15)):
        ref = odec.aligned_key_rows(full["k"][b, h], full["w"][b, h], full["beta"][b, h], rows,
                                    L + n_dec - 1)
        ek = max(ek, float(np.max(np.abs(kc_np[b, h, rows] - ref))))
    _log(f"  max|do|={eo:.3g} max|dlse|={el:.3g} max|dk| (sampled)={ek:.3g}")
    assert eo <= tol_o and el <= tol_l and ek <= 1e-3


def test_decode_workspace_needs_no_initialisation():
    """The decode workspace holds only the split partials, written by every
    step before the merge reads them: a workspace filled with garbage (NaN
    bytes) before the first step gives the same outputs as a zeroed one, and
    they match the oracle's rows."""
    import torch
    dtype, d, B, H, L, n_dec, T_cap = "bf16", 64, 2, 3, 64, 5, 1100
    inp = workloads.small(dtype, B, H, L + n_dec, d, seed=5)
    import householder_position_encoding_amd as pa
    orig = pa.DecodeCache.__init__

    def garbage_init(self, *a, **kw):
        orig(self, *a, **kw)
        self.workspace.fill_(0xFF)
    pa.DecodeCache.__init__ = garbage_init
    try:
        outs, lses, _ = _run(inp, dtype, "f32", L, n_dec, T_cap)
    finally:
        pa.DecodeCache.__init__ = orig
    outs0, lses0, _ = _run(inp, dtype, "f32", L, n_dec, T_cap)
    assert np.array_equal(outs, outs0) and np.array_equal(lses, lses0)
    for b in range(B):
        for h in range(H):
            o_ref, l_ref = _oracle_rows(inp, b, h, list(range(L, L + n_dec)))
            assert np.max(np.abs(outs[:, b, h] - o_ref)) <= TOL["bf16"][0]
            assert np.max(np.abs(lses[:, b, h] - l_ref)) <= TOL["bf16"][1]
