"""GPU parity of strided and packed (variable-length) batches:
path_attn_fwd_varlen and path_attn_bwd_varlen through the C ABI.

  * Strided: q, k, v, w are slices of one fused [B, T, 4, H, d] projection
    buffer and beta, logf slices of a [B, T, H, 2] buffer, so no tensor is
    dense in [B, H, T, ...] order; out and lse go to [B, T, H, ...] buffers.
  * Packed: sequences of different lengths (one of length 0, one of length
    1, others across chunk boundaries) stored token-major one after another
    ([total, H, d]), with cu_seqlens giving each sequence's first token;
    every sequence must match the oracle run on that sequence alone.  Both
    row-copy widths are exercised (16-byte rows where base and strides allow,
    4-byte words where the base is offset by one bf16 pair).
  * Equal lengths: a packed batch whose sequences all have the same length
    T (a multiple of 64) stages exactly the values the dense entry point
    reads, so out, lse and every gradient but dbeta must be bit-identical to
    path_attn_fwd / path_attn_bwd on the dense copy (dbeta adds its parts in
    an unfixed order and must agree to float32 rounding).

Bars: the forward parity bars (float32 1e-4 on o and lse; bf16 2e-2 on o,
1e-2 on lse) and the backward bars (max |g - r| <= tol * max(1, max |r|),
tol 2e-4 float32 / 2e-2 bf16), against the float64 oracles.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from oracle.backward import gradients as oracle_gradients
from tests.gpu_util import TOL

pytestmark = pytest.mark.gpu

GTOL = {"f32": 2e-4, "bf16": 2e-2}
GRADS = ("dq", "dk", "dv", "dw", "dbeta", "dlogf")


def _log(msg):
    print(msg, flush=True)


def _tdt(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check_fwd(tag, dtype, out, lse, o_ref, l_ref):
    tol_o, tol_l = TOL[dtype]
    eo = float(np.max(np.abs(out - o_ref))) if out.size else 0.0
    el = float(np.max(np.abs(lse - l_ref))) if lse.size else 0.0
    _log(f"{tag}: max|do|={eo:.3g} (tol {tol_o}) max|dlse|={el:.3g} (tol {tol_l})")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert eo <= tol_o and el <= tol_l, tag


def _check_grads(tag, dtype, got, ref):
    tol = GTOL[dtype]
    for n in GRADS:
        r = ref[n]
        if r is None:
            assert got[n] is None, f"{tag}: {n} returned without the gate"
            continue
        g = got[n]
        assert np.all(np.isfinite(g)), f"{tag}: {n} not finite"
        err = float(np.max(np.abs(g - r))) / max(1.0, float(np.max(np.abs(r))))
        _log(f"{tag} {n}: max|err|/max(1,max|ref|) = {err:.3g} (tol {tol})")
        assert err <= tol, f"{tag}: {n} off by {err:.3g} > {tol}"
    if ref["dlogf"] is not None:
        assert got["dlogf"][0] == 0.0, f"{tag}: dlogf at the first token must be 0"


# ------------------------------------------------------------------ strided

STRIDED = [
    # dtype, d, fox, B, H, T   (bf16 with T a multiple of 64 is read and
    # written in place; the others go through the staging)
    ("bf16", 64, True, 2, 3, 100),
    ("f32", 128, False, 1, 2, 128),
    ("f32", 64, True, 2, 1, 65),
    ("bf16", 64, True, 2, 3, 256),
    ("bf16", 128, False, 2, 2, 192),
    ("bf16", 64, False, 1, 2, 512),
]


def _strided_inputs(inp, dtype, B, H, T, d):
    """Device views of inp's arrays inside fused token-major buffers."""
    import torch
    fused = torch.zeros(B, T, 4, H, d, dtype=_tdt(dtype), device="cuda")
    for i, n in enumerate(("q", "k", "v", "w")):
        fused[:, :, i] = torch.from_numpy(inp[n].transpose(0, 2, 1, 3)).to("cuda", _tdt(dtype))
    sc = torch.zeros(B, T, H, 2, dtype=torch.float32, device="cuda")
    sc[..., 0] = torch.from_numpy(inp["beta"].transpose(0, 2, 1)).cuda()
    if inp["logf"] is not None:
        sc[..., 1] = torch.from_numpy(inp["logf"].transpose(0, 2, 1)).cuda()
    views = {n: fused[:, :, i].permute(0, 2, 1, 3) for i, n in enumerate(("q", "k", "v", "w"))}
    views["beta"] = sc[..., 0].permute(0, 2, 1)
    views["logf"] = None if inp["logf"] is None else sc[..., 1].permute(0, 2, 1)
    return views


@pytest.mark.parametrize("case", STRIDED, ids=lambda c: "-".join(map(str, c)))
def test_strided_forward_and_backward(case):
    import torch
    import householder_position_encoding_amd as pa
    dtype, d, fox, B, H, T = case
    _log(f"strided {case}")
    inp = workloads.small(dtype, B, H, T, d, seed=300 + T + d, fox=fox, beta_sigma=1.5)
    cot = workloads.cotangents(dtype, B, H, T, d, seed=400 + T + d)
    x = _strided_inputs(inp, dtype, B, H, T, d)
    assert not x["q"].is_contiguous() and not x["beta"].is_contiguous()
    out_buf = torch.zeros(B, T, H, d, dtype=_tdt(dtype), device="cuda")
    lse_buf = torch.zeros(B, T, H, dtype=torch.float32, device="cuda")
    out, lse = pa.path_attn_fwd_varlen(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"],
                                       out=out_buf.permute(0, 2, 1, 3),
                                       lse=lse_buf.permute(0, 2, 1))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.path_attn(inp["q"], inp["k"], inp["v"], inp["w"], inp["beta"],
                                    inp["logf"])
    _check_fwd(f"strided fwd {case}", dtype, _np(out), _np(lse), o_ref, l_ref)
    # the cotangents as strided views too
    dout_buf = torch.from_numpy(cot["dout"].transpose(0, 2, 1, 3).copy()).to("cuda", _tdt(dtype))
    dlse_buf = torch.from_numpy(cot["dlse"].transpose(0, 2, 1).copy()).cuda()
    grads = pa.path_attn_bwd_varlen(x["q"], x["k"], x["v"], x["w"], x["beta"], x["logf"],
                                    out, lse, dout_buf.permute(0, 2, 1, 3),
                                    dlse_buf.permute(0, 2, 1))
    torch.cuda.synchronize()
    got = {n: (None if g is None else _np(g)) for n, g in zip(GRADS, grads)}
    sel = lambda a, b, h: None if a is None else np.asarray(a[b, h], dtype=np.float64)
    for b in range(B):
        for h in range(H):
            ref = oracle_gradients(*(sel(inp[n], b, h) for n in ("q", "k", "v", "w", "beta",
                                                                    "logf")),
                                   sel(cot["dout"], b, h), sel(cot["dlse"], b, h))
            _check_grads(f"strided bwd {case} head ({b},{h})", dtype,
                         {n: (None if g is None else g[b, h]) for n, g in got.items()}, ref)


# ------------------------------------------------------------------- packed

PACKED = [
    # dtype, d, fox, H, lengths, misaligned (4-byte row copies)
    ("bf16", 64, True, 2, (1, 130, 0, 64, 77), False),
    ("bf16", 64, False, 2, (70, 5, 128), True),
    ("f32", 128, True, 1, (33, 100), False),
    ("f32", 64, False, 2, (64, 1, 191), True),
]


def _pack(parts, key):
    """Concatenate per-sequence [1, H, L, ...] arrays token-major: [total, H, ...]."""
    arrs = [np.swapaxes(p[key][0], 0, 1) for p in parts if p is not None]
    return np.concatenate(arrs, axis=0)


def _packed_device(arr, dtype, H, d, misaligned, slot):
    """A [total, H, d] (or [total, H]) device view of arr inside a wider buffer:
    vectors interleaved 4 to a token, scalars 2 to a token; `misaligned`
    shifts the vector views by two elements (4 bytes in bf16, 8 in float32)
    and widens the token stride by two, so rows are not 16-byte aligned."""
    import torch
    total = arr.shape[0]
    if arr.ndim == 3:
        shift = 2 if misaligned else 0
        width = 4 * H * d + shift
        tdt = _tdt(dtype)
        buf = torch.zeros(total * width + shift + 8, dtype=tdt, device="cuda")
        view = buf.as_strided((total, H, d), (width, d, 1), shift + slot * H * d)
        view.copy_(torch.from_numpy(arr).to(tdt))
        return view
    buf = torch.zeros(total, H, 2, dtype=torch.float32, device="cuda")
    buf[..., slot] = torch.from_numpy(np.ascontiguousarray(arr)).cuda()
    return buf[..., slot]


@pytest.mark.parametrize("case", PACKED, ids=lambda c: "-".join(map(str, c)))
def test_packed_forward_and_backward(case):
    import torch
    import householder_position_encoding_amd as pa
    dtype, d, fox, H, lengths, misaligned = case
    _log(f"packed {case}")
    parts, cots = [], []
    for n, L in enumerate(lengths):
        if L == 0:
            parts.append(None)
            cots.append(None)
            continue
        parts.append(workloads.small(dtype, 1, H, L, d, seed=500 + 7 * n + L, fox=fox,
                                     beta_sigma=1.5))
        cots.append(workloads.cotangents(dtype, 1, H, L, d, seed=600 + 7 * n + L))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    dev = {}
    for slot, n in enumerate(("q", "k", "v", "w")):
        dev[n] = _packed_device(_pack(parts, n), dtype, H, d, misaligned, slot)
    dev["beta"] = _packed_device(_pack(parts, "beta"), dtype, H, d, misaligned, 0)
    dev["logf"] = _packed_device(_pack(parts, "logf"), dtype, H, d, misaligned, 1) if fox else None
    cu_t = torch.from_numpy(cu).cuda()
    out, lse = pa.path_attn_fwd_varlen(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"],
                                       dev["logf"], cu_seqlens=cu_t)
    dout = _packed_device(_pack(cots, "dout"), dtype, H, d, misaligned, 1)
    dlse = _packed_device(_pack(cots, "dlse"), dtype, H, d, misaligned, 0)
    grads = pa.path_attn_bwd_varlen(dev["q"], dev["k"], dev["v"], dev["w"], dev["beta"],
                                    dev["logf"], out, lse, dout, dlse, cu_seqlens=cu_t)
    torch.cuda.synchronize()
    assert out.shape == (int(cu[-1]), H, d) and lse.shape == (int(cu[-1]), H)
    out_np, lse_np = _np(out), _np(lse)
    got = {n: (None if g is None else _np(g)) for n, g in zip(GRADS, grads)}
    for n, (p, c) in enumerate(zip(parts, cots)):
        if p is None:
            continue
        a, b = int(cu[n]), int(cu[n + 1])
        o_ref, l_ref = oracle.path_attn(p["q"], p["k"], p["v"], p["w"], p["beta"], p["logf"])
        _check_fwd(f"packed fwd {case} seq {n} (L={b - a})", dtype,
                   np.swapaxes(out_np[a:b], 0, 1), lse_np[a:b].T, o_ref[0], l_ref[0])
        for h in range(H):
            sel = lambda x: None if x is None else np.asarray(x[0, h], dtype=np.float64)
            ref = oracle_gradients(*(sel(p[k]) for k in ("q", "k", "v", "w", "beta", "logf")),
                                   sel(c["dout"]), sel(c["dlse"]))
            mine = {}
            for k, g in got.items():
                if g is None:
                    mine[k] = None
                else:
                    mine[k] = g[a:b, h]
            _check_grads(f"packed bwd {case} seq {n} head {h}", dtype, mine, ref)


def test_packed_equal_lengths_match_dense_bit_for_bit():
    """All sequences of one length T = 128: the staged values equal what the
    dense path reads, so every result is identical."""
    import torch
    import householder_position_encoding_amd as pa
    dtype, d, B, H, T = "bf16", 64, 3, 2, 128
    inp = workloads.small(dtype, B, H, T, d, seed=77, fox=True, beta_sigma=1.5)
    cot = workloads.cotangents(dtype, B, H, T, d, seed=78)
    tdt = _tdt(dtype)
    dense = {n: torch.from_numpy(inp[n]).to("cuda", tdt).contiguous() for n in ("q", "k", "v", "w")}
    for n in ("beta", "logf"):
        dense[n] = torch.from_numpy(inp[n]).cuda().contiguous()
    dout = torch.from_numpy(cot["dout"]).to("cuda", tdt).contiguous()
    dlse = torch.from_numpy(cot["dlse"]).cuda().contiguous()
    out_d, lse_d = pa.path_attn_fwd(dense["q"], dense["k"], dense["v"], dense["w"],
                                    dense["beta"], dense["logf"])
    g_d = pa.path_attn_bwd(dense["q"], dense["k"], dense["v"], dense["w"], dense["beta"],
                           dense["logf"], out_d, lse_d, dout, dlse)
    # packed token-major copies: [B*T, H, ...]
    pk = lambda t: t.permute(0, 2, 1, *range(3, t.dim())).reshape(B * T, H, *t.shape[3:]).contiguous()
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device="cuda")
    out_p, lse_p = pa.path_attn_fwd_varlen(pk(dense["q"]), pk(dense["k"]), pk(dense["v"]),
                                           pk(dense["w"]), pk(dense["beta"]), pk(dense["logf"]),
                                           cu_seqlens=cu, max_seqlen=T)
    g_p = pa.path_attn_bwd_varlen(pk(dense["q"]), pk(dense["k"]), pk(dense["v"]), pk(dense["w"]),
                                  pk(dense["beta"]), pk(dense["logf"]), out_p, lse_p, pk(dout),
                                  pk(dlse), cu_seqlens=cu, max_seqlen=T)
    torch.cuda.synchronize()
    assert torch.equal(pk(out_d), out_p) and torch.equal(pk(lse_d), lse_p)
    for n, a, b in zip(GRADS, g_d, g_p):
        if n == "dbeta":
            # dbeta sums per-thread parts with shared-memory atomics, whose order
            # is not fixed: equal up to float32 rounding of the sum order
            err = float((pk(a) - b).abs().max()) / max(1.0, float(a.abs().max()))
            assert err <= 1e-5, f"dbeta differs by {err:.3g}"
            continue
        assert torch.equal(pk(a), b), f"{n} differs between the dense and the packed call"
    _log("packed equal lengths: forward and backward identical to the dense call")


def test_strided_misaligned_rows_are_staged():
    """bf16 views of whole chunks whose rows start 4 bytes off a 16-byte
    boundary cannot be read in place (the chunk preparation copies 16-byte
    pieces): the call falls back to the staging copies and still matches the
    oracle, inputs and outputs alike."""
    import torch
    import householder_position_encoding_amd as pa
    B, H, T, d = 1, 2, 128, 64
    inp = workloads.small("bf16", B, H, T, d, seed=777, fox=True)
    n = B * H * T * d

    def shifted(arr):
        buf = torch.zeros(n + 8, dtype=torch.bfloat16, device="cuda")
        view = buf.as_strided((B, H, T, d), (H * T * d, T * d, d, 1), 2)
        if arr is not None:
            view.copy_(torch.from_numpy(arr).to(torch.bfloat16))
        return view

    x = {k: shifted(inp[k]) for k in ("q", "k", "v", "w")}
    beta = torch.from_numpy(inp["beta"]).cuda()
    logf = torch.from_numpy(inp["logf"]).cuda()
    out = shifted(None)
    lse = torch.zeros(B, H, T, dtype=torch.float32, device="cuda")
    assert x["q"].data_ptr() % 16 == 4
    out, lse = pa.path_attn_fwd_varlen(x["q"], x["k"], x["v"], x["w"], beta, logf, out=out,
                                       lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.path_attn(inp["q"], inp["k"], inp["v"], inp["w"], inp["beta"],
                                    inp["logf"])
    _check_fwd("strided misaligned", "bf16", _np(out), _np(lse), o_ref, l_ref)
