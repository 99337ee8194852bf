"""Parity of attention_forward (softmax attention with S_max taken from the
same pass) against the fp64 oracle.

Tolerances, from the arithmetic: the kernel rounds each probability to bf16
for the value product (relative error <= 2^-9 per weight, while the row sum
uses the fp32 probabilities) and rounds the output to bf16 once, so
|o - o_ref| <= 2^-9 (max_j |v_j| + |o_ref|) up to fp32 terms; the tests allow
twice that. lse is fp32, formed as scale m + ln(l) with the kernel's
reference max m up to 128 binary orders (89 in natural log) above the row
max: each term is rounded at about 2^-24 of a magnitude below |lse| + 89, and
the row sum of up to T terms adds T 2^-24, so |lse - lse_ref| <= T 2^-24 +
2^-22 (|lse| + 128). S_max is the fp32 max of fp32 dot
products: rtol 1e-3 against the oracle (as for max_logits_per_head), and
1e-5 against max_logits_per_head itself (the same products summed in a
different order).
"""
import math

import numpy as np
import pytest
import torch

import muonclip_step_amd as mc
import oracle
import workloads as wl
from gpu_harness import dev_tensor, host64

pytestmark = pytest.mark.gpu


def to_dev(q, k, ks, v):
    return (dev_tensor(q, "bf16"), dev_tensor(k, "bf16"),
            dev_tensor(ks, "bf16") if ks is not None else None, dev_tensor(v, "bf16"))


def run(qd, kd, ksd, vd, causal, want_lse=True, want_smax=True):
    B, T, H, _ = qd.shape
    lse = torch.empty(B, H, T, dtype=torch.float32, device="cuda") if want_lse else None
    smax = torch.empty(H, dtype=torch.float32, device="cuda") if want_smax else None
    o = mc.attention_forward(qd, kd, ksd, vd, causal=causal, lse=lse, s_max=smax)
    torch.cuda.synchronize()
    return o, lse, smax


def check_rows(o_gpu, lse_gpu, o_ref, lse_ref, v, T):
    """Element-wise bound of the module docstring; o_* [B,R,H,dv], lse [B,H,R]."""
    vmax = np.abs(v).max(axis=(1, 3))                       # [B, H]
    bound = 2.0 ** -8 * (vmax[:, None, :, None] + np.abs(o_ref)) + 1e-6
    err = np.abs(o_gpu - o_ref)
    assert np.all(np.isfinite(o_gpu))
    assert np.all(err <= bound), f"max excess {np.max(err - bound):.3g} (max err {err.max():.3g})"
    if lse_gpu is not None:
        tol = T * 2.0 ** -24 + 2.0 ** -22 * (np.abs(lse_ref) + 128.0)
        assert np.all(np.abs(lse_gpu - lse_ref) <= tol), np.max(np.abs(lse_gpu - lse_ref) - tol)


CASES = {
    # name: (B, T, H, d_s, causal, q_std, k_std) -- T spans several 256-row
    # query tiles and 64-key tiles with a ragged tail
    "mha_causal": (2, 333, 3, 0, True, 1.0, 1.0),
    "mha_full": (2, 333, 3, 0, False, 1.0, 1.0),
    "mla_causal": (1, 300, 2, 64, True, 1.0, 1.0),
    "mha_spiky": (1, 600, 2, 0, True, 3.0, 3.0),       # logits with std ~9: peaked softmax, rescales
    "mla_full_spiky": (1, 200, 2, 64, False, 2.5, 2.5),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_attention_matches_oracle(name):
    B, T, H, ds, causal, qs, ks_ = CASES[name]
    print("attention case", name, flush=True)
    q, k, ks, v = wl.draw_attention_case(100 + len(name), B, T, H, 128, ds, 128, q_std=qs, k_std=ks_)
    scale = 1.0 / math.sqrt(128 + ds)
    qd, kd, ksd, vd = to_dev(q, k, ks, v)
    o, lse, smax = run(qd, kd, ksd, vd, causal)
    o_ref, lse_ref = oracle.attention_forward(q, k, ks, v, causal, scale)
    check_rows(host64(o), host64(lse), o_ref, lse_ref, v, T)
    s_ref = oracle.max_logits(q, k, ks, causal, scale)
    assert np.allclose(host64(smax), s_ref, rtol=1e-3, atol=0)
    s_sep = host64(mc.max_logits_per_head(qd, kd, ksd, causal=causal, scale=scale))
    assert np.allclose(host64(smax), s_sep, rtol=1e-5, atol=0)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 256, 257])
def test_attention_edge_lengths(T):
    print("attention T =", T, flush=True)
    q, k, ks, v = wl.draw_attention_case(7, 1, T, 2, 128, 0, 128)
    qd, kd, ksd, vd = to_dev(q, k, ks, v)
    for causal in (True, False):
        o, lse, smax = run(qd, kd, ksd, vd, causal)
        o_ref, lse_ref = oracle.attention_forward(q, k, None, v, causal, 1.0 / math.sqrt(128))
        check_rows(host64(o), host64(lse), o_ref, lse_ref, v, T)
        assert np.allclose(host64(smax), oracle.max_logits(q, k, None, causal, 1.0 / math.sqrt(128)), rtol=1e-3)
    if T == 1:   # one key: the output is that key's value row, exactly
        o, _, _ = run(qd, kd, ksd, vd, True)
        assert torch.equal(o.cpu(), vd.cpu())


def test_attention_optional_outputs_and_empty():
    q, k, ks, v = wl.draw_attention_case(8, 2, 130, 2, 128, 64, 128)
    qd, kd, ksd, vd = to_dev(q, k, ks, v)
    full, lse, smax = run(qd, kd, ksd, vd, True)
    bare, _, _ = run(qd, kd, ksd, vd, True, want_lse=False, want_smax=False)
    # the S_max bookkeeping changes nothing in the output
    assert torch.equal(full, bare)
    # empty batch: nothing computed, every head -inf
    e = torch.empty(0, 5, 2, 192, dtype=torch.bfloat16, device="cuda")
    ek = torch.empty(0, 5, 2, 128, dtype=torch.bfloat16, device="cuda")
    er = torch.empty(0, 5, 64, dtype=torch.bfloat16, device="cuda")
    sm = torch.zeros(2, dtype=torch.float32, device="cuda")
    mc.attention_forward(e, ek, er, ek.clone(), causal=True, s_max=sm)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(sm.cpu()))


def test_attention_strided_views():
    # q, k, v as views into one packed [B, T, H, 3, 128] projection output,
    # the output into a wider buffer: only the strides change
    B, T, H = 2, 200, 3
    q, k, _, v = wl.draw_attention_case(9, B, T, H, 128, 0, 128)
    packed = torch.zeros(B, T, H, 3, 128, dtype=torch.bfloat16, device="cuda")
    packed[:, :, :, 0] = dev_tensor(q, "bf16")
    packed[:, :, :, 1] = dev_tensor(k, "bf16")
    packed[:, :, :, 2] = dev_tensor(v, "bf16")
    qv, kv, vv = packed[:, :, :, 0], packed[:, :, :, 1], packed[:, :, :, 2]
    wide = torch.full((B, T, H, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    out = wide[..., 64:192]
    smax = torch.empty(H, dtype=torch.float32, device="cuda")
    mc.attention_forward(qv, kv, None, vv, causal=True, out=out, s_max=smax)
    torch.cuda.synchronize()
    o_ref, _ = oracle.attention_forward(q, k, None, v, True, 1.0 / math.sqrt(128))
    check_rows(host64(out), None, o_ref, None, v, T)
    w = wide.cpu()
    assert torch.all(w[..., :64] == 7.0) and torch.all(w[..., 192:] == 7.0)   # nothing outside the view
    contig, _, _ = run(*to_dev(q, k, None, v), True)
    assert torch.equal(out.cpu(), contig.cpu())


def test_attention_nan_key_is_ignored_by_smax():
    # a NaN key poisons every output row that attends to it (as softmax
    # does) but not S_max, whose max ignores NaN logits
    q, k, _, v = wl.draw_attention_case(10, 1, 150, 2, 128, 0, 128)
    k[0, 100, 1, 5] = np.nan
    qd, kd, _, vd = to_dev(q, k, None, v)
    o, _, smax = run(qd, kd, None, vd, True, want_lse=False)
    oh = host64(o)
    assert np.all(np.isfinite(oh[0, :100])) and np.all(np.isfinite(oh[0, :, 0]))
    assert np.all(np.isnan(oh[0, 100:, 1]))
    assert np.allclose(host64(smax), oracle.max_logits(q, k, None, True, 1.0 / math.sqrt(128)), rtol=1e-3)
    k2 = k.copy()
    k2[0, 100, 1, 5] = 0.0
    o_ref, _ = oracle.attention_forward(q, k2, None, v, True, 1.0 / math.sqrt(128))
    check_rows(oh[:, :100], None, o_ref[:, :100], None, v, 150)


# ----------------------------------------------------------------- full sizes

def _layer_inputs(idx):
    cfg = wl.config(idx)
    wts = {s.name: wl.draw_weight(cfg, i) for i, s in enumerate(cfg.matrices) if not s.device_drawn}
    q, k, ks = wl.draw_attention_inputs(cfg, wts)
    v = wl.draw_attention_values(cfg, wts)
    return cfg, q, k, ks, v


@pytest.mark.slow
@pytest.mark.timeout(300)
@pytest.mark.parametrize("idx", [2, 3])
def test_attention_layer_sampled(idx):
    """The MHA layer (B4 T4096 H16 d128) and the MLA layer (B2 T4096 H64,
    d 192 / 128) at full size, in the launch configuration bench.py times:
    S_max against max_logits_per_head for every head and the oracle for the
    boosted and two plain heads, and sampled output rows (first, tile
    boundaries, last) of those heads against the oracle."""
    print("attention full size, configuration", idx, flush=True)
    cfg, q, k, ks, v = _layer_inputs(idx)
    a = cfg.attn
    scale = 1.0 / math.sqrt(a.d_q)
    qd, kd, ksd, vd = to_dev(q, k, ks, v)
    o, lse, smax = run(qd, kd, ksd, vd, True)
    s_sep = host64(mc.max_logits_per_head(qd, kd, ksd, causal=True))
    assert np.allclose(host64(smax), s_sep, rtol=1e-5, atol=0)
    heads = [0, 3, a.H // 2, a.H - 1]
    rows = [0, 1, 63, 64, 255, 256, 1000, a.T - 257, a.T - 1]
    oh, lh = host64(o), host64(lse)
    for h in heads:
        kh = k[:, :, h:h + 1]
        s_ref = oracle.max_logits(q[:, :, h:h + 1], kh, ks, True, scale)[0]
        assert math.isclose(float(smax[h]), s_ref, rel_tol=1e-3)
        o_ref, lse_ref = oracle.attention_forward(q[:, :, h:h + 1], kh, ks, v[:, :, h:h + 1], True, scale, rows=rows)
        check_rows(oh[:, rows, h:h + 1], lh[:, h:h + 1][:, :, rows], o_ref, lse_ref, v[:, :, h:h + 1], a.T)
