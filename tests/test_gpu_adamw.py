"""GPU parity of the AdamW entry point (the parameters Muon does not cover)
against the fp64 oracle, through the C ABI, over several steps.

Bounds, each step from the GPU's own previous state: m = fma(b1, m, (1-b1) g)
rounds the product and the sum, so it is within an ulp of m plus half an
ulp of (1-b1) g (the sum can cancel far below the product); v likewise with
(1-b2) g g (two product roundings, no cancellation). The parameter: one
rounding to its dtype (half an ulp on each side), the fp32 evaluation of
lr * m_hat / (sqrt(v_hat) + eps) (a few fp32 ulps of that term) and of
p (1 - lr wd), plus what the m difference moves the step term.
"""
import numpy as np
import pytest
import torch

import muonclip_step_amd as mc
import oracle
import workloads as wl
from gpu_harness import host64

pytestmark = pytest.mark.gpu


def ulp(x, bits):
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e - bits, -126 - bits + 1))


def make(n, seed, p_dtype, g_dtype, offset=0):
    p = wl.quantize_bf16(wl.normal(seed, 0, (n,), 0.5)) if p_dtype == "bf16" else wl.quantize_f32(wl.normal(seed, 0, (n,), 0.5))
    pt = torch.zeros(n + offset, dtype=torch.bfloat16 if p_dtype == "bf16" else torch.float32, device="cuda")
    gt = torch.zeros(n + offset, dtype=torch.bfloat16 if g_dtype == "bf16" else torch.float32, device="cuda")
    mt = torch.zeros(n + offset, dtype=torch.float32, device="cuda")
    vt = torch.zeros(n + offset, dtype=torch.float32, device="cuda")
    pt[offset:] = torch.from_numpy(p.astype(np.float32)).to(pt.dtype).cuda()
    return pt[offset:], gt[offset:], mt[offset:], vt[offset:], p.astype(np.float64)


@pytest.mark.parametrize("sizes,p_dtype,g_dtype,offset", [
    ((1, 3, 4, 4097), "bf16", "f32", 0),
    ((5000, 64, 12345), "f32", "f32", 0),
    ((333, 1024, 7), "bf16", "bf16", 1),     # unaligned views: element-wise path
    ((0, 70000), "bf16", "f32", 0),
])
def test_adamw_matches_oracle_over_steps(sizes, p_dtype, g_dtype, offset):
    print("adamw", sizes, p_dtype, g_dtype, offset, flush=True)
    bufs = [make(n, 40 + i, p_dtype, g_dtype, offset) for i, n in enumerate(sizes)]
    vecs = [mc.vector(p, g, m, v) for (p, g, m, v, _) in bufs]
    kw = dict(lr=1e-2, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    p_prev = [b[4] for b in bufs]
    m_prev = [np.zeros(len(b[4])) for b in bufs]
    v_prev = [np.zeros(len(b[4])) for b in bufs]
    for t in (1, 2, 3):
        grads = []
        for i, (p, g, m, v, _) in enumerate(bufs):
            gh = wl.normal(100 + t, i, (p.numel(),), 1.0 if i % 2 else 1e-3)
            gh = wl.quantize_bf16(gh) if g_dtype == "bf16" else wl.quantize_f32(gh)
            g.copy_(torch.from_numpy(gh.astype(np.float32)).to(g.dtype))
            grads.append(gh.astype(np.float64))
        mc.adamw_step(vecs, mc.adamw_hparams(step=t, **kw))
        torch.cuda.synchronize()
        for i, (p, g, m, v, _) in enumerate(bufs):
            if p.numel() == 0:
                continue
            po, mo, vo = oracle.adamw_step(p_prev[i], grads[i], m_prev[i], v_prev[i], step=t,
                                           p_dtype=p_dtype, **{k: oracle.f32(x) for k, x in kw.items()})
            mg, vg, pg = host64(m), host64(v), host64(p)
            g64 = grads[i]
            m_bound = 2 * ulp(mo, 24) + ulp(0.1 * np.abs(g64), 24) + 1e-45
            v_bound = 2 * ulp(vo, 24) + 2 * ulp(0.05 * g64 * g64, 24) + 1e-45
            assert np.all(np.abs(mg - mo) <= m_bound), (t, i, "m")
            assert np.all(np.abs(vg - vo) <= v_bound), (t, i, "v")
            c1 = 1.0 / (1.0 - 0.9 ** t)
            c2 = 1.0 / (1.0 - 0.95 ** t)
            den = np.sqrt(vo * c2) + 1e-8
            step_term = 1e-2 * np.abs(mo * c1) / den
            bits = 8 if p_dtype == "bf16" else 24
            bound = (1.001 * ulp(np.maximum(np.abs(po), np.abs(pg)), bits) + 8 * ulp(step_term, 24)
                     + 2 * ulp(np.abs(p_prev[i]), 24) + 1e-2 * c1 * m_bound / den
                     + step_term * (v_bound / np.maximum(vo, 1e-300)) + 1e-30)
            assert np.all(np.abs(pg - po) <= bound), (t, i, "p", float(np.max(np.abs(pg - po) - bound)))
            # continue from the GPU's own state (the bounds are per step)
            p_prev[i], m_prev[i], v_prev[i] = pg, mg, vg
