"""Several optimizer steps in a row on the GPU against the fp64 oracle's own
trajectory, resume from a saved (W, M) state, and the QK-Clip factor of an
infinite S_max.

Trajectory (Notes on Moonlight, "Background": M_t = mu M_{t-1} + G_t feeds
every later step): the oracle and the HIP path each run three steps from the
same drawn state with the same per-step gradients and the same per-head S_max
vector (held fixed, standing in for three forwards). Neither side ever sees
the other's state, so the comparison bounds carry the previous step's
difference forward: |dM_t| <= mu |dM_{t-1}| + 1 ulp, and the W bound of one
step plus decay times the carried bound. lr = 0.02 so that the bf16 weights
of the MHA-layer shapes move by tens of ulps per step.
"""
import numpy as np
import pytest
import torch

import muonclip_step_amd as mc
import oracle
import workloads as wl
from gpu_harness import (State, assert_within, check_matrix, host64, hp_for, load_config_states, rel_fro, ulp,
                         w_bound)

pytestmark = pytest.mark.gpu

STEPS = 3


def _upload_grad(state, g):
    state.g.copy_(torch.from_numpy(np.ascontiguousarray(g, np.float32)).to(state.g.dtype).to("cuda"))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg_idx", [1, 2])
def test_three_step_trajectory_matches_oracle(cfg_idx):
    cfg = wl.config(cfg_idx)
    hp = hp_for(cfg, lr=0.02)
    s_in = wl.draw_smax(cfg, n_over=2 if cfg_idx == 1 else 4)
    heads = cfg.attn.H
    s_max = torch.from_numpy(s_in).cuda()
    g_orc = oracle.clip_factor(s_in.astype(np.float64), cfg.tau)
    assert np.any(g_orc < 1.0) and np.any(g_orc == 1.0)
    ref = load_config_states(cfg)          # o_out requested: O of every step is compared
    fused = load_config_states(cfg)        # no O copy: the update rides on the last apply where it can
    n = len(cfg.matrices)
    # oracle state, fp64 values of what each step stores (W in its dtype, M in fp32)
    w_o = [s.w0.astype(np.float64) for s in ref]
    m_o = [s.m0.astype(np.float64) for s in ref]
    carried_w = [None] * n
    carried_m = [np.zeros_like(x) for x in m_o]
    gamma = torch.empty(heads, dtype=torch.float32, device="cuda")
    for t in range(1, STEPS + 1):
        print(f"config {cfg_idx}: step {t}", flush=True)
        grads = [wl.draw_grad(cfg, i, step=t) for i in range(n)]
        for st_r, st_f, g in zip(ref, fused, grads):
            _upload_grad(st_r, g)
            _upload_grad(st_f, g)
        mc.muonclip_step([s.desc() for s in ref], hp, s_max=s_max, slots=1, heads=heads, gamma_out=gamma)
        mc.muonclip_step([s.desc(with_o=False) for s in fused], hp, s_max=s_max, slots=1, heads=heads)
        torch.cuda.synchronize()
        g_gpu = host64(gamma)
        assert np.allclose(g_gpu, g_orc, rtol=1e-6, atol=0)
        for i, st in enumerate(ref):
            spec = st.spec
            w_new, m_new, o_new = oracle.muonclip_step_matrix(
                w_o[i], grads[i].astype(np.float64), m_o[i],
                lr=oracle.f32(hp.lr), mu=oracle.f32(hp.mu), weight_decay=oracle.f32(hp.weight_decay),
                rms_scale=oracle.f32(hp.rms_scale), ns_steps=hp.ns_steps, ns_a=oracle.f32(hp.ns_a),
                ns_b=oracle.f32(hp.ns_b), ns_c=oracle.f32(hp.ns_c), ns_eps=oracle.f32(hp.ns_eps),
                gamma=g_orc if spec.clip_slot >= 0 else None, period=spec.period, segments=spec.segments,
                w_dtype=spec.w_dtype)
            m_new = m_new.astype(np.float64)
            m_g = host64(st.m)
            # momentum: each side rounds mu M + G once to fp32
            carried_m[i] = oracle.f32(hp.mu) * carried_m[i] + ulp(np.maximum(np.abs(m_new), np.abs(m_g)), "f32")
            assert_within(m_g, m_new, carried_m[i] + 1e-45, f"{spec.name} M step {t}")
            o_g = host64(st.o)
            err = rel_fro(o_g, o_new)
            assert err <= 2e-2, (spec.name, t, err)
            w_g = host64(st.w)
            bound = w_bound(spec, hp, w_o[i], w_new, w_g, o_g, o_new,
                            g_orc if spec.clip_slot >= 0 else None, g_gpu, carried_w[i])
            assert_within(w_g, w_new, bound, f"{spec.name} W step {t}")
            carried_w[i] = bound
            # the fused-update run is the same arithmetic, bit for bit
            assert torch.equal(fused[i].w, st.w) and torch.equal(fused[i].m, st.m), (spec.name, t)
            w_o[i], m_o[i] = w_new, m_new
            print(f"  {spec.name}: NS rel err {err:.2e}", flush=True)
    # over the three steps the weights moved well above rounding; the moves agree
    for i, st in enumerate(ref):
        d_g = host64(st.w) - st.w0
        d_o = w_o[i] - st.w0
        assert np.linalg.norm(d_o) > 0
        assert rel_fro(d_g, d_o) < 3e-2, (st.spec.name, rel_fro(d_g, d_o))


@pytest.mark.timeout(300)
def test_resume_from_saved_state_is_bit_identical():
    """The library keeps no state between calls: saving (W, M) after step 1,
    reloading them into fresh buffers (fresh, unfilled workspace too) and
    running steps 2 and 3 gives the bits of an uninterrupted run."""
    cfg2 = wl.config(2)
    cfg1 = wl.config(1)
    picks = [(cfg2, 0), (cfg2, 2), (cfg1, 0), (cfg1, 1)]

    def fresh():
        return [load_config_states(c, indices=[i])[0] for c, i in picks]

    s_max = torch.from_numpy(wl.draw_smax(cfg2, n_over=4)).cuda()
    hp = hp_for(cfg2, lr=0.02)

    def step(states, t, ws):
        for (c, i), st in zip(picks, states):
            _upload_grad(st, wl.draw_grad(c, i, step=t))
        mc.muonclip_step([st.desc(with_o=False) for st in states], hp, s_max=s_max, slots=1, heads=16,
                         workspace=ws)

    probe = fresh()
    ws_bytes = mc.workspace_size([st.desc(with_o=False) for st in probe], hp)
    del probe
    ws_a = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    a = fresh()
    for t in (1, 2, 3):
        step(a, t, ws_a)
    b = fresh()
    ws_b = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    step(b, 1, ws_b)
    torch.cuda.synchronize()
    saved = [(st.w.cpu().clone(), st.m.cpu().clone()) for st in b]
    del b, ws_b
    torch.cuda.empty_cache()
    c = fresh()
    for st, (w, m) in zip(c, saved):
        st.w.copy_(w.cuda())
        st.m.copy_(m.cuda())
    ws_c = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bytes everywhere
    for t in (2, 3):
        step(c, t, ws_c)
    torch.cuda.synchronize()
    for (cfg, i), x, y in zip(picks, a, c):
        assert torch.equal(x.w, y.w), cfg.matrices[i].name
        assert torch.equal(x.m, y.m), cfg.matrices[i].name


@pytest.mark.parametrize("w_dtype", ["bf16", "f32"])
def test_infinite_smax_gives_gamma_zero(w_dtype):
    """gamma_h = min(1, tau / S) with the guard of the essay's MHA code
    sample (1 when S is not positive): S = +inf gives gamma = 0 and zeroes
    the head's clipped rows; -inf and NaN give 1; S = 5 tau gives 0.2. bf16
    weights take the update fused into the last Newton-Schulz product, fp32
    weights the update kernel; qk_clip_apply zeroes the rows too."""
    import dataclasses
    heads, period, cols = 5, 32, 96
    spec = dataclasses.replace(wl.config(2).matrices[0], rows=heads * period, cols=cols, w_dtype=w_dtype,
                               row_boost=(), clip_slot=0, period=period, segments=((0, period, 0.5),))
    rng_w = wl.normal(41, 0, (spec.rows, cols), 0.05)
    w = wl.quantize_bf16(rng_w) if w_dtype == "bf16" else wl.quantize_f32(rng_w)
    g = wl.quantize_f32(wl.normal(41, 1, (spec.rows, cols), 1e-2))
    m = wl.quantize_f32(wl.normal(41, 2, (spec.rows, cols), 1e-2))
    tau = 100.0
    s_in = np.array([np.inf, 50.0, np.nan, 500.0, -np.inf], np.float32)
    g_orc = oracle.clip_factor(s_in.astype(np.float64), tau)
    assert np.array_equal(g_orc, [0.0, 1.0, 1.0, 0.2, 1.0])
    s_max = torch.from_numpy(s_in).cuda()
    hp = hp_for(wl.config(2), lr=0.01, tau=tau)
    clipped = free = None
    gamma = torch.empty(heads, dtype=torch.float32, device="cuda")
    for with_o in (True, False):
        c, f = State(spec, w, g, m), State(spec, w, g, m)
        mc.muonclip_step([c.desc(with_o)], hp, s_max=s_max, slots=1, heads=heads, gamma_out=gamma)
        mc.muonclip_step([f.desc(with_o)], hp)
        torch.cuda.synchronize()
        g_gpu = host64(gamma)
        assert np.allclose(g_gpu, g_orc, rtol=1e-6, atol=0)
        assert g_gpu[0] == 0.0
        wc = host64(c.w)
        assert np.all(wc[:period] == 0.0)                       # head 0: gamma 0
        assert torch.equal(c.w[period:3 * period], f.w[period:3 * period])   # gamma 1 heads
        assert torch.equal(c.w[4 * period:], f.w[4 * period:])
        if with_o:
            clipped, free = c, f
    check_matrix(clipped, hp, g_orc, gamma_gpu=host64(gamma))
    # the standalone clip on the drawn weights
    plain = State(spec, w, g, m)
    gamma2 = torch.empty(heads, dtype=torch.float32, device="cuda")
    mc.qk_clip_apply([plain.desc(False)], s_max, 1, heads, tau, gamma_out=gamma2)
    torch.cuda.synchronize()
    assert np.array_equal(host64(gamma2), host64(gamma))
    got = host64(plain.w)
    assert np.all(got[:period] == 0.0)
    assert np.array_equal(got[period:3 * period], w[period:3 * period].astype(np.float64))
    assert np.array_equal(got[4 * period:], w[4 * period:].astype(np.float64))
    want = oracle.qk_clip_rows(w.astype(np.float64), g_orc, period, spec.segments)
    # fp32 sqrt(gamma) and product, then one rounding to the dtype
    assert np.all(np.abs(got - want) <= 1.001 * ulp(np.abs(want), w_dtype) + 1e-30)
