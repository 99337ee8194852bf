"""GPU parity of the HIP library against the fp64 oracle, through the C ABI.

Tolerances: S_max 1e-3 relative; gamma 1e-3 relative; Newton-Schulz output
2e-2 relative Frobenius; momentum within 1 fp32 ulp; parameters within 1 ulp
of their dtype plus the part of the update the NS difference moves; rows the
clip leaves alone bit-identical to an unclipped run.
"""
import math

import numpy as np
import pytest
import torch

import muonclip_step_amd as mc
import oracle
import workloads as wl
from gpu_harness import (State, check_matrix, dev_tensor, host64, hp_for, load_config_states, oracle_step,
                         qk_to_device, rel_fro)

pytestmark = pytest.mark.gpu


def smax_oracle(cfg, q, k, ks):
    a = cfg.attn
    return oracle.max_logits(q, k, ks, a.causal, 1.0 / math.sqrt(a.d_q))


def weights_of(cfg):
    return {s.name: wl.draw_weight(cfg, i) for i, s in enumerate(cfg.matrices)
            if not s.device_drawn}


# ----------------------------------------------------------------- config 1

@pytest.mark.parametrize("lr", [2e-4, 0.02])
def test_config1_tiny_mha_full_step(lr):
    print("config 1 tiny MHA, lr", lr, flush=True)
    cfg = wl.config(1)
    q, k, ks = wl.draw_attention_inputs(cfg, weights_of(cfg))
    qd, kd, _ = qk_to_device(q, k, ks, "f32")
    s_gpu = mc.max_logits_per_head(qd, kd, None, causal=False)
    s_orc = smax_oracle(cfg, q, k, None)
    assert np.allclose(host64(s_gpu), s_orc, rtol=1e-3, atol=0)
    gam_orc = oracle.clip_factor(s_orc, cfg.tau)
    assert np.all(gam_orc < 1.0)          # tau = 10: every head clips
    states = load_config_states(cfg)
    hp = hp_for(cfg, lr=lr)
    gamma = torch.empty(4, dtype=torch.float32, device="cuda")
    mc.muonclip_step([s.desc() for s in states], hp, s_max=s_gpu, slots=1, heads=4, gamma_out=gamma)
    torch.cuda.synchronize()
    assert np.allclose(host64(gamma), gam_orc, rtol=1e-3, atol=0)
    for s in states:
        check_matrix(s, hp, gam_orc, gamma_gpu=host64(gamma))
    if lr == 0.02:
        # the update is visible above rounding: W0 (never clipped) moves by
        # the RMS-matched step; compare the change itself
        s0 = states[0]
        w_o, _, _ = oracle_step(s0, hp, None)
        d_g = host64(s0.w) - s0.w0
        d_o = w_o - s0.w0
        assert rel_fro(d_g, d_o) < 2e-2


def test_nesterov_step_matches_oracle():
    # Nesterov-style momentum: the stored buffer is mu M + G, the matrix
    # orthogonalised is G + mu (mu M + G)
    print("config 1, nesterov", flush=True)
    cfg = wl.config(1)
    states = load_config_states(cfg)
    hp = hp_for(cfg, lr=0.02, nesterov=1)
    mc.muonclip_step([s.desc() for s in states], hp)
    torch.cuda.synchronize()
    for s in states:
        check_matrix(s, hp)
    # the variant is visible: the plain step's O differs
    plain = load_config_states(cfg, indices=[0])
    hp0 = hp_for(cfg, lr=0.02)
    mc.muonclip_step([plain[0].desc()], hp0)
    torch.cuda.synchronize()
    assert rel_fro(host64(plain[0].o), host64(states[0].o)) > 5e-2


@pytest.mark.parametrize("alpha", [0.5, 0.3])
def test_global_clip_step_matches_oracle(alpha):
    # the all-head variant: one gamma from the largest S_max of the layer,
    # W_q rows scaled by gamma^alpha and W_k rows by gamma^(1 - alpha)
    import dataclasses
    print("config 1, global clip, alpha", alpha, flush=True)
    cfg = wl.config(1)
    q, k, ks = wl.draw_attention_inputs(cfg, weights_of(cfg))
    qd, kd, _ = qk_to_device(q, k, ks, "f32")
    s_gpu = mc.max_logits_per_head(qd, kd, None, causal=False)
    s_orc = smax_oracle(cfg, q, k, None)
    g_glob = oracle.clip_factor_global(s_orc, cfg.tau)
    assert g_glob < min(oracle.clip_factor(s_orc, cfg.tau)) * 1.0000001
    states = load_config_states(cfg)
    for s in states:
        if s.spec.name == "wq":
            s.spec = dataclasses.replace(s.spec, segments=((0, s.spec.period, alpha),))
        elif s.spec.name == "wk":
            s.spec = dataclasses.replace(s.spec, segments=((0, s.spec.period, 1.0 - alpha),))
    hp = hp_for(cfg, lr=0.02, clip_global=1)
    gamma = torch.empty(4, dtype=torch.float32, device="cuda")
    mc.muonclip_step([s.desc() for s in states], hp, s_max=s_gpu, slots=1, heads=4, gamma_out=gamma)
    torch.cuda.synchronize()
    g_gpu = host64(gamma)
    assert np.allclose(g_gpu, g_glob, rtol=1e-3, atol=0) and np.all(g_gpu == g_gpu[0])
    for s in states:
        check_matrix(s, hp, np.full(4, g_glob), gamma_gpu=g_gpu)


def test_cold_start_momentum_is_gradient():
    cfg = wl.config(1)
    states = load_config_states(cfg, indices=[0], cold=True)
    hp = hp_for(cfg)
    mc.muonclip_step([states[0].desc()], hp)
    torch.cuda.synchronize()
    assert np.array_equal(host64(states[0].m), states[0].g0.astype(np.float64))
    check_matrix(states[0], hp)


# ----------------------------------------------------------------- ragged / edge shapes

@pytest.mark.parametrize("shape,w_dtype,g_dtype,ld_pad", [
    ((1, 7), "bf16", "f32", 0),
    ((7, 1), "f32", "f32", 3),
    ((100, 37), "bf16", "bf16", 5),
    ((37, 100), "f32", "f32", 0),
    ((130, 300), "bf16", "f32", 2),
    ((300, 130), "bf16", "f32", 0),
    ((1000, 257), "bf16", "f32", 8),
    ((257, 1100), "f32", "bf16", 0),
])
def test_ragged_shapes(shape, w_dtype, g_dtype, ld_pad):
    print("ragged", shape, w_dtype, g_dtype, ld_pad, flush=True)
    rows, cols = shape
    spec = wl.MatrixSpec("r", rows, cols, w_dtype, init_std=0.5, grad_std=1.0, mom_std=1.0)
    seed = 1000 + rows * 7 + cols
    w = wl.normal(seed, 0, shape, 0.5)
    w = wl.quantize_bf16(w) if w_dtype == "bf16" else wl.quantize_f32(w)
    g = wl.normal(seed, 1, shape, 1.0)
    g = wl.quantize_bf16(g) if g_dtype == "bf16" else wl.quantize_f32(g)
    m = wl.quantize_f32(wl.normal(seed, 2, shape, 1.0))
    st = State(spec, w, g, m, g_dtype=g_dtype, ld_pad=ld_pad)
    hp = mc.hparams(lr=0.01)
    mc.muonclip_step([st.desc()], hp)
    torch.cuda.synchronize()
    check_matrix(st, hp)
    # the padding columns of the row stride are untouched
    if ld_pad:
        assert torch.all(st.w_full[:, cols:] == 0) and torch.all(st.m_full[:, cols:] == 0)


def test_group_on_128_tiles_against_oracle():
    """Four matrices of one shape group (m = 1024, n = 1100: two wide, two
    tall, padded rows) whose symmetric products run unsplit on 128x128 tiles
    (144 of them), the path where the Gram hands A to the Poly epilogue in
    fp32 fragment order; every matrix against the oracle."""
    states = []
    for k, shape in enumerate([(1024, 1100), (1100, 1024), (1024, 1100), (1100, 1024)]):
        spec = wl.MatrixSpec("g", *shape, "bf16", init_std=0.5, grad_std=1.0, mom_std=1.0)
        seed = 3000 + k
        w = wl.quantize_bf16(wl.normal(seed, 0, shape, 0.5))
        g = wl.quantize_f32(wl.normal(seed, 1, shape, 1.0))
        m = wl.quantize_f32(wl.normal(seed, 2, shape, 1.0))
        states.append(State(spec, w, g, m, ld_pad=8 * k))
    hp = mc.hparams(lr=0.01)
    mc.muonclip_step([st.desc() for st in states], hp)
    torch.cuda.synchronize()
    for st in states:
        check_matrix(st, hp)


@pytest.mark.parametrize("ns_steps,f32_weight,coef", [(5, False, None), (5, True, None), (4, False, None),
                                                     (4, True, None), (3, False, None), (7, False, None),
                                                     (5, False, (2.0, -1.5, 0.5))])
def test_gram_space_head_against_oracle(ns_steps, f32_weight, coef):
    """Six matrices of one group with n >= 2 m (m = 1100, n = 2300: wide and
    tall, padded rows, ragged against the 128 tiles) whose first three
    Newton-Schulz iterations run in Gram space (A_{j+1} = P_j A_j P_j, the
    accumulated product kept as P_j .. P_0 - a^{j+1} I, then one apply to X0);
    ns_steps = 4 leaves one X-space iteration after the head, ns_steps = 3
    none, so it takes the plain path; ns_steps = 7 four. The oracle check
    requests O copies, so the update runs as its own kernel and reads O from
    whichever X buffer holds it; a second run without O copies (the update in
    the last apply's epilogue, unless an f32 weight keeps the wave on the
    update kernel) must give the same weights bit for bit. coef: other
    quintic coefficients (a, b, c), whose a sets the shifts a^j of the
    accumulated product."""
    print("gram head", ns_steps, f32_weight, coef, flush=True)
    states = []
    for k in range(6):
        shape = (1100, 2300) if k % 2 == 0 else (2300, 1100)
        w_dtype = "f32" if f32_weight and k == 3 else "bf16"
        spec = wl.MatrixSpec("h", *shape, w_dtype, init_std=0.5, grad_std=1.0, mom_std=1.0)
        seed = 3100 + k
        w = wl.normal(seed, 0, shape, 0.5)
        w = wl.quantize_f32(w) if w_dtype == "f32" else wl.quantize_bf16(w)
        g = wl.quantize_f32(wl.normal(seed, 1, shape, 1.0))
        m = wl.quantize_f32(wl.normal(seed, 2, shape, 1.0))
        states.append(State(spec, w, g, m, ld_pad=8 * (k % 3)))
    kw = {} if coef is None else dict(ns_a=coef[0], ns_b=coef[1], ns_c=coef[2])
    hp = mc.hparams(lr=0.01, ns_steps=ns_steps, **kw)
    mc.muonclip_step([st.desc() for st in states], hp)
    torch.cuda.synchronize()
    for st in states:
        check_matrix(st, hp)
    _same_weights_without_o(states, hp)


def _same_weights_without_o(states, hp):
    """Rerun the step from the drawn inputs without O copies and require the
    weights of the run just checked, bit for bit."""
    want = [s.w.cpu().clone() for s in states]
    _fresh(states)
    mc.muonclip_step([s.desc(with_o=False) for s in states], hp)
    torch.cuda.synchronize()
    for a, s in zip(want, states):
        assert torch.equal(a, s.w.cpu())


def test_gram_space_head_eight_wave_apply_against_oracle():
    """Four 1024 x 2304 matrices (two wide, two tall): the head's m x m
    products run on 128 tiles and its final apply on 144 tiles of 256, one
    per CU, so that apply takes the eight-wave kernel. Against the oracle
    with O copies, then bit for bit without them (fused update)."""
    states = []
    for k in range(4):
        shape = (1024, 2304) if k % 2 == 0 else (2304, 1024)
        spec = wl.MatrixSpec("h8", *shape, "bf16", init_std=0.02, grad_std=1e-3, mom_std=1e-3)
        seed = 3200 + k
        w = wl.quantize_bf16(wl.normal(seed, 0, shape, 0.02))
        g = wl.quantize_f32(wl.normal(seed, 1, shape, 1e-3))
        m = wl.quantize_f32(wl.normal(seed, 2, shape, 1e-3))
        states.append(State(spec, w, g, m))
    hp = mc.hparams(lr=0.01)
    mc.muonclip_step([st.desc() for st in states], hp)
    torch.cuda.synchronize()
    for st in states:
        check_matrix(st, hp)
    _same_weights_without_o(states, hp)


def test_nesterov_bf16_gradients_through_the_gram_space_head():
    """Nesterov momentum with bf16 gradients and padded rows on a group that
    takes the Gram-space head (1024 x 2304, two wide and two tall): the
    matrix the head orthogonalises is the look-ahead G + mu (mu M + G).
    Against the oracle with O copies, then bit for bit without them (the
    update in the last apply's epilogue)."""
    states = []
    for k in range(4):
        shape = (1024, 2304) if k % 2 == 0 else (2304, 1024)
        spec = wl.MatrixSpec("hn", *shape, "bf16", init_std=0.02, grad_std=1e-3, mom_std=1e-3)
        seed = 3600 + k
        w = wl.quantize_bf16(wl.normal(seed, 0, shape, 0.02))
        g = wl.quantize_bf16(wl.normal(seed, 1, shape, 1e-3))
        m = wl.quantize_f32(wl.normal(seed, 2, shape, 1e-3))
        states.append(State(spec, w, g, m, g_dtype="bf16", ld_pad=8 * k))
    hp = mc.hparams(lr=0.01, nesterov=1)
    mc.muonclip_step([st.desc() for st in states], hp)
    torch.cuda.synchronize()
    for st in states:
        check_matrix(st, hp)
    _same_weights_without_o(states, hp)


@pytest.mark.parametrize("shapes", [[(1024, 4096)], [(4096, 1024), (1024, 4096)]])
def test_gram_space_head_split_k_against_oracle(shapes):
    """One or two 1024 x 4096 matrices: too few tiles to fill the chip, so the
    symmetric products run split-K and A reaches the Poly as the bf16 pair
    A_hi + A_lo from the split-K finish (which also adds the head's diagonal
    shifts and a^j P_j term), while the applies run unsplit and the head is
    taken. Against the oracle with O copies, then bit for bit without."""
    print("gram head split-K", shapes, flush=True)
    states = []
    for k, shape in enumerate(shapes):
        spec = wl.MatrixSpec("hs", *shape, "bf16", init_std=0.02, grad_std=1e-3, mom_std=1e-3)
        seed = 3300 + k
        w = wl.quantize_bf16(wl.normal(seed, 0, shape, 0.02))
        g = wl.quantize_f32(wl.normal(seed, 1, shape, 1e-3))
        m = wl.quantize_f32(wl.normal(seed, 2, shape, 1e-3))
        states.append(State(spec, w, g, m, ld_pad=8 * k))
    hp = mc.hparams(lr=0.01)
    mc.muonclip_step([st.desc() for st in states], hp)
    torch.cuda.synchronize()
    for st in states:
        check_matrix(st, hp)
    _same_weights_without_o(states, hp)


@pytest.mark.parametrize("shape,count", [((96, 160), 1), ((1024, 2304), 4)])
def test_zero_gradient_and_momentum_decay_only(shape, count):
    """G = M = 0: O is exactly zero and W only decays. The 1024 x 2304 group
    takes the Gram-space head, whose shifts (a^j P_j - a^{j+1} I, with P_j's
    diagonal rounded to bf16) do not cancel exactly: they must still multiply
    X0 = 0 and leave O zero."""
    states = []
    for k in range(count):
        rows, cols = shape if k % 2 == 0 else shape[::-1]
        spec = wl.MatrixSpec("z", rows, cols, "f32")
        w = wl.quantize_f32(wl.normal(77, k, (rows, cols), 1.0))
        z = np.zeros((rows, cols), np.float32)
        states.append(State(spec, w, z, z))
    hp = mc.hparams(lr=0.05)
    mc.muonclip_step([st.desc() for st in states], hp)
    torch.cuda.synchronize()
    decay = np.float32(1.0 - np.float64(np.float32(0.05)) * np.float64(np.float32(0.1)))
    for st in states:
        assert torch.all(st.o == 0)
        assert np.array_equal(host64(st.w), (st.w0 * decay).astype(np.float32).astype(np.float64))


# ----------------------------------------------------------------- config 2

def test_config2_mha_layer_full_step():
    print("config 2 MHA layer", flush=True)
    cfg = wl.config(2)
    q, k, _ = wl.draw_attention_inputs(cfg, weights_of(cfg))
    qd, kd, _ = qk_to_device(q, k, None, "bf16")
    s_gpu = mc.max_logits_per_head(qd, kd, None, causal=True)
    s_orc = smax_oracle(cfg, q, k, None)
    assert np.allclose(host64(s_gpu), s_orc, rtol=1e-3, atol=0)
    gam_orc = oracle.clip_factor(s_orc, cfg.tau)
    assert np.all(gam_orc[:4] < 1.0) and np.all(gam_orc[4:] == 1.0)
    states = load_config_states(cfg)
    hp = hp_for(cfg)
    gamma = torch.empty(16, dtype=torch.float32, device="cuda")
    mc.muonclip_step([s.desc() for s in states], hp, s_max=s_gpu, slots=1, heads=16, gamma_out=gamma)
    torch.cuda.synchronize()
    assert np.allclose(host64(gamma), gam_orc, rtol=1e-3, atol=0)
    for s in states:
        err = check_matrix(s, hp, gam_orc, gamma_gpu=host64(gamma))
        print(s.spec.name, "NS rel err %.3e" % err, flush=True)


def test_clip_rows_versus_unclipped_run():
    """gamma = 1 heads are bit-identical to the run without QK-Clip; clipped
    rows equal that run's rows times gamma^expo (one rounding)."""
    cfg = wl.config(2)
    idx = [0]
    a = load_config_states(cfg, idx)
    b = load_config_states(cfg, idx)
    s_max = torch.tensor([1000.0, 150.0, 100.0, 50.0] + [1.0] * 12, device="cuda")
    hp = hp_for(cfg)
    mc.muonclip_step([a[0].desc()], hp, s_max=s_max, slots=1, heads=16)
    mc.muonclip_step([b[0].desc()], hp)
    torch.cuda.synchronize()
    wa, wb = host64(a[0].w), host64(b[0].w)
    assert np.array_equal(wa[256:], wb[256:])          # heads 2..15: gamma == 1
    for h, sm in enumerate([1000.0, 150.0]):
        g = np.float32(100.0) / np.float32(sm)
        want = oracle.round_to_bf16(wb[h * 128:(h + 1) * 128] * math.sqrt(g))
        diff = np.abs(wa[h * 128:(h + 1) * 128] - want)
        assert np.all(diff <= 1.001 * np.ldexp(1.0, np.frexp(np.abs(want))[1] - 8) + 1e-30)
    assert np.array_equal(host64(a[0].m), host64(b[0].m))  # the clip does not touch momentum


def test_determinism_and_wave_split():
    """Bit-identical results run to run; a group run in several waves (a
    minimal workspace) still matches the oracle."""
    cfg = wl.config(1)
    outs = []
    for ws_mode in ("full", "full", "min"):
        states = load_config_states(cfg, indices=[1, 2])   # two 64x64 matrices: one group
        descs = [s.desc() for s in states]
        hp = hp_for(cfg)
        size = mc.workspace_size(descs, hp, minimal=(ws_mode == "min"))
        ws = torch.empty(size, dtype=torch.uint8, device="cuda")
        mc.muonclip_step(descs, hp, workspace=ws)
        torch.cuda.synchronize()
        outs.append([(s.w.cpu().clone(), s.m.cpu().clone(), s.o.cpu().clone()) for s in states])
        if ws_mode == "min":
            for s in states:
                check_matrix(s, hp)
    for (w0, m0, o0), (w1, m1, o1) in zip(outs[0], outs[1]):
        assert torch.equal(w0, w1) and torch.equal(m0, m1) and torch.equal(o0, o1)


def test_two_lanes_match_one_lane_bit_for_bit():
    """A step with two chains (two shape groups) runs them on two streams
    when the workspace holds both; the results are bit-identical to the
    one-stream run with the smallest workspace, and match the oracle."""
    cfg = wl.config(1)
    q, k, ks = wl.draw_attention_inputs(cfg, weights_of(cfg))
    qd, kd, _ = qk_to_device(q, k, ks, "f32")
    s_gpu = mc.max_logits_per_head(qd, kd, None, causal=False)
    gam_orc = oracle.clip_factor(smax_oracle(cfg, q, k, None), cfg.tau)
    outs = []
    for ws_mode in ("full", "min", "full"):
        print("two lanes vs one:", ws_mode, flush=True)
        states = load_config_states(cfg)               # 256x512 and two 64x64: two groups
        descs = [s.desc() for s in states]
        hp = hp_for(cfg, lr=0.02)
        size = mc.workspace_size(descs, hp, minimal=(ws_mode == "min"))
        if ws_mode == "full":
            assert size >= 2 * mc.workspace_size([descs[0]], hp)
        ws = torch.empty(size, dtype=torch.uint8, device="cuda")
        mc.muonclip_step(descs, hp, s_max=s_gpu, slots=1, heads=4, workspace=ws)
        torch.cuda.synchronize()
        outs.append([(s.w.cpu().clone(), s.m.cpu().clone(), s.o.cpu().clone()) for s in states])
        for s in states:
            check_matrix(s, hp, gam_orc)
    for run in outs[1:]:
        for (w0, m0, o0), (w1, m1, o1) in zip(outs[0], run):
            assert torch.equal(w0, w1) and torch.equal(m0, m1) and torch.equal(o0, o1)



def test_large_and_small_waves_on_two_lanes_bit_for_bit():
    """Eight 2048^2 matrices (their Gram launch has a tile for every CU: a
    large wave, on the caller's stream) and two 256 x 512 ones (a small wave,
    on the auxiliary stream beside it): the weights, momenta and O must equal
    bit for bit those of the same waves run on one stream (kernel timing on,
    which keeps every chain on the caller's stream; the waves are the same, so
    are the kernels), and sampled matrices of both groups match the oracle."""
    states = []
    for k in range(10):
        shape = (2048, 2048) if k < 8 else (256, 512)
        spec = wl.MatrixSpec("ls", *shape, "bf16", init_std=0.02, grad_std=1e-3, mom_std=1e-3)
        seed = 3400 + k
        w = wl.quantize_bf16(wl.normal(seed, 0, shape, 0.02))
        g = wl.quantize_f32(wl.normal(seed, 1, shape, 1e-3))
        m = wl.quantize_f32(wl.normal(seed, 2, shape, 1e-3))
        states.append(State(spec, w, g, m))
    hp = mc.hparams(lr=0.01)
    descs = [st.desc() for st in states]
    ws = torch.empty(mc.workspace_size(descs, hp), dtype=torch.uint8, device="cuda")
    outs = []
    for one_stream in (False, True):
        print("large and small waves, one stream:", one_stream, flush=True)
        _fresh(states)
        mc.profile_enable(one_stream)
        try:
            mc.muonclip_step(descs, hp, workspace=ws)
            torch.cuda.synchronize()
        finally:
            mc.profile_enable(False)
        outs.append([(st.w.cpu().clone(), st.m.cpu().clone(), st.o.cpu().clone()) for st in states])
    for (w0, m0, o0), (w1, m1, o1) in zip(outs[0], outs[1]):
        assert torch.equal(w0, w1) and torch.equal(m0, m1) and torch.equal(o0, o1)
    for k in (0, 9):
        check_matrix(states[k], hp)

def test_two_groups_of_large_waves_run_on_one_lane():
    """Two shape groups whose waves are all large (eight 2048^2 matrices and
    eight 2048 x 4096 ones, the latter through the Gram-space head): nothing
    is left for a second lane, so the step runs on the caller's stream with
    waves planned for the whole workspace, the same waves as with kernel
    timing on. Weights, momenta and O must match that run bit for bit, and
    a matrix of each group matches the oracle."""
    states = []
    for k in range(16):
        shape = (2048, 2048) if k < 8 else (2048, 4096)
        spec = wl.MatrixSpec("ll", *shape, "bf16", init_std=0.02, grad_std=1e-3, mom_std=1e-3)
        seed = 3500 + k
        w = wl.quantize_bf16(wl.normal(seed, 0, shape, 0.02))
        g = wl.quantize_f32(wl.normal(seed, 1, shape, 1e-3))
        m = wl.quantize_f32(wl.normal(seed, 2, shape, 1e-3))
        states.append(State(spec, w, g, m))
    hp = mc.hparams(lr=0.01)
    descs = [st.desc() for st in states]
    ws = torch.empty(mc.workspace_size(descs, hp), dtype=torch.uint8, device="cuda")
    outs = []
    for one_stream in (False, True):
        print("two groups of large waves, one stream:", one_stream, flush=True)
        _fresh(states)
        mc.profile_enable(one_stream)
        try:
            mc.muonclip_step(descs, hp, workspace=ws)
            torch.cuda.synchronize()
        finally:
            mc.profile_enable(False)
        outs.append([(st.w.cpu().clone(), st.m.cpu().clone(), st.o.cpu().clone()) for st in states])
    for (w0, m0, o0), (w1, m1, o1) in zip(outs[0], outs[1]):
        assert torch.equal(w0, w1) and torch.equal(m0, m1) and torch.equal(o0, o1)
    for k in (0, 15):
        check_matrix(states[k], hp)

# ----------------------------------------------------------------- QK-Clip alone

def test_qk_clip_apply_essay_invariants():
    """After qk_clip_apply the max logit recomputed from the clipped weights
    is before*gamma and <= tau; gamma <= 1; gamma = 1 heads untouched."""
    cfg = wl.config(2)
    wts = weights_of(cfg)
    q, k, _ = wl.draw_attention_inputs(cfg, wts)
    qd, kd, _ = qk_to_device(q, k, None, "bf16")
    before = mc.max_logits_per_head(qd, kd, None, causal=True)
    wq = dev_tensor(wts["wq"], "bf16")
    wk = dev_tensor(wts["wk"], "bf16")
    dummy = torch.zeros_like(wq, dtype=torch.float32)
    seg = ((0, 128, 0.5),)
    mats = [mc.matrix(wq, dummy, dummy, clip_slot=0, period=128, segments=seg),
            mc.matrix(wk, dummy, dummy, clip_slot=0, period=128, segments=seg)]
    gamma = torch.empty(16, dtype=torch.float32, device="cuda")
    mc.qk_clip_apply(mats, before, 1, 16, cfg.tau, gamma_out=gamma)
    torch.cuda.synchronize()
    g = host64(gamma)
    assert np.all(g <= 1.0) and np.all(g[:4] < 1.0) and np.all(g[4:] == 1.0)
    wq_h, wk_h = host64(wq), host64(wk)
    assert np.array_equal(wq_h[512:], wts["wq"][512:].astype(np.float64))
    assert np.array_equal(wk_h[512:], wts["wk"][512:].astype(np.float64))
    # recompute Q, K from the clipped weights (same activations) -> S_max
    cfg_c = wl.config(2)
    q2, k2, _ = wl.draw_attention_inputs(cfg_c, {"wq": wq_h.astype(np.float32), "wk": wk_h.astype(np.float32)})
    q2d, k2d, _ = qk_to_device(q2, k2, None, "bf16")
    after = host64(mc.max_logits_per_head(q2d, k2d, None, causal=True))
    b = host64(before)
    # bf16 rounding of the clipped weights and of the recomputed Q/K moves
    # the product by a few bf16 ulps
    assert np.allclose(after, b * g, rtol=2e-2)
    assert np.all(after <= cfg.tau * 1.02)


# ----------------------------------------------------------------- max logits

@pytest.mark.parametrize("B,T,H,dk,ds,causal,dtype", [
    (1, 1, 2, 128, 0, True, "bf16"),
    (2, 63, 3, 128, 0, True, "bf16"),
    (2, 65, 2, 128, 64, True, "bf16"),
    (1, 300, 4, 128, 64, False, "bf16"),
    (1, 16384 + 77, 2, 128, 64, True, "bf16"),   # MLA at a length that runs 64-row waves
    (3, 257, 2, 64, 0, True, "bf16"),
    (2, 513, 2, 128, 0, False, "bf16"),
    (2, 40, 3, 16, 0, True, "bf16"),      # generic kernel
    (2, 33, 2, 16, 8, False, "f32"),      # generic kernel, fp32
])
def test_max_logits_shapes(B, T, H, dk, ds, causal, dtype):
    print("max_logits", B, T, H, dk, ds, causal, dtype, flush=True)
    seed = B * 1000 + T * 10 + H
    q = wl.normal(seed, 0, (B, T, H, dk + ds), 2.0)
    k = wl.normal(seed, 1, (B, T, H, dk), 2.0)
    ks = wl.normal(seed, 2, (B, T, ds), 2.0) if ds else None
    qz = wl.quantize_bf16 if dtype == "bf16" else wl.quantize_f32
    q, k = qz(q), qz(k)
    ks = qz(ks) if ds else None
    qd, kd, ksd = qk_to_device(q, k, ks, dtype)
    got = host64(mc.max_logits_per_head(qd, kd, ksd, causal=causal))
    want = oracle.max_logits(q, k, ks, causal, 1.0 / math.sqrt(dk + ds))
    assert np.allclose(got, want, rtol=1e-3, atol=0), (got, want)


def test_max_logits_strided_views_and_nan():
    B, T, H, d = 2, 130, 3, 128
    big = wl.quantize_bf16(wl.normal(5, 0, (B, T, H + 1, 2 * d), 1.0))
    q = big[:, :, :H, :d]
    k = big[:, :, 1:, d:]
    qd_full = dev_tensor(big, "bf16")
    qd, kd = qd_full[:, :, :H, :d], qd_full[:, :, 1:, d:]
    got = host64(mc.max_logits_per_head(qd, kd, None, causal=True))
    want = oracle.max_logits(q, k, None, True, 1.0 / math.sqrt(d))
    assert np.allclose(got, want, rtol=1e-3)
    # one NaN key element: that key's logits are NaN and ignored
    k2 = np.array(k)
    k2[0, 5, 1, 3] = np.nan
    kd2 = dev_tensor(k2, "bf16")
    qd2 = dev_tensor(np.ascontiguousarray(q), "bf16")
    got2 = host64(mc.max_logits_per_head(qd2, kd2, None, causal=True))
    want2 = oracle.max_logits(q, k2, None, True, 1.0 / math.sqrt(d))
    assert np.allclose(got2, want2, rtol=1e-3)


def test_max_logits_huge_key_stride():
    """A key view whose t stride (2^23 elements) exceeds the MFMA kernels'
    32-bit tile offsets runs the generic kernel and still matches the
    oracle."""
    B, T, H, d = 1, 3, 2, 128
    rng = np.random.default_rng(77)
    q = wl.quantize_bf16(rng.standard_normal((B, T, H, d)))
    k = wl.quantize_bf16(rng.standard_normal((B, T, H, d)))
    big = torch.zeros(T, 1 << 23, dtype=torch.bfloat16, device="cuda")
    kv = big[:, : H * d].view(T, H, d).unsqueeze(0)          # [1, T, H, d], t stride 2^23
    kv.copy_(dev_tensor(k, "bf16"))
    got = host64(mc.max_logits_per_head(dev_tensor(q, "bf16"), kv, None, causal=True))
    ref = oracle.max_logits(q, k, None, True, 1.0 / math.sqrt(d))
    assert np.allclose(got, ref, rtol=1e-3, atol=0)


def test_max_logits_empty_gives_neg_inf_and_gamma_one():
    q = torch.zeros(0, 4, 2, 128, dtype=torch.bfloat16, device="cuda")
    out = mc.max_logits_per_head(q, q, None, causal=True)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(out))


@pytest.mark.parametrize("dk,ds,dtype", [(128, 0, "bf16"), (128, 64, "bf16"), (64, 0, "bf16"), (16, 0, "f32")])
def test_max_logits_negative_and_zero(dk, ds, dtype):
    """Per-head maxima that are negative (every query u, every key -u: all
    logits -|u|^2 scale) or zero (zero queries: all logits 0, the result +0,
    not -0 or -inf), next to a head with a positive maximum, through every
    kernel family; checked against the oracle."""
    B, T, H = 2, 150, 3
    print("negative/zero S_max", dk, ds, dtype, flush=True)
    rng = np.random.default_rng(dk + ds)
    d = dk + ds
    q = rng.standard_normal((B, T, H, d))
    k = rng.standard_normal((B, T, H, dk))
    ks = rng.standard_normal((B, T, ds)) if ds else None
    u = rng.standard_normal(d)
    q[:, :, 0] = u                       # head 0: all logits -|u|^2
    k[:, :, 0] = -u[:dk]
    if ds:
        ks[:] = 0.0                      # (the shared rotary key adds nothing)
        q[:, :, 0, dk:] = 0.0
    q[:, :, 1] = 0.0                     # head 1: all logits 0
    q = wl.quantize_bf16(q) if dtype == "bf16" else wl.quantize_f32(q)
    k = wl.quantize_bf16(k) if dtype == "bf16" else wl.quantize_f32(k)
    ks = (wl.quantize_bf16(ks) if dtype == "bf16" else wl.quantize_f32(ks)) if ds else None
    qd, kd, ksd = qk_to_device(q, k, ks, dtype)
    scale = 1.0 / math.sqrt(d)
    got = host64(mc.max_logits_per_head(qd, kd, ksd, causal=True, scale=scale))
    ref = oracle.max_logits(q, k, ks, True, scale)
    assert got[0] < 0 and np.isclose(got[0], ref[0], rtol=1e-5, atol=0)
    assert got[1] == 0.0 and not np.signbit(got[1])
    assert got[2] > 0 and np.isclose(got[2], ref[2], rtol=1e-3, atol=0)
    if dk == 128 and dtype == "bf16":   # the same merge inside attention_forward
        smax = torch.empty(H, dtype=torch.float32, device="cuda")
        v = torch.zeros(B, T, H, 128, dtype=torch.bfloat16, device="cuda")
        mc.attention_forward(qd, kd, ksd, v, causal=True, s_max=smax)
        torch.cuda.synchronize()
        assert np.array_equal(host64(smax), got)


def test_gamma_out_without_matrices_and_with_two_lanes():
    """gamma_out is written once per step: with no matrices at all, and when
    the step's waves run on two streams (two shape groups)."""
    s = torch.tensor([50.0, 400.0, -3.0, float("nan"), 100.0, 1e6], dtype=torch.float32, device="cuda")
    want = oracle.clip_factor(host64(s), 100.0)
    hp = mc.hparams(tau=100.0)
    g0 = torch.full((6,), -7.0, dtype=torch.float32, device="cuda")
    mc.muonclip_step([], hp, s_max=s, slots=2, heads=3, gamma_out=g0)
    torch.cuda.synchronize()
    assert np.allclose(host64(g0), want, rtol=1e-6, atol=0)
    cfg = wl.config(1)
    states = load_config_states(cfg)                    # 256x512 and two 64x64: two groups
    descs = [st.desc() for st in states]
    s4 = s[:4].contiguous()                             # config 1: one layer of 4 heads
    g1 = torch.full((4,), -7.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(mc.workspace_size(descs, hp), dtype=torch.uint8, device="cuda")
    mc.muonclip_step(descs, hp, s_max=s4, slots=1, heads=4, gamma_out=g1, workspace=ws)
    torch.cuda.synchronize()
    assert np.allclose(host64(g1), want[:4], rtol=1e-6, atol=0)


# ----------------------------------------------------------------- fused update

def _step_weights(states, hp, s_max, heads, with_o, ws_mode="full"):
    descs = [s.desc(with_o=with_o) for s in states]
    ws = torch.empty(mc.workspace_size(descs, hp, minimal=(ws_mode == "min")), dtype=torch.uint8, device="cuda")
    gam = torch.full((s_max.numel(),), -7.0, dtype=torch.float32, device="cuda") if s_max is not None else None
    mc.muonclip_step(descs, hp, s_max=s_max, slots=1 if s_max is not None else 0, heads=heads,
                     gamma_out=gam, workspace=ws)
    torch.cuda.synchronize()
    return [s.w.cpu().clone() for s in states], (gam.cpu() if gam is not None else None)


def _fresh(states):
    for s in states:
        s.w.copy_(dev_tensor(s.w0, s.spec.w_dtype))
        s.g.copy_(dev_tensor(s.g0, "f32"))
        s.m.copy_(dev_tensor(s.m0, "f32"))


@pytest.mark.parametrize("case", ["mha_layer", "ragged_tall_wide", "many_clipped", "global_clip", "many_tiles"])
def test_update_fused_into_last_apply_is_bit_identical(case):
    """Without an O output the update runs in the last Newton-Schulz apply's
    epilogue. It must give bit for bit the weights and gamma of the separate
    update kernel (which the oracle parity tests check, since they request
    O): the MHA layer's four 2048^2 matrices with clipped W_q, W_k (apply
    tiles of eight waves); a tall and a wide matrix of one ragged shape group
    with padded rows, clipped; eleven clipped matrices (past the fused path's
    clip table: the update kernel runs); the global-gamma variant; seventeen
    2048x1024 / 1024x2048 matrices, a tall and a wide one clipped, whose 544
    apply tiles run the four-wave kernel."""
    print("fused update case", case, flush=True)
    rng = np.random.default_rng(sum(map(ord, case)))
    heads = 4
    kw = {}
    if case == "mha_layer":
        cfg = wl.config(2)
        states = load_config_states(cfg)
        heads = cfg.attn.H
    else:
        if case == "ragged_tall_wide":
            shapes = [(200, 136), (136, 200)]
        elif case == "many_clipped":
            shapes = [(96, 64)] * 11
        elif case == "many_tiles":
            shapes = [(2048, 1024)] * 4 + [(1024, 2048)] * 9 + [(2048, 1024)] * 4
        else:
            shapes = [(128, 256), (256, 128)]
            kw = dict(clip_global=1)
        states = []
        for idx, (r, c) in enumerate(shapes):
            period = r // heads
            clipped = case != "many_tiles" or idx in (0, 4)   # a tall and a wide one
            spec = wl.MatrixSpec("m", r, c, clip_slot=0 if clipped else -1, period=period,
                                 segments=((0, period // 2, 0.5), (period // 2, 8, 1.0)))
            w = (rng.standard_normal((r, c)) * 0.02).astype(np.float32)
            g = (rng.standard_normal((r, c)) * 1e-3).astype(np.float32)
            m = (rng.standard_normal((r, c)) * 1e-3).astype(np.float32)
            states.append(State(spec, w, g, m, ld_pad=8))
    s_max = torch.tensor(rng.uniform(20.0, 400.0, heads), dtype=torch.float32, device="cuda")
    hp = hp_for(wl.config(2), **kw)
    # (the smallest workspace runs one matrix per wave, with other tiles and
    # split-K, so each workspace size is compared with itself)
    for ws_mode in ("full", "min"):
        _fresh(states)
        w_sep, g_sep = _step_weights(states, hp, s_max, heads, with_o=True, ws_mode=ws_mode)
        _fresh(states)
        w_fus, g_fus = _step_weights(states, hp, s_max, heads, with_o=False, ws_mode=ws_mode)
        for a, b in zip(w_sep, w_fus):
            assert torch.equal(a, b)
        assert torch.equal(g_sep, g_fus)
    assert torch.all(g_sep <= 1.0) and torch.any(g_sep < 1.0)
    # and the padding past each row stayed untouched
    for s in states:
        assert torch.all(s.w_full[:, s.spec.cols:].cpu() == 0)


# ----------------------------------------------------------------- S_max on another stream

def _smax_then_step(states, hp, attn, heads, slots, overlapped, with_o):
    """S_max of `attn` then one step; with `overlapped` the S_max pass runs on
    a second stream and only the launches that read it wait (the event)."""
    q, k, ks, causal = attn
    _fresh(states)
    descs = [s.desc(with_o=with_o) for s in states]
    ws = torch.empty(max(mc.workspace_size(descs, hp), 256), dtype=torch.uint8, device="cuda")
    s_max = torch.full((slots * heads,), -5.0, dtype=torch.float32, device="cuda")
    gam = torch.full((slots * heads,), -7.0, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    if overlapped:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for sl in range(slots):
                mc.max_logits_per_head(q, k, ks, causal=causal, out=s_max[sl * heads:(sl + 1) * heads])
            ready = torch.cuda.Event()
            ready.record(side)
        mc.muonclip_step(descs, hp, s_max=s_max, slots=slots, heads=heads, gamma_out=gam, workspace=ws,
                         s_max_ready=ready)
        torch.cuda.current_stream().wait_stream(side)
    else:
        for sl in range(slots):
            mc.max_logits_per_head(q, k, ks, causal=causal, out=s_max[sl * heads:(sl + 1) * heads])
        mc.muonclip_step(descs, hp, s_max=s_max, slots=slots, heads=heads, gamma_out=gam, workspace=ws)
    torch.cuda.synchronize()
    return ([(s.w.cpu().clone(), s.m.cpu().clone()) for s in states], gam.cpu(), s_max.cpu())


@pytest.mark.parametrize("case", ["mha_layer", "two_lanes_with_o"])
def test_step_overlapped_with_smax_pass_is_bit_identical(case):
    """muonclip_step_overlapped with S_max computed on a second stream gives
    bit for bit the weights, momenta, gamma and S_max of S_max followed by
    muonclip_step on one stream: the MHA layer (update inside the last apply,
    one lane) and the tiny layer's two shape groups on two lanes with O
    requested (separate update kernel)."""
    print("overlapped step case", case, flush=True)
    cfg = wl.config(2 if case == "mha_layer" else 1)
    states = load_config_states(cfg)
    q, k, ks = wl.draw_attention_inputs(cfg, weights_of(cfg))
    if case == "mha_layer":
        qd, kd, ksd = qk_to_device(q, k, ks, "bf16")
    else:
        qd, kd, ksd = qk_to_device(q, k, ks, "f32")
    attn = (qd, kd, ksd, cfg.attn.causal)
    hp = hp_for(cfg, lr=0.02)
    with_o = case != "mha_layer"
    base = _smax_then_step(states, hp, attn, cfg.attn.H, 1, False, with_o)
    over = _smax_then_step(states, hp, attn, cfg.attn.H, 1, True, with_o)
    for (w0, m0), (w1, m1) in zip(base[0], over[0]):
        assert torch.equal(w0, w1) and torch.equal(m0, m1)
    assert torch.equal(base[1], over[1]) and torch.equal(base[2], over[2])
    assert torch.all(base[1] <= 1.0) and torch.all(base[1] > 0.0)


def test_step_overlapped_without_matrices_writes_gamma():
    """With no matrices the overlapped step still writes gamma from the
    S_max the event guards."""
    s = torch.tensor([50.0, 400.0, -3.0, 100.0], dtype=torch.float32, device="cuda")
    want = oracle.clip_factor(host64(s), 100.0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    s2 = torch.empty_like(s)
    with torch.cuda.stream(side):
        s2.copy_(s)
        ready = torch.cuda.Event()
        ready.record(side)
    g = torch.full((4,), -7.0, dtype=torch.float32, device="cuda")
    mc.muonclip_step([], mc.hparams(tau=100.0), s_max=s2, slots=1, heads=4, gamma_out=g, s_max_ready=ready)
    torch.cuda.synchronize()
    assert np.allclose(host64(g), want, rtol=1e-6, atol=0)


def test_qk_clip_apply_batches_mixed_layouts():
    """One qk_clip_apply call over eleven matrices: bf16 and fp32, row widths
    that are and are not whole 16-byte vectors, padded row strides, MHA and
    MLA segment layouts (more than one batched launch). Every clipped row is
    the drawn row times gamma_h^expo rounded once (fp32 factor), every other
    row is bit-identical (essay, gamma equation and MHA / MLA rules)."""
    heads, tau = 6, 10.0
    s_in = np.array([40.0, 5.0, 12.5, np.inf, 10.0, 80.0], np.float32)
    g_orc = oracle.clip_factor(s_in.astype(np.float64), tau)
    s_max = torch.from_numpy(s_in).cuda()
    cases = []   # (rows, cols, ld_pad, dtype, period, segments)
    for k in range(11):
        dt = "bf16" if k % 2 == 0 else "f32"
        cols = [64, 37, 96, 130, 8, 512][k % 6]
        ld_pad = [0, 3, 8, 0, 1, 4][k % 6]
        if k % 3 == 0:
            period, segs = 16, ((0, 16, 0.5),)
        elif k % 3 == 1:
            period, segs = 12, ((0, 8, 0.5), (8, 4, 1.0))
        else:
            period, segs = 10, ((2, 5, 0.5),)
        cases.append((heads * period, cols, ld_pad, dt, period, segs))
    mats, keep = [], []
    for k, (rows, cols, ld_pad, dt, period, segs) in enumerate(cases):
        w = wl.normal(60 + k, 0, (rows, cols), 1.0)
        w = wl.quantize_bf16(w) if dt == "bf16" else wl.quantize_f32(w)
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        full = torch.zeros(rows, cols + ld_pad, dtype=tdt, device="cuda")
        full[:, :cols] = torch.from_numpy(w).to(tdt).cuda()
        z = torch.zeros(rows, cols + ld_pad, dtype=torch.float32, device="cuda")[:, :cols]
        view = full[:, :cols]
        mats.append(mc.matrix(view, z, z, clip_slot=0, period=period, segments=segs))
        keep.append((w, full, view, dt, period, segs))
    gamma = torch.empty(heads, dtype=torch.float32, device="cuda")
    mc.qk_clip_apply(mats, s_max, 1, heads, tau, gamma_out=gamma)
    torch.cuda.synchronize()
    assert np.allclose(host64(gamma), g_orc, rtol=1e-6, atol=0)
    for w, full, view, dt, period, segs in keep:
        got = host64(view)
        want = oracle.qk_clip_rows(w.astype(np.float64), g_orc, period, segs)
        # fp32 factor and product, then one rounding to the dtype (fp32: the
        # factor's and the product's roundings, up to two ulps of the result)
        ulps = 1.001 if dt == "bf16" else 2.001
        tol = ulps * (2.0 ** (np.frexp(np.abs(want))[1] - (8 if dt == "bf16" else 24))) + 1e-30
        assert np.all(np.abs(got - want) <= tol), (dt, view.shape, period)
        untouched = np.isclose(want, w, rtol=0, atol=0)
        assert np.array_equal(got[untouched], w.astype(np.float64)[untouched])
        if full.shape[1] > view.shape[1]:   # the padding is never written
            assert not bool(full[:, view.shape[1]:].any())
