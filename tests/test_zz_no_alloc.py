"""muonclip_step_noalloc (static per-device scratch, no allocation) against
muonclip_step with a caller workspace of the same size, through the C ABI:
two calls in a row, the second on a smaller input, each bit-identical to the
reference (same wave plan, one stream)."""
import numpy as np
import pytest
import torch

import muonclip_step_amd as mc
import workloads as wl
from gpu_harness import State, load_config_states

pytestmark = pytest.mark.gpu


def _ragged_states(n, rows, cols, seed):
    cfg = wl.config(2)
    import dataclasses
    out = []
    for i in range(n):
        spec = dataclasses.replace(cfg.matrices[2], name=f"r{i}", rows=rows, cols=cols, row_boost=())
        w = wl.quantize_bf16(wl.normal(seed, 3 * i, (rows, cols), 0.02))
        g = wl.quantize_f32(wl.normal(seed, 3 * i + 1, (rows, cols), 1e-3))
        m = wl.quantize_f32(wl.normal(seed, 3 * i + 2, (rows, cols), 1e-3))
        out.append(State(spec, w, g, m))
    return out


def _run_pair(make, hp, s_max=None, heads=0):
    ref, new = make(), make()
    gamma_r = torch.full((max(heads, 1),), -1.0, device="cuda")
    gamma_n = torch.full((max(heads, 1),), -2.0, device="cuda")
    ws = torch.empty(mc.NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    kw = dict(s_max=s_max, slots=1 if s_max is not None else 0, heads=heads)
    mc.muonclip_step([s.desc(with_o=False) for s in ref], hp, gamma_out=gamma_r if s_max is not None else None,
                     workspace=ws, **kw)
    mc.muonclip_step_noalloc([s.desc(with_o=False) for s in new], hp,
                             gamma_out=gamma_n if s_max is not None else None, **kw)
    torch.cuda.synchronize()
    del ws
    for a, b in zip(ref, new):
        assert torch.equal(a.w, b.w), a.spec.name
        assert torch.equal(a.m, b.m), a.spec.name
        assert not torch.equal(b.w, torch.from_numpy(b.w0).to(b.w.dtype).cuda()), "step did not run"
    if s_max is not None:
        assert torch.equal(gamma_r, gamma_n)


def test_noalloc_matches_the_workspace_step_on_two_calls():
    cfg = wl.config(2)
    hp = mc.hparams(**{**cfg.hparams, "tau": cfg.tau, "lr": 0.02})
    s_max = torch.from_numpy(wl.draw_smax(cfg, n_over=4)).cuda()
    print("no-alloc: MHA layer, 4 x 2048^2 with QK-Clip", flush=True)
    _run_pair(lambda: load_config_states(cfg), hp, s_max, 16)
    print("no-alloc: smaller input, 3 x 300 x 130 ragged", flush=True)
    _run_pair(lambda: _ragged_states(3, 300, 130, 17), hp)


def test_noalloc_rejects_a_matrix_beyond_the_scratch():
    w = torch.zeros(7168, 18432, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(7168, 18432, dtype=torch.float32, device="cuda")
    with pytest.raises(mc.MuonClipError, match="static scratch"):
        mc.muonclip_step_noalloc([mc.matrix(w, g, g)], mc.hparams())
    torch.cuda.synchronize()
    assert not bool(w.any())
