"""Shared GPU-test plumbing: upload seeded workloads, run the library, and
compute the matching oracle values on the host. The oracle only ever sees
values drawn by the workloads package (never anything the HIP path wrote)."""
from __future__ import annotations

import math

import numpy as np
import torch

import muonclip_step_amd as mc
import oracle
import workloads as wl

DEV = "cuda"


def dev_tensor(x: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(DEV)


def host64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class State:
    """One matrix's host inputs and device buffers."""

    def __init__(self, spec, w, g, m, g_dtype="f32", ld_pad=0):
        self.spec = spec
        self.w0, self.g0, self.m0 = w, g, m
        rows, cols = w.shape
        ld = cols + ld_pad
        wdt = torch.bfloat16 if spec.w_dtype == "bf16" else torch.float32
        gdt = torch.bfloat16 if g_dtype == "bf16" else torch.float32
        self.w_full = torch.zeros(rows, ld, dtype=wdt, device=DEV)
        self.g_full = torch.zeros(rows, ld, dtype=gdt, device=DEV)
        self.m_full = torch.zeros(rows, ld, dtype=torch.float32, device=DEV)
        self.w = self.w_full[:, :cols]
        self.g = self.g_full[:, :cols]
        self.m = self.m_full[:, :cols]
        self.w.copy_(dev_tensor(w, spec.w_dtype))
        self.g.copy_(dev_tensor(g, g_dtype))
        self.m.copy_(dev_tensor(m, "f32"))
        self.o = torch.empty(rows, cols, dtype=torch.bfloat16, device=DEV)

    def desc(self, with_o=True):
        s = self.spec
        return mc.matrix(self.w, self.g, self.m, o_out=self.o if with_o else None, clip_slot=s.clip_slot,
                         period=s.period, segments=s.segments)


def load_config_states(cfg, indices=None, cold=False):
    idx = range(len(cfg.matrices)) if indices is None else indices
    out = []
    for i in idx:
        out.append(State(cfg.matrices[i], wl.draw_weight(cfg, i), wl.draw_grad(cfg, i),
                         wl.draw_momentum(cfg, i, cold=cold)))
    return out


def hp_for(cfg, **kw):
    h = dict(cfg.hparams)
    h["tau"] = cfg.tau
    h.update(kw)
    return mc.hparams(**h)


def oracle_step(state: State, hp, gamma=None):
    """fp64 oracle of one matrix's step from the drawn inputs; gamma is the
    oracle's own per-head factor vector for the matrix's clip slot."""
    s = state.spec
    g64 = state.g0.astype(np.float64)
    return oracle.muonclip_step_matrix(
        state.w0.astype(np.float64), g64, state.m0.astype(np.float64),
        lr=oracle.f32(hp.lr), mu=oracle.f32(hp.mu), weight_decay=oracle.f32(hp.weight_decay),
        rms_scale=oracle.f32(hp.rms_scale), ns_steps=hp.ns_steps, ns_a=oracle.f32(hp.ns_a),
        ns_b=oracle.f32(hp.ns_b), ns_c=oracle.f32(hp.ns_c), ns_eps=oracle.f32(hp.ns_eps),
        gamma=gamma if s.clip_slot >= 0 else None, period=s.period, segments=s.segments,
        w_dtype=s.w_dtype, nesterov=bool(getattr(hp, "nesterov", 0)))


def rel_fro(a, b) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the param dtype grid at |x| (normal range)."""
    bits = 8 if dtype == "bf16" else 24
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e - bits, -126 - bits + 1))


def clip_scales(spec, gamma_oracle=None, gamma_gpu=None):
    """Per-row clip factor gamma_h^expo of the oracle (rows x 1) and the
    relative difference of the GPU's factor from it."""
    rows = spec.rows
    sc = np.ones((rows, 1))
    sc_rel = np.zeros((rows, 1))
    if gamma_oracle is not None and spec.clip_slot >= 0:
        for h, gh in enumerate(gamma_oracle):
            for off, ln, ex in spec.segments:
                r0 = h * spec.period + off
                sc[r0:r0 + ln] = gh ** ex
                if gamma_gpu is not None and gh > 0:
                    sc_rel[r0:r0 + ln] = abs((gamma_gpu[h] / gh) ** ex - 1.0)
    return sc, sc_rel


def w_bound(spec, hp, w_prev, w_o, w_g, o_g, o_o, gamma_oracle=None, gamma_gpu=None, carried=None):
    """Elementwise bound on |W_gpu - W_oracle| after one step whose previous
    weights differed by at most `carried` (None: identical inputs).

    The oracle rounds once from fp64 (half an ulp of the param dtype). The
    kernel computes t = w*decay, f = fma(-lr*rms, o, t), f*s in fp32 with
    decay, lr*rms and s themselves rounded to fp32, which adds at most
    s*(ulp(t) + ulp(lr*rms*o) + ulp(f)) + ulp(w') in fp32 ulps of those
    intermediates (they can be far larger than w' when the update cancels w).
    On top come the NS difference (lr*rms*|dO|, times the clip factor), for
    clipped rows the relative difference of the GPU's and the oracle's
    gamma^expo, and the carried difference times decay and the clip factor."""
    rows, cols = spec.rows, spec.cols
    lr_rms = oracle.f32(hp.lr) * oracle.f32(hp.rms_scale) * math.sqrt(max(rows, cols))
    lr_wd = oracle.f32(hp.lr) * oracle.f32(hp.weight_decay)
    decay = 1.0 - lr_wd
    sc, sc_rel = clip_scales(spec, gamma_oracle, gamma_gpu)
    c = 0.0 if carried is None else carried
    t = np.abs(w_prev * decay) + c
    u = lr_rms * np.abs(o_o)
    f = np.abs(w_prev * decay - lr_rms * o_o) + c
    fp32_part = sc * (ulp(t, "f32") + ulp(u, "f32") + ulp(f, "f32")) + ulp(w_o, "f32")
    # each side rounds its own value to the dtype: half an ulp at each
    w_big = np.maximum(np.abs(w_o), np.abs(w_g))
    return (1.001 * ulp(w_big, spec.w_dtype) + fp32_part + lr_rms * np.abs(o_g - o_o) * sc
            + np.abs(w_o) * sc_rel * 1.01 + sc * decay * c + 1e-30)


def assert_within(w_g, w_o, bound, what="W", extra=None):
    excess = np.abs(w_g - w_o) - bound
    if (excess > 0).any():
        i = np.unravel_index(np.argmax(excess), excess.shape)
        more = "" if extra is None else " " + " ".join(f"{k} {v[i]!r}" for k, v in extra.items())
        raise AssertionError(f"{what}: {(excess > 0).sum()} elements beyond bound; worst at {i}: gpu {w_g[i]!r} "
                             f"oracle {w_o[i]!r} bound {bound[i]!r}{more}")


def check_matrix(state: State, hp, gamma_oracle=None, ns_tol=2e-2, gamma_gpu=None):
    """Compare one matrix after the GPU step against the oracle (momentum
    within 1 fp32 ulp, O within ns_tol relative Frobenius, W within
    w_bound). Returns the NS relative Frobenius error."""
    w_o, m_o, o_o = oracle_step(state, hp, gamma_oracle)
    # momentum: one rounding of mu*M + G -> within 1 fp32 ulp
    m_g = host64(state.m)
    assert np.all(np.abs(m_g - m_o) <= ulp(m_o, "f32") + 1e-45), "momentum"
    # Newton-Schulz output
    o_g = host64(state.o)
    err = rel_fro(o_g, o_o)
    assert err <= ns_tol, f"NS rel Frobenius {err:.3e} > {ns_tol}"
    w_g = host64(state.w)
    w0 = state.w0.astype(np.float64)
    bound = w_bound(state.spec, hp, w0, w_o, w_g, o_g, o_o, gamma_oracle, gamma_gpu)
    assert_within(w_g, w_o, bound, "W", {"w0": w0, "o_gpu": o_g, "o_orc": o_o})
    return err


def qk_to_device(q, k, ks, dtype):
    qd = dev_tensor(q, dtype)
    kd = dev_tensor(k, dtype)
    ksd = dev_tensor(ks, dtype) if ks is not None else None
    return qd, kd, ksd
