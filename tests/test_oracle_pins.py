"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

None of these re-types the oracle's own formula: each checks it against a
different route to the same number (an SVD closed form, a brute-force loop, a
scalar recurrence, an identity the pages state, or a library routine).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import muonclip_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def phi_n(x, n, a=O.NS_A, b=O.NS_B, c=O.NS_C):
    """phi(x) = a x + b x^3 + c x^5 composed n times (scalar route)."""
    for _ in range(n):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def closed_form_ns(m, steps=5, eps=1e-7):
    """U phi^N(S / (||M||_F + eps)) V^T from numpy's SVD (Notes on Muon blog,
    "Newton-Schulz": N steps of the iteration act on singular values only)."""
    u, s, vt = np.linalg.svd(m, full_matrices=False)
    sn = s / (np.linalg.norm(m) + eps)
    return (u * phi_n(sn, steps)) @ vt


@pytest.mark.parametrize("shape", [(16, 64), (64, 16), (64, 64), (8, 8), (48, 200), (200, 48), (1, 7), (7, 1)])
def test_ns_matches_svd_closed_form(shape):
    rng = np.random.default_rng(11)
    m = rng.standard_normal(shape)
    got = oracle.newton_schulz(m)
    want = closed_form_ns(m)
    assert np.linalg.norm(got - want) <= 1e-12 * max(1.0, np.linalg.norm(want))


def test_ns_rank_one_value():
    # rank-1 M = u v^T has one normalised singular value ~1 -> phi^5(1) u^ v^T
    rng = np.random.default_rng(3)
    u, v = rng.standard_normal(37), rng.standard_normal(53)
    m = np.outer(u, v)
    got = oracle.newton_schulz(m)
    s1 = np.linalg.norm(m) / (np.linalg.norm(m) + 1e-7)
    want = phi_n(s1, 5) * np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    assert np.allclose(got, want, atol=1e-12)
    # the value printed in the band table below: phi^5(1) = 0.69643...
    assert abs(phi_n(1.0, 5) - 0.6964364) < 1e-6


def test_ns_zero_matrix_gives_zero():
    got = oracle.newton_schulz(np.zeros((5, 9)))
    assert np.all(got == 0.0)


def test_ns_scale_and_transpose_invariance():
    # Ortho(cM) = Ortho(M) (Notes on Muon blog, rescaling); the transpose rule
    # of newtonschulz5 makes NS(M^T) = NS(M)^T exactly in exact arithmetic.
    rng = np.random.default_rng(5)
    m = rng.standard_normal((24, 40))
    o = oracle.newton_schulz(m)
    assert np.allclose(oracle.newton_schulz(m * 1e3), o, atol=1e-9)
    assert np.allclose(oracle.newton_schulz(m.T), o.T, atol=1e-12)


def test_ns_singular_values_in_band():
    # the band phi^5 reaches on [0.002, 1] (brute force on a fine grid) holds
    # every normalised singular value of a well-conditioned Gaussian matrix
    xs = np.linspace(0.002, 1.0, 200001)
    ys = phi_n(xs, 5)
    lo, hi = ys.min(), ys.max()
    assert 0.68 < lo < 0.69 and 1.20 < hi < 1.21
    rng = np.random.default_rng(9)
    for shape in [(32, 128), (128, 32), (50, 300)]:
        m = rng.standard_normal(shape)
        s = np.linalg.svd(oracle.newton_schulz(m), compute_uv=False)
        assert s.min() >= lo - 1e-9 and s.max() <= hi + 1e-9


def test_ns_coefficient_sign():
    # with b = -4.7750 phi(1) lies in the [0.7, 1.3] target band of "Coefficient
    # Optimization"; with the +4.7750 printed in the Moonlight notes it is 10.25
    assert O.NS_B < 0
    assert 0.7 <= phi_n(1.0, 1) <= 1.3
    assert phi_n(1.0, 1, b=+4.7750) > 10.0
    assert (O.NS_A, O.NS_C, O.NS_STEPS, O.NS_EPS) == (3.4445, 2.0315, 5, 1e-7)


def test_rms_lemma():
    # Notes on Moonlight, "Scaling up Muon": RMS(U V^T) = sqrt(r/(AB)); for a
    # full-rank [A, B] matrix 0.2*sqrt(max(A,B))*UV^T has RMS exactly 0.2
    rng = np.random.default_rng(2)
    for A, B in [(30, 70), (70, 30), (40, 40)]:
        u, _, vt = np.linalg.svd(rng.standard_normal((A, B)), full_matrices=False)
        upd = oracle.rms_matched(u @ vt, A, B, 0.2)
        assert abs(np.sqrt(np.mean(upd ** 2)) - 0.2) < 1e-12
        # with the NS approximation the RMS sits in 0.2 x the phi^5 band
        o = oracle.newton_schulz(rng.standard_normal((A, B)))
        r = np.sqrt(np.mean(oracle.rms_matched(o, A, B) ** 2))
        assert 0.2 * 0.68 < r < 0.2 * 1.21


def test_decay_only_special_case():
    # G = 0 and M = 0 -> O = 0 -> W' = (1 - lr*lambda) W
    rng = np.random.default_rng(4)
    w = rng.standard_normal((12, 20)).astype(np.float32).astype(np.float64)
    z = np.zeros_like(w)
    w_new, m_new, o = oracle.muonclip_step_matrix(w, z, z, lr=0.01, mu=0.95, weight_decay=0.1,
                                                  w_dtype="f32")
    assert np.all(o == 0) and np.all(m_new == 0)
    assert np.array_equal(w_new, (w * (1 - 0.01 * 0.1)).astype(np.float32).astype(np.float64))


def test_momentum_cold_start_and_closed_form():
    rng = np.random.default_rng(6)
    g1, g2 = rng.standard_normal((3, 4)), rng.standard_normal((3, 4))
    m1 = oracle.momentum(np.zeros((3, 4)), g1, 0.9)      # M_0 = 0
    assert np.array_equal(m1, g1)
    m2 = oracle.momentum(m1, g2, 0.9)
    assert np.allclose(m2, 0.9 * g1 + g2, rtol=0, atol=0)


def test_update_step_order_against_hand_expansion():
    # one full step on a tiny matrix, against the update written out by hand
    # from the Moonlight rule with the closed-form NS
    rng = np.random.default_rng(8)
    w = rng.standard_normal((6, 10))
    g = rng.standard_normal((6, 10))
    m = rng.standard_normal((6, 10))
    lr, mu, wd = 0.05, 0.9, 0.1
    w_new, m_new, o = oracle.muonclip_step_matrix(w, g, m, lr=lr, mu=mu, weight_decay=wd, w_dtype="f64")
    mm = mu * m + g
    upd = 0.2 * math.sqrt(10) * closed_form_ns(mm)
    want = w - lr * upd - lr * wd * w
    assert np.allclose(w_new, want, rtol=0, atol=1e-12)


def _clip_by_hand(w, gamma, period, segments):
    """Row-block rescale written out row by row: row r of head h = r // period
    at offset r % period inside a segment (off, len, expo) is multiplied by
    gamma_h ** expo (essay, MHA sqrt(gamma) equations and the MLA table)."""
    out = np.array(w, np.float64, copy=True)
    for r in range(out.shape[0]):
        h, o = divmod(r, period)
        for off, ln, ex in segments:
            if off <= o < off + ln:
                out[r, :] = out[r, :] * gamma[h] ** ex
    return out


@pytest.mark.parametrize("segments,period", [(((0, 4, 0.5),), 4), (((0, 3, 0.5), (3, 2, 1.0)), 6)])
def test_clip_runs_after_the_update(segments, period):
    # The clip rescales the weights once the optimizer update is done (essay,
    # section on why neither a logit soft-cap nor QK-Norm is used; K2 report,
    # "Taming Muon with QK-Clip": the rescale is post-update). Expected value:
    # the Moonlight update with the closed-form NS, then the row rescale by
    # hand. A plausible mistake, clipping W before the update (so that the
    # update term escapes the clip), must not pass the same check.
    rng = np.random.default_rng(31)
    heads = 3
    rows, cols = heads * period, 11
    w = rng.standard_normal((rows, cols))
    g = rng.standard_normal((rows, cols))
    m = rng.standard_normal((rows, cols))
    lr, mu, wd = 0.05, 0.9, 0.1
    gamma = np.array([0.3, 1.0, 0.05])
    kw = dict(lr=lr, mu=mu, weight_decay=wd, w_dtype="f64", period=period, segments=segments)
    w_clip, m_clip, o_clip = oracle.muonclip_step_matrix(w, g, m, gamma=gamma, **kw)
    w_free, m_free, o_free = oracle.muonclip_step_matrix(w, g, m, gamma=None, **kw)
    # the clip touches neither the momentum nor the orthogonalised update
    assert np.array_equal(m_clip, m_free) and np.array_equal(o_clip, o_free)
    upd = 0.2 * math.sqrt(max(rows, cols)) * closed_form_ns(mu * m + g)
    want = _clip_by_hand(w - lr * upd - lr * wd * w, gamma, period, segments)
    assert np.allclose(w_clip, want, rtol=0, atol=1e-12)
    # composition: the clipped step is the clip of the unclipped step
    assert np.array_equal(w_clip, oracle.qk_clip_rows(w_free, gamma, period, segments))
    # planted wrong order: clip first, then the update
    w_pre = _clip_by_hand(w, gamma, period, segments)
    wrong = w_pre - lr * upd - lr * wd * w_pre
    assert not np.allclose(wrong, want, rtol=0, atol=1e-6)
    assert np.abs(wrong - w_clip).max() > 1e-3
    # heads with gamma = 1 and rows outside every segment are the same either way
    assert np.array_equal(w_clip[period:2 * period], w_free[period:2 * period])


# ---------------------------------------------------------------- S_max

def _tiny_qk(rng, B, T, H, dk, ds):
    q = rng.standard_normal((B, T, H, dk + ds))
    k = rng.standard_normal((B, T, H, dk))
    ks = rng.standard_normal((B, T, ds)) if ds else None
    return q, k, ks


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ds", [0, 3])
def test_max_logits_blocked_equals_bruteforce(causal, ds):
    rng = np.random.default_rng(12 + ds)
    q, k, ks = _tiny_qk(rng, 2, 9, 3, 4, ds)
    a = oracle.max_logits(q, k, ks, causal, 0.5, block=4)
    b = oracle.max_logits_bruteforce(q, k, ks, causal, 0.5)
    assert np.allclose(a, b, rtol=1e-14, atol=1e-14)


def test_max_logits_torch_route():
    # the same quantity computed through torch CPU einsum projections (the
    # route the essay's MHA sample takes): x -> Q, K per head -> QK^T -> amax
    import torch
    g = torch.Generator().manual_seed(1)
    x = torch.randn(2, 7, 6, generator=g, dtype=torch.float64)
    wq = torch.randn(3, 6, 4, generator=g, dtype=torch.float64)
    wk = torch.randn(3, 6, 4, generator=g, dtype=torch.float64)
    qh = torch.einsum("btd,hdf->bthf", x, wq)
    kh = torch.einsum("btd,hdf->bthf", x, wk)
    ref = torch.einsum("bihf,bjhf->bhij", qh, kh).amax(dim=(0, 2, 3)) / 2.0
    got = oracle.max_logits(qh.numpy(), kh.numpy(), None, False, 0.5)
    assert np.allclose(got, ref.numpy(), rtol=1e-14)


def test_max_logits_ignores_nan_and_empty():
    q = np.ones((1, 2, 1, 2))
    k = np.ones((1, 2, 1, 2))
    k[0, 1, 0, 0] = np.nan
    got = oracle.max_logits(q, k, None, False, 1.0)
    assert got[0] == 2.0
    empty = oracle.max_logits(np.zeros((0, 3, 2, 4)), np.zeros((0, 3, 2, 4)), None, True, 1.0)
    assert np.all(np.isneginf(empty))


# ---------------------------------------------------------------- gamma / clip

def test_gamma_policy_special_cases():
    s = np.array([-3.0, 0.0, np.nan, 50.0, 100.0, 200.0, np.inf])
    g = oracle.clip_factor(s, 100.0)
    assert list(g[:5]) == [1.0, 1.0, 1.0, 1.0, 1.0]
    assert g[5] == 0.5 and g[6] == 0.0
    assert np.all(g <= 1.0)


def test_essay_worked_example_invariants():
    # the essay's MHA sample: seeded x, W_q, W_k (scaled by 8), tau = 10;
    # after the per-head sqrt(gamma) rescale the max logit equals before*gamma
    # and does not exceed tau; gamma <= 1.
    import torch
    spec = json.load(open(os.path.join(GOLDEN, "essay_mha_example.json")))
    torch.manual_seed(spec["seed"])
    x = torch.randn(*spec["x_shape"])
    wq = torch.randn(*spec["w_shape"]) * spec["w_scale"]
    wk = torch.randn(*spec["w_shape"]) * spec["w_scale"]
    tau = spec["tau"]
    x64, wq64, wk64 = (t.double().numpy() for t in (x, wq, wk))
    H, dm, dh = wq64.shape

    def smax(wqm, wkm):
        q = np.einsum("btd,hdf->bthf", x64, wqm)
        k = np.einsum("btd,hdf->bthf", x64, wkm)
        return oracle.max_logits(q, k, None, False, 1.0 / math.sqrt(dh))

    before = smax(wq64, wk64)
    gamma = oracle.clip_factor(before, tau)
    # as projection matrices [H*dh, dm]: row h*dh+f = W[h, :, f]
    def as_rows(w):
        return w.transpose(0, 2, 1).reshape(H * dh, dm)

    def from_rows(m):
        return m.reshape(H, dh, dm).transpose(0, 2, 1)
    seg = [(0, dh, 0.5)]
    wq2 = from_rows(oracle.qk_clip_rows(as_rows(wq64), gamma, dh, seg))
    wk2 = from_rows(oracle.qk_clip_rows(as_rows(wk64), gamma, dh, seg))
    after = smax(wq2, wk2)
    assert np.allclose(after, before * gamma, rtol=1e-12)
    assert np.all(after <= tau * (1 + spec["rel_slack"]))
    assert np.all(gamma <= 1.0)
    assert np.any(gamma < 1.0)


def test_mla_clip_identity_and_shared_rope_untouched():
    # tiny MLA: per-head q rows [q^C | q^R], kv_b rows [k^C | v], shared k^R.
    # After clipping with the MLA exponents every head's max logit becomes
    # before*gamma (content sqrt*sqrt, rope gamma*1), k^R rows are unchanged.
    rng = np.random.default_rng(21)
    H, dc, dr, dv, dm, lq, lkv, B, T = 3, 4, 2, 4, 10, 6, 5, 2, 8
    q_a = rng.standard_normal((lq, dm))
    q_b = rng.standard_normal((H * (dc + dr), lq))
    q_b[: dc + dr] *= 8.0  # head 0 hot
    kv_a = rng.standard_normal((lkv + dr, dm))
    kv_b = rng.standard_normal((H * (dc + dv), lkv))
    kv_b[: dc + dv] *= 8.0
    x = rng.standard_normal((B, T, dm))

    def smax(q_b_, kv_a_, kv_b_):
        q = (x @ q_a.T) @ q_b_.T
        q = q.reshape(B, T, H, dc + dr)
        ckv = x @ kv_a_[:lkv].T
        kr = x @ kv_a_[lkv:].T
        kc = (ckv @ kv_b_.reshape(H, dc + dv, lkv)[:, :dc].reshape(H * dc, lkv).T).reshape(B, T, H, dc)
        return oracle.max_logits(q, kc, kr, True, 1.0 / math.sqrt(dc + dr))

    before = smax(q_b, kv_a, kv_b)
    tau = float(np.sort(before)[-1]) / 3.0
    gamma = oracle.clip_factor(before, tau)
    assert gamma[0] < 1.0
    q_b2 = oracle.qk_clip_rows(q_b, gamma, dc + dr, [(0, dc, 0.5), (dc, dr, 1.0)])
    kv_b2 = oracle.qk_clip_rows(kv_b, gamma, dc + dv, [(0, dc, 0.5)])
    after = smax(q_b2, kv_a, kv_b2)
    assert np.allclose(after, before * gamma, rtol=1e-12)
    assert np.all(after <= tau * (1 + 1e-12))
    # untouched: v rows of kv_b and all of kv_a (holds k^R)
    for h in range(H):
        r0 = h * (dc + dv)
        assert np.array_equal(kv_b2[r0 + dc: r0 + dc + dv], kv_b[r0 + dc: r0 + dc + dv])
    # heads with gamma == 1 are bit-identical
    for h in np.nonzero(gamma == 1.0)[0]:
        r0 = h * (dc + dr)
        assert np.array_equal(q_b2[r0:r0 + dc + dr], q_b[r0:r0 + dc + dr])


def test_wrong_exponent_breaks_the_identity():
    # the identity above is a real pin: swapping the rope exponent to 1/2 fails it
    rng = np.random.default_rng(22)
    H, dc, dr = 2, 3, 2
    q = rng.standard_normal((1, 6, H, dc + dr)) * 5
    kc = rng.standard_normal((1, 6, H, dc)) * 5
    kr = rng.standard_normal((1, 6, dr)) * 5
    before = oracle.max_logits(q, kc, kr, False, 1.0)
    gamma = np.array([0.25, 0.5])
    q_ok = q.copy()
    q_bad = q.copy()
    for h in range(H):
        q_ok[..., h, :dc] *= math.sqrt(gamma[h]); q_ok[..., h, dc:] *= gamma[h]
        q_bad[..., h, :dc] *= math.sqrt(gamma[h]); q_bad[..., h, dc:] *= math.sqrt(gamma[h])
    kc_ok = kc * np.sqrt(gamma)[None, None, :, None]
    assert np.allclose(oracle.max_logits(q_ok, kc_ok, kr, False, 1.0), before * gamma)
    assert not np.allclose(oracle.max_logits(q_bad, kc_ok, kr, False, 1.0), before * gamma)


# ---------------------------------------------------------------- rounding

def test_round_to_bf16_against_torch_and_ties():
    import torch
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
    # ties to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert oracle.round_to_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert oracle.round_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    # a single rounding from fp64: just above the tie goes up
    assert oracle.round_to_bf16(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == 1 + 2 ** -7
    assert np.isinf(oracle.round_to_bf16(np.array([3.5e38]))[0])


def test_ns_flops_formula():
    # Notes on Muon blog, "Analysis": 2(2nm^2 + m^3) per step, m <= n
    assert oracle.ns_flops(2048, 7168, 1) == 2 * (2 * 7168 * 2048 ** 2 + 2048 ** 3)
    assert oracle.ns_flops(7168, 2048, 5) == oracle.ns_flops(2048, 7168, 5)


# ---------------------------------------------------------------- variants

def test_nesterov_direction_is_the_lookahead_of_plain_momentum():
    # Nesterov momentum in Sutskever's look-ahead form: the direction at step t
    # is M_t + mu (M_t - M_{t-1}) of the plain buffer sequence; built here from
    # two plain momentum steps, never from the oracle's direction formula
    rng = np.random.default_rng(21)
    mu = 0.95
    g1, g2 = rng.standard_normal((2, 6, 9))
    m0 = rng.standard_normal((6, 9))
    m1 = oracle.momentum(m0, g1, mu)
    m2 = oracle.momentum(m1, g2, mu)
    lookahead = m2 + mu * (m2 - m1)
    assert np.allclose(oracle.nesterov_direction(m2, g2, mu), lookahead, rtol=0, atol=1e-12)
    # mu = 0: no momentum at all, the direction is the gradient
    assert np.array_equal(oracle.nesterov_direction(oracle.momentum(m0, g1, 0.0), g1, 0.0), g1)


def test_nesterov_cold_start_orthogonalises_the_gradient():
    # M_0 = 0: the look-ahead is (1 + mu) G, and Newton-Schulz is scale
    # invariant up to eps, so the update equals a plain step on G alone
    rng = np.random.default_rng(22)
    w = rng.standard_normal((12, 20))
    g = rng.standard_normal((12, 20))
    kw = dict(lr=0.01, mu=0.9, weight_decay=0.1, w_dtype="f64")
    _, _, o_nest = oracle.muonclip_step_matrix(w, g, np.zeros_like(g), nesterov=True, **kw)
    want = closed_form_ns(g * 1.9)
    assert np.linalg.norm(o_nest - want) <= 1e-12 * np.linalg.norm(want)
    # and with a warm buffer the two variants differ
    m = rng.standard_normal((12, 20))
    _, _, o_plain = oracle.muonclip_step_matrix(w, g, m, nesterov=False, **kw)
    _, _, o_n2 = oracle.muonclip_step_matrix(w, g, m, nesterov=True, **kw)
    assert np.linalg.norm(o_plain - o_n2) > 1e-3


@pytest.mark.parametrize("alpha", [0.5, 0.3])
def test_global_clip_scales_every_logit_by_gamma(alpha):
    # the naive variant (K2 report 2.1): W_q by gamma^alpha, W_k by
    # gamma^(1-alpha) on every head; each logit q.k is bilinear in (W_q, W_k),
    # so every head's max logit scales by exactly gamma and the layer max lands
    # on tau. Logits are recomputed here with plain einsum, not the oracle.
    rng = np.random.default_rng(23)
    H, dm, dh, T, tau = 3, 12, 4, 9, 5.0
    x = rng.standard_normal((1, T, dm))
    wq = rng.standard_normal((H * dh, dm)) * 2.0
    wk = rng.standard_normal((H * dh, dm)) * 2.0

    def head_max(wq_, wk_):
        q = np.einsum("btd,od->bto", x, wq_).reshape(1, T, H, dh)
        k = np.einsum("btd,od->bto", x, wk_).reshape(1, T, H, dh)
        lg = np.einsum("bihf,bjhf->hij", q, k) / math.sqrt(dh)
        return lg.reshape(H, -1).max(axis=1)

    before = head_max(wq, wk)
    gam = oracle.clip_factor_global(before, tau)
    assert gam < 1.0 and abs(gam - tau / before.max()) < 1e-15
    g_all = np.full(H, gam)
    wq2 = oracle.qk_clip_rows(wq, g_all, dh, ((0, dh, alpha),))
    wk2 = oracle.qk_clip_rows(wk, g_all, dh, ((0, dh, 1.0 - alpha),))
    after = head_max(wq2, wk2)
    assert np.allclose(after, before * gam, rtol=1e-12)
    assert abs(after.max() - tau) < 1e-9


def test_global_clip_special_cases():
    # one head: the global rule is the per-head rule
    for s in (250.0, 40.0, -3.0, 0.0, math.inf):
        assert oracle.clip_factor_global(np.array([s]), 100.0) == oracle.clip_factor(np.array([s]), 100.0)[0]
    # NaN heads are ignored by the max; all-NaN gives gamma = 1
    assert oracle.clip_factor_global(np.array([np.nan, 400.0, 20.0]), 100.0) == 0.25
    assert oracle.clip_factor_global(np.array([np.nan, np.nan]), 100.0) == 1.0


# ---------------------------------------------------------------- AdamW

def test_adamw_first_step_is_a_sign_step():
    # t = 1 from zero moments: both bias corrections undo (1 - beta), so the
    # step is g / (|g| + eps), i.e. the sign of g up to eps
    rng = np.random.default_rng(31)
    p, g = rng.standard_normal((2, 50))
    z = np.zeros(50)
    kw = dict(lr=0.01, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0, step=1, p_dtype="f64")
    p1, m1, v1 = oracle.adamw_step(p, g, z, z, **kw)
    assert np.allclose(p1, p - 0.01 * g / (np.abs(g) + 1e-8), rtol=0, atol=1e-15)
    assert np.allclose(m1, 0.1 * g, rtol=1e-6) and np.allclose(v1, 0.05 * g * g, rtol=1e-6)


def test_adamw_constant_gradient_closed_form():
    # a constant gradient keeps m_hat = g and v_hat = g^2 exactly at every
    # step (the bias corrections are what make this so), so after t steps
    # without decay p_t = p_0 - t lr g / (|g| + eps); with decay each step
    # also multiplies by (1 - lr lambda): a scalar recurrence, not the oracle
    g = np.array([0.5, -2.0, 3e-3])
    p0 = np.array([1.0, -1.0, 0.25])
    lr, eps, lam = 1e-3, 1e-8, 0.1
    p, m, v = p0.copy(), np.zeros(3), np.zeros(3)
    for t in range(1, 41):
        p, m, v = oracle.adamw_step(p, g, m, v, lr=lr, beta1=0.9, beta2=0.95, eps=eps,
                                    weight_decay=lam, step=t, p_dtype="f64")
        m, v = m.astype(np.float64), v.astype(np.float64)
    want = p0.copy()
    for _ in range(40):
        want = want * (1.0 - lr * lam) - lr * g / (np.abs(g) + eps)
    # m and v pass through fp32 each step: their rounding (2^-24 relative,
    # at most ~2^-22 on m_hat / sqrt(v_hat)) is the only slack, 40 steps of lr
    assert np.allclose(p, want, rtol=0, atol=40 * lr * 2.0 ** -21)
    # a dropped bias correction or decay term is off by far more
    assert abs(want[0] - (p0[0] - 40 * lr * g[0] / (abs(g[0]) + eps))) > 1e-3


def test_adamw_decay_only_and_rounding():
    # zero gradient and zero moments: only the decoupled decay acts, and the
    # bf16 result is one round-to-nearest-even of p (1 - lr lambda)
    p = oracle.round_to_bf16(np.linspace(-3.0, 3.0, 101))
    z = np.zeros_like(p)
    p1, _, _ = oracle.adamw_step(p, z, z, z, lr=0.01, beta1=0.9, beta2=0.95, eps=1e-8,
                                 weight_decay=0.1, step=3, p_dtype="bf16")
    import torch
    want = torch.tensor(p * (1.0 - 0.001), dtype=torch.float64).to(torch.bfloat16).double().numpy()
    assert np.array_equal(p1, want)


# ---------------------------------------------------------------- attention forward

def _tiny_qkv(rng, B, T, H, dk, ds, dv):
    q, k, ks = _tiny_qk(rng, B, T, H, dk, ds)
    v = rng.standard_normal((B, T, H, dv))
    return q, k, ks, v


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ds", [0, 3])
def test_attention_matches_torch_sdpa(causal, ds):
    # a library route: torch's scaled_dot_product_attention in fp64 on the
    # CPU, fed [B,H,T,d] with the shared key appended to every head's key
    import torch
    rng = np.random.default_rng(40 + ds)
    q, k, ks, v = _tiny_qkv(rng, 2, 11, 3, 4, ds, 5)
    scale = 0.37
    o, lse = oracle.attention_forward(q, k, ks, v, causal, scale)
    kk = k if ks is None else np.concatenate([k, np.repeat(ks[:, :, None, :], 3, axis=2)], axis=3)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(kk).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    assert np.allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)
    # lse through scipy's logsumexp of torch's logits
    from scipy.special import logsumexp
    logits = (torch.einsum("bhid,bhjd->bhij", qt, kt) * scale).numpy()
    if causal:
        logits = np.where(np.tril(np.ones((11, 11), bool)), logits, -np.inf)
    assert np.allclose(lse, logsumexp(logits, axis=3), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_identical_keys_average_the_values(causal):
    # every key equal -> every allowed key gets the same weight: o_i is the
    # mean of v over j <= i (causal) or over all j, and lse_i = scale q_i.k + ln(count)
    rng = np.random.default_rng(7)
    B, T, H, d = 1, 9, 2, 4
    q = rng.standard_normal((B, T, H, d))
    k = np.broadcast_to(rng.standard_normal((1, 1, H, d)), (B, T, H, d)).copy()
    v = rng.standard_normal((B, T, H, 3))
    o, lse = oracle.attention_forward(q, k, None, v, causal, 0.5)
    for i in range(T):
        n = i + 1 if causal else T
        assert np.allclose(o[0, i], v[0, :n].mean(axis=0), rtol=1e-13, atol=1e-13)
        for h in range(H):
            assert math.isclose(lse[0, h, i], 0.5 * float(q[0, i, h] @ k[0, 0, h]) + math.log(n), rel_tol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(8)
    q, k, ks, v = _tiny_qkv(rng, 2, 6, 2, 4, 2, 3)
    # causal row 0 sees key 0 only: o = v_0 and lse = its logit
    o, lse = oracle.attention_forward(q, k, ks, v, True, 0.25)
    assert np.array_equal(o[:, 0], v[:, 0])
    for b in range(2):
        for h in range(2):
            s = float(q[b, 0, h, :4] @ k[b, 0, h] + q[b, 0, h, 4:] @ ks[b, 0])
            assert math.isclose(lse[b, h, 0], 0.25 * s, rel_tol=1e-14)
    # constant values come back unchanged (the weights sum to one)
    vc = np.full_like(v, 2.5)
    oc, _ = oracle.attention_forward(q, k, ks, vc, False, 0.25)
    assert np.allclose(oc, 2.5, rtol=1e-14)
    # one dominant logit selects its value row
    qd = np.zeros((1, 4, 1, 2)); kd = np.zeros((1, 4, 1, 2)); vd = rng.standard_normal((1, 4, 1, 3))
    qd[0, :, 0, 0] = 1.0
    kd[0, 2, 0, 0] = 200.0
    od, _ = oracle.attention_forward(qd, kd, None, vd, False, 1.0)
    assert np.allclose(od[0, :, 0], vd[0, 2, 0], rtol=1e-12, atol=1e-12)
    # selected rows equal the same rows of the full output
    orow, lrow = oracle.attention_forward(q, k, ks, v, True, 0.25, rows=[5, 1])
    assert np.array_equal(orow[:, 0], o[:, 5]) and np.array_equal(orow[:, 1], o[:, 1])
    assert np.array_equal(lrow[:, :, 0], lse[:, :, 5])

