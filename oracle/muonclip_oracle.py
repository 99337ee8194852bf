"""Plain fp64 CPU oracle of one MuonClip optimizer step.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The product
path (the HIP library and its Python binding) never touches it, and this module
imports nothing from the product package.

Everything here is written straight from the pages' definitions, in fp64,
with no blocking, fusion or reordering beyond what a definition states
(S_max is evaluated one query block at a time only to bound memory; max is
order independent, so the result is the plain definition).

Sources, by page title and section:
  [K2-essay]  "Kimi K2：1T MoE、MuonClip 与 Agentic 训练系统" — section
              "Muon 为何在规模扩大后撞上 attention logit" (S_max, gamma_h and the
              MHA sqrt(gamma) rescale equations) and section "MLA 为什么要非对称缩放"
              (the MLA component / scale table).
  [K2-report] "Kimi K2: Open Agentic Intelligence" — the MuonClip paragraphs
              (Muon update factor sqrt(max(n,m))*0.2, "Taming Muon with QK-Clip",
              per-head MLA clipping).
  [K2-cn]     "2 预训练" translation, section "2.1 MuonClip:通过权重裁剪实现稳定训练"
              (S_max definition, per-head gamma_h, MLA q^C/k^C/q^R/k^R rule).
  [Moonlight] "Notes on Moonlight" — section "Method / Background" (momentum
              M_t = mu M_{t-1} + G_t with M_0 = 0, Newton-Schulz iteration),
              "Scaling up Muon" (decoupled weight decay, RMS lemma, 0.2*sqrt(max(A,B))).
  [Muon-blog] "Notes on Muon blog" — sections "Newton-Schulz" (quintic
              polynomial phi, U phi^N(S) V^T), "Coefficient Optimization", "Algorithm"
              (newtonschulz5: bf16 copy, Frobenius normalisation with eps=1e-7,
              transpose when rows > cols, 5 steps, (a,b,c) = (3.4445, -4.7750, 2.0315))
              and "Analysis" (2(2nm^2+m^3) FLOPs per step; Nesterov-style momentum).

Readings where the pages are silent or garbled:
  * Algorithm 1's body is absent on every page; the step is assembled from the
    Muon update paragraph, the Moonlight update rule and the QK-Clip equations.
  * The sign of b: the Moonlight notes print +4.7750, the newtonschulz5 listing
    prints -4.7750; with +b phi(1) = 10.25 and the iteration diverges, so b < 0.
  * The oracle normalises by the fp64 norm of the fp64 momentum (not of a bf16
    copy) and runs every step in fp64.
  * gamma_h = 1 when S_max^h is not > 0 (so S<=0 and NaN give 1; +inf gives 0),
    mirroring the guard in the essay's MHA code sample.
  * d in 1/sqrt(d) is the per-head q.k dimension (the essay's code divides by
    q.size(-1)); NaN logits are ignored by the max (IEEE maxNum).
  * Nesterov-style momentum (the Muon blog notes say only that Muon uses it):
    the buffer update is unchanged and the matrix orthogonalised is the
    look-ahead G_t + mu M_t.
  * Global clip ([K2-cn] 2.1, the naive variant): gamma from the largest
    S_max^h of the layer, NaN heads ignored by that max.
  * The attention forward that S_max is observed in ([K2-report] "Taming Muon
    with QK-Clip", [K2-cn] 2.1) is the plain softmax attention the pages
    write down, with the same logits (and MLA shared rotary key) as S_max and
    the causal mask j <= i; no dropout, no bias, no soft-cap.
  * AdamW for the parameters Muon does not cover ([Muon-blog] "Limitation":
    only 2-D parameters; the rest still need AdamW; [Moonlight] "Scaling up
    Muon": Muon and AdamW share the learning rate and weight decay). The pages
    give no AdamW formula: the textbook form with bias correction and the
    same decoupled decay as the Muon update is used; beta1, beta2 and eps are
    arguments.
"""

from __future__ import annotations

import math

import numpy as np

# Newton-Schulz quintic coefficients and step count ([Muon-blog] "Algorithm";
# sign of b per the reading in the module docstring).
NS_A, NS_B, NS_C = 3.4445, -4.7750, 2.0315
NS_STEPS = 5
NS_EPS = 1e-7


def f32(x) -> float:
    """The fp64 value of x after rounding to fp32 (hyper-parameters reach the
    GPU as fp32, so the oracle uses the same values)."""
    return float(np.float32(x))


# ---------------------------------------------------------------------------
# rounding to the parameter dtype
# ---------------------------------------------------------------------------

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values once, to nearest-even, onto the bfloat16 grid.

    bfloat16 keeps 8 significant bits with fp32's exponent range, so the
    spacing for |x| in [2^e, 2^(e+1)) is 2^(e-7), and 2^-133 in the subnormal
    range. x / spacing is exact (power-of-two scale); numpy's round is
    half-to-even. Returns fp64 values that are exactly representable in bf16.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)                  # xf = f * 2^e, f in [0.5, 1)
    spacing = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.round(xf / spacing) * spacing
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    out[~fin] = x[~fin]
    return out


# ---------------------------------------------------------------------------
# the Muon part of the step
# ---------------------------------------------------------------------------

def momentum(m_prev: np.ndarray, g: np.ndarray, mu: float) -> np.ndarray:
    """M_t = mu * M_{t-1} + G_t  ([Moonlight] "Background"; M_0 = 0)."""
    return mu * np.asarray(m_prev, np.float64) + np.asarray(g, np.float64)


def nesterov_direction(m_new: np.ndarray, g: np.ndarray, mu: float) -> np.ndarray:
    """The matrix a Nesterov-style Muon step orthogonalises: the look-ahead
    G_t + mu M_t of the plain buffer M_t = mu M_{t-1} + G_t ([Muon-blog]
    "Analysis": Nesterov-style momentum is used instead of plain SGD momentum)."""
    return np.asarray(g, np.float64) + mu * np.asarray(m_new, np.float64)


def newton_schulz(m: np.ndarray, steps: int = NS_STEPS, a: float = NS_A,
                  b: float = NS_B, c: float = NS_C, eps: float = NS_EPS) -> np.ndarray:
    """Approximate orthogonalisation of a 2-D matrix by the quintic
    Newton-Schulz iteration ([Muon-blog] "Newton-Schulz" and "Algorithm").

    X0 = M / (||M||_F + eps); iterate on the transpose when the matrix has
    more rows than columns so the Gram matrix X X^T is the smaller one; each
    step X <- a X + (b A + c A A) X with A = X X^T; transpose back.
    """
    x = np.asarray(m, np.float64)
    x = x / (np.linalg.norm(x) + eps)
    tall = x.shape[0] > x.shape[1]
    if tall:
        x = x.T
    for _ in range(steps):
        gram = x @ x.T
        poly = b * gram + c * (gram @ gram)
        x = a * x + poly @ x
    return x.T if tall else x


def rms_matched(o: np.ndarray, rows: int, cols: int, rms_scale: float = 0.2) -> np.ndarray:
    """Scale the orthogonalised update by rms_scale * sqrt(max(rows, cols)) so
    its RMS matches an AdamW-style update ([Moonlight] "Scaling up Muon";
    [K2-report] Muon update paragraph)."""
    return rms_scale * math.sqrt(max(rows, cols)) * np.asarray(o, np.float64)


def decoupled_update(w: np.ndarray, u: np.ndarray, lr: float, weight_decay: float) -> np.ndarray:
    """W_t = W_{t-1} - lr * (U_t + lambda * W_{t-1})  ([Moonlight] "Scaling up Muon")."""
    w = np.asarray(w, np.float64)
    return w - lr * (np.asarray(u, np.float64) + weight_decay * w)


# ---------------------------------------------------------------------------
# the QK-Clip part of the step
# ---------------------------------------------------------------------------

def max_logits(q: np.ndarray, k: np.ndarray, k_shared: np.ndarray | None,
               causal: bool, scale: float, block: int = 512) -> np.ndarray:
    """Per-head max attention logit ([K2-essay] S_max^h equation; [K2-cn] 2.1).

    q: [B, T, H, d_q]; k: [B, T, H, d_k]; k_shared: [B, T, d_s] or None with
    d_q == d_k + d_s. The logit of (query i, key j, head h) in sample b is
    q[b,i,h,:d_k].k[b,j,h,:] + q[b,i,h,d_k:].k_shared[b,j,:]. Pairs are all
    (i, j) of one sample (j <= i when causal). Returns scale * max over samples
    and pairs, per head, as fp64 (NaN logits ignored; -inf if no pair).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, T, H, dq = q.shape
    out = np.full(H, -np.inf)
    if B == 0 or T == 0:
        return out * scale
    for h in range(H):
        best = -np.inf
        for b in range(B):
            kk = k[b, :, h, :]
            if k_shared is not None:
                kk = np.concatenate([kk, np.asarray(k_shared[b], np.float64)], axis=1)
            qq = q[b, :, h, :]
            for i0 in range(0, T, block):
                i1 = min(T, i0 + block)
                jmax = i1 if causal else T
                logits = qq[i0:i1] @ kk[:jmax].T
                if causal:
                    ii = np.arange(i0, i1)[:, None]
                    jj = np.arange(jmax)[None, :]
                    logits = np.where(jj <= ii, logits, -np.inf)
                logits = np.where(np.isnan(logits), -np.inf, logits)
                best = max(best, float(logits.max()))
        out[h] = best
    return out * scale


def max_logits_bruteforce(q, k, k_shared, causal: bool, scale: float) -> np.ndarray:
    """The same definition as max_logits as explicit loops (tiny inputs only)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, T, H, dq = q.shape
    dk = k.shape[3]
    out = []
    for h in range(H):
        best = -math.inf
        for b in range(B):
            for i in range(T):
                for j in range(T):
                    if causal and j > i:
                        continue
                    s = 0.0
                    for f in range(dk):
                        s += q[b, i, h, f] * k[b, j, h, f]
                    for f in range(dq - dk):
                        s += q[b, i, h, dk + f] * float(k_shared[b, j, f])
                    if not math.isnan(s) and s > best:
                        best = s
        out.append(best * scale)
    return np.array(out)


def clip_factor(s_max: np.ndarray, tau: float) -> np.ndarray:
    """gamma_h = min(1, tau / S_max^h), and 1 when S_max^h is not positive
    ([K2-essay] gamma_h equation and the guard of its code sample)."""
    s = np.asarray(s_max, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        g = np.where(s > 0, np.minimum(1.0, tau / np.where(s > 0, s, 1.0)), 1.0)
    return g


def clip_factor_global(s_max_layer: np.ndarray, tau: float) -> float:
    """The naive all-head variant ([K2-cn] 2.1): gamma = min(1, tau / S_max)
    with S_max the largest S_max^h of the layer; W_q is then scaled by
    gamma**alpha and W_k by gamma**(1 - alpha) (alpha = 1/2 typically). NaN
    heads are ignored by the max; gamma is 1 when that max is not positive."""
    s = np.asarray(s_max_layer, np.float64)
    s = s[~np.isnan(s)]
    top = float(s.max()) if s.size else float("nan")
    return float(clip_factor(np.array([top]), tau)[0])


def qk_clip_rows(w: np.ndarray, gamma: np.ndarray, period: int, segments) -> np.ndarray:
    """Scale the head-specific row blocks of a projection weight [out, in].

    Head h owns rows [h*period, (h+1)*period); each (offset, length, expo)
    segment of those rows is multiplied by gamma_h ** expo. MHA: one segment,
    expo 1/2 on W_q and W_k ([K2-essay] MHA equations). MLA: q^C and k^C
    segments expo 1/2, q^R expo 1, k^R and v rows in no segment
    ([K2-essay] MLA table; [K2-report], [K2-cn] 2.1).
    """
    w = np.array(w, np.float64, copy=True)
    for h, gh in enumerate(np.asarray(gamma, np.float64)):
        for off, length, expo in segments:
            r0 = h * period + off
            w[r0:r0 + length] *= gh ** expo
    return w


# ---------------------------------------------------------------------------
# one full step for one matrix
# ---------------------------------------------------------------------------

def muonclip_step_matrix(w, g, m, *, lr, mu, weight_decay, rms_scale=0.2,
                         ns_steps=NS_STEPS, ns_a=NS_A, ns_b=NS_B, ns_c=NS_C,
                         ns_eps=NS_EPS, gamma=None, period=0, segments=(),
                         w_dtype="bf16", nesterov=False):
    """One MuonClip update of one 2-D parameter, in the pages' order:
    momentum -> Newton-Schulz -> RMS matching -> decoupled decay/update ->
    post-update QK-Clip of the head row blocks (gamma from this step's
    forward, computed on the pre-update weights). With nesterov the
    orthogonalised matrix is the look-ahead G + mu M_t (nesterov_direction);
    gamma is per head (clip_factor) or one value repeated over the heads
    (clip_factor_global).

    Returns (w_new rounded once to w_dtype as fp64 values, m_new as fp32,
    the fp64 Newton-Schulz output O).
    """
    rows, cols = np.shape(w)
    m_new = momentum(m, g, mu)
    d = nesterov_direction(m_new, g, mu) if nesterov else m_new
    o = newton_schulz(d, ns_steps, ns_a, ns_b, ns_c, ns_eps)
    u = rms_matched(o, rows, cols, rms_scale)
    w_new = decoupled_update(w, u, lr, weight_decay)
    if gamma is not None and segments:
        w_new = qk_clip_rows(w_new, gamma, period, segments)
    if w_dtype == "bf16":
        w_out = round_to_bf16(w_new)
    elif w_dtype == "f32":
        w_out = w_new.astype(np.float32).astype(np.float64)
    else:                                   # "f64": unrounded, for pins
        w_out = w_new
    return w_out, m_new.astype(np.float32), o


# ---------------------------------------------------------------------------
# the attention forward whose logits S_max is taken from
# ---------------------------------------------------------------------------

def attention_forward(q, k, k_shared, v, causal: bool, scale: float, rows=None):
    """Attention output of one layer with its per-row log-sum-exp
    ([K2-report] "Taming Muon with QK-Clip": O^h = softmax(Q^h K^h^T / sqrt(d)) V^h;
    [K2-cn] 2.1, the same equation).

    q [B,T,H,d_q], k [B,T,H,d_k], k_shared [B,T,d_s] or None, v [B,T,H,d_v].
    The logit of (query i, key j, head h) in sample b is the one max_logits
    uses, times scale; keys j > i are left out when causal. `rows` (optional
    list of query indices) restricts the output to those queries, which the
    definition computes independently of each other.
    Returns fp64 (o [B,R,H,d_v], lse [B,H,R]) with R = T or len(rows); lse is
    the natural log of the sum of exp(scaled logit) over the row's keys. A row
    with no key (not reachable: the diagonal is always kept) gives o = NaN.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, H, _ = q.shape
    dv = v.shape[3]
    ridx = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(ridx)
    o = np.zeros((B, R, H, dv))
    lse = np.zeros((B, H, R))
    for b in range(B):
        for h in range(H):
            kk = k[b, :, h, :]
            if k_shared is not None:
                kk = np.concatenate([kk, np.asarray(k_shared[b], np.float64)], axis=1)
            logits = scale * (q[b, ridx, h, :] @ kk.T)              # [R, T]
            if causal:
                logits = np.where(np.arange(T)[None, :] <= ridx[:, None], logits, -np.inf)
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            ssum = e.sum(axis=1, keepdims=True)
            o[b, :, h, :] = (e / ssum) @ v[b, :, h, :]
            lse[b, h, :] = (m + np.log(ssum))[:, 0]
    return o, lse


# ---------------------------------------------------------------------------
# AdamW for the non-matrix parameters
# ---------------------------------------------------------------------------

def adamw_step(p, g, m, v, *, lr, beta1, beta2, eps, weight_decay, step, p_dtype="bf16"):
    """One AdamW update of a parameter vector (reading in the module
    docstring): m <- b1 m + (1 - b1) g; v <- b2 v + (1 - b2) g^2;
    p <- p - lr (m / (1 - b1^t) / (sqrt(v / (1 - b2^t)) + eps) + lambda p).
    Returns (p_new rounded once to p_dtype as fp64 values, m_new and v_new as
    fp32 values)."""
    p = np.asarray(p, np.float64)
    g = np.asarray(g, np.float64)
    m_new = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v_new = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    p_new = p - lr * (m_hat / (np.sqrt(v_hat) + eps) + weight_decay * p)
    if p_dtype == "bf16":
        p_out = round_to_bf16(p_new)
    elif p_dtype == "f32":
        p_out = p_new.astype(np.float32).astype(np.float64)
    else:
        p_out = p_new
    return p_out, m_new.astype(np.float32), v_new.astype(np.float32)


def ns_flops(rows: int, cols: int, steps: int = NS_STEPS) -> float:
    """Algorithmic Newton-Schulz FLOPs: 2(2 n m^2 + m^3) per step with
    m = min, n = max ([Muon-blog] "Analysis")."""
    m, n = min(rows, cols), max(rows, cols)
    return float(steps) * 2.0 * (2.0 * n * m * m + m ** 3)
