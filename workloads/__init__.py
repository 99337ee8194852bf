"""Seeded synthetic workloads for the MuonClip step.

This package only draws inputs: the configurations' shapes and value
distributions, counter-based random streams, and the quantisation of drawn
values onto the fp32 / bf16 grids. It holds none of the optimizer's
arithmetic, imports neither the oracle nor the HIP binding, and is the one
piece of code both of them are fed from.

Streams: every tensor has its own counter-based Philox stream keyed by
(seed, tensor id), so any single tensor can be re-drawn alone. Large expert
tensors (the MoE configurations) are drawn on the device with torch's Philox
generator, one seed per tensor, because drawing 1.7e10 values on the host is
too slow; their parity samples are copied to the host before the step runs.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

KIND_W, KIND_G, KIND_M, KIND_X, KIND_S, KIND_V = 0, 1, 2, 3, 4, 5

# Hyper-parameters of the step, as the configurations use them.
DEFAULT_HPARAMS = dict(lr=2e-4, mu=0.95, weight_decay=0.1, rms_scale=0.2,
                       ns_a=3.4445, ns_b=-4.7750, ns_c=2.0315, ns_eps=1e-7, ns_steps=5)


def stream(seed: int, tensor_id: int) -> np.random.Generator:
    """Independent counter-based stream for one tensor."""
    return np.random.Generator(np.random.Philox(key=(int(seed) << 64) | int(tensor_id)))


def normal(seed: int, tensor_id: int, shape, std: float = 1.0) -> np.ndarray:
    return std * stream(seed, tensor_id).standard_normal(size=shape)


def quantize_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def quantize_bf16(x) -> np.ndarray:
    """Round to fp32, then to the nearest-even bfloat16; returns float32 values
    that lie on the bf16 grid (finite inputs)."""
    f = np.ascontiguousarray(quantize_f32(x))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def bf16_bits_of(x_bf16_valued_f32: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(np.asarray(x_bf16_valued_f32, np.float32))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# configurations
# ---------------------------------------------------------------------------

@dataclass
class MatrixSpec:
    name: str
    rows: int
    cols: int
    w_dtype: str = "bf16"          # "bf16" or "f32"
    init_std: float = 0.02
    row_boost: tuple = ()          # ((r0, r1, factor), ...) applied before rounding
    grad_std: float = 1e-3
    mom_std: float = 1e-3          # warm momentum; 0 => cold start M_0 = 0
    clip_slot: int = -1
    period: int = 0
    segments: tuple = ()           # ((offset, length, expo), ...)
    device_drawn: bool = False     # drawn on the device (expert / dense FFN tensors)


@dataclass
class AttnSpec:
    kind: str                      # "mha" or "mla"
    B: int
    T: int
    H: int
    d_model: int
    causal: bool
    dtype: str                     # "bf16" or "f32"
    d_q: int
    d_k: int
    d_shared: int

    @property
    def d_v(self) -> int:
        """Value width per head: the head width for MHA, 128 for MLA."""
        return 128 if self.kind == "mla" else self.d_q


@dataclass
class Config:
    idx: int
    name: str
    matrices: list
    tau: float
    attn: AttnSpec | None
    hparams: dict = field(default_factory=lambda: dict(DEFAULT_HPARAMS))

    @property
    def seed(self) -> int:
        return self.idx


def _mha_tiny() -> Config:
    # one fp32 256x512 weight plus W_q, W_k [H=4, d_model=64, d_head=16] drawn
    # N(0,1)*8, laid out as [H*d_head, d_model] projection matrices.
    seg = ((0, 16, 0.5),)
    mats = [MatrixSpec("w0", 256, 512, "f32", 8.0, grad_std=1.0, mom_std=1.0),
            MatrixSpec("wq", 64, 64, "f32", 8.0, grad_std=1.0, mom_std=1.0,
                       clip_slot=0, period=16, segments=seg),
            MatrixSpec("wk", 64, 64, "f32", 8.0, grad_std=1.0, mom_std=1.0,
                       clip_slot=0, period=16, segments=seg)]
    attn = AttnSpec("mha", 2, 64, 4, 64, False, "f32", 16, 16, 0)
    return Config(1, "tiny_mha", mats, 10.0, attn)


def _mha_layer(all_heads: bool = False) -> Config:
    boost = ((0, 2048, 20.0),) if all_heads else ((0, 4 * 128, 20.0),)
    seg = ((0, 128, 0.5),)
    mats = [MatrixSpec("wq", 2048, 2048, row_boost=boost, clip_slot=0, period=128, segments=seg),
            MatrixSpec("wk", 2048, 2048, row_boost=boost, clip_slot=0, period=128, segments=seg),
            MatrixSpec("wv", 2048, 2048),
            MatrixSpec("wo", 2048, 2048)]
    attn = AttnSpec("mha", 4, 4096, 16, 2048, True, "bf16", 128, 128, 0)
    return Config(2, "mha_layer" + ("_all_heads" if all_heads else ""), mats, 100.0, attn)


def _mla_matrices(boost_heads: int = 4, factor: float = 30.0):
    H = 64
    qb_boost = ((0, boost_heads * 192, factor),)
    kvb_boost = ((0, boost_heads * 256, factor),)
    return [MatrixSpec("q_a", 1536, 7168),
            MatrixSpec("q_b", H * 192, 1536, row_boost=qb_boost, clip_slot=0, period=192,
                       segments=((0, 128, 0.5), (128, 64, 1.0))),
            MatrixSpec("kv_a", 512 + 64, 7168),
            MatrixSpec("kv_b", H * 256, 512, row_boost=kvb_boost, clip_slot=0, period=256,
                       segments=((0, 128, 0.5),)),
            MatrixSpec("o", 7168, H * 128)]


def _mla_layer() -> Config:
    attn = AttnSpec("mla", 2, 4096, 64, 7168, True, "bf16", 192, 128, 64)
    return Config(3, "mla_layer", _mla_matrices(), 100.0, attn)


def _expert_matrices(n_experts: int = 385):
    mats = []
    for e in range(n_experts):
        mats.append(MatrixSpec(f"e{e}.gate", 7168, 2048, device_drawn=True))
        mats.append(MatrixSpec(f"e{e}.up", 7168, 2048, device_drawn=True))
        mats.append(MatrixSpec(f"e{e}.down", 2048, 7168, device_drawn=True))
    return mats


def _moe_experts(n_experts: int = 385) -> Config:
    return Config(4, "moe_experts", _expert_matrices(n_experts), 100.0, None)


def _full_layer(n_experts: int = 385) -> Config:
    mats = _mla_matrices()
    mats += [MatrixSpec("dense.gate", 7168, 18432, device_drawn=True),
             MatrixSpec("dense.up", 7168, 18432, device_drawn=True),
             MatrixSpec("dense.down", 18432, 7168, device_drawn=True)]
    mats += _expert_matrices(n_experts)
    attn = AttnSpec("mla", 1, 32768, 64, 7168, True, "bf16", 192, 128, 64)
    return Config(5, "full_layer", mats, 100.0, attn)


def config(idx: int, **kw) -> Config:
    """Configurations 1..5 of the workload (see the module docstring)."""
    if idx == 1:
        return _mha_tiny()
    if idx == 2:
        return _mha_layer(**kw)
    if idx == 3:
        return _mla_layer()
    if idx == 4:
        return _moe_experts(**kw)
    if idx == 5:
        return _full_layer(**kw)
    raise ValueError(f"no configuration {idx}")


def tensor_id(matrix_index: int, kind: int) -> int:
    return matrix_index * 16 + kind


# ---------------------------------------------------------------------------
# drawing the tensors
# ---------------------------------------------------------------------------

def _boosted(w: np.ndarray, spec: MatrixSpec) -> np.ndarray:
    for r0, r1, f in spec.row_boost:
        w[r0:r1] *= f
    return w


def draw_weight(cfg: Config, i: int) -> np.ndarray:
    """Parameter W of matrix i as float32 values (on the bf16 grid for bf16)."""
    s = cfg.matrices[i]
    if cfg.idx == 1 and s.name in ("wq", "wk"):
        # drawn as [H, d_model, d_head]; projection row h*d_head+f is W[h, :, f]
        a = cfg.attn
        t = normal(cfg.seed, tensor_id(i, KIND_W), (a.H, a.d_model, a.d_q), s.init_std)
        w = np.ascontiguousarray(t.transpose(0, 2, 1).reshape(a.H * a.d_q, a.d_model))
    else:
        w = normal(cfg.seed, tensor_id(i, KIND_W), (s.rows, s.cols), s.init_std)
    w = _boosted(w, s)
    return quantize_bf16(w) if s.w_dtype == "bf16" else quantize_f32(w)


KIND_G_LATER = 6                   # kinds 6..15: gradients of steps 2..11


def draw_grad(cfg: Config, i: int, step: int = 1) -> np.ndarray:
    """Gradient of matrix i at optimizer step `step` (1..11), each step its
    own stream (step 1 is the gradient every configuration starts from)."""
    s = cfg.matrices[i]
    if not 1 <= step <= 11:
        raise ValueError("step must be in 1..11")
    kind = KIND_G if step == 1 else KIND_G_LATER + step - 2
    return quantize_f32(normal(cfg.seed, tensor_id(i, kind), (s.rows, s.cols), s.grad_std))


def draw_momentum(cfg: Config, i: int, cold: bool = False) -> np.ndarray:
    s = cfg.matrices[i]
    if cold or s.mom_std == 0.0:
        return np.zeros((s.rows, s.cols), np.float32)
    return quantize_f32(normal(cfg.seed, tensor_id(i, KIND_M), (s.rows, s.cols), s.mom_std))


def draw_device_tensors(cfg: Config, i: int, device):
    """(W, G, M) of a device-drawn matrix as torch tensors on `device`:
    W bf16 N(0, init_std^2), G and M fp32 N(0, std^2), one torch Philox seed
    per tensor."""
    import torch
    s = cfg.matrices[i]
    out = []
    for kind, std, dt in ((KIND_W, s.init_std, torch.bfloat16),
                          (KIND_G, s.grad_std, torch.float32),
                          (KIND_M, s.mom_std, torch.float32)):
        gen = torch.Generator(device=device)
        gen.manual_seed(cfg.seed * 1_000_003 + tensor_id(i, kind))
        t = torch.randn((s.rows, s.cols), generator=gen, device=device, dtype=torch.float32)
        t.mul_(std)
        out.append(t.to(dt))
    return tuple(out)


def _matmul_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    import torch
    return (torch.from_numpy(np.ascontiguousarray(a, np.float32))
            @ torch.from_numpy(np.ascontiguousarray(b, np.float32))).numpy()


def draw_attention_inputs(cfg: Config, weights: dict):
    """Q, K (and the MLA shared rotary key) of this step's forward, computed
    from seeded activations x and the pre-update weights.

    Returns float32 arrays (on the bf16 grid for bf16 configurations):
    q [B,T,H,d_q], k [B,T,H,d_k], k_shared [B,T,d_s] or None.
    MHA: Q = x W_q^T, K = x W_k^T split into heads. MLA (no RoPE, no norm):
    c_Q = x q_a^T; Q = c_Q q_b^T (per head [q^C | q^R]); c_KV = x kv_a[:512]^T;
    K^C = c_KV kv_b[k^C rows]^T; k^R = x kv_a[512:]^T.
    """
    a = cfg.attn
    xid = tensor_id(len(cfg.matrices), KIND_X)
    x = normal(cfg.seed, xid, (a.B * a.T, a.d_model), 1.0)
    if a.dtype == "f32":
        x = quantize_f32(x).astype(np.float64)
        q = (x @ weights["wq"].astype(np.float64).T).astype(np.float32)
        k = (x @ weights["wk"].astype(np.float64).T).astype(np.float32)
        return (q.reshape(a.B, a.T, a.H, a.d_q), k.reshape(a.B, a.T, a.H, a.d_k), None)
    x = quantize_bf16(x)
    if a.kind == "mha":
        q = quantize_bf16(_matmul_f32(x, weights["wq"].T))
        k = quantize_bf16(_matmul_f32(x, weights["wk"].T))
        return (q.reshape(a.B, a.T, a.H, a.d_q), k.reshape(a.B, a.T, a.H, a.d_k), None)
    # MLA
    H = a.H
    c_q = quantize_bf16(_matmul_f32(x, weights["q_a"].T))
    q = quantize_bf16(_matmul_f32(c_q, weights["q_b"].T)).reshape(a.B, a.T, H, 192)
    kv_a = weights["kv_a"]
    c_kv = quantize_bf16(_matmul_f32(x, kv_a[:512].T))
    k_r = quantize_bf16(_matmul_f32(x, kv_a[512:576].T)).reshape(a.B, a.T, 64)
    kv_b = weights["kv_b"].reshape(H, 256, 512)[:, :128, :].reshape(H * 128, 512)
    k_c = quantize_bf16(_matmul_f32(c_kv, kv_b.T)).reshape(a.B, a.T, H, 128)
    return q, k_c, k_r


def draw_attention_values(cfg: Config, weights: dict) -> np.ndarray:
    """V [B,T,H,d_v] of the same forward (float32 on the bf16 grid for bf16
    configurations). MHA: V = x W_v^T from the same seeded x. MLA: v =
    c_KV kv_b[v rows]^T, the v rows being 128..255 of every head's 256 rows of
    kv_b. The tiny fp32 configuration has no W_v: V ~ N(0, 1) is drawn."""
    a = cfg.attn
    if a.dtype == "f32":
        v = normal(cfg.seed, tensor_id(len(cfg.matrices), KIND_V), (a.B, a.T, a.H, a.d_v), 1.0)
        return quantize_f32(v)
    xid = tensor_id(len(cfg.matrices), KIND_X)
    x = quantize_bf16(normal(cfg.seed, xid, (a.B * a.T, a.d_model), 1.0))
    if a.kind == "mha":
        v = quantize_bf16(_matmul_f32(x, weights["wv"].T))
        return v.reshape(a.B, a.T, a.H, a.d_v)
    H = a.H
    c_kv = quantize_bf16(_matmul_f32(x, weights["kv_a"][:512].T))
    kv_b = weights["kv_b"].reshape(H, 256, 512)[:, 128:, :].reshape(H * 128, 512)
    return quantize_bf16(_matmul_f32(c_kv, kv_b.T)).reshape(a.B, a.T, H, 128)


def draw_attention_case(seed: int, B: int, T: int, H: int, d_k: int, d_s: int, d_v: int,
                        q_std: float = 1.0, k_std: float = 1.0, v_std: float = 1.0):
    """A free-standing attention input on the bf16 grid (float32 arrays):
    q [B,T,H,d_k+d_s], k [B,T,H,d_k], k_shared [B,T,d_s] or None, v [B,T,H,d_v],
    each from its own stream of `seed`."""
    q = quantize_bf16(normal(seed, 1, (B, T, H, d_k + d_s), q_std))
    k = quantize_bf16(normal(seed, 2, (B, T, H, d_k), k_std))
    ks = quantize_bf16(normal(seed, 3, (B, T, d_s), k_std)) if d_s else None
    v = quantize_bf16(normal(seed, 4, (B, T, H, d_v), v_std))
    return q, k, ks, v


def draw_smax(cfg: Config, n_over: int = 4) -> np.ndarray:
    """A per-head max-logit vector standing in for a forward pass (float32):
    heads below n_over lie in (1.1, 4) x tau, the rest in (0.1, 0.95) x tau."""
    a = cfg.attn
    u = stream(cfg.seed, tensor_id(len(cfg.matrices), KIND_S)).uniform(size=a.H)
    s = cfg.tau * (0.1 + 0.85 * u)
    s[:n_over] = cfg.tau * (1.1 + 2.9 * u[:n_over])
    return quantize_f32(s)


def elements(cfg: Config) -> int:
    return sum(m.rows * m.cols for m in cfg.matrices)
