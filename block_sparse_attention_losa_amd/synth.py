"""Seeded synthetic Q/K/V shaped like the video-DiT attention layers LoSA
accelerates.

This module only draws inputs; it contains none of the method's arithmetic,
and both the HIP path and the fp64 oracle consume exactly the tensors it
produces.  The pages evaluate on real activations of Wan2.1, HunyuanVideo and
CogVideoX (mlsanity.com paper index, "Abstract (arXiv)"; legiblepapers,
FAQ Q8), which are not available; these tensors stand in for them.

Recipe (per configuration, numpy PCG64 streams keyed by
``SeedSequence([seed, purpose, ...])``):

* tokens are the cells of a ``(T, H, W)`` grid flattened t-major, w fastest
  (token = (t*H + h)*W + w), optionally preceded by ``text_tokens`` text
  tokens;
* a video token's normalised position is ``(t/(T-1), h/(H-1), w/(W-1))``;
* ``phi(p)_d = cos(omega_d . p + beta_d)`` for 64 random Fourier features,
  ``omega_d ~ N(0, 4^2 I_3)``, ``beta_d ~ U[0, 2pi)`` (purpose 1, once per
  configuration, shared by Q and K of every head and batch item); when the
  head dim exceeds 64 the features fill dims 0..63 and the rest is zero;
  text tokens have no positional term;
* ``Q = eps_Q + alpha_h * phi``, ``K = eps_K + alpha_h * phi``, ``V = eps_V``
  with independent standard normal noise per (tensor, batch item, head)
  (purposes 2, 3, 4);
* ``alpha_h`` per head (purpose 0): fixed, uniform over {0,...,4}, or
  ``U[0, 4]`` depending on the configuration;
* the float64 values are rounded once, round-to-nearest-even, to bf16 (or
  to fp32 for fp32 configurations).

Later denoising steps perturb the step-3 tensors on the device:
``X_t = bf16(X_3 + 0.05 * eps_t)`` with ``eps_t`` drawn by torch's seeded
device generator (seed derived from ``(seed, 5, t, tensor)``).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

PURPOSE_ALPHA = 0
PURPOSE_RFF = 1
PURPOSE_Q = 2
PURPOSE_K = 3
PURPOSE_V = 4
PURPOSE_STEP = 5

RFF_FEATURES = 64
RFF_FREQ_STD = 4.0
CONSTRUCTION_STEP = 3
PERTURB_STD = 0.05


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    batch: int
    heads: int
    head_dim: int
    grid: tuple  # (T, H, W) video grid
    block: int
    dtype: str  # "bf16" or "fp32"
    alpha: object  # tuple of per-head values, "choice" ({0..4}) or "uniform" (U[0,4])
    text_tokens: int = 0
    taus: tuple = (0.99,)
    seed: int = 1
    later_steps: tuple = ()

    @property
    def seq_len(self) -> int:
        t, h, w = self.grid
        return self.text_tokens + t * h * w

    @property
    def num_blocks(self) -> int:
        return (self.seq_len + self.block - 1) // self.block

    @property
    def tau(self) -> float:
        return 0.99 if 0.99 in self.taus else self.taus[0]


# The five model-shaped workloads.
CONFIGS = {
    1: Config("tiny-ref B1 H2 D64 N1024 (4x16x16) block64 fp32",
              1, 2, 64, (4, 16, 16), 64, "fp32", (3.0, 0.0), seed=1),
    2: Config("Wan2.1-1.3B layer B1 H12 D128 N32760 (21x30x52) block64 bf16",
              1, 12, 128, (21, 30, 52), 64, "bf16", "choice", seed=2,
              later_steps=tuple(range(4, 51))),
    3: Config("Wan2.1-14B layer B1 H40 D128 N32760 (21x30x52) block64 bf16",
              1, 40, 128, (21, 30, 52), 64, "bf16", "uniform", seed=3),
    4: Config("HunyuanVideo-13B layer B1 H24 D128 N118800 (33x45x80) block128 bf16",
              1, 24, 128, (33, 45, 80), 128, "bf16", "uniform", seed=4),
    5: Config("CogVideoX-5B joint layer B2 H48 D64 N17776 (226 text + 13x30x45) block64 bf16",
              2, 48, 64, (13, 30, 45), 64, "bf16", "uniform", text_tokens=226,
              taus=(0.95, 0.99, 0.999, 1.0), seed=5),
}


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(x) for x in key])))


def round_bf16(x) -> np.ndarray:
    """Round float64 values once, to nearest-even, onto the bf16 grid.

    Works on the binary64 encoding: the 52-bit fraction is rounded to bf16's
    7 bits (carries into the exponent are the usual round-up).  Only values
    inside bf16's normal range (or zero) are accepted.  The integer
    arithmetic runs on torch's multithreaded CPU kernels.
    """
    import torch

    bits = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).view(torch.int64)
    out = ((bits >> 45) & 1) + ((1 << 44) - 1)
    out += bits
    out &= -(1 << 45)
    res = out.view(torch.float64)
    mag = res.abs()
    if not bool((mag < 2.0 ** 128).all()) or bool(((mag < 2.0 ** -126) & (mag != 0)).any()):
        raise ValueError("value outside bf16's normal range")
    return res.numpy()


def round_dtype(x, dtype: str) -> np.ndarray:
    """Round float64 values to the configuration's element type; the result
    is float32 holding values exactly representable in that type."""
    if dtype == "bf16":
        return round_bf16(x).astype(np.float32)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def alphas(cfg: Config) -> np.ndarray:
    """Per-head positional strength alpha_h."""
    if isinstance(cfg.alpha, tuple):
        if len(cfg.alpha) != cfg.heads:
            raise ValueError("need one alpha per head")
        return np.asarray(cfg.alpha, dtype=np.float64)
    rng = _rng(cfg.seed, PURPOSE_ALPHA)
    if cfg.alpha == "choice":
        return rng.integers(0, 5, size=cfg.heads).astype(np.float64)
    if cfg.alpha == "uniform":
        return rng.uniform(0.0, 4.0, size=cfg.heads)
    raise ValueError(cfg.alpha)


def positions(cfg: Config) -> np.ndarray:
    """Normalised 3D positions of the video tokens, ``[T*H*W, 3]``."""
    t, h, w = cfg.grid
    tt, hh, ww = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")

    def norm(a, size):
        return a.reshape(-1) / (size - 1) if size > 1 else np.zeros(a.size)

    return np.stack([norm(tt, t), norm(hh, h), norm(ww, w)], axis=1)


def fourier_features(cfg: Config) -> np.ndarray:
    """``phi`` for every token, ``[N, head_dim]`` float64 (text rows zero)."""
    rng = _rng(cfg.seed, PURPOSE_RFF)
    omega = rng.normal(0.0, RFF_FREQ_STD, size=(RFF_FEATURES, 3))
    beta = rng.uniform(0.0, 2.0 * math.pi, size=RFF_FEATURES)
    feats = np.cos(positions(cfg) @ omega.T + beta)
    out = np.zeros((cfg.seq_len, cfg.head_dim))
    m = min(RFF_FEATURES, cfg.head_dim)
    out[cfg.text_tokens:, :m] = feats[:, :m]
    return out


def make_head(cfg: Config, b: int, h: int, phi=None, alpha=None, step: int = CONSTRUCTION_STEP):
    """Q, K, V of one (batch item, head) as float32 ``[N, D]`` arrays whose
    values are exactly representable in ``cfg.dtype``."""
    if phi is None:
        phi = fourier_features(cfg)
    if alpha is None:
        alpha = alphas(cfg)[h]
    n, d = cfg.seq_len, cfg.head_dim
    out = []
    for purpose in (PURPOSE_Q, PURPOSE_K, PURPOSE_V):
        x = _rng(cfg.seed, purpose, b, h, step).standard_normal((n, d))
        if purpose != PURPOSE_V:
            x += alpha * phi
        out.append(round_dtype(x, cfg.dtype))
    return tuple(out)


def make_inputs(cfg: Config, step: int = CONSTRUCTION_STEP):
    """Q, K, V of the whole configuration, float32 ``[B, H, N, D]``."""
    phi = fourier_features(cfg)
    al = alphas(cfg)
    shape = (cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim)
    q, k, v = (np.empty(shape, dtype=np.float32) for _ in range(3))
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            q[b, h], k[b, h], v[b, h] = make_head(cfg, b, h, phi, al[h], step)
    return q, k, v


def step_seed(cfg: Config, step: int, tensor: int) -> int:
    """Seed of torch's device generator for the step-``step`` perturbation
    of tensor ``tensor`` (0 = Q, 1 = K, 2 = V)."""
    ss = np.random.SeedSequence([cfg.seed, PURPOSE_STEP, step, tensor])
    return int(ss.generate_state(2, dtype=np.uint32).view(np.uint64)[0] & ((1 << 63) - 1))


def perturb_on_device(cfg: Config, x3, step: int, tensor: int, out=None):
    """Later-step input ``X_t = round(X_3 + 0.05 * eps_t)`` drawn on the
    tensor's device with torch's seeded generator (float32 arithmetic, one
    rounding to the tensor's dtype)."""
    import torch

    gen = torch.Generator(device=x3.device)
    gen.manual_seed(step_seed(cfg, step, tensor))
    eps = torch.randn(x3.shape, generator=gen, device=x3.device, dtype=torch.float32)
    y = (x3.float() + PERTURB_STD * eps).to(x3.dtype)
    if out is not None:
        out.copy_(y)
        return out
    return y


def small_config(n_grid=(3, 5, 7), text=0, heads=2, batch=1, head_dim=64, block=64,
                 dtype="bf16", alpha=(3.0, 0.0), seed=11, taus=(0.99,)) -> Config:
    """A small configuration for tests (ragged tails, few blocks)."""
    if isinstance(alpha, (list, tuple)):
        alpha = tuple(float(a) for a in alpha)
    return Config(f"test B{batch} H{heads} D{head_dim} grid{n_grid}+{text} block{block} {dtype}",
                  batch, heads, head_dim, tuple(n_grid), block, dtype, alpha,
                  text_tokens=text, taus=tuple(taus), seed=seed)
