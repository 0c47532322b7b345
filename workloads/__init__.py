"""Seeded synthetic Q/K/V shaped like video-DiT self-attention.

This module only makes inputs. It holds none of the attention arithmetic, so both the HIP
path and the CPU oracle may consume what it produces.

Recipe (the pages' workloads are video diffusion models whose weights and prompts are not
available, so these inputs stand in for them; LiteAttention, page 1 "Core Concept": the
model attends over flattened spatio-temporal tiles and the sparsity pattern is stable
across denoising steps):

* tokens sit on an (F, Hh, Ww) latent grid, raster order f, h, w, optionally preceded by a
  text-like prefix;
* per head, 64 random Fourier features of the normalised coordinate
  x = (f/(F-1), h/(Hh-1), w/(Ww-1)):  phi_k(x) = sqrt(2) cos(omega_k . x + beta_k),
  omega_k ~ N(0, bw^2 I_3), beta_k ~ U[0, 2 pi).  The same phi serves Q and K of a head, so
  q . k is large for nearby tokens (a Gaussian kernel of bandwidth bw) and small far away;
* Q0 = a phi + b N(0,1),  K0 = a phi + b N(0,1) (independent noise), phi filling dims 0..63;
  V ~ N(0,1), fixed across steps;
* step t: Q_t = Q0 + sigma_t eps_t, K_t = K0 + sigma_t eps'_t with fresh noise every step
  (not a random walk), emulating the slow drift of attention between denoising steps;
* prefix tokens (when present) have isotropic Q0, K0 ~ N(0,1) and get the same perturbation.

Seeding: every random draw comes from its own generator seeded by
(20251114, config id, batch, head, tensor id, step), so any single head can be regenerated
alone. Small per-head parameters (omega, beta, bandwidth) are drawn on the CPU so they are
identical on every device; the large noise tensors are drawn on the device that holds the
workload (torch's CPU and GPU generators give different streams for the same seed, so a
comparison always takes both sides' inputs from the same device's draw).
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import List, Optional, Sequence, Tuple

import torch

__all__ = [
    "WorkloadConfig",
    "CONFIGS",
    "get_config",
    "Workload",
    "derive",
]

_ROOT_SEED = 20251114
_T_OMEGA, _T_Q0, _T_K0, _T_V, _T_QPERT, _T_KPERT, _T_HEADS = range(7)
_RFF_FEATURES = 64


@dataclasses.dataclass(frozen=True)
class HeadRecipe:
    """Q/K recipe of one head: RFF weight a, noise weight b, bandwidth bw."""

    a: float
    b: float
    bw: float


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    """One synthetic attention workload and its denoising schedule."""

    name: str
    cid: int
    batch: int
    heads: int
    head_dim: int
    grid: Tuple[int, int, int]
    prefix: int
    dtype: torch.dtype
    tile_q: int
    tile_k: int
    steps: int
    sigmas: Tuple[float, ...]          # per-step perturbation std
    log_eps: Tuple[float, ...]         # per-step error budget (natural log)
    head_recipes: Tuple[HeadRecipe, ...]  # per head (shared by all batch items)
    softmax_scale: float = 1.0
    order: str = "alt"
    dense_prefix: int = 0
    description: str = ""

    @property
    def seq_len(self) -> int:
        f, h, w = self.grid
        return self.prefix + f * h * w

    @property
    def tiles_q(self) -> int:
        return -(-self.seq_len // self.tile_q)

    @property
    def tiles_k(self) -> int:
        return -(-self.seq_len // self.tile_k)

    def dense_flops(self) -> float:
        """Dense-equivalent flops of one step: 4 B H N^2 D (QK^T and PV, no causal halving)."""
        n = self.seq_len
        return 4.0 * self.batch * self.heads * n * n * self.head_dim


def _linear(a: float, b: float, n: int) -> Tuple[float, ...]:
    if n == 1:
        return (a,)
    return tuple(a + (b - a) * t / (n - 1) for t in range(n))


def _seed(*parts: int) -> int:
    h = hashlib.sha256(repr((_ROOT_SEED,) + tuple(int(p) for p in parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _cpu_gen(*parts: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(_seed(*parts))
    return g


def _dev_gen(device: torch.device, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _config3_bandwidths(heads: int) -> Tuple[float, ...]:
    g = _cpu_gen(3, 0, 0, _T_HEADS, 0)
    u = torch.rand(heads, generator=g, dtype=torch.float64)
    return tuple(float(2.0 + 8.0 * x) for x in u)


def _build_configs() -> dict:
    lin10_sigma = _linear(0.1, 0.01, 10)
    lin10_eps = _linear(-14.0, -8.0, 10)
    cfgs = [
        WorkloadConfig(
            name="tiny_ref", cid=1, batch=1, heads=2, head_dim=64, grid=(4, 16, 16), prefix=0,
            dtype=torch.float32, tile_q=64, tile_k=64, steps=4,
            sigmas=tuple(0.05 * math.sqrt(4 - t) for t in range(4)),
            log_eps=(-math.inf, -12.0, -10.0, -9.0),
            head_recipes=(HeadRecipe(0.8, 0.6, 4.0),) * 2,
            description="1x2 heads, D=64, 4x16x16 grid = 1024 tokens, fp32, 64x64 tiles, 4 steps",
        ),
        WorkloadConfig(
            name="wan2.1_1.3b", cid=2, batch=1, heads=12, head_dim=128, grid=(21, 30, 52),
            prefix=0, dtype=torch.bfloat16, tile_q=128, tile_k=64, steps=10,
            sigmas=lin10_sigma, log_eps=lin10_eps,
            head_recipes=(HeadRecipe(0.8, 0.6, 6.0),) * 12,
            description="Wan2.1-1.3B-shaped: 1x12 heads, D=128, 21x30x52 = 32760 tokens, bf16",
        ),
        WorkloadConfig(
            name="wan14b_720p", cid=3, batch=1, heads=40, head_dim=128, grid=(21, 45, 80),
            prefix=0, dtype=torch.bfloat16, tile_q=128, tile_k=64, steps=10,
            sigmas=lin10_sigma, log_eps=lin10_eps,
            head_recipes=tuple(HeadRecipe(0.8, 0.6, bw) for bw in _config3_bandwidths(40)),
            description="Wan-14B-shaped 720p: 1x40 heads, D=128, 21x45x80 = 75600 tokens, bf16, "
                        "per-head bandwidth U[2,10]",
        ),
        WorkloadConfig(
            name="hunyuan_720p", cid=4, batch=1, heads=24, head_dim=128, grid=(33, 45, 80),
            prefix=256, dtype=torch.bfloat16, tile_q=128, tile_k=64, steps=10,
            sigmas=lin10_sigma, log_eps=lin10_eps,
            head_recipes=(HeadRecipe(0.8, 0.6, 6.0),) * 24, dense_prefix=256,
            description="HunyuanVideo-shaped 720p: 1x24 heads, D=128, 256 prefix + 33x45x80 = "
                        "119056 tokens, bf16, dense prefix",
        ),
        WorkloadConfig(
            name="stress_edge", cid=5, batch=2, heads=16, head_dim=64, grid=(17, 32, 32),
            prefix=0, dtype=torch.bfloat16, tile_q=128, tile_k=64, steps=20,
            sigmas=_linear(0.1, 0.01, 20), log_eps=(-10.0,) * 20,
            head_recipes=(HeadRecipe(0.1, 0.6, 6.0),) * 8 + (HeadRecipe(1.5, 0.6, 12.0),) * 8,
            description="stress: 2x16 heads, D=64, 17x32x32 = 17408 tokens, bf16; heads 0-7 "
                        "near-uniform, heads 8-15 sharply local; 20 steps at log_eps=-10",
        ),
    ]
    return {c.name: c for c in cfgs}


CONFIGS = _build_configs()
_BY_ID = {c.cid: c for c in CONFIGS.values()}


def get_config(key) -> WorkloadConfig:
    """Look a config up by name or by its 1-based id."""
    if isinstance(key, int) or (isinstance(key, str) and key.isdigit()):
        return _BY_ID[int(key)]
    return CONFIGS[key]


def derive(cfg: WorkloadConfig, *, name: Optional[str] = None, batch: Optional[int] = None,
           heads: Optional[Sequence[int]] = None, grid: Optional[Tuple[int, int, int]] = None,
           prefix: Optional[int] = None, steps: Optional[int] = None,
           dense_prefix: Optional[int] = None, **kw) -> WorkloadConfig:
    """A smaller or altered workload with the same recipe (for tests at sizes the oracle
    finishes in seconds). `heads` picks which of the config's head recipes to keep."""
    recipes = cfg.head_recipes if heads is None else tuple(cfg.head_recipes[h] for h in heads)
    st = cfg.steps if steps is None else steps
    sig = cfg.sigmas[:st] if steps is not None and steps <= cfg.steps else cfg.sigmas
    eps = cfg.log_eps[:st] if steps is not None and steps <= cfg.steps else cfg.log_eps
    out = dataclasses.replace(
        cfg,
        name=name or (cfg.name + "_derived"),
        batch=cfg.batch if batch is None else batch,
        heads=len(recipes), head_recipes=recipes,
        grid=cfg.grid if grid is None else tuple(grid),
        prefix=cfg.prefix if prefix is None else prefix,
        steps=st, sigmas=tuple(sig), log_eps=tuple(eps),
        dense_prefix=cfg.dense_prefix if dense_prefix is None else dense_prefix,
        **kw,
    )
    return out


def _coords(grid: Tuple[int, int, int]) -> torch.Tensor:
    f, h, w = grid
    axes = []
    for n in (f, h, w):
        axes.append(torch.arange(n, dtype=torch.float64) / (n - 1) if n > 1
                    else torch.zeros(n, dtype=torch.float64))
    ff, hh, ww = torch.meshgrid(*axes, indexing="ij")
    return torch.stack([ff.reshape(-1), hh.reshape(-1), ww.reshape(-1)], dim=1)  # [F*H*W, 3]


class Workload:
    """Materialises a config's inputs on one device.

    base(b, h)        -> (q0, k0, v) float32 [N, D] for one head
    inputs(t)         -> (q_t, k_t, v) in the config dtype, [B, H, N, D] contiguous
    head_inputs(t,b,h)-> (q_t, k_t, v) float32 [N, D] for one head (same values as inputs(t))
    """

    def __init__(self, cfg: WorkloadConfig, device="cpu"):
        self.cfg = cfg
        self.device = torch.device(device)
        self._coords = None
        self._base_cache = {}

    # -- per-head pieces ------------------------------------------------------------------
    def _phi(self, b: int, h: int) -> torch.Tensor:
        cfg = self.cfg
        rec = cfg.head_recipes[h]
        g = _cpu_gen(cfg.cid, b, h, _T_OMEGA, 0)
        omega = torch.randn(_RFF_FEATURES, 3, generator=g, dtype=torch.float64) * rec.bw
        beta = torch.rand(_RFF_FEATURES, generator=g, dtype=torch.float64) * (2.0 * math.pi)
        if self._coords is None:
            self._coords = _coords(cfg.grid).to(self.device, torch.float32)
        arg = self._coords @ omega.T.to(self.device, torch.float32) + beta.to(self.device, torch.float32)
        return math.sqrt(2.0) * torch.cos(arg)  # [F*H*W, 64]

    def base(self, b: int, h: int):
        key = (b, h)
        if key in self._base_cache:
            return self._base_cache[key]
        cfg = self.cfg
        n, d, p = cfg.seq_len, cfg.head_dim, cfg.prefix
        rec = cfg.head_recipes[h]
        dev = self.device
        q0 = torch.randn(n, d, generator=_dev_gen(dev, cfg.cid, b, h, _T_Q0, 0), device=dev)
        k0 = torch.randn(n, d, generator=_dev_gen(dev, cfg.cid, b, h, _T_K0, 0), device=dev)
        v = torch.randn(n, d, generator=_dev_gen(dev, cfg.cid, b, h, _T_V, 0), device=dev)
        # video tokens: a * phi + b * noise (phi fills the first 64 dims)
        phi = self._phi(b, h)
        f = min(_RFF_FEATURES, d)
        q0[p:] *= rec.b
        k0[p:] *= rec.b
        q0[p:, :f] += rec.a * phi[:, :f]
        k0[p:, :f] += rec.a * phi[:, :f]
        # prefix tokens stay isotropic N(0,1)
        self._base_cache[key] = (q0, k0, v)
        return q0, k0, v

    def head_inputs(self, t: int, b: int, h: int):
        cfg = self.cfg
        q0, k0, v = self.base(b, h)
        sig = cfg.sigmas[t]
        dev = self.device
        eq = torch.randn(q0.shape, generator=_dev_gen(dev, cfg.cid, b, h, _T_QPERT, t), device=dev)
        ek = torch.randn(k0.shape, generator=_dev_gen(dev, cfg.cid, b, h, _T_KPERT, t), device=dev)
        return q0 + sig * eq, k0 + sig * ek, v

    # -- whole tensors --------------------------------------------------------------------
    def inputs(self, t: int, dtype: Optional[torch.dtype] = None, cache_base: bool = True):
        cfg = self.cfg
        dt = cfg.dtype if dtype is None else dtype
        shape = (cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim)
        q = torch.empty(shape, dtype=dt, device=self.device)
        k = torch.empty(shape, dtype=dt, device=self.device)
        v = torch.empty(shape, dtype=dt, device=self.device)
        for b in range(cfg.batch):
            for h in range(cfg.heads):
                qt, kt, vt = self.head_inputs(t, b, h)
                q[b, h].copy_(qt)
                k[b, h].copy_(kt)
                v[b, h].copy_(vt)
                if not cache_base:
                    self._base_cache.pop((b, h), None)
        return q, k, v

    def drop_cache(self):
        self._base_cache.clear()
