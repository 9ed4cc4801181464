"""Seeded synthetic inputs for block-sparse video attention.

This module only draws and shapes input tensors. It holds none of the
attention method's arithmetic (no scores, softmax, masks or lists): both the
HIP path and the fp64 oracle consume the exact bytes it produces.

Workloads stand in for the video-DiT layers the pages measure (Wan2.1-1.3B
480p and Wan2.1-14B 720p layers on the VMoBA and Pyramid Sparse Attention
pages, HunyuanVideo at 4x length on the Radial Attention page), whose weights
and prompts are not available. Values follow the structure the pages report
for real attention maps (the LiteAttention page, section 七, and the
PAROAttention page, section 一: diagonal, multi-diagonal and local patterns):

* Z ~ N(0, 1) per tensor, per (batch, head), from a PCG64 stream keyed on
  (seed, tensor, batch, head);
* a smooth per-token component shared by Q and K and by every head,
  c(t, y, x)_k = A sin(2 pi (ft_k t / T + fy_k y / Hs + fx_k x / Ws) + phi_k),
  A = 1, integer frequencies in {0, 1, 2}, phases uniform in [0, 2 pi);
* Q = Z_q + c, K = Z_k + c, then (for the video-sized workloads) a 3D rotary
  position encoding over (t, y, x); V = Z_v;
* bf16 workloads are rounded fp64 -> fp32 -> bf16, round-to-nearest-even at
  each step.

Tokens are flattened t-major: i = (t * Hs + y) * Ws + x.
Layout of every tensor: [B][N][H][d], head_dim contiguous.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "make_qkv", "make_step_qk",
    "step_sigma", "f32_to_bf16_bits", "bf16_bits_to_f32",
]

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2
_SMOOTH_STREAM = 7
_THREADS = max(1, min(16, os.cpu_count() or 1))


@dataclass(frozen=True)
class Workload:
    """Shape and knobs of one synthetic attention call."""
    name: str
    B: int
    H: int
    d: int
    T: int
    Hs: int
    Ws: int
    Bq: int
    Bk: int
    dtype: str            # "bf16" or "f32"
    mask: str             # "radial", "pooled", "skip", "ones"
    seed: int
    rope: bool
    h0: int = 0           # radial window half-width at frame distance 0 (tokens)
    beta: int = 2         # radial decay base
    pooled_mode: int = 1  # 0 = top-k, 1 = cumulative mass
    pooled_param: float = 0.0
    tau: float = 0.0      # skip threshold, natural-log units of scaled scores
    steps: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return self.T * self.Hs * self.Ws

    @property
    def F(self) -> int:
        return self.Hs * self.Ws

    @property
    def nQ(self) -> int:
        return -(-self.N // self.Bq)

    @property
    def nK(self) -> int:
        return -(-self.N // self.Bk)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads. The pooled threshold for the 480p layer was set by
# bisection on the oracle for ~85% tile sparsity on seed 1002
# (tests/golden/tune_pooled_threshold.py writes tests/golden/pooled_tau.json).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, 4, 8, 8, 64, 64, "f32", "radial", 1001,
                     False, h0=64, beta=2),
    "wan13b_480p": Workload("wan13b_480p", 1, 12, 128, 21, 30, 52, 64, 64,
                            "bf16", "pooled", 1002, True, pooled_mode=1,
                            pooled_param=0.5),
    "wan14b_720p": Workload("wan14b_720p", 1, 40, 128, 21, 45, 80, 128, 64,
                            "bf16", "radial", 1003, True, h0=512, beta=2),
    "skip_carry_480p": Workload("skip_carry_480p", 1, 12, 128, 21, 30, 52, 64,
                                64, "bf16", "skip", 1004, True, tau=10.0,
                                steps=10),
    "hunyuan_4x": Workload("hunyuan_4x", 1, 24, 128, 132, 45, 80, 128, 64,
                           "bf16", "radial", 1005, True, h0=480, beta=2),
}


def _load_pooled_tau():
    import json
    p = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "tests", "golden", "pooled_tau.json")
    try:
        with open(p) as f:
            tau = float(json.load(f)["tau_p"])
    except (OSError, KeyError, ValueError):
        return
    WORKLOADS["wan13b_480p"] = WORKLOADS["wan13b_480p"].with_(pooled_param=tau)


_load_pooled_tau()


def workload(name: str) -> Workload:
    return WORKLOADS[name]


# ---------------------------------------------------------------- bf16 bytes
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------ the generator
def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _coords(w: Workload):
    i = np.arange(w.N, dtype=np.int64)
    t = i // w.F
    y = (i % w.F) // w.Ws
    x = i % w.Ws
    return t, y, x


def _smooth(w: Workload, seed: int) -> np.ndarray:
    """[N][d] fp64 smooth component shared by Q and K of every head."""
    r = _rng(seed, _SMOOTH_STREAM)
    f = r.integers(0, 3, size=(3, w.d))
    phi = r.uniform(0.0, 2.0 * np.pi, size=w.d)
    t, y, x = _coords(w)
    arg = (np.outer(t / w.T, f[0]) + np.outer(y / w.Hs, f[1])
           + np.outer(x / w.Ws, f[2]))
    return np.sin(2.0 * np.pi * arg + phi[None, :])


def _rope_tables(w: Workload):
    """cos/sin [N][d/2] for a 3D rotary encoding over (t, y, x).

    head_dim splits into (d - 2*2*(d//6), 2*(d//6), 2*(d//6)) channels for
    (t, y, x); within an axis of width da, pair m rotates by pos * 10000^(-2m/da).
    """
    d = w.d
    dy = dx = 2 * (d // 6)
    dt = d - dy - dx
    t, y, x = _coords(w)
    angles = []
    for pos, da in ((t, dt), (y, dy), (x, dx)):
        m = np.arange(da // 2, dtype=np.float64)
        inv = 10000.0 ** (-2.0 * m / da)
        angles.append(np.outer(pos.astype(np.float64), inv))
    ang = np.concatenate(angles, axis=1)
    return np.cos(ang), np.sin(ang)


def _apply_rope(z: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    a = z[:, 0::2]
    b = z[:, 1::2]
    out = np.empty_like(z)
    out[:, 0::2] = a * cos - b * sin
    out[:, 1::2] = a * sin + b * cos
    return out


def _cast(w: Workload, x64: np.ndarray) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if w.dtype == "f32":
        return x32
    return f32_to_bf16_bits(x32)


def _alloc(w: Workload, heads):
    dt = np.float32 if w.dtype == "f32" else np.uint16
    return np.empty((w.B, w.N, len(heads), w.d), dtype=dt)


def step_sigma(s: int) -> float:
    """Noise level of denoising step s for the skip-carry workload (0.5 -> 0.05)."""
    return 0.5 - 0.05 * s


def make_qkv(w: Workload, seed: int | None = None, heads=None, step: int | None = None,
             want=("q", "k", "v")):
    """Return dict of arrays [B][N][len(heads)][d] (bf16 bits as uint16, or float32).

    heads: subset of head indices to generate (default all); each head's values
    do not depend on which other heads are generated.
    step: for the skip-carry workload, Q_s = Q_0 + sigma_s Z and K_s likewise,
    with fresh noise keyed on (4000 + s) for Q and (5000 + s) for K.
    """
    seed = w.seed if seed is None else seed
    heads = list(range(w.H)) if heads is None else list(heads)
    c = _smooth(w, seed)
    rope = _rope_tables(w) if w.rope else None
    out = {name: _alloc(w, heads) for name in want}

    def one(job):
        b, hi = job
        h = heads[hi]
        for name in want:
            tid = {"q": TENSOR_Q, "k": TENSOR_K, "v": TENSOR_V}[name]
            z = _rng(seed, tid, b, h).standard_normal((w.N, w.d))
            if name in ("q", "k"):
                z += c
                if step is not None:
                    base = 4000 if name == "q" else 5000
                    z += step_sigma(step) * _rng(base + step, b, h).standard_normal((w.N, w.d))
                if rope is not None:
                    z = _apply_rope(z, rope[0], rope[1])
            out[name][b, :, hi, :] = _cast(w, z)

    jobs = [(b, hi) for b in range(w.B) for hi in range(len(heads))]
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(one, jobs))
    return out


def make_step_qk(w: Workload, step: int, seed: int | None = None, heads=None):
    """Q_s, K_s of denoising step s (skip-carry workload); V is unchanged."""
    return make_qkv(w, seed=seed, heads=heads, step=step, want=("q", "k"))
