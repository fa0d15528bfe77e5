"""Seeded synthetic Q/K/V for the SparsePR workloads.

This module only draws random numbers and builds the inputs; it holds none of the
attention method's arithmetic.  Both the GPU path (tests, benchmark) and the oracle
consume what it returns.

Recipe (per KV head kappa, token n at grid position x_n = (t, h, w), raster order
n = (t*H + h)*W + w):

* 16 random Fourier features phi_k(x) = cos(omega_k . x + b_k), omega_k = z_k / ell
  (element-wise), z_k ~ N(0, I_3), b_k ~ U(0, 2 pi); phi is normalised per token to unit
  l2 norm.  Head types follow the local / cross-shaped / global taxonomy of the Compact
  Attention news item (paragraph on the three attention patterns):
  local ell = (1.5, 3, 3); cross-shaped as local, but features 0-3 have omega_w = 0
  (row corridors) and 4-7 have omega_h = 0 (column corridors), those eight amplified x2
  before normalisation; global ell = (12, 24, 24).
* signal = phi G with G ~ N(0, 1)^{16 x d} per KV head.
* Q_h = a s_h signal + 0.3 eps_Q,  K = a s signal + 0.3 eps_K  (eps ~ N(0, 1)),
  V ~ N(0, 1).  a is the per-type amplitude found by calibration (``amplitudes.json``),
  s the per-head feature scale (C2: on Q and K; C4: on Q only; otherwise 1).
* RNG: numpy PCG64 seeded with [cfg_id, head, stream]; streams 0 = omega and b,
  1 = G, 2 = Q noise (query head), 3 = K noise, 4 = V, 5 = per-head scale (query head).
* Cast: bf16 workloads are rounded to bfloat16 (round to nearest, ties to even,
  directly from float64); fp32 workloads to float32.  Values are returned as float32
  arrays that hold exactly the values the kernels receive.
"""
import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Workload

_AMP_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "amplitudes.json")

LENGTH_SCALES = {"local": (1.5, 3.0, 3.0), "cross": (1.5, 3.0, 3.0), "global": (12.0, 24.0, 24.0)}
N_FEATURES = 16
NOISE_STD = 0.3


def rng(cfg_id: int, head: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([cfg_id, head, stream]))


def positions(grid):
    t, h, w = grid
    tt, hh, ww = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")
    return np.stack([tt.ravel(), hh.ravel(), ww.ravel()], axis=1).astype(np.float64)


def fourier_features(cfg: Workload, kv_head: int) -> np.ndarray:
    kind = cfg.head_types[kv_head]
    r = rng(cfg.cfg_id, kv_head, 0)
    z = r.standard_normal((N_FEATURES, 3))
    b = r.uniform(0.0, 2.0 * np.pi, N_FEATURES)
    omega = z / np.asarray(LENGTH_SCALES[kind])[None, :]
    amp = np.ones(N_FEATURES)
    if kind == "cross":
        omega[0:4, 2] = 0.0          # row corridors: constant along w
        omega[4:8, 1] = 0.0          # column corridors: constant along h
        amp[0:8] = 2.0
    x = positions(cfg.grid)
    phi = np.cos(x @ omega.T + b[None, :]) * amp[None, :]
    phi /= np.linalg.norm(phi, axis=1, keepdims=True)
    return phi


def signal(cfg: Workload, kv_head: int) -> np.ndarray:
    phi = fourier_features(cfg, kv_head)
    G = rng(cfg.cfg_id, kv_head, 1).standard_normal((N_FEATURES, cfg.d))
    return phi @ G


def head_scale(cfg: Workload, q_head: int) -> float:
    if cfg.scale_on == "none":
        return 1.0
    lo, hi = cfg.scale_range
    return float(rng(cfg.cfg_id, q_head, 5).uniform(lo, hi))


def noise(cfg: Workload, head: int, stream: int) -> np.ndarray:
    return rng(cfg.cfg_id, head, stream).standard_normal((cfg.n, cfg.d))


def load_amplitudes():
    if not os.path.exists(_AMP_FILE):
        raise FileNotFoundError(
            f"{_AMP_FILE} is missing: run `python -m oracle.calibrate` to produce it")
    with open(_AMP_FILE) as f:
        return json.load(f)


def amplitude(cfg: Workload, kv_head: int, table=None) -> float:
    table = table if table is not None else load_amplitudes()
    return float(table[str(cfg.cfg_id)][cfg.head_types[kv_head]])


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even); returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    u = x.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    u = (u + (np.uint64((1 << 44) - 1) + lsb)) & ~np.uint64((1 << 45) - 1)
    return u.view(np.float64).astype(np.float32)


def cast(cfg: Workload, x: np.ndarray) -> np.ndarray:
    if cfg.dtype == "bf16":
        return round_to_bf16(x)
    if cfg.dtype == "fp32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(cfg.dtype)


def head_inputs_fp64(cfg: Workload, kv_head: int, amp: float):
    """Uncast float64 (Q [g,N,d], K [N,d], V [N,d]) for one KV head and its query heads."""
    sig = signal(cfg, kv_head)
    g = cfg.g
    qs = []
    for j in range(g):
        h = kv_head * g + j
        s = head_scale(cfg, h)
        qs.append(amp * s * sig + NOISE_STD * noise(cfg, h, 2))
    sk = head_scale(cfg, kv_head) if cfg.scale_on == "qk" else 1.0
    k = amp * sk * sig + NOISE_STD * noise(cfg, kv_head, 3)
    v = noise(cfg, kv_head, 4)
    return np.stack(qs), k, v


def head_inputs(cfg: Workload, kv_head: int, table=None):
    """Cast (Q [g,N,d], K [N,d], V [N,d]) float32 arrays for one KV head."""
    q, k, v = head_inputs_fp64(cfg, kv_head, amplitude(cfg, kv_head, table))
    return cast(cfg, q), cast(cfg, k), cast(cfg, v)


def make_inputs(cfg: Workload, threads: int = 8):
    """Q [Hq,N,d], K [Hkv,N,d], V [Hkv,N,d] as float32 arrays holding the cast values."""
    table = load_amplitudes()
    Q = np.empty((cfg.heads_q, cfg.n, cfg.d), np.float32)
    K = np.empty((cfg.heads_kv, cfg.n, cfg.d), np.float32)
    V = np.empty((cfg.heads_kv, cfg.n, cfg.d), np.float32)

    def one(kv):
        q, k, v = head_inputs(cfg, kv, table)
        Q[kv * cfg.g:(kv + 1) * cfg.g] = q
        K[kv] = k
        V[kv] = v

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(cfg.heads_kv)))
    return Q, K, V
