"""Seeded synthetic inputs for the draft -> schedule -> verify step.

This module holds no arithmetic of the method: it only draws random tensors
with the shapes and value laws of the five workloads and builds the SPS cost
tables.  Both the HIP path and the CPU oracle consume its tensors (the oracle
after a copy to float64 NumPy), so neither depends on the other.

Workloads (shapes follow the pages' target families: Qwen3 vocabulary 151936,
DeepSeek vocabulary 129280; decaying per-position confidence mimics the
suffix decay of the DSpark paper's Figure 2):

  tiny        B=4, K=7, V=1024, r=16, fp32 logits.  Target t ~ N(0, 2^2),
              U = t[:, :7] + N(0, 1); W1, W2 ~ N(0, 0.05^2) -> bf16;
              c ~ U(0.5, 1); SPS(B) = 1000 / (1 + B/32) steps/s.
  qwen_verify B=64, K=7, V=151936, bf16.  t ~ N(0, 3^2); draft base logits
              D = 0.8 t[:, :7] + 0.6 N(0, 3^2) (correlation 0.8); every
              position verified.
  ds_stepped  B=256, K=5, V=129280, bf16.  t ~ N(0, 3^2); rho_r ~ U(0.5, 0.95),
              D = rho_r t + sqrt(1 - rho_r^2) N(0, 3^2); c_{r,k} ~ Beta(8-k, 1+k);
              staircase SPS(B) = 1000 min(1, 1024 / (64 ceil(B/64))).
  sched_stress B=1024, K=7, V=32768, fp32.  c_{r,.} = 7 i.i.d. Beta(a_r, b_r)
              sorted descending, a_r ~ U(2, 9), b_r ~ U(1, 3); t, D as qwen_verify;
              sawtooth SPS over [1024, 8192].
  full_step   B=512, K=7, V=151936, r=256, bf16.  U = 2 * StudentT(4);
              W1, W2 ~ N(0, 0.02^2) -> bf16; x0 ~ U{0..V-1};
              c_{r,k} ~ Beta(8-k, 1+k); target rows t_k = 0.85 U_k + 0.5268 s eps
              (k = 1..7, s = 2 sqrt(2) the standard deviation of U) and a bonus
              row t_8 = s eps; staircase SPS(B) = 1000 min(1, 2048 / (64 ceil(B/64))).

RNN-head inputs (rnn_head): backbone hidden states H [B, K, d] ~ N(0, 1) and
the head's projection W [3r, 2r + d] ~ N(0, 1 / (2r + d)), both bf16, so that
gate, candidate and output pre-activations have about unit variance; the
full-size case uses the full_step workload with r = 256 and d = 4096.

Float values are drawn in float32 and rounded to nearest-even bfloat16 where
the workload is bf16.  Randomness: a torch generator seeded with
1000 + workload number drives the large logit tensors (on the requested
device); a NumPy generator with the same seed draws the small per-request
quantities.  The per-decision uniforms of the method use seed
0x5EED0000 + workload number.
"""
import math
from dataclasses import dataclass, field

import numpy as np
import torch

WORKLOADS = {"tiny": 1, "qwen_verify": 2, "ds_stepped": 3, "sched_stress": 4, "full_step": 5}


@dataclass
class Workload:
    name: str
    B: int
    K: int
    V: int
    r: int
    temperature: float
    U: torch.Tensor                 # [B, K, V] draft base logits
    t: torch.Tensor                 # [B, K+1, V] target logits of every possible verify row
    W1: torch.Tensor = None         # [V, r] bf16
    W2: torch.Tensor = None         # [V, r] bf16: column-major storage of the r x V factor
    x0: torch.Tensor = None         # [B] int32
    c: torch.Tensor = None          # [B, K] float32
    sps: torch.Tensor = None        # [L] float64 steps/s indexed by verify tokens
    rng_seed: int = 0
    notes: dict = field(default_factory=dict)


def sps_hyperbolic(n, beta=32.0, scale=1000.0):
    b = np.arange(n, dtype=np.float64)
    return scale / (1.0 + b / beta)


def sps_staircase(n, flat_until, step=64, scale=1000.0):
    b = np.arange(n, dtype=np.float64)
    steps = step * np.ceil(np.maximum(b, 1) / step)
    return scale * np.minimum(1.0, flat_until / steps)


def sps_sawtooth(n, lo=1024, hi=8192, tooth=512, scale=1000.0):
    b = np.clip(np.arange(n, dtype=np.float64), lo, hi)
    x = (b - lo)
    frac = x / tooth - np.floor(x / tooth)
    return scale * (1.0 - 0.5 * x / (hi - lo)) * (1.0 - 0.08 * frac)


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, device, std=1.0):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _student_t4(shape, g, device):
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    u1 = 1.0 - torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    u2 = 1.0 - torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    chi2_over_nu = (-torch.log(u1 * u2) / 2.0).clamp_min(1e-30)   # chi^2_4 / 4
    return z / torch.sqrt(chi2_over_nu)


def make(name, device="cpu", B=None, V=None):
    """Generate workload `name`; B and V may be shrunk for small parity cases."""
    num = WORKLOADS[name]
    seed = 1000 + num
    g = _gen(seed, device)
    npr = np.random.default_rng(seed)
    rng_seed = 0x5EED0000 + num
    dev = torch.device(device)

    if name == "tiny":
        B, K, V, r = B or 4, 7, V or 1024, 16
        t = _normal((B, K + 1, V), g, device, 2.0)
        U = t[:, :K] + _normal((B, K, V), g, device, 1.0)
        W1 = _normal((V, r), g, device, 0.05).to(torch.bfloat16)
        W2 = _normal((V, r), g, device, 0.05).to(torch.bfloat16)
        x0 = torch.from_numpy(npr.integers(0, V, size=B).astype(np.int32)).to(dev)
        c = torch.from_numpy(npr.uniform(0.5, 1.0, size=(B, K)).astype(np.float32)).to(dev)
        sps = torch.from_numpy(sps_hyperbolic(B * (K + 1) + 1)).to(dev)
        return Workload(name, B, K, V, r, 1.0, U.contiguous(), t.contiguous(), W1, W2, x0, c, sps, rng_seed,
                        {"sps": "1000/(1+B/32) steps/s"})

    if name in ("qwen_verify", "sched_stress"):
        if name == "qwen_verify":
            B, K, V, dt = B or 64, 7, V or 151936, torch.bfloat16
        else:
            B, K, V, dt = B or 1024, 7, V or 32768, torch.float32
        t = _normal((B, K + 1, V), g, device, 3.0)
        D = 0.8 * t[:, :K] + 0.6 * _normal((B, K, V), g, device, 3.0)
        x0 = torch.from_numpy(npr.integers(0, V, size=B).astype(np.int32)).to(dev)
        if name == "qwen_verify":
            c = torch.ones((B, K), dtype=torch.float32, device=dev)
            sps = torch.from_numpy(np.full(B * (K + 1) + 1, 1000.0)).to(dev)
        else:
            a = npr.uniform(2, 9, size=B)
            b = npr.uniform(1, 3, size=B)
            cc = np.sort(npr.beta(a[:, None], b[:, None], size=(B, K)), axis=1)[:, ::-1]
            c = torch.from_numpy(np.ascontiguousarray(cc).astype(np.float32)).to(dev)
            sps = torch.from_numpy(sps_sawtooth(max(8193, B * (K + 1) + 1))).to(dev)
        return Workload(name, B, K, V, 0, 1.0, D.to(dt).contiguous(), t.to(dt).contiguous(), None, None, x0, c,
                        sps, rng_seed)

    if name == "ds_stepped":
        B, K, V = B or 256, 5, V or 129280
        t = _normal((B, K + 1, V), g, device, 3.0)
        rho = torch.from_numpy(npr.uniform(0.5, 0.95, size=B).astype(np.float32)).to(dev).view(B, 1, 1)
        D = rho * t[:, :K] + torch.sqrt(1 - rho * rho) * _normal((B, K, V), g, device, 3.0)
        x0 = torch.from_numpy(npr.integers(0, V, size=B).astype(np.int32)).to(dev)
        k = np.arange(1, K + 1)
        c = torch.from_numpy(npr.beta(8 - k, 1 + k, size=(B, K)).astype(np.float32)).to(dev)
        sps = torch.from_numpy(sps_staircase(B * (K + 1) + 1, flat_until=1024)).to(dev)
        return Workload(name, B, K, V, 0, 1.0, D.to(torch.bfloat16).contiguous(),
                        t.to(torch.bfloat16).contiguous(), None, None, x0, c, sps, rng_seed)

    if name == "full_step":
        B, K, V, r = B or 512, 7, V or 151936, 256
        s = 2.0 * math.sqrt(2.0)
        U = torch.empty((B, K, V), dtype=torch.bfloat16, device=dev)
        t = torch.empty((B, K + 1, V), dtype=torch.bfloat16, device=dev)
        for k in range(K):                       # per position to bound temporaries
            u = 2.0 * _student_t4((B, V), g, device)
            U[:, k] = u.to(torch.bfloat16)
            t[:, k] = (0.85 * u + 0.5268 * s * _normal((B, V), g, device)).to(torch.bfloat16)
        t[:, K] = (s * _normal((B, V), g, device)).to(torch.bfloat16)
        W1 = _normal((V, r), g, device, 0.02).to(torch.bfloat16)
        W2 = _normal((V, r), g, device, 0.02).to(torch.bfloat16)
        x0 = torch.from_numpy(npr.integers(0, V, size=B).astype(np.int32)).to(dev)
        kk = np.arange(1, K + 1)
        c = torch.from_numpy(npr.beta(8 - kk, 1 + kk, size=(B, K)).astype(np.float32)).to(dev)
        sps = torch.from_numpy(sps_staircase(B * (K + 1) + 1, flat_until=2048)).to(dev)
        return Workload(name, B, K, V, r, 1.0, U, t, W1, W2, x0, c, sps, rng_seed,
                        {"target": "correlated 0.85 with the base logits U"})
    raise KeyError(name)


def rnn_head(B, K, r, d, seed, device="cpu"):
    """Hidden states H [B, K, d] and the RNN head's projection W [3r, 2r + d]
    (gate rows, candidate rows, output rows), bf16."""
    g = _gen(seed, device)
    H = _normal((B, K, d), g, device).to(torch.bfloat16)
    W = _normal((3 * r, 2 * r + d), g, device, 1.0 / math.sqrt(2 * r + d)).to(torch.bfloat16)
    return H.contiguous(), W.contiguous()


def flat_target_rows(t, cu_seqlens):
    """Stand-in for the target model's verification pass: the flat [N, V]
    batch holding rows 0..l_r of request r's target logits, request-major
    (cu_seqlens[r] .. cu_seqlens[r+1]-1)."""
    B, K1, V = t.shape
    cu = cu_seqlens.to("cpu", torch.int64)
    lengths = (cu[1:] - cu[:-1])
    idx = torch.cat([torch.arange(int(lengths[r])) + r * K1 for r in range(B)])
    return t.reshape(B * K1, V).index_select(0, idx.to(t.device)).contiguous()


def all_rows_cu(B, K, device="cpu"):
    """cu_seqlens verifying every draft position (no scheduling)."""
    return torch.arange(0, B * (K + 1) + 1, K + 1, dtype=torch.int32, device=device)


def to_f64(x):
    """Exact float64 NumPy copy of a (float32 or bfloat16) tensor."""
    return x.detach().to("cpu", torch.float64).numpy()
