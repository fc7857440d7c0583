"""Seeded synthetic workloads for decode-step block-sparse attention.

This module only draws inputs: it holds none of the method's arithmetic (no
scoring, selection, softmax or fusion).  Both the oracle-side tests and the
HIP-side tests/benchmarks take their inputs from here; the oracle always
receives the host copy of exactly the bf16 tensors handed to the library.

Every tensor draws from its own seeded torch generator (seed, tensor id), so a
(config, seed) pair fixes all inputs on a given device type.  Values are drawn
in fp32 and rounded to bf16 (round to nearest even).

Workloads (shapes of the pages' measurement points; no dataset items):
  tiny     B=1, Hq=4, Hkv=1, d=64, N=1024, S=16, budget 25% of N (k=16 blocks),
           4 sinks + 64 recent tokens dense; 3 planted blocks.
  llama32k B=8, Hq=32, Hkv=8, d=128, N=32768, S=32, budget 5%, 4 sinks + 512
           recent; sink rows (K and V) scaled x4; 2% of blocks planted.
  sweep    tiny head geometry at N=32768 for B in {1,8,32,64},
           S in {16,32,64}, budget in {2%,5%,10%}; 2% planted.
  qwen128k B=4, Hq=28, Hkv=4, d=128, N=131072, per-KV-head budget uniform in
           [1%, 20%] and S in {16, 64}; 4 sinks + 1024 recent; four planted
           sets that drift every 64 decode steps.
  loop32   32 layers x 256 decode steps, B=16, Hq=32, Hkv=8, d=128,
           N=65536 -> 65791, S=32, 5%, 4 sinks + 512 recent, MAW beta=1.

Planted keys are 3*u + 0.5*N(0,1) with u a unit direction: for single-step
workloads u = unit(sum of the group's query heads); for the loop workloads u is
a fixed random unit direction per (layer, sequence, KV head) and each query is
N(0,1) + 3u (the drift workload uses one direction per epoch).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    N: int
    block_size: List[int]          # per KV head
    budget_ppm: List[int]          # per KV head
    n_sink: int
    window: int
    plant_frac: float = 0.0        # fraction of blocks planted per (seq, kvh)
    n_plant: int = 0               # explicit planted-block count (overrides)
    sink_scale: float = 1.0
    layers: int = 1
    steps: int = 1
    maw_beta: float = 0.0
    maw_decay: float = 0.95

    @property
    def G(self):
        return self.Hq // self.Hkv


def tiny(seed: int = 0) -> Workload:
    return Workload("tiny", B=1, Hq=4, Hkv=1, d=64, N=1024, block_size=[16],
                    budget_ppm=[250000], n_sink=4, window=64, n_plant=3)


def llama32k() -> Workload:
    return Workload("llama32k", B=8, Hq=32, Hkv=8, d=128, N=32768,
                    block_size=[32] * 8, budget_ppm=[50000] * 8, n_sink=4,
                    window=512, plant_frac=0.02, sink_scale=4.0)


def sweep(B: int, S: int, budget_pct: int) -> Workload:
    return Workload("sweep_B%d_S%d_b%d" % (B, S, budget_pct), B=B, Hq=4, Hkv=1,
                    d=64, N=32768, block_size=[S], budget_ppm=[budget_pct * 10000],
                    n_sink=4, window=64, plant_frac=0.02)


def qwen128k(seed: int = 0) -> Workload:
    """Per-KV-head budgets (integer ppm uniform in [10000, 200000]) and block
    sizes (16 or 64, probability 1/2 each), drawn once per seed."""
    g = torch.Generator().manual_seed(1_000_003 * (seed + 1) + 7)
    budgets = torch.randint(10000, 200001, (4,), generator=g).tolist()
    sizes = [16 if b else 64 for b in torch.randint(0, 2, (4,), generator=g).tolist()]
    return Workload("qwen128k", B=4, Hq=28, Hkv=4, d=128, N=131072,
                    block_size=sizes, budget_ppm=budgets, n_sink=4, window=1024,
                    plant_frac=0.02, steps=256)


def loop32() -> Workload:
    return Workload("loop32", B=16, Hq=32, Hkv=8, d=128, N=65536,
                    block_size=[32] * 8, budget_ppm=[50000] * 8, n_sink=4,
                    window=512, plant_frac=0.02, layers=32, steps=256,
                    maw_beta=1.0)


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def _gen(seed: int, tensor_id: int, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed((int(seed) * 0x9E3779B1 + int(tensor_id) * 0x85EBCA77) % (2**63 - 1))
    return g


def randn(shape, seed, tensor_id, device="cpu", std=1.0, mean=None):
    g = _gen(seed, tensor_id, device)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean is not None:
        x.add_(mean)
    return x.to(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def n_blocks(N: int, S: int) -> int:
    return (N + S - 1) // S


def plantable_blocks(N: int, S: int, n_sink: int, window: int) -> np.ndarray:
    """Blocks wholly outside the dense sink/window ranges and not block 0:
    where planted tokens can only be reached through selection."""
    nb = n_blocks(N, S)
    idx = np.arange(nb)
    lo = idx * S
    hi = np.minimum(lo + S, N)
    outside = (lo >= n_sink) & (hi <= N - window)
    outside &= idx != 0
    return idx[outside]


def choose_planted(N, S, n_sink, window, count, seed, tensor_id) -> np.ndarray:
    pool = plantable_blocks(N, S, n_sink, window)
    count = min(count, pool.shape[0])
    g = torch.Generator().manual_seed((seed * 7919 + tensor_id * 104729) % (2**63 - 1))
    perm = torch.randperm(pool.shape[0], generator=g).numpy()
    return np.sort(pool[perm[:count]])


def plant_count(w: Workload, S: int, N: int) -> int:
    if w.n_plant:
        return w.n_plant
    return int(round(w.plant_frac * n_blocks(N, S)))


def unit_dir(x: torch.Tensor) -> torch.Tensor:
    x = x.float()
    return x / x.norm(dim=-1, keepdim=True)


# ----------------------------------------------------------------------------
# single decode step workloads (tiny, llama32k, sweep)
# ----------------------------------------------------------------------------

def single_step(w: Workload, seed: int, device="cpu", N: Optional[int] = None):
    """K, V: [B, N, Hkv, d] bf16; q: [B, Hq, d] bf16; planted: list per
    (b, g) of planted block indices.  Tensors live on `device`."""
    N = w.N if N is None else N
    B, Hq, Hkv, d, G = w.B, w.Hq, w.Hkv, w.d, w.G
    q = randn((B, Hq, d), seed, 1, device)
    K = randn((B, N, Hkv, d), seed, 2, device)
    V = randn((B, N, Hkv, d), seed, 3, device)
    planted = {}
    for b in range(B):
        for g in range(Hkv):
            S = w.block_size[g]
            cnt = plant_count(w, S, N)
            blocks = choose_planted(N, S, w.n_sink, w.window, cnt, seed,
                                    1000 + b * Hkv + g)
            planted[(b, g)] = blocks
            if blocks.size == 0:
                continue
            u = unit_dir(q[b, g * G:(g + 1) * G].float().sum(0))
            toks = torch.from_numpy((blocks[:, None] * S + np.arange(S)[None, :]).reshape(-1))
            toks = toks[toks < N].to(device)
            noise = randn((toks.numel(), d), seed, 5000 + b * Hkv + g, device,
                          std=0.5).float()
            K[b, toks, g] = (3.0 * u[None, :] + noise).to(torch.bfloat16)
    if w.sink_scale != 1.0 and w.n_sink > 0:
        ns = min(w.n_sink, N)
        K[:, :ns] = (K[:, :ns].float() * w.sink_scale).to(torch.bfloat16)
        V[:, :ns] = (V[:, :ns].float() * w.sink_scale).to(torch.bfloat16)
    return dict(q=q, K=K, V=V, planted=planted, N=N)


# ----------------------------------------------------------------------------
# multi-step workloads (qwen128k drift, loop32)
# ----------------------------------------------------------------------------

def directions(w: Workload, seed: int, layer: int, n_dir: int, device="cpu"):
    """Fixed random unit directions [B, Hkv, n_dir, d] (float32)."""
    x = torch.randn(w.B, w.Hkv, n_dir, w.d,
                    generator=_gen(seed, 90000 + layer, device), device=device)
    return unit_dir(x)


def prefill_with_directions(w: Workload, seed: int, layer: int, N0: int,
                            dirs: torch.Tensor, device="cpu"):
    """Prefill K, V [B, N0, Hkv, d] with len(dirs[b,g]) planted sets per
    (b, g): set e holds keys 3*dirs[b,g,e] + 0.5*N(0,1).  The sets are
    disjoint.  Returns K, V, planted[(b,g)] = list of arrays."""
    B, Hkv, d = w.B, w.Hkv, w.d
    K = randn((B, N0, Hkv, d), seed, 10 + 7 * layer, device)
    V = randn((B, N0, Hkv, d), seed, 11 + 7 * layer, device)
    n_dir = dirs.shape[2]
    planted = {}
    for b in range(B):
        for g in range(Hkv):
            S = w.block_size[g]
            cnt = plant_count(w, S, N0)
            allb = choose_planted(N0, S, w.n_sink, w.window, cnt * n_dir, seed,
                                  20000 + layer * 4096 + b * Hkv + g)
            g2 = torch.Generator().manual_seed(seed * 31 + layer * 131 + b * 17 + g)
            allb = allb[torch.randperm(allb.shape[0], generator=g2).numpy()]
            sets = [np.sort(allb[e * cnt:(e + 1) * cnt]) for e in range(n_dir)]
            planted[(b, g)] = sets
            for e, blocks in enumerate(sets):
                if blocks.size == 0:
                    continue
                toks = torch.from_numpy((blocks[:, None] * S + np.arange(S)[None, :]).reshape(-1))
                toks = toks[toks < N0].to(device)
                noise = randn((toks.numel(), d), seed,
                              30000 + layer * 65536 + (b * Hkv + g) * 8 + e,
                              device, std=0.5).float()
                K[b, toks, g] = (3.0 * dirs[b, g, e][None, :] + noise).to(torch.bfloat16)
    if w.sink_scale != 1.0 and w.n_sink > 0:
        ns = min(w.n_sink, N0)
        K[:, :ns] = (K[:, :ns].float() * w.sink_scale).to(torch.bfloat16)
        V[:, :ns] = (V[:, :ns].float() * w.sink_scale).to(torch.bfloat16)
    return K, V, planted


def loop_query(w: Workload, seed: int, layer: int, step: int,
               dirs: torch.Tensor, device="cpu"):
    """loop32: q = N(0,1) + 3u, u the (layer, seq, kvh) direction."""
    G = w.G
    base = torch.randn(w.B, w.Hq, w.d, generator=_gen(seed, 200000 + layer * 1024 + step, device),
                       device=device)
    u = dirs[:, :, 0, :].repeat_interleave(G, dim=1)  # [B, Hq, d]
    return (base + 3.0 * u).to(torch.bfloat16)


def drift_query(w: Workload, seed: int, step: int, epoch_q: torch.Tensor,
                device="cpu"):
    """qwen128k: q_t = q^(e) + 0.25*N(0,1), e = step // 64."""
    e = min(step // 64, epoch_q.shape[0] - 1)
    noise = torch.randn(w.B, w.Hq, w.d, generator=_gen(seed, 300000 + step, device),
                        device=device)
    return (epoch_q[e].float() + 0.25 * noise).to(torch.bfloat16)


def drift_setup(w: Workload, seed: int, n_epoch: int = 4, device="cpu"):
    """Epoch base queries q^(e) [n_epoch, B, Hq, d] and their group
    directions [B, Hkv, n_epoch, d]."""
    G = w.G
    qe = torch.stack([randn((w.B, w.Hq, w.d), seed, 400 + e, device)
                      for e in range(n_epoch)])
    dirs = torch.stack([unit_dir(qe[e].float().view(w.B, w.Hkv, G, w.d).sum(2))
                        for e in range(n_epoch)], dim=2)
    return qe, dirs


def step_kv(w: Workload, seed: int, layer: int, step: int, device="cpu"):
    """New decode token per sequence: K, V [B, 1, Hkv, d] ~ N(0,1)."""
    K = randn((w.B, 1, w.Hkv, w.d), seed, 500000 + layer * 4096 + 2 * step, device)
    V = randn((w.B, 1, w.Hkv, w.d), seed, 500001 + layer * 4096 + 2 * step, device)
    return K, V


# ----------------------------------------------------------------------------
# adversarial inputs for the approximate block score's error bound
# ----------------------------------------------------------------------------

ADVERSARIAL_KINDS = ("spread", "cancel", "denormal")


def adversarial(kind: str, B: int, Hkv: int, G: int, d: int, N: int, S: int, seed: int):
    """Keys and queries that stress an fp32 score bound (no method arithmetic
    here: only how the values are drawn).

      spread    every (sequence, KV head, block of S tokens) draws a scale
                2^e, e uniform in [-40, 40]; key elements are
                +-2^(e + f) (1 + u), f uniform in [-3, 3], u in [0, 1);
                queries N(0, 1).
      cancel    query channels come in equal pairs (2j, 2j+1); every token
                of a block is the same vector; in 97% of the blocks (chosen
                at random) channel 2j+1 is the negation of channel 2j, so
                their exact scores are 0 and a 5% budget ends among exact
                ties; the rest are drawn as in `spread`.
      denormal  keys as in `spread`; queries N(0, 1) * 2^-124, so that a part
                of their elements fall below the smallest normal bf16.
    Returns dict(q [B][G*Hkv][d], K, V [B][N][Hkv][d]) as bf16 tensors.
    """
    if kind not in ADVERSARIAL_KINDS:
        raise ValueError(kind)
    nb = n_blocks(N, S)
    g = _gen(seed, 900, "cpu")
    e_blk = torch.randint(-40, 41, (B, nb, Hkv), generator=g).to(torch.float32)
    e_tok = e_blk.repeat_interleave(S, dim=1)[:, :N]                       # [B][N][Hkv]
    f = torch.randint(-3, 4, (B, N, Hkv, d), generator=g).to(torch.float32)
    u = torch.rand(B, N, Hkv, d, generator=g)
    sgn = torch.where(torch.rand(B, N, Hkv, d, generator=g) < 0.5, -1.0, 1.0)
    K = sgn * torch.exp2(e_tok[..., None] + f) * (1.0 + u)
    q = torch.randn(B, Hkv * G, d, generator=g)
    if kind == "cancel":
        first = torch.arange(nb).repeat_interleave(S)[:N] * S              # first token of its block
        K = K[:, first]                                                     # one vector per block
        zero = torch.rand(B, nb, Hkv, generator=g) < 0.97
        zt = zero.repeat_interleave(S, dim=1)[:, :N]
        paired = K.clone()
        paired[..., 1::2] = -K[..., 0::2]
        K = torch.where(zt[..., None], paired, K)
        q[..., 1::2] = q[..., 0::2]
    elif kind == "denormal":
        q = q * 2.0 ** -124
    V = torch.randn(B, N, Hkv, d, generator=_gen(seed, 901, "cpu"))
    return dict(q=q.to(torch.bfloat16), K=K.to(torch.bfloat16), V=V.to(torch.bfloat16))
