"""Seeded synthetic inputs for the Gated DSA layer.

This module only draws random tensors; it holds none of the layer's
arithmetic.  The same tensors feed the HIP library and the CPU oracle.

Recipe (shapes and distributions of the workloads named in the design notes):
  - q_idx, q, gate, k_idx (bf16), k_cache, v_cache: N(0, 1) drawn in fp32 by
    torch's seeded generator, rounded to bf16 (round-to-nearest-even).
  - w (indexer head weights): U(0, 1), rounded to bf16.
  - fp8 indexer keys: N(0, 1) rounded to fp8 e4m3fn (RNE); per-token fp32
    scale U(0.5, 2).
  - fp8 indexer query heads (the fp8 prefill contraction): the same, with one
    fp32 scale U(0.5, 2) per (query, head).
  - "planted" keys: each position independently with probability
    plant_frac has its indexer key row multiplied by plant_mult (exact in
    bf16 for powers of two), giving a long-tailed score distribution.
  - ragged lengths: floor(exp(U(ln lo, ln hi))) per sequence.
Every tensor has its own seed derived from (seed, name) so any one tensor
can be regenerated without the others.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field

import torch

_CHUNK = 1 << 26  # elements drawn per generator call (bounds fp32 temporaries)


def _seed(seed: int, name: str) -> int:
    return (int(seed) * 1000003 + zlib.crc32(name.encode())) & 0x7FFFFFFFFFFF


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, name))
    return g


def randn_bf16(shape, seed: int, name: str, device="cpu") -> torch.Tensor:
    g = _gen(seed, name, device)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), _CHUNK):
        n = min(_CHUNK, flat.numel() - s)
        flat[s:s + n] = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    return out


def rand_bf16(shape, seed: int, name: str, lo=0.0, hi=1.0, device="cpu") -> torch.Tensor:
    g = _gen(seed, name, device)
    x = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return (lo + (hi - lo) * x).to(torch.bfloat16)


def randn_fp8(shape, seed: int, name: str, device="cpu") -> torch.Tensor:
    g = _gen(seed, name, device)
    out = torch.empty(shape, dtype=torch.float8_e4m3fn, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), _CHUNK):
        n = min(_CHUNK, flat.numel() - s)
        flat[s:s + n] = torch.randn(n, generator=g, device=device,
                                    dtype=torch.float32).to(torch.float8_e4m3fn)
    return out


def rand_f32(shape, seed: int, name: str, lo: float, hi: float, device="cpu") -> torch.Tensor:
    g = _gen(seed, name, device)
    return lo + (hi - lo) * torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def plant_rows(k: torch.Tensor, seed: int, frac: float, mult: float) -> torch.Tensor:
    """Multiply a random subset (probability frac per row) of rows by mult."""
    if frac <= 0:
        return k
    g = _gen(seed, "plant", k.device)
    mask = torch.rand(k.shape[0], generator=g, device=k.device) < frac
    k[mask] = (k[mask].float() * mult).to(k.dtype)
    return k


def log_uniform_lengths(n: int, lo: int, hi: int, seed: int) -> list[int]:
    g = torch.Generator().manual_seed(_seed(seed, "len"))
    u = torch.rand(n, generator=g, dtype=torch.float64)
    return [int(math.floor(math.exp(math.log(lo) + float(x) * (math.log(hi) - math.log(lo)))))
            for x in u]


@dataclass
class Workload:
    """Shapes of one DSA layer call (decode when n_q == 1 for every sequence)."""
    name: str
    ctx_lens: list
    n_q: list
    H_I: int
    d_I: int
    Hq: int
    D: int
    K: int
    key_dtype: str = "bf16"
    q_dtype: str = "bf16"
    plant_frac: float = 0.0
    plant_mult: float = 4.0
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def B(self):
        return len(self.ctx_lens)

    @property
    def T(self):
        return sum(self.n_q)

    @property
    def decode(self):
        return all(n == 1 for n in self.n_q)


# The named workloads (sizes of the pages' configurations; see the design notes).
def tiny_decode(seed=0):
    return Workload("tiny_decode_ctx4096", [4096], [1], 4, 64, 8, 64, 256, seed=seed)


def decode_128k(seed=1):
    return Workload("dsa_decode_b1_ctx131072", [131072], [1], 32, 128, 64, 128, 2048,
                    plant_frac=0.05, plant_mult=4.0, seed=seed)


def prefill_8k(seed=2):
    return Workload("dsa_prefill_q8192_ctx139264", [139264], [8192], 16, 128, 64, 128, 2048,
                    seed=seed)


def prefill_8k_fp8(seed=2):
    return Workload("dsa_prefill_q8192_ctx139264_fp8", [139264], [8192], 16, 128, 64, 128, 2048,
                    key_dtype="fp8", q_dtype="fp8", seed=seed)


def decode_1m_b32_fp8(seed=3):
    return Workload("dsa_decode_b32_ctx1048576_fp8", [1 << 20] * 32, [1] * 32, 32, 128, 64,
                    128, 2048, key_dtype="fp8", seed=seed)


def hybrid_5to1(seed=5):
    lens = log_uniform_lengths(8, 4096, 1 << 20, seed)
    return Workload("hybrid_swa5_dsa1_b8_ragged", lens, [1] * 8, 16, 128, 64, 128, 2048,
                    seed=seed, extra={"swa_layers": 5, "window": 128})


WORKLOADS = {
    "tiny": tiny_decode,
    "dec128k": decode_128k,
    "prefill8k": prefill_8k,
    "prefill8k_fp8": prefill_8k_fp8,
    "dec1m_b32_fp8": decode_1m_b32_fp8,
    "hybrid51": hybrid_5to1,
}


def make_inputs(wl: Workload, device="cpu", seed_offset: int = 0) -> dict:
    """Draw every tensor of one layer call for workload wl on `device`."""
    s = wl.seed + seed_offset
    B, T = wl.B, wl.T
    L_tot = sum(wl.ctx_lens)
    cu_ctx = [0]
    for L in wl.ctx_lens:
        cu_ctx.append(cu_ctx[-1] + L)
    cu_q = [0]
    for n in wl.n_q:
        cu_q.append(cu_q[-1] + n)
    t = {}
    if wl.q_dtype == "fp8":
        t["q_idx"] = randn_fp8((T, wl.H_I, wl.d_I), s, "q_idx", device)
        t["q_scale"] = rand_f32((T, wl.H_I), s, "q_scale", 0.5, 2.0, device)
    else:
        t["q_idx"] = randn_bf16((T, wl.H_I, wl.d_I), s, "q_idx", device)
        t["q_scale"] = None
    t["w"] = rand_bf16((T, wl.H_I), s, "w", 0.0, 1.0, device)
    if wl.key_dtype == "fp8":
        t["k_idx"] = randn_fp8((L_tot, wl.d_I), s, "k_idx", device)
        t["k_scale"] = rand_f32((L_tot,), s, "k_scale", 0.5, 2.0, device)
    else:
        t["k_idx"] = plant_rows(randn_bf16((L_tot, wl.d_I), s, "k_idx", device), s,
                                wl.plant_frac, wl.plant_mult)
        t["k_scale"] = None
    t["q"] = randn_bf16((T, wl.Hq, wl.D), s, "q", device)
    t["k_cache"] = randn_bf16((L_tot, wl.D), s, "k_cache", device)
    t["v_cache"] = randn_bf16((L_tot, wl.D), s, "v_cache", device)
    t["gate"] = randn_bf16((T, wl.Hq, wl.D), s, "gate", device)
    t["ctx_len"] = torch.tensor(wl.ctx_lens, dtype=torch.int32, device=device)
    t["cu_ctx"] = torch.tensor(cu_ctx, dtype=torch.int64, device=device)
    t["cu_q"] = torch.tensor(cu_q, dtype=torch.int32, device=device)
    return t
