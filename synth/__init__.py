"""Seeded synthetic workloads for one IndexShare layer group.

This module only draws random tensors and names their shapes. It holds none of
the method's arithmetic, so both the CPU oracle's tests and the GPU path's
tests and benchmark can take their inputs from here without sharing any
computation.

Shapes and value distributions follow the statement of the problem: an
indexer of H_I heads x D_I dims with int8 queries and keys drawn uniformly
from [-8, 7] and fp32 per-(query, head) weights drawn from {1/4, 1/2, 1, 2};
per layer, absorbed-MLA queries Q of H heads x D dims and a latent cache C of
D = D_c + D_r dims per token, both N(0, 1) rounded to bf16.  The sizes come
from the pages' workloads: the 2048-entry top-k and the group of four layers
that share it (GLM-5.2 configuration keys ``index_topk`` and
``index_topk_freq``), 64 attention heads and a 512-wide latent plus a 64-wide
RoPE slice, the 128K mid-training length and the 1M serving context, and the
seven-step MTP draft that reuses one index set.

Draw order (fixed, so a seed names one workload): qI, w, kI, then for each
layer l: Q_l, C_l (or, for an FP8 cache, Q_l and the layer's FP8 cache).  Per-layer indexer inputs (the per-layer-indexer
ablation) come from their own seeds, and per-step MTP queries from seed
``mtp_q_seed0 + step``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import torch

W_TABLE = (0.25, 0.5, 1.0, 2.0)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int            # sequences
    Tq: int           # query tokens per sequence (appended at the end of the cache)
    kv_len: int       # cache entries visible to the last query of every sequence
    L_cap: int        # allocated cache length (>= kv_len)
    H_I: int          # indexer heads
    D_I: int          # indexer dim
    k: int            # top-k
    H: int            # attention heads
    D: int            # latent row width (D_c + D_r)
    D_v: int          # value width (the first D_v entries of a latent row)
    n_layers: int     # layers sharing one index set
    seed: int
    mtp_steps: int = 1          # > 1: steps 2.. reuse the step-1 index set
    mtp_q_seed0: int = 5000     # per-step query seed base (step s uses seed0 + s)
    ablation_seeds: tuple = ()  # per-layer indexer seeds for the per-layer-indexer ablation
    causal_prefill: bool = False

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def tokens_per_group(self) -> int:
        return self.B * self.Tq * self.mtp_steps

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # tiny causal prefill: 1024 queries over their own 1024 keys, top-64
    "C1": Workload("C1", B=1, Tq=1024, kv_len=1024, L_cap=1024, H_I=4, D_I=32, k=64,
                   H=16, D=160, D_v=128, n_layers=4, seed=0, causal_prefill=True),
    # decode, batch 8 at 32K
    "C2": Workload("C2", B=8, Tq=1, kv_len=32768, L_cap=32768, H_I=64, D_I=128, k=2048,
                   H=64, D=576, D_v=512, n_layers=4, seed=2),
    # decode, batch 8 at 128K (the headline decode group)
    "C2_128K": Workload("C2_128K", B=8, Tq=1, kv_len=131072, L_cap=131072, H_I=64, D_I=128,
                        k=2048, H=64, D=576, D_v=512, n_layers=4, seed=6),
    # 4096-token prefill chunk appended to a 131072-token cache
    "C3": Workload("C3", B=1, Tq=4096, kv_len=131072 + 4096, L_cap=131072 + 4096, H_I=64,
                   D_I=128, k=2048, H=64, D=576, D_v=512, n_layers=4, seed=3,
                   causal_prefill=True),
    # 1M-context decode, batch 2; ablation indexers from seeds 40..43
    "C4": Workload("C4", B=2, Tq=1, kv_len=1 << 20, L_cap=1 << 20, H_I=64, D_I=128, k=2048,
                   H=64, D=576, D_v=512, n_layers=4, seed=4, ablation_seeds=(40, 41, 42, 43)),
    # MTP draft: batch 16 at 256K, 7 steps reusing the step-1 index set
    "C5": Workload("C5", B=16, Tq=1, kv_len=262144, L_cap=262144, H_I=64, D_I=128, k=2048,
                   H=64, D=576, D_v=512, n_layers=4, seed=5, mtp_steps=7, mtp_q_seed0=5000),
    # multi-query decode (e.g. verifying 8 draft tokens): batch 8 x 8 queries
    # at 128K, each query with its own index set, causal among the 8
    "C2_128K_MQ8": Workload("C2_128K_MQ8", B=8, Tq=8, kv_len=131072, L_cap=131072, H_I=64,
                            D_I=128, k=2048, H=64, D=576, D_v=512, n_layers=4, seed=7),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def int8_uniform(shape, g: torch.Generator, device, lo: int = -8, hi: int = 7) -> torch.Tensor:
    return torch.randint(lo, hi + 1, shape, generator=g, device=device, dtype=torch.int8)


def pow2_weights(shape, g: torch.Generator, device) -> torch.Tensor:
    sel = torch.randint(0, len(W_TABLE), shape, generator=g, device=device)
    table = torch.tensor(W_TABLE, dtype=torch.float32, device=device)
    return table[sel]


def normal_bf16(shape, g: torch.Generator, device) -> torch.Tensor:
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def fp8_cache(B: int, L_cap: int, D_c: int, D_r: int, g: torch.Generator, device):
    """An FP8 latent cache (C8, Ce, Cr).  Per row: an exponent byte e drawn
    uniformly from [124, 130] (row scale 2^(e-127) in [1/8, 8]); the E4M3 codes
    (torch's float8_e4m3fn rounding) of N(0,1) latent values divided by the
    row scale; N(0,1) bf16 RoPE dims.  C8 [B,L_cap,D_c] uint8, Ce [B,L_cap]
    uint8, Cr [B,L_cap,D_r] bf16."""
    e = torch.randint(124, 131, (B, L_cap), generator=g, device=device, dtype=torch.int32)
    x = torch.randn((B, L_cap, D_c), generator=g, device=device, dtype=torch.float32)
    C8 = torch.ldexp(x, (127 - e)[..., None].float()).to(torch.float8_e4m3fn).view(torch.uint8)
    Cr = normal_bf16((B, L_cap, D_r), g, device)
    return C8.contiguous(), e.to(torch.uint8), Cr


def page_layout(B: int, L_cap: int, block_size: int, g: torch.Generator, device,
                extra_pages: int = 0) -> torch.Tensor:
    """A block table [B, L_cap / block_size] int32 that places the logical
    blocks of every sequence on distinct pages of a pool of
    B * L_cap / block_size + extra_pages pages, in a random order."""
    nb = L_cap // block_size
    perm = torch.randperm(B * nb + extra_pages, generator=g, device=device)[: B * nb]
    return perm.view(B, nb).to(torch.int32).contiguous()


def to_pages(cache: torch.Tensor, table: torch.Tensor, block_size: int, n_pages: int) -> torch.Tensor:
    """The page pool [n_pages, block_size, row...] holding cache [B, L_cap, row...]
    at the pages the table names (pages no block uses stay zero)."""
    B, L = cache.shape[0], cache.shape[1]
    nb = L // block_size
    pool = torch.zeros((n_pages, block_size) + tuple(cache.shape[2:]), dtype=cache.dtype,
                       device=cache.device)
    pool[table.reshape(-1).long()] = cache.reshape((B * nb, block_size) + tuple(cache.shape[2:]))
    return pool


def indexer_inputs(wl: Workload, seed: Optional[int] = None, device="cpu") -> Dict[str, torch.Tensor]:
    """qI [B,Tq,H_I,D_I] int8, w [B,Tq,H_I] fp32, kI [B,L_cap,D_I] int8, kv_len [B] int32."""
    g = _gen(wl.seed if seed is None else seed, device)
    qI = int8_uniform((wl.B, wl.Tq, wl.H_I, wl.D_I), g, device)
    w = pow2_weights((wl.B, wl.Tq, wl.H_I), g, device)
    kI = int8_uniform((wl.B, wl.L_cap, wl.D_I), g, device)
    kv_len = torch.full((wl.B,), wl.kv_len, dtype=torch.int32, device=device)
    return {"qI": qI, "w": w, "kI": kI, "kv_len": kv_len}


def group_inputs(wl: Workload, device="cpu", layers: Optional[int] = None,
                 kv8: bool = False) -> Dict[str, object]:
    """Indexer inputs plus, per layer, Q_l [B,Tq,H,D] and C_l [B,L_cap,D] (bf16),
    or with kv8 the layer's FP8 cache (lists C8, Ce, Cr; C is then None).

    One generator stream in the fixed draw order, so the indexer tensors are
    identical to ``indexer_inputs(wl)`` on the same device.
    """
    n_layers = wl.n_layers if layers is None else layers
    g = _gen(wl.seed, device)
    qI = int8_uniform((wl.B, wl.Tq, wl.H_I, wl.D_I), g, device)
    w = pow2_weights((wl.B, wl.Tq, wl.H_I), g, device)
    kI = int8_uniform((wl.B, wl.L_cap, wl.D_I), g, device)
    Q: List[torch.Tensor] = []
    C: List[torch.Tensor] = []
    C8: List[torch.Tensor] = []
    Ce: List[torch.Tensor] = []
    Cr: List[torch.Tensor] = []
    for _ in range(n_layers):
        Q.append(normal_bf16((wl.B, wl.Tq, wl.H, wl.D), g, device))
        if kv8:
            c8, ce, cr = fp8_cache(wl.B, wl.L_cap, wl.D_v, wl.D - wl.D_v, g, device)
            C8.append(c8); Ce.append(ce); Cr.append(cr)
        else:
            C.append(normal_bf16((wl.B, wl.L_cap, wl.D), g, device))
    kv_len = torch.full((wl.B,), wl.kv_len, dtype=torch.int32, device=device)
    d = {"qI": qI, "w": w, "kI": kI, "kv_len": kv_len, "Q": Q, "C": None if kv8 else C}
    if kv8:
        d.update(C8=C8, Ce=Ce, Cr=Cr)
    return d


def mtp_queries(wl: Workload, step: int, device="cpu", layers: Optional[int] = None) -> List[torch.Tensor]:
    """Per-step draft queries; steps count from 1 and every step, the first
    included, draws its queries from seed ``mtp_q_seed0 + step``."""
    n_layers = wl.n_layers if layers is None else layers
    g = _gen(wl.mtp_q_seed0 + step, device)
    return [normal_bf16((wl.B, wl.Tq, wl.H, wl.D), g, device) for _ in range(n_layers)]


def ablation_indexers(wl: Workload, device="cpu") -> List[Dict[str, torch.Tensor]]:
    """One independent indexer draw per layer (the per-layer-indexer baseline)."""
    return [indexer_inputs(wl, seed=s, device=device) for s in wl.ablation_seeds]
