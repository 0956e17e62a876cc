"""Seeded synthetic workloads for MoE token dispatch / combine.

This module only draws inputs: token rows ``x``, routing ``topk_idx`` /
``topk_weights`` and expert-output rows ``y``.  It holds none of the
dispatch/combine arithmetic, so the CPU oracle and the HIP path can both take
their inputs from it without sharing any of the method.

Shapes and distributions follow the workloads the TileScale "EP v2 intranode
dispatch/combine" pull request measures on (PR summary and Performance
section: 8192 tokens per rank, hidden 7168, top-8 of 256 experts), plus a
tiny, a mid-sized, a skewed+masked and a grouped one-GPU-receive-share case.
The pages benchmark with a script, not a dataset; these synthetic tensors
stand in for it.

Conventions
-----------
* ``x``: bf16 ``[T, H]``, N(0,1) drawn in fp32 and rounded to bf16 by torch.
* ``topk_idx``: int64 ``[T, K]``; ``-1`` marks "no selection" (DeepEP's marker,
  PR commit on masked top-k).  Experts of one token are distinct.
* ``topk_weights``: fp32 ``[T, K]``, softmax of N(0,1) logits over the K picks.
* ``y``: bf16 ``[rows, H]`` expert-output rows in the expert-major receive
  order; ``rows`` defaults to ``T*K`` (an upper bound on the selections), of
  which the combine reads only the first ``N_sel``.

Every tensor comes from its own sub-stream ``seed * 1000 + stream`` so that
changing one tensor's shape never shifts another's values.
"""
from __future__ import annotations

import dataclasses

import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "by_name",
    "make_x",
    "make_routing",
    "make_y",
    "tiny_expert_outputs",
    "make_expert_weights",
    "make_rows",
]

# sub-stream ids
_S_X, _S_ROUTE, _S_PERM, _S_MASK, _S_FULLMASK, _S_W, _S_Y, _S_EW, _S_RX, _S_INT = range(10)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int  # tokens
    H: int  # hidden
    K: int  # top-k
    E: int  # experts
    G: int = 1  # expert groups (1 = no grouped dedup)
    routing: str = "uniform"  # "uniform" or "zipf"
    zipf_s: float = 0.0
    mask_p: float = 0.0  # per-entry probability of -1
    full_mask_frac: float = 0.0  # fraction of tokens with every entry -1
    fp8: bool = False  # dispatch payload is the packed fp8 row
    y_kind: str = "normal"  # "normal" or "tiny_scaled" (rows x (1+e/16))
    seed: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = (
    Workload("tiny", T=128, H=256, K=2, E=16, y_kind="tiny_scaled"),
    Workload("mid", T=4096, H=4096, K=4, E=64),
    Workload("pages", T=8192, H=7168, K=8, E=256, fp8=True),
    Workload(
        "skewed_masked",
        T=8192,
        H=7168,
        K=8,
        E=256,
        routing="zipf",
        zipf_s=1.2,
        mask_p=0.1,
        full_mask_frac=0.01,
    ),
    Workload("grouped", T=65536, H=7168, K=8, E=256, G=8),
)


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def _gen(w: Workload, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000 + stream)
    return g


def make_x(w: Workload, device="cpu") -> torch.Tensor:
    """bf16 [T, H], N(0,1) rounded to bf16."""
    g = _gen(w, _S_X, device)
    return torch.randn(w.T, w.H, generator=g, device=device, dtype=torch.float32).to(
        torch.bfloat16
    )


def make_routing(w: Workload, device="cpu"):
    """(topk_idx int64 [T,K], topk_weights fp32 [T,K]).

    Uniform: K distinct experts per token, every subset equally likely
    (top-K of i.i.d. uniforms).  Zipf: expert of popularity rank r has weight
    r^-s over a seeded random permutation of the experts; K distinct experts
    are drawn without replacement proportionally to it (Gumbel top-K).  Then
    each entry is set to -1 with probability ``mask_p`` and
    ``round(full_mask_frac * T)`` distinct tokens are masked entirely.
    """
    T, K, E = w.T, w.K, w.E
    if K > E:
        raise ValueError("K distinct experts need K <= E")
    g = _gen(w, _S_ROUTE, device)
    if w.routing == "uniform":
        keys = torch.rand(T, E, generator=g, device=device)
    elif w.routing == "zipf":
        gp = _gen(w, _S_PERM, device)
        perm = torch.randperm(E, generator=gp, device=device)
        ranks = torch.empty(E, device=device, dtype=torch.float64)
        ranks[perm] = torch.arange(1, E + 1, device=device, dtype=torch.float64)
        logp = (-w.zipf_s * torch.log(ranks)).to(torch.float32)
        u = torch.rand(T, E, generator=g, device=device).clamp_(min=1e-20)
        keys = logp[None, :] - torch.log(-torch.log(u))
    else:
        raise ValueError(w.routing)
    idx = keys.topk(K, dim=1).indices.to(torch.int64)
    if w.mask_p > 0:
        gm = _gen(w, _S_MASK, device)
        m = torch.rand(T, K, generator=gm, device=device) < w.mask_p
        idx[m] = -1
    nfull = int(round(w.full_mask_frac * T))
    if nfull > 0:
        gf = _gen(w, _S_FULLMASK, device)
        toks = torch.randperm(T, generator=gf, device=device)[:nfull]
        idx[toks] = -1
    gw = _gen(w, _S_W, device)
    logits = torch.randn(T, K, generator=gw, device=device, dtype=torch.float32)
    weights = torch.softmax(logits, dim=1).contiguous()
    return idx.contiguous(), weights


def make_y(w: Workload, rows: int | None = None, device="cpu") -> torch.Tensor:
    """bf16 [rows, H] expert-output rows, N(0,1); rows defaults to T*K."""
    if rows is None:
        rows = w.T * w.K
    g = _gen(w, _S_Y, device)
    return torch.randn(rows, w.H, generator=g, device=device, dtype=torch.float32).to(
        torch.bfloat16
    )


def tiny_expert_outputs(recv: torch.Tensor, row_expert: torch.Tensor) -> torch.Tensor:
    """Tiny workload's expert outputs: each dispatched row times (1 + e/16).

    ``recv`` bf16 [N, H] holds dispatched rows in receive order and
    ``row_expert`` int [N] the expert each row belongs to.  The product is
    taken in fp32 and rounded to bf16 by torch.  This is a stand-in for an
    expert network, not part of dispatch or combine.
    """
    f = 1.0 + row_expert.to(torch.float32) / 16.0
    return (recv.to(torch.float32) * f[:, None]).to(torch.bfloat16)



def make_expert_weights(w: Workload, n_out: int, device="cpu") -> torch.Tensor:
    """bf16 [E, n_out, H] random expert weights, N(0, 1/H), so a row of N(0,1)
    inputs maps to outputs of unit scale (random init: no trained weights)."""
    g = _gen(w, _S_EW, device)
    out = torch.empty(w.E, n_out, w.H, dtype=torch.bfloat16, device=device)
    for e in range(w.E):  # one expert at a time keeps the fp32 temporary small
        out[e] = (torch.randn(n_out, w.H, generator=g, device=device) * w.H**-0.5).to(torch.bfloat16)
    return out


def make_rows(w: Workload, rows: int, device="cpu") -> torch.Tensor:
    """bf16 [rows, H] N(0,1) receive rows for a consumer of the dispatch."""
    g = _gen(w, _S_RX, device)
    return torch.randn(rows, w.H, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_small_ints(w: Workload, shape, lo: int = -2, hi: int = 2, stream: int = 0,
                    device="cpu") -> torch.Tensor:
    """bf16 tensor of integers drawn uniformly from [lo, hi]: products and
    sums of a few thousand of them are exact in fp32, so any summation order
    gives the same value."""
    g = _gen(w, _S_INT * 16 + stream, device)
    return torch.randint(lo, hi + 1, tuple(shape), generator=g, device=device).to(torch.bfloat16)
