"""Seeded synthetic inputs for the ZeRO-2 shard step.

This module holds workload shapes and random-number recipes only. It does no
part of the optimizer's arithmetic (no flatten, no reduction, no Adam, no
rounding of results), so both the HIP path and the CPU oracle can be fed the
same bytes from here without sharing any of the method's code.

Recipe (applies to every workload):
  * parameters: fp32 N(0, 0.02), generator seed PARAM_SEED;
  * gradient of replica q at step t: N(0, std) drawn in fp32 with seed
    grad_seed(t, q), then rounded to the gradient dtype by torch's own
    round-to-nearest-even cast;
  * optional outliers: a Bernoulli(frac) mask drawn with seed
    mask_seed(t, q) multiplies the fp32 sample by `scale` before the cast.

Shapes follow the model families the workloads are named after (GPT-2 small,
Llama 7B / 13B / 70B dense layouts); no weights or data are involved.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import torch

PARAM_SEED = 0
PARAM_STD = 0.02


def grad_seed(t: int, q: int) -> int:
    """Seed of replica q's gradient at step t (t >= 1)."""
    return 123 + 1000 * t + q


def mask_seed(t: int, q: int) -> int:
    """Seed of replica q's outlier mask at step t."""
    return 7 + 1000 * t + q


# --------------------------------------------------------------------------
# shape lists
# --------------------------------------------------------------------------

def gpt2_small_shapes(layers: int = 12, d: int = 768, vocab: int = 50257,
                      context: int = 1024) -> List[Tuple[int, ...]]:
    """GPT-2-small parameter list: token and position embeddings, then per
    block ln_1 (w, b), attention qkv (w, b), attention proj (w, b), ln_2
    (w, b), MLP up (w, b), MLP down (w, b); final LayerNorm (w, b). The LM
    head is tied to the token embedding. 148 tensors, 124,439,808 elements."""
    shapes: List[Tuple[int, ...]] = [(vocab, d), (context, d)]
    for _ in range(layers):
        shapes += [(d,), (d,),
                   (d, 3 * d), (3 * d,),
                   (d, d), (d,),
                   (d,), (d,),
                   (d, 4 * d), (4 * d,),
                   (4 * d, d), (d,)]
    shapes += [(d,), (d,)]
    return shapes


def llama_shapes(layers: int, d: int, ffn: int, vocab: int = 32000,
                 kv_dim: Optional[int] = None,
                 trailing_scalar: bool = False) -> List[Tuple[int, ...]]:
    """Llama-style dense decoder list in the usual checkpoint order:
    embedding; per layer q, k, v, o, gate, up, down, input norm, post-attention
    norm; final norm; untied LM head. `trailing_scalar` appends one
    1-element tensor (used to force a non-multiple-of-N total)."""
    kv = d if kv_dim is None else kv_dim
    shapes: List[Tuple[int, ...]] = [(vocab, d)]
    for _ in range(layers):
        shapes += [(d, d), (kv, d), (kv, d), (d, d),
                   (ffn, d), (ffn, d), (d, ffn),
                   (d,), (d,)]
    shapes += [(d,), (vocab, d)]
    if trailing_scalar:
        shapes.append((1,))
    return shapes


def numel_of(shapes: Sequence[Tuple[int, ...]]) -> int:
    return sum(math.prod(s) for s in shapes)


def ragged_shapes(seed: int, count: int, max_numel: int) -> List[Tuple[int, ...]]:
    """Random list of 1-D/2-D shapes with odd sizes (exercise misaligned
    offsets). Deterministic in `seed`."""
    g = torch.Generator().manual_seed(seed)
    out: List[Tuple[int, ...]] = []
    for _ in range(count):
        n = int(torch.randint(1, max_numel + 1, (1,), generator=g))
        if n > 8 and int(torch.randint(0, 2, (1,), generator=g)):
            r = int(torch.randint(1, 8, (1,), generator=g))
            out.append((r, max(1, n // r)))
        else:
            out.append((n,))
    return out


# --------------------------------------------------------------------------
# random tensors
# --------------------------------------------------------------------------

def _gen(seed: int, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return g


# Large draws are made in chunks of CHUNK elements so that the fp32 scratch
# stays small; chunk c > 0 uses seed + c * 2^40 (chunk 0 uses the seed
# itself, so draws of at most CHUNK elements are one plain draw).
CHUNK = 1 << 27


def _chunk_seed(seed: int, c: int) -> int:
    return seed if c == 0 else seed + (c << 40)


def fill_gaussian(out: torch.Tensor, std: float, seed: int,
                  mseed: Optional[int] = None, frac: float = 0.01,
                  scale: float = 100.0) -> torch.Tensor:
    """Fill `out` (any float dtype, contiguous) with N(0, std) drawn in fp32
    and cast with torch's round-to-nearest-even; with `mseed`, a
    Bernoulli(frac) subset is multiplied by `scale` before the cast."""
    flat = out.view(-1)
    n = flat.numel()
    dev = out.device
    for c, start in enumerate(range(0, n, CHUNK)):
        k = min(CHUNK, n - start)
        x = torch.randn(k, generator=_gen(_chunk_seed(seed, c), dev),
                        dtype=torch.float32, device=dev)
        x.mul_(std)
        if mseed is not None:
            mask = torch.rand(k, generator=_gen(_chunk_seed(mseed, c), dev),
                              device=dev) < frac
            x[mask] *= scale
            del mask
        flat[start:start + k].copy_(x)
        del x
    return out


def gaussian(n: int, std: float, seed: int, dtype=torch.float32,
             device="cpu") -> torch.Tensor:
    """n samples of N(0, std) drawn in fp32, then cast to `dtype`."""
    out = torch.empty(n, dtype=dtype, device=device)
    return fill_gaussian(out, std, seed)


def gaussian_with_outliers(n: int, std: float, seed: int, mseed: int,
                           frac: float = 0.01, scale: float = 100.0,
                           dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """N(0, std) in fp32; a Bernoulli(frac) subset is multiplied by `scale`
    before the cast to `dtype`."""
    out = torch.empty(n, dtype=dtype, device=device)
    return fill_gaussian(out, std, seed, mseed, frac, scale)


def params(n: int, device="cpu") -> torch.Tensor:
    """Initial fp32 parameters, N(0, 0.02)."""
    return gaussian(n, PARAM_STD, PARAM_SEED, torch.float32, device)


def split_to_shapes(flat: torch.Tensor, shapes) -> List[torch.Tensor]:
    """Cut a 1-D tensor into independent contiguous tensors of `shapes`
    (each a fresh allocation, so the list is a genuine ragged list)."""
    out, off = [], 0
    for s in shapes:
        k = math.prod(s)
        out.append(flat[off:off + k].reshape(s).clone())
        off += k
    return out


def split_views(flat: torch.Tensor, shapes) -> List[torch.Tensor]:
    """Cut a 1-D tensor into contiguous views of `shapes` (no copies; for
    lists too large to duplicate)."""
    out, off = [], 0
    for s in shapes:
        k = math.prod(s)
        out.append(flat[off:off + k].view(s))
        off += k
    return out


# --------------------------------------------------------------------------
# named workloads
# --------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    numel: int
    world: int
    rank: int
    grad_dtype: torch.dtype
    grad_std: float
    steps: int
    shapes: Optional[List[Tuple[int, ...]]] = None   # tensor list, if any
    outliers: bool = False
    slice_only: bool = False      # replicas hold only this rank's slice
    lr: float = 1e-3
    betas: Tuple[float, float] = (0.9, 0.999)
    eps: float = 1e-8
    extra_ranks: Tuple[int, ...] = field(default_factory=tuple)


def workloads() -> dict:
    """The five shard-step workloads, smallest first."""
    llama13 = llama_shapes(40, 5120, 13824, trailing_scalar=True)
    return {
        "flat1m_n4": Workload(
            "flat1m_n4: 1,000,003 fp32 params, one flat tensor, N=4",
            1_000_003, 4, 0, torch.float32, 0.01, 10,
            shapes=[(1_000_003,)], extra_ranks=(3,)),
        "gpt2s_n8": Workload(
            "gpt2s_n8: GPT-2-small list (148 tensors), N=8, rank 3",
            numel_of(gpt2_small_shapes()), 8, 3, torch.bfloat16, 1e-3, 10,
            shapes=gpt2_small_shapes()),
        "flat7b_n8": Workload(
            "flat7b_n8: 7e9-element flat vector, N=8, rank 0",
            7_000_000_000, 8, 0, torch.bfloat16, 1e-3, 10,
            shapes=[(7_000_000_000,)], slice_only=True),
        "llama13b_n8": Workload(
            "llama13b_n8: Llama-13B list + 1 scalar (364 tensors), N=8, rank 7",
            numel_of(llama13), 8, 7, torch.bfloat16, 1e-3, 5,
            shapes=llama13, outliers=True),
        "flat70b_n64": Workload(
            "flat70b_n64: 70e9-element state, N=64, rank 0, slice-only replicas",
            70_000_000_000, 64, 0, torch.bfloat16, 1e-3, 3,
            slice_only=True),
    }
