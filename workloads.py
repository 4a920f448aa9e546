"""Seeded synthetic inputs for 64-token block-sparse (VSA) attention.

This module only draws random inputs; it holds none of the attention arithmetic. Both the CPU
oracle (``oracle/``) and the HIP path (through ``block_sparse_attention_attn_amd``) take their
inputs from here, so the two sides see bit-identical tensors.

The workloads mirror the test generator on the FastVideo sm_100a backward test page
(``make_case``: randn bf16 q/k/v/grad_o, per-q-block random distinct kv selections sorted
ascending, full or ragged ``variable_block_sizes``, a kv pool that leaves some kv blocks
unselected) and its 65536-token stability case (1024 kv blocks, 12.5 % density, top-k 128).

Draw order (fixed, so a case is reproducible from its seed): q, k, v, dO as fp32 ``randn`` on a
CPU ``torch.Generator`` rounded to bf16 (round-to-nearest-even), then per (b, h, q-block) the
top-k size (only where it varies), then the selection ``randperm(pool)[:topk]`` sorted ascending.
Activation tensors above 2**27 elements (the 524k-token workload) are drawn in 2**24-element
chunks, chunk c of tensor t (q, k, v, dO = 0..3) from its own generator seeded
seed * 1000003 + t * 65536 + c, so they can be drawn in parallel.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

BLOCK = 64
HEAD_DIM = 128


@dataclass
class Case:
    """One synthetic problem. Activations are [B, H, S, 128] bf16 (BHSD, contiguous); metadata int32."""
    name: str
    B: int
    H: int
    nb: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor
    q2k_idx: torch.Tensor          # [B, H, nb, K] int32, rows padded with 0 past q2k_num
    q2k_num: torch.Tensor          # [B, H, nb] int32
    vbs: torch.Tensor              # [nb] int32 valid kv tokens per block (<= 64)
    sm_scale: float = field(default=1.0 / HEAD_DIM ** 0.5)

    @property
    def S(self) -> int:
        return self.nb * BLOCK

    @property
    def pairs(self) -> int:
        """Selected (q block, kv block) pairs: the unit of the selected-block FLOP count."""
        return int(self.q2k_num.to(torch.int64).sum())


# The five workloads (BHSD, head_dim 128, bf16), by number.
CONFIG_TEXT = {
    1: "B=1 H=1 S=256 (4 blocks), top-k 2, all blocks full",
    2: "B=2 H=2 S=1024 (16 blocks), top-k in {1,2,3,5,7}, kv blocks 4 and 11 unselected, "
       "vbs[7]=50, vbs[15]=37",
    3: "B=1 H=8 S=32768 (512 blocks), 25% density (top-k 128), all blocks full",
    4: "B=1 H=8 S=65536 (1024 blocks), 12.5% density (top-k 128), all blocks full",
    5: "B=1 H=8 S=524288 (8192 blocks), 25% density (top-k 2048), inputs x0.5, "
       "last block 40 valid tokens",
}


# Tensors with more elements than this are drawn in fixed chunks, each from its own generator,
# on a thread pool (the single-stream draw runs at ~5e7 samples/s, a minute for 524k tokens).
CHUNKED_ABOVE = 1 << 27
CHUNK = 1 << 24


def _randn_bf16(shape, gen: torch.Generator, scale: float = 1.0, *, seed: int = 0,
                tensor: int = 0) -> torch.Tensor:
    numel = 1
    for d in shape:
        numel *= d
    if numel <= CHUNKED_ABOVE:
        x = torch.randn(shape, generator=gen, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)  # a power of two: exact, so rounding before or after is the same
        return x.to(torch.bfloat16)
    # chunk c of tensor t comes from generator seed * 1000003 + t * 65536 + c: the result does
    # not depend on the number of threads
    from concurrent.futures import ThreadPoolExecutor
    out = torch.empty(numel, dtype=torch.bfloat16)

    def draw(c):
        g = torch.Generator(device="cpu")
        g.manual_seed(seed * 1000003 + tensor * 65536 + c)
        lo = c * CHUNK
        n = min(CHUNK, numel - lo)
        x = torch.randn(n, generator=g, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        out[lo:lo + n] = x.to(torch.bfloat16)

    chunks = (numel + CHUNK - 1) // CHUNK
    with ThreadPoolExecutor(max_workers=min(16, torch.get_num_threads(), chunks)) as ex:
        list(ex.map(draw, range(chunks)))
    return out.view(shape)


def _select(gen: torch.Generator, rows: int, pool: torch.Tensor, topk: Sequence[int] | int,
            width: int) -> torch.Tensor:
    """Per row: ``randperm(len(pool))[:topk_r]`` of the pool, sorted ascending, padded with 0."""
    out = torch.zeros((rows, width), dtype=torch.int32)
    n = pool.numel()
    fixed = isinstance(topk, int)
    for r in range(rows):
        t = topk if fixed else int(topk[r])
        pick = pool[torch.randperm(n, generator=gen)[:t]]
        out[r, :t] = pick.sort().values.to(torch.int32)
    return out


def make_case(B: int, H: int, nb: int, topk, *, seed: int, kv_pool: Optional[Sequence[int]] = None,
              vbs: Optional[Sequence[int]] = None, scale: float = 1.0, topk_choices=None,
              name: str = "custom") -> Case:
    """General generator.

    ``topk`` is an int, or None with ``topk_choices`` given: then each (b, h, q block) draws its
    top-k uniformly from ``topk_choices`` (one ``randint`` over all rows, before the selections).
    ``kv_pool`` restricts which kv blocks may be selected. ``vbs`` defaults to all 64.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    S = nb * BLOCK
    shape = (B, H, S, HEAD_DIM)
    q = _randn_bf16(shape, gen, scale, seed=seed, tensor=0)
    k = _randn_bf16(shape, gen, scale, seed=seed, tensor=1)
    v = _randn_bf16(shape, gen, scale, seed=seed, tensor=2)
    do = _randn_bf16(shape, gen, scale, seed=seed, tensor=3)
    pool = torch.arange(nb) if kv_pool is None else torch.as_tensor(list(kv_pool))
    rows = B * H * nb
    if topk is None:
        choices = torch.as_tensor(list(topk_choices), dtype=torch.int64)
        pick = torch.randint(0, choices.numel(), (rows,), generator=gen)
        ks = choices[pick]
        width = int(choices.max())
        assert width <= pool.numel()
        idx = _select(gen, rows, pool, ks.tolist(), width)
        num = ks.to(torch.int32)
    else:
        assert topk <= pool.numel()
        idx = _select(gen, rows, pool, topk, topk)
        num = torch.full((rows,), topk, dtype=torch.int32)
    vbs_t = torch.full((nb,), BLOCK, dtype=torch.int32)
    if vbs is not None:
        vbs_t = torch.as_tensor(list(vbs), dtype=torch.int32)
        assert vbs_t.numel() == nb
    return Case(name=name, B=B, H=H, nb=nb, q=q, k=k, v=v, do=do,
                q2k_idx=idx.view(B, H, nb, -1).contiguous(), q2k_num=num.view(B, H, nb).contiguous(),
                vbs=vbs_t)


def config(n: int, seed: Optional[int] = None) -> Case:
    """Workload ``n`` (1..5); the seed defaults to ``n``."""
    seed = n if seed is None else seed
    if n == 1:
        return make_case(1, 1, 4, 2, seed=seed, name="c1")
    if n == 2:
        vbs = [BLOCK] * 16
        vbs[7] = 50
        vbs[15] = 37
        pool = [kb for kb in range(16) if kb not in (4, 11)]
        return make_case(2, 2, 16, None, topk_choices=(1, 2, 3, 5, 7), seed=seed, kv_pool=pool,
                         vbs=vbs, name="c2")
    if n == 3:
        return make_case(1, 8, 512, 128, seed=seed, name="c3")
    if n == 4:
        return make_case(1, 8, 1024, 128, seed=seed, name="c4")
    if n == 5:
        vbs = [BLOCK] * 8192
        vbs[-1] = 40
        return make_case(1, 8, 8192, 2048, seed=seed, vbs=vbs, scale=0.5, name="c5")
    raise ValueError(f"no workload {n}")
