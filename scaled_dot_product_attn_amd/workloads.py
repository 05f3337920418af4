"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path and the fp64 oracle are fed the exact
tensors produced here.  Every draw is made on a CPU ``torch.Generator`` so the
values do not depend on where they are sent afterwards; floating-point draws
are float32 ``randn`` rounded to bfloat16 (round-to-nearest-even) where the
workload is bf16.

Workloads (the shapes of the pages' use cases; no dataset is involved):

* ``tiny_f32``        B=1, H=Hkv=4, Sq=Sk=128, D=64, causal, float32.
* ``gqa_causal``      B=2, H=32, Hkv=8, Sq=Sk=4096, D=128, causal, bf16.
* ``window_offset``   B=1, H=32, Hkv=8, Sq=2048 new queries after 14336 cached
                      keys (Sk=16384), window 4096, D=128, k_lengths=[16384].
* ``image_clustered`` B=1, H=Hkv=32, 4096 tokens of a 64x64 grid in raster
                      order, D=128, no mask; each key is its 4x4 patch's shared
                      N(0,1) mean plus 0.5*N(0,1) per token.  Stands in for the
                      image self-attention of a 1024x1024 image at 64x64
                      tokens with 32 heads, whose trained weights are absent.
* ``gqa_documents``   the ``gqa_causal`` tensors (same seed, same draws) as
                      packed training sequences: each of the two 4096-token
                      sequences is cut into 16 documents at 15 distinct cut
                      points drawn uniformly from 1..4095 (ids 0..15 in order,
                      ``meta["doc"]`` (B, S) int32); attention stays causal
                      inside each document.
* ``decode_split``    B=64 sequences, H=32, Hkv=8, one query per head, D=128,
                      lengths uniform in [512, 32768], cache padded to 32768,
                      n_splits=8, TILE_N=64.
* ``decode_paged``    the same sequences (same seed, same draws) stored in a
                      paged serving cache: (num_blocks, block_size=16, Hkv=8,
                      D=128) with the physical blocks of all sequences dealt
                      from a seeded random permutation, plus spare blocks.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass
class Prefill:
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    causal: bool = False
    window: int = 0
    input_pos: int = 0
    k_lengths: torch.Tensor | None = None
    meta: dict = field(default_factory=dict)


@dataclass
class Decode:
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    lengths: torch.Tensor
    n_splits: int = 8
    meta: dict = field(default_factory=dict)


def _randn(gen, shape, dtype):
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(dtype)


def prefill_random(B, H, Hkv, Sq, Sk, D, dtype=torch.bfloat16, seed=0,
                   causal=False, window=0, input_pos=0, k_lengths=None,
                   device="cpu", name="random") -> Prefill:
    """iid N(0,1) Q, K, V drawn in that order from ``seed``."""
    gen = torch.Generator().manual_seed(seed)
    q = _randn(gen, (B, H, Sq, D), dtype)
    k = _randn(gen, (B, Hkv, Sk, D), dtype)
    v = _randn(gen, (B, Hkv, Sk, D), dtype)
    kl = None
    if k_lengths is not None:
        kl = torch.as_tensor(k_lengths, dtype=torch.int32).to(device)
    return Prefill(name, q.to(device), k.to(device), v.to(device), causal,
                   window, input_pos, kl,
                   dict(B=B, H=H, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, seed=seed))


def raster_patch_index(grid: int = 64, patch: int = 4) -> torch.Tensor:
    """Patch id of each token of a grid x grid image in raster order."""
    t = torch.arange(grid * grid)
    row, col = t // grid, t % grid
    return (row // patch) * (grid // patch) + (col // patch)


def image_clustered(B=1, H=32, grid=64, patch=4, D=128, seed=4,
                    dtype=torch.bfloat16, device="cpu") -> Prefill:
    """Clustered keys: per (head, patch) a shared mean, plus 0.5 x token noise.

    Draw order: Q, patch means (H, n_patches, D), token noise (H, S, D), V.
    """
    gen = torch.Generator().manual_seed(seed)
    S = grid * grid
    n_patches = (grid // patch) ** 2
    q = _randn(gen, (B, H, S, D), dtype)
    means = torch.randn(B, H, n_patches, D, generator=gen)
    noise = torch.randn(B, H, S, D, generator=gen)
    pid = raster_patch_index(grid, patch)
    k = (means[:, :, pid, :] + 0.5 * noise).to(dtype)
    v = _randn(gen, (B, H, S, D), dtype)
    return Prefill("image_clustered", q.to(device), k.to(device), v.to(device),
                   False, 0, 0, None,
                   dict(B=B, H=H, Hkv=H, Sq=S, Sk=S, D=D, seed=seed, grid=grid))


def decode_random(B=64, H=32, Hkv=8, D=128, smin=512, smax=32768, n_splits=8,
                  seed=5, dtype=torch.bfloat16, device="cpu", pad_value=0.0,
                  name="decode_split") -> Decode:
    """Per-sequence lengths uniform in [smin, smax], then Q, then per sequence K_b, V_b.

    The cache is (B, Hkv, smax, D) filled with ``pad_value`` past each length
    (0 by default; NaN for the poison variant).  Sequences are written one at a
    time so the host holds one sequence's draws at once.
    """
    gen = torch.Generator().manual_seed(seed)
    lengths = torch.randint(smin, smax + 1, (B,), generator=gen, dtype=torch.int64)
    q = _randn(gen, (B, H, D), dtype)
    k = torch.full((B, Hkv, smax, D), pad_value, dtype=dtype, device=device)
    v = torch.full((B, Hkv, smax, D), pad_value, dtype=dtype, device=device)
    for b in range(B):
        n = int(lengths[b])
        k[b, :, :n] = _randn(gen, (Hkv, n, D), dtype).to(device)
        v[b, :, :n] = _randn(gen, (Hkv, n, D), dtype).to(device)
    return Decode(name, q.to(device), k, v,
                  lengths.to(torch.int32).to(device), n_splits,
                  dict(B=B, H=H, Hkv=Hkv, Smax=smax, D=D, seed=seed))


@dataclass
class PagedDecode:
    name: str
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_tables: torch.Tensor
    lengths: torch.Tensor
    n_splits: int = 8
    meta: dict = field(default_factory=dict)


def decode_paged(B=64, H=32, Hkv=8, D=128, smin=512, smax=32768, block_size=16,
                 n_splits=8, seed=5, dtype=torch.bfloat16, device="cpu",
                 pad_value=0.0, spare_blocks=64, name="decode_paged") -> PagedDecode:
    """The draws of ``decode_random`` (same seed, same order) in a paged cache.

    Cache (num_blocks, block_size, Hkv, D), num_blocks = sum of ceil(len /
    block_size) + spare_blocks.  Physical blocks are dealt to the sequences'
    logical blocks in order from a random permutation drawn on a second
    generator, so K/V values equal ``decode_random``'s.  Unused token slots and
    spare blocks hold ``pad_value``; unused table entries are -1.
    """
    gen = torch.Generator().manual_seed(seed)
    perm_gen = torch.Generator().manual_seed(seed * 7919 + 1)
    lengths = torch.randint(smin, smax + 1, (B,), generator=gen, dtype=torch.int64)
    q = _randn(gen, (B, H, D), dtype)
    nblk = [(int(n) + block_size - 1) // block_size for n in lengths]
    num_blocks = sum(nblk) + spare_blocks
    perm = torch.randperm(num_blocks, generator=perm_gen)
    max_blocks = max((smax + block_size - 1) // block_size, 1)
    tables = torch.full((B, max_blocks), -1, dtype=torch.int32)
    kc = torch.full((num_blocks, block_size, Hkv, D), pad_value, dtype=dtype, device=device)
    vc = torch.full((num_blocks, block_size, Hkv, D), pad_value, dtype=dtype, device=device)
    pos = 0
    for b in range(B):
        n, nb = int(lengths[b]), nblk[b]
        phys = perm[pos:pos + nb]
        pos += nb
        tables[b, :nb] = phys.to(torch.int32)
        for cache in (kc, vc):
            x = torch.full((Hkv, nb * block_size, D), pad_value, dtype=dtype)
            x[:, :n] = _randn(gen, (Hkv, n, D), dtype)
            cache[phys.to(device)] = x.view(Hkv, nb, block_size, D).permute(1, 2, 0, 3).to(device)
    return PagedDecode(name, q.to(device), kc, vc, tables.to(device),
                       lengths.to(torch.int32).to(device), n_splits,
                       dict(B=B, H=H, Hkv=Hkv, D=D, block_size=block_size,
                            num_blocks=num_blocks, max_blocks=max_blocks, seed=seed))


def document_ids(B: int, S: int, n_docs: int, seed: int) -> torch.Tensor:
    """(B, S) int32 ids of packed sequences: each of the B rows of S tokens is
    cut into n_docs documents at n_docs - 1 distinct cut points drawn
    uniformly from 1..S-1; the documents take ids 0, 1, ... in order."""
    gen = torch.Generator().manual_seed(seed)
    out = torch.empty(B, S, dtype=torch.int32)
    for b in range(B):
        cuts = torch.sort(torch.randperm(S - 1, generator=gen)[:n_docs - 1] + 1).values
        edges = [0] + cuts.tolist() + [S]
        for d, (a, c) in enumerate(zip(edges, edges[1:])):
            out[b, a:c] = d
    return out


def documents_of(w: Prefill, n_docs: int = 16, seed: int = 9) -> torch.Tensor:
    """The ``gqa_documents`` ids for a prefill of that shape, on its device."""
    return document_ids(w.q.shape[0], w.k.shape[2], n_docs, seed).to(w.q.device)


def make(name: str, device="cpu"):
    """The five named workloads at their full sizes."""
    if name == "tiny_f32":
        return prefill_random(1, 4, 4, 128, 128, 64, torch.float32, seed=1,
                              causal=True, device=device, name=name)
    if name == "gqa_causal":
        return prefill_random(2, 32, 8, 4096, 4096, 128, torch.bfloat16, seed=2,
                              causal=True, device=device, name=name)
    if name == "window_offset":
        return prefill_random(1, 32, 8, 2048, 16384, 128, torch.bfloat16, seed=3,
                              causal=True, window=4096, input_pos=14336,
                              k_lengths=[16384], device=device, name=name)
    if name == "gqa_documents":
        w = make("gqa_causal", device=device)
        w.name = name
        w.meta["doc"] = documents_of(w)
        return w
    if name == "image_clustered":
        return image_clustered(device=device)
    if name == "decode_split":
        return decode_random(device=device)
    if name == "decode_paged":
        return decode_paged(device=device)
    raise KeyError(name)


NAMES = ("tiny_f32", "gqa_causal", "gqa_documents", "window_offset", "image_clustered",
         "decode_split", "decode_paged")
