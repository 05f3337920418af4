"""Plain fp64 CPU oracle for masked multi-head attention and split-KV decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this module imports nothing from the product package: the two share no code.

Everything here is written out from the definitions on the pages, slowly and
plainly, in float64 NumPy:

* the attention statement: the output is the softmax of the scaled, masked
  query-key scores applied to the values (Tylo.jl "Primitives", ``attention!``;
  vllm_mlx.attention, ``MLXAttentionImpl.forward`` calling
  ``scaled_dot_product_attention`` with ``scale``);
* the default scale 1/sqrt(Dk) (Tylo.jl "Primitives", ``flex_attention!``
  keyword ``qk_scale``);
* masks are additive, 0 where a pair attends and -inf where it is blocked, of
  shape (1, 1, Sq, offset + Sq) (mlx-arsenal "Attention", ``causal_mask`` and
  ``sliding_window_mask``, and the ``video_masks`` module note);
* causal means key position <= query position, with absolute positions shifted
  by ``input_pos`` (Tylo.jl "Primitives", ``CausalMask`` and ``attention!``
  keyword ``input_pos``);
* a sliding window of ``window_size`` lets a query see at most that many
  previous positions, itself included (mlx-arsenal "Attention",
  ``sliding_window_mask``);
* keys at or past ``k_lengths[b]`` are invalid (Tylo.jl "Primitives",
  ``attention!`` keyword ``k_lengths``);
* grouped-query attention: Heads is a multiple of Heads_KV (Tylo.jl
  "Primitives", ``flex_attention!``);
* the saved softmax statistics M (row max) and L (row sum of exp) (Tylo.jl
  "Primitives", ``attention!`` keyword ``checkpoints``), returned here as
  LSE = M + ln L;
* split-KV decode: one query per head and sequence, valid KV length per
  sequence, the cache processed as ``n_splits`` slices (Tylo.jl "Primitives",
  ``decode_attention!``);
* the backward: input gradients from the output gradient (Tylo.jl
  "Primitives", ``∇attention!``);
* the flex variants: ``SoftCapScore``, ``AliBiScore``, ``BiasScore``,
  ``PrefixMask`` / ``prefix_lm``, ``DocumentMask`` and ``q_lengths``
  (Tylo.jl "Primitives", ``flex_attention!`` and its mods), and the coarse
  block classes of a mask (Tylo.jl "Primitives", ``BlockMask`` /
  ``build_block_mask``);
* block-sparse prefill: centroid / radius-bounded (RBS) and min/max block
  scores, relative and top-k block masks, attention on the kept blocks
  (mlx-arsenal "Radius-bounded block scores (RBS)");
* the paged KV cache of a serving engine: a (num_blocks, block_size,
  num_kv_heads, head_size) cache addressed through per-sequence block tables
  and ``seq_lens`` (vllm_mlx.attention, ``get_kv_cache_shape`` and
  ``MLXAttentionMetadata``).

Readings taken where the pages are silent or disagree (each is listed in the
repository's design notes):

* window width: the mlx-arsenal reading (at most ``window`` keys, itself
  included), i.e. keys j with p - window + 1 <= j <= p.  Tylo's
  ``SlidingWindowMask(w)`` (q - w <= kv <= q) is this mask with window = w + 1;
* GQA grouping: query head h reads KV head h // (H // Hkv);
* a window is only defined together with causal masking; window > 0 without
  causal is rejected;
* a row with no allowed key has output 0 and LSE = -inf;
* ``k_lengths`` / ``lengths`` values are clamped to [0, Sk];
* the decode slices hold C = ceil(ceil(len / TILE_N) / n_splits) * TILE_N keys
  each; the slice merge weighs each slice by exp(LSE_s - max LSE);
* flex: score mods act on the scaled score, bias and ALiBi are added first
  and soft-capping comes last; ALiBi adds slope * (q - kv) literally, with
  absolute positions; the bias is indexed by the local query row; doc_q
  holds the document ids of the Sq query rows (row i at absolute position
  input_pos + i, so a single id vector doc of a whole sequence gives
  doc_q[i] = doc[input_pos + i] and doc_kv[j] = doc[j]);
  a prefix ORs keys j < prefix into the causal / window set (with a window
  a row may then see two key intervals); rows at or past q_lengths[b] attend
  to nothing;
* block classes: a block counts only the rows and keys that exist (a ragged
  last block is classed on its existing pairs);
* block scores: radius quantiles per KV head with linear interpolation; a
  ragged last block summarises its existing keys; top-k ties go to the lower
  block index;
* block tables: entry i of a sequence's row names the physical block holding
  its tokens [i * block_size, (i + 1) * block_size); a paged length is clamped
  to [0, max_blocks * block_size].

Layouts are row-major: Q/O (B, H, Sq, D), K/V (B, Hkv, Sk, D), LSE (B, H, Sq);
decode Q/O (B, H, D), K/V (B, Hkv, Smax, D).  This is Tylo's column-major
(D, S, H, B) read in row-major order.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf

# Tile classes of the block plan (Tylo.jl "Primitives", ``BlockMask``): a
# (query tile, key tile) pair is empty (no allowed pair), full (every pair
# allowed) or partial.
TILE_EMPTY = 0
TILE_PARTIAL = 1
TILE_FULL = 2


# ---------------------------------------------------------------------------
# masks
# ---------------------------------------------------------------------------

def _check_mask_args(causal: bool, window: int) -> None:
    if window > 0 and not causal:
        raise ValueError("a sliding window is defined only for causal attention")


def allowed_mask(Sq: int, Sk: int, causal: bool = False, window: int = 0,
                 input_pos: int = 0, k_len: int | None = None) -> np.ndarray:
    """Boolean (Sq, Sk) matrix: True where query i may attend to key j.

    Query i sits at absolute position p = input_pos + i (Tylo ``attention!``
    keyword ``input_pos``; mlx-arsenal ``causal_mask`` offset = cached KV
    length).  Conditions, all of which must hold:

    * j < k_len                 (``k_lengths``, clamped to [0, Sk])
    * j <= p        if causal   (``CausalMask``: q >= kv)
    * j >= p - window + 1  if window > 0  (``sliding_window_mask``: at most
      ``window`` positions including itself)
    """
    _check_mask_args(causal, window)
    kl = Sk if k_len is None else min(max(int(k_len), 0), Sk)
    i = np.arange(Sq, dtype=np.int64)[:, None]
    j = np.arange(Sk, dtype=np.int64)[None, :]
    p = input_pos + i
    ok = j < kl
    if causal:
        ok = ok & (j <= p)
    if window > 0:
        ok = ok & (j >= p - window + 1)
    return np.broadcast_to(ok, (Sq, Sk)).copy()


def additive_mask(seq_len: int, offset: int = 0, window: int = 0) -> np.ndarray:
    """The mlx-arsenal causal / sliding-window mask as an additive array.

    Shape (1, 1, seq_len, offset + seq_len); 0.0 where attention is allowed and
    -inf where it is blocked (mlx-arsenal "Attention", ``causal_mask`` and
    ``sliding_window_mask``).  The queries are the last ``seq_len`` positions
    of an ``offset + seq_len`` long key sequence.
    """
    ok = allowed_mask(seq_len, offset + seq_len, causal=True, window=window,
                      input_pos=offset)
    m = np.where(ok, 0.0, NEG_INF)
    return m.reshape(1, 1, seq_len, offset + seq_len)


def tile_plan_ref(Sq: int, Sk: int, causal: bool, window: int, input_pos: int,
                  k_len: int | None, tile_m: int, tile_n: int) -> np.ndarray:
    """Per (query tile, key tile) class: empty, partial or full.

    A tile covers the existing query rows [qt*tile_m, min(Sq, (qt+1)*tile_m))
    and the nominal key range [kt*tile_n, (kt+1)*tile_n); keys at or past Sk do
    not exist and so are never allowed.  Empty: no allowed pair.  Full: every
    (existing row, nominal key) pair allowed.  Partial: anything else.  This is
    Tylo's ``BlockMask`` notion evaluated by brute force from the element mask.
    """
    nqt = -(-Sq // tile_m)
    nkt = -(-Sk // tile_n)
    pad_k = nkt * tile_n
    ok = np.zeros((Sq, pad_k), dtype=bool)
    ok[:, :Sk] = allowed_mask(Sq, Sk, causal, window, input_pos, k_len)
    plan = np.empty((nqt, nkt), dtype=np.int8)
    for qt in range(nqt):
        rows = ok[qt * tile_m:min(Sq, (qt + 1) * tile_m)]
        for kt in range(nkt):
            blk = rows[:, kt * tile_n:(kt + 1) * tile_n]
            if not blk.any():
                plan[qt, kt] = TILE_EMPTY
            elif blk.all():
                plan[qt, kt] = TILE_FULL
            else:
                plan[qt, kt] = TILE_PARTIAL
    return plan


# ---------------------------------------------------------------------------
# attention, step by step
# ---------------------------------------------------------------------------

def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * q @ k^T for q (n, D), k (Sk, D)."""
    return scale * (q @ k.T)


def apply_mask(s: np.ndarray, ok: np.ndarray) -> np.ndarray:
    """Blocked pairs get -inf (additive 0 / -inf mask)."""
    return np.where(ok, s, NEG_INF)


def softmax_stats(s: np.ndarray):
    """Numerically stable row softmax of masked scores.

    Returns (P, M, L): M the row max, L = sum exp(s - M), P = exp(s - M) / L.
    A row with no finite score has M = -inf, L = 0 and P = 0 (the reading for
    fully masked rows).
    """
    M = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], NEG_INF)
    finite = np.isfinite(M)
    M_safe = np.where(finite, M, 0.0)
    E = np.exp(s - M_safe[:, None])          # exp(-inf) = 0 for blocked pairs
    E[~finite] = 0.0
    L = E.sum(axis=1)
    P = np.zeros_like(E)
    P[finite] = E[finite] / L[finite, None]
    return P, M, L


def combine(P: np.ndarray, v: np.ndarray) -> np.ndarray:
    """O = P @ V."""
    return P @ v


def lse_from_stats(M: np.ndarray, L: np.ndarray) -> np.ndarray:
    """LSE = M + ln L; -inf for a row without allowed keys."""
    out = np.full(M.shape, NEG_INF)
    ok = L > 0
    out[ok] = M[ok] + np.log(L[ok])
    return out


def attn_ref(Q, K, V, causal: bool = False, window: int = 0, input_pos: int = 0,
             k_lengths=None, scale: float | None = None, heads=None, rows=None,
             row_chunk: int = 1024):
    """Masked grouped-query attention forward in float64.

    Q (B, H, Sq, D); K, V (B, Hkv, Sk, D); returns (O, LSE) with O (B, H, Sq, D)
    float64 and LSE (B, H, Sq) float64.  ``heads`` (iterable of (b, h)) and
    ``rows`` (array of query indices) restrict the work to a sample; entries
    not computed are left as NaN.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, Sq, D = Q.shape
    Bk, Hkv, Sk, Dk = K.shape
    if Bk != B or Dk != D or V.shape[:3] != K.shape[:3]:
        raise ValueError("shape mismatch between Q, K and V")
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError("Heads must be a multiple of Heads_KV")
    _check_mask_args(causal, window)
    G = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Dv = V.shape[3]
    O = np.full((B, H, Sq, Dv), np.nan)
    LSE = np.full((B, H, Sq), np.nan)
    row_idx = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    masks = {}
    for b, h in pairs:
        if b not in masks:
            kl = None if k_lengths is None else int(k_lengths[b])
            masks[b] = allowed_mask(Sq, Sk, causal, window, input_pos, kl)
        g = h // G
        for c0 in range(0, len(row_idx), row_chunk):
            r = row_idx[c0:c0 + row_chunk]
            s = apply_mask(scores(Q[b, h, r], K[b, g], scale), masks[b][r])
            P, M, L = softmax_stats(s)
            O[b, h, r] = combine(P, V[b, g])
            LSE[b, h, r] = lse_from_stats(M, L)
    return O, LSE


def decode_ref(Q, K, V, lengths, scale: float | None = None, batches=None):
    """Single-query decode attention in float64: the plain definition.

    Q (B, H, D); K, V (B, Hkv, Smax, D); lengths (B,).  Sequence b attends to
    its keys j < clamp(lengths[b], 0, Smax) (Tylo ``decode_attention!``;
    vllm_mlx ``MLXAttentionMetadata.seq_lens``).  The result does not depend on
    how the cache is split.  Returns (O (B, H, D), LSE (B, H)).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, D = Q.shape
    _, Hkv, Smax, _ = K.shape
    if H % Hkv != 0:
        raise ValueError("Heads must be a multiple of Heads_KV")
    G = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = np.full((B, H, V.shape[3]), np.nan)
    LSE = np.full((B, H), np.nan)
    for b in (range(B) if batches is None else batches):
        n = min(max(int(lengths[b]), 0), Smax)
        for h in range(H):
            g = h // G
            s = scores(Q[b, h][None, :], K[b, g, :n], scale)
            P, M, L = softmax_stats(s)
            O[b, h] = combine(P, V[b, g, :n])[0] if n else 0.0
            LSE[b, h] = lse_from_stats(M, L)[0]
    return O, LSE


def split_bounds(length: int, n_splits: int, tile_n: int):
    """Key ranges of the decode slices: C = ceil(ceil(len/TILE_N)/n_splits)*TILE_N."""
    tiles = -(-length // tile_n)
    per = -(-tiles // n_splits) * tile_n
    return [(s * per, min((s + 1) * per, length)) for s in range(n_splits)]


def decode_split_ref(Q, K, V, lengths, n_splits: int, tile_n: int = 64,
                     scale: float | None = None):
    """Flash-Decoding in float64: per-slice softmax, then an LSE-weighted merge.

    Each slice s yields a normalised partial output O_s and LSE_s over its keys
    (LSE_s = -inf for an empty slice).  The merge takes M = max_s LSE_s,
    w_s = exp(LSE_s - M) and O = sum_s w_s O_s / sum_s w_s, which is the
    softmax over the union of the slices.  Used to pin the merge algebra.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, D = Q.shape
    _, Hkv, Smax, _ = K.shape
    G = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = np.zeros((B, H, V.shape[3]))
    LSE = np.full((B, H), NEG_INF)
    for b in range(B):
        n = min(max(int(lengths[b]), 0), Smax)
        for h in range(H):
            g = h // G
            parts = []
            for lo, hi in split_bounds(n, n_splits, tile_n):
                if hi <= lo:
                    parts.append((np.zeros(V.shape[3]), NEG_INF))
                    continue
                s = scores(Q[b, h][None, :], K[b, g, lo:hi], scale)
                P, M, L = softmax_stats(s)
                parts.append((combine(P, V[b, g, lo:hi])[0], lse_from_stats(M, L)[0]))
            lses = np.array([p[1] for p in parts])
            Mx = lses.max()
            if not np.isfinite(Mx):
                continue
            w = np.exp(lses - Mx)
            O[b, h] = sum(wi * oi for wi, (oi, _) in zip(w, parts)) / w.sum()
            LSE[b, h] = Mx + np.log(w.sum())
    return O, LSE


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def softmax_backward(P: np.ndarray, dP: np.ndarray) -> np.ndarray:
    """Row-wise softmax vector-Jacobian product: dS = P * (dP - sum_j dP P)."""
    return P * (dP - (dP * P).sum(axis=1, keepdims=True))


def attn_bwd_ref(Q, K, V, dO, causal: bool = False, window: int = 0, input_pos: int = 0,
                 k_lengths=None, scale: float | None = None, heads=None):
    """Gradients of the masked attention forward, in float64.

    Tylo.jl "Primitives", ``∇attention!``: from the output gradient dO (Ō) and
    the primals, the input gradients dQ, dK, dV.  Written out from the chain
    rule of O = P V with P = softmax(S), S = scale * Q K^T + mask:

      dV   = P^T dO
      dP   = dO V^T
      dS   = P * (dP - rowsum(dP * P))       (softmax Jacobian, row by row)
      dQ   = scale * dS K,   dK = scale * dS^T Q

    With GQA, a KV head's dK / dV sum the contributions of every query head
    that reads it.  Rows without an allowed key contribute nothing.  Returns
    (dQ (B, H, Sq, D), dK, dV (B, Hkv, Sk, D)); ``heads`` restricts dQ to the
    listed (b, h) pairs (dK / dV are then partial sums and not meaningful).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, H, Sq, D = Q.shape
    _, Hkv, Sk, _ = K.shape
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError("Heads must be a multiple of Heads_KV")
    _check_mask_args(causal, window)
    G = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dQ = np.full(Q.shape, np.nan)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in pairs:
        kl = None if k_lengths is None else int(k_lengths[b])
        ok = allowed_mask(Sq, Sk, causal, window, input_pos, kl)
        g = h // G
        s = apply_mask(scores(Q[b, h], K[b, g], scale), ok)
        P, _, _ = softmax_stats(s)
        dV[b, g] += P.T @ dO[b, h]
        dP = dO[b, h] @ V[b, g].T
        dS = softmax_backward(P, dP)
        dQ[b, h] = scale * (dS @ K[b, g])
        dK[b, g] += scale * (dS.T @ Q[b, h])
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# flex variants: score mods and mask mods
# ---------------------------------------------------------------------------

def flex_mask(Sq: int, Sk: int, causal: bool = False, window: int = 0,
              input_pos: int = 0, k_len: int | None = None, q_len: int | None = None,
              prefix: int = 0, doc_q=None, doc_kv=None) -> np.ndarray:
    """Boolean (Sq, Sk) mask of the flex variants (Tylo.jl "Primitives").

    * the causal / sliding-window set of ``allowed_mask`` (``CausalMask``,
      ``SlidingWindowMask``; without causal it is ``FullMask``);
    * OR keys j < prefix (``PrefixMask(len)``; ``prefix_lm(len)`` is
      ``CausalMask() | PrefixMask(len)``);
    * AND j < k_len, AND i < q_len (``k_lengths`` / ``q_lengths``: per-batch
      valid lengths; query rows at or past q_len attend to nothing);
    * AND doc_q[i] == doc_kv[j] (``DocumentMask(doc_q, doc_kv)``: a pair
      attends iff its document ids match; doc_q is indexed by the local query
      row, whose absolute position is input_pos + i).
    """
    base = allowed_mask(Sq, Sk, causal, window, input_pos, None)
    j = np.arange(Sk)[None, :]
    i = np.arange(Sq)[:, None]
    if prefix > 0:
        base = base | (j < prefix)
    kl = Sk if k_len is None else min(max(int(k_len), 0), Sk)
    ok = base & (j < kl)
    if q_len is not None:
        ok = ok & (i < min(max(int(q_len), 0), Sq))
    if doc_q is not None:
        ok = ok & (np.asarray(doc_q)[:Sq, None] == np.asarray(doc_kv)[None, :Sk])
    return np.broadcast_to(ok, (Sq, Sk)).copy()


def score_mods(s: np.ndarray, rows: np.ndarray, input_pos: int, bias=None,
               alibi_slope: float | None = None, softcap: float = 0.0) -> np.ndarray:
    """Score mods applied to scaled scores s (len(rows), Sk), in this order:

    * ``BiasScore``: s + bias[i, j] (indexed by the local query row i);
    * ``AliBiScore``: s + slope * (q - kv), q = input_pos + i the absolute query
      position and kv the key position;
    * ``SoftCapScore(cap)``: cap * tanh(s / cap), last.
    The additive mods commute; soft-capping their sum is the composition
    ``SoftCapScore ∘ ...`` (``ComposeScore`` applies its first mod first).
    """
    out = s.copy()
    Sk = s.shape[1]
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float64)[rows][:, :Sk]
    if alibi_slope is not None:
        q = (input_pos + np.asarray(rows, dtype=np.int64))[:, None]
        kv = np.arange(Sk, dtype=np.int64)[None, :]
        out = out + float(alibi_slope) * (q - kv)
    if softcap and softcap > 0:
        out = softcap * np.tanh(out / softcap)
    return out


def flex_ref(Q, K, V, causal: bool = False, window: int = 0, input_pos: int = 0,
             k_lengths=None, q_lengths=None, prefix: int = 0, softcap: float = 0.0,
             alibi_slopes=None, bias=None, doc_q=None, doc_kv=None,
             scale: float | None = None, heads=None, rows=None, row_chunk: int = 1024):
    """FlexAttention forward in float64 (Tylo.jl "Primitives", ``flex_attention!``).

    Scores s = scale * q.k (``qk_scale``, default 1/sqrt(D)); then the score
    mods of ``score_mods``; then the mask of ``flex_mask`` (-inf where
    blocked); softmax, O = P V, LSE = M + ln L.  ``bias`` is (Bb, Hb, Sq, Sk)
    with Bb in {1, B} and Hb in {1, H}, broadcast when 1 (``BiasScore``);
    ``alibi_slopes`` (H,); ``doc_q`` (B, Sq) and ``doc_kv`` (B, Sk) ints;
    ``k_lengths`` / ``q_lengths`` (B,).  Returns (O, LSE) like ``attn_ref``.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, Sq, D = Q.shape
    _, Hkv, Sk, _ = K.shape
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError("Heads must be a multiple of Heads_KV")
    _check_mask_args(causal, window)
    G = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = np.full((B, H, Sq, V.shape[3]), np.nan)
    LSE = np.full((B, H, Sq), np.nan)
    row_idx = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    masks = {}
    for b, h in pairs:
        if b not in masks:
            masks[b] = flex_mask(
                Sq, Sk, causal, window, input_pos,
                None if k_lengths is None else int(k_lengths[b]),
                None if q_lengths is None else int(q_lengths[b]), prefix,
                None if doc_q is None else np.asarray(doc_q)[b],
                None if doc_kv is None else np.asarray(doc_kv)[b])
        g = h // G
        bh = None
        if bias is not None:
            bias_a = np.asarray(bias)
            bh = bias_a[b if bias_a.shape[0] > 1 else 0, h if bias_a.shape[1] > 1 else 0]
        slope = None if alibi_slopes is None else float(alibi_slopes[h])
        for c0 in range(0, len(row_idx), row_chunk):
            r = row_idx[c0:c0 + row_chunk]
            s = score_mods(scores(Q[b, h, r], K[b, g], scale), r, input_pos, bh, slope,
                           softcap)
            s = apply_mask(s, masks[b][r])
            P, M, L = softmax_stats(s)
            O[b, h, r] = combine(P, V[b, g])
            LSE[b, h, r] = lse_from_stats(M, L)
    return O, LSE


def block_mask_ref(ok, tile_m: int = 64, tile_n: int = 64) -> np.ndarray:
    """Coarse block classes of a boolean (..., Sq, Sk) pair mask (Tylo.jl
    "Primitives", ``BlockMask`` / ``build_block_mask``): each (query block, key
    block) pair is empty, partial or full according to how many of its pairs
    attend.

    Query block qb covers the rows [qb * tile_m, (qb + 1) * tile_m) that exist
    (< Sq), key block kb the keys [kb * tile_n, (kb + 1) * tile_n) that exist
    (< Sk).  The class is 0 when no pair of the block attends, 2 when every
    pair does and 1 otherwise.  Returns uint8 (..., ceil(Sq / tile_m),
    ceil(Sk / tile_n)).  ``ok`` is the predicate evaluated at every pair, e.g.
    ``flex_mask`` (which already shifts the queries by ``input_pos``).
    """
    ok = np.asarray(ok, dtype=bool)
    Sq, Sk = ok.shape[-2:]
    nqb, nkb = -(-Sq // tile_m), -(-Sk // tile_n)
    out = np.zeros(ok.shape[:-2] + (nqb, nkb), dtype=np.uint8)
    for qb in range(nqb):
        for kb in range(nkb):
            blk = ok[..., qb * tile_m:(qb + 1) * tile_m, kb * tile_n:(kb + 1) * tile_n]
            some = blk.any(axis=(-2, -1))
            every = blk.all(axis=(-2, -1))
            out[..., qb, kb] = np.where(every, 2, np.where(some, 1, 0))
    return out


# ---------------------------------------------------------------------------
# block-sparse prefill: block-score estimators, block masks, masked attention
# ---------------------------------------------------------------------------

def key_block_stats(k: np.ndarray, block_size: int):
    """Per key block of k (Sk, D): centroid c_b, radius r_b = max ||k - c_b||_2,
    and the element-wise min / max (mlx-arsenal "Radius-bounded block scores":
    centroid summary, RBS radius, SPADE's element-wise min/max box).  The last
    block holds the remaining keys."""
    k = np.asarray(k, dtype=np.float64)
    Sk = k.shape[0]
    nb = -(-Sk // block_size)
    c = np.empty((nb, k.shape[1]))
    r = np.empty(nb)
    lo = np.empty((nb, k.shape[1]))
    hi = np.empty((nb, k.shape[1]))
    for b in range(nb):
        blk = k[b * block_size:(b + 1) * block_size]
        c[b] = blk.mean(axis=0)
        r[b] = np.sqrt(((blk - c[b]) ** 2).sum(axis=1)).max()
        lo[b] = blk.min(axis=0)
        hi[b] = blk.max(axis=0)
    return c, r, lo, hi


def radius_weights(r: np.ndarray, low: float = 0.5, high: float = 0.9) -> np.ndarray:
    """beta_b = clip((r_b - r_low) / (r_high - r_low), 0, 1) with r_low / r_high the
    `low` / `high` quantiles (linear interpolation) of one head's block radii; when
    the two coincide, beta_b = 1 for blocks strictly wider than r_low, else 0."""
    r_low = float(np.quantile(r, low))
    r_high = float(np.quantile(r, high))
    if r_high == r_low:
        return (r > r_low).astype(np.float64)
    return np.clip((r - r_low) / (r_high - r_low), 0.0, 1.0)


def _block_lse(ell: np.ndarray, block_size: int) -> np.ndarray:
    """Log of the sum of exp over each query block's tokens: ell (Sq, nk) -> (nq, nk)."""
    Sq = ell.shape[0]
    nq = -(-Sq // block_size)
    out = np.empty((nq, ell.shape[1]))
    for a in range(nq):
        rows = ell[a * block_size:(a + 1) * block_size]
        m = rows.max(axis=0)
        out[a] = m + np.log(np.exp(rows - m).sum(axis=0))
    return out


def rbs_block_scores_ref(Q, K, block_size: int = 64, low: float = 0.5, high: float = 0.9):
    """Radius-bounded block scores (mlx-arsenal "Radius-bounded block scores (RBS)").

    Per query token q and key block b: base = q.c_b / sqrt(D) and rescue =
    (q.c_b + ||q|| r_b beta_b) / sqrt(D); each block score is the log of the sum of
    exp over the query block's tokens.  Radii quantiles are taken per KV head.
    Q (B, H, Sq, D), K (B, Hkv, Sk, D); returns (base, rescue) (B, H, nq, nk).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    B, H, Sq, D = Q.shape
    Hkv = K.shape[1]
    G = H // Hkv
    nq, nk = -(-Sq // block_size), -(-K.shape[2] // block_size)
    base = np.empty((B, H, nq, nk))
    rescue = np.empty((B, H, nq, nk))
    for b in range(B):
        for g in range(Hkv):
            c, r, _, _ = key_block_stats(K[b, g], block_size)
            beta = radius_weights(r, low, high)
            for h in range(g * G, (g + 1) * G):
                qc = Q[b, h] @ c.T
                qn = np.sqrt((Q[b, h] ** 2).sum(axis=1))[:, None]
                base[b, h] = _block_lse(qc / math.sqrt(D), block_size)
                rescue[b, h] = _block_lse((qc + qn * (r * beta)[None, :]) / math.sqrt(D),
                                          block_size)
    return base, rescue


def minmax_block_scores_ref(Q, K, block_size: int = 64):
    """SPADE-style box bound: per query token, sum_d max(q_d lo_bd, q_d hi_bd) /
    sqrt(D) bounds q.k / sqrt(D) for every key of block b; block score = log-sum-exp
    over the query block's tokens.  Returns (B, H, nq, nk)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    B, H, Sq, D = Q.shape
    Hkv = K.shape[1]
    G = H // Hkv
    nq, nk = -(-Sq // block_size), -(-K.shape[2] // block_size)
    out = np.empty((B, H, nq, nk))
    for b in range(B):
        for g in range(Hkv):
            _, _, lo, hi = key_block_stats(K[b, g], block_size)
            for h in range(g * G, (g + 1) * G):
                q = Q[b, h][:, None, :]
                bound = np.maximum(q * lo[None], q * hi[None]).sum(axis=2)
                out[b, h] = _block_lse(bound / math.sqrt(D), block_size)
    return out


def relative_block_mask_ref(scores, alpha: float, dtype=np.float64) -> np.ndarray:
    """Keep the blocks whose exp(score) is at least alpha times the row maximum
    (mlx-arsenal ``relative_block_mask``), i.e. score >= max + ln(alpha).

    ``dtype`` is the precision the threshold is formed and compared in (the
    page fixes none): float64 by default; float32 takes the keep/drop decision
    exactly as a float32 implementation does (max and ln(alpha) rounded to
    float32, their sum rounded once)."""
    s = np.asarray(scores, dtype=dtype)
    return s >= s.max(axis=-1, keepdims=True) + dtype(math.log(alpha))


def top_k_block_mask_ref(scores, k: int) -> np.ndarray:
    """Keep the k highest-scoring blocks of each row (``top_k_block_mask``); equal
    scores are ranked by block index, lower first."""
    s = np.asarray(scores, dtype=np.float64)
    keep = np.zeros(s.shape, dtype=bool)
    flat = s.reshape(-1, s.shape[-1])
    kf = keep.reshape(-1, s.shape[-1])
    for row in range(flat.shape[0]):
        order = sorted(range(flat.shape[1]), key=lambda j: (-flat[row, j], j))
        kf[row, order[:k]] = True
    return keep


def band_block_mask_ref(nq: int, nk: int, diagonal: int) -> np.ndarray:
    """Forced blocks |row - col| < diagonal (the recipe's band)."""
    a = np.arange(nq)[:, None]
    c = np.arange(nk)[None, :]
    return np.abs(a - c) < diagonal


def block_sparse_attn_ref(Q, K, V, keep, block_size: int = 64, causal: bool = False,
                          window: int = 0, input_pos: int = 0, k_lengths=None,
                          heads=None, rows=None):
    """Attention restricted to the kept (query block, key block) pairs of ``keep``
    (B, H, nq, nk), together with the causal / window / k_lengths mask: a pair is
    allowed iff both allow it (the block mask expanded to tokens)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, Sq, D = Q.shape
    _, Hkv, Sk, _ = K.shape
    G = H // Hkv
    scale = 1.0 / math.sqrt(D)
    keep = np.asarray(keep, dtype=bool)
    O = np.full((B, H, Sq, V.shape[3]), np.nan)
    LSE = np.full((B, H, Sq), np.nan)
    row_idx = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    tok_q = row_idx // block_size
    tok_k = np.arange(Sk) // block_size
    for b, h in pairs:
        kl = None if k_lengths is None else int(k_lengths[b])
        ok = allowed_mask(Sq, Sk, causal, window, input_pos, kl)[row_idx]
        ok = ok & keep[b, h][tok_q][:, tok_k]
        g = h // G
        s = apply_mask(scores(Q[b, h, row_idx], K[b, g], scale), ok)
        P, M, L = softmax_stats(s)
        O[b, h, row_idx] = combine(P, V[b, g])
        LSE[b, h, row_idx] = lse_from_stats(M, L)
    return O, LSE


# ---------------------------------------------------------------------------
# paged KV cache (serving layout)
# ---------------------------------------------------------------------------

def gather_paged(cache, table_row, n: int, g: int) -> np.ndarray:
    """Logical rows 0..n-1 of KV head g of one sequence from a paged cache.

    The cache is (num_blocks, block_size, num_kv_heads, head_size)
    (vllm_mlx.attention, ``MLXAttentionBackend.get_kv_cache_shape``); the
    sequence's block table (``MLXAttentionMetadata.block_tables``) lists, for
    its i-th run of block_size tokens, the physical block holding them, so
    token t lives in block table_row[t // block_size] at slot t % block_size.
    Entries past the sequence's last block are never read.
    """
    cache = np.asarray(cache)
    bs = cache.shape[1]
    t = np.arange(n)
    blocks = np.asarray(table_row, dtype=np.int64)[t // bs]
    return np.asarray(cache[blocks, t % bs, g], dtype=np.float64)


def decode_paged_ref(Q, K_cache, V_cache, block_tables, lengths,
                     scale: float | None = None, batches=None):
    """Single-query decode over a paged KV cache, in float64.

    Q (B, H, D); K_cache, V_cache (num_blocks, block_size, Hkv, D);
    block_tables (B, max_blocks) int; lengths (B,) (``seq_lens``), clamped to
    [0, max_blocks * block_size].  Sequence b attends to its first lengths[b]
    tokens, gathered through its block table; the result is the plain decode
    of those rows.  Returns (O (B, H, D), LSE (B, H)).
    """
    Q = np.asarray(Q, dtype=np.float64)
    B, H, D = Q.shape
    _, bs, Hkv, _ = K_cache.shape
    tables = np.asarray(block_tables)
    cap = tables.shape[1] * bs
    if H % Hkv != 0:
        raise ValueError("Heads must be a multiple of Heads_KV")
    G = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = np.full((B, H, V_cache.shape[3]), np.nan)
    LSE = np.full((B, H), np.nan)
    for b in (range(B) if batches is None else batches):
        n = min(max(int(lengths[b]), 0), cap)
        for g in range(Hkv):
            kb = gather_paged(K_cache, tables[b], n, g)
            vb = gather_paged(V_cache, tables[b], n, g)
            for h in range(g * G, (g + 1) * G):
                s = scores(Q[b, h][None, :], kb, scale)
                P, M, L = softmax_stats(s)
                O[b, h] = combine(P, vb)[0] if n else 0.0
                LSE[b, h] = lse_from_stats(M, L)[0]
    return O, LSE


def allowed_pairs(Sq: int, Sk: int, causal: bool, window: int, input_pos: int,
                  k_len: int | None) -> int:
    """Number of allowed (query, key) pairs, by counting the mask."""
    return int(allowed_mask(Sq, Sk, causal, window, input_pos, k_len).sum())
