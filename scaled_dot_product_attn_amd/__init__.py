"""MI355X (gfx950) fused attention: a thin Python binding over libattn_mi355x.so.

The functions below carry the names of the C entry points declared in
``include/attn.h`` and only marshal arguments: they read shapes from torch
tensors, pass raw device pointers and the current HIP stream, and turn a
non-zero status into ``RuntimeError`` (like vllm_mlx.attention's forward,
which logs and re-raises).  Every step of the computation runs in the HIP
kernels; there is no fallback.  Every tensor's shape is checked against the
sizes passed to the library (it addresses them through raw pointers).  ``fwd``
(also ``sdpa``) and ``decode`` are allocating conveniences on top.

Layouts (row-major, contiguous): prefill Q/O (B, H, Sq, D), K/V (B, Hkv, Sk, D),
LSE (B, H, Sq) float32; decode Q/O (B, H, D), K/V (B, Hkv, Smax, D).
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_mi355x.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP = 0, 1, 2, 3
TILE_M, TILE_N = 256, 64  # prefill tile sizes (ATTN_FWD_TILE_M / _N)
BLOCK = 64                 # block-sparse block size (ATTN_BLOCK)
DECODE_STATIC_SCRATCH_BYTES = 32 << 20  # ATTN_DECODE_STATIC_SCRATCH_BYTES
BLOCK_SCORES_RBS, BLOCK_SCORES_MINMAX = 0, 1
BLOCK_MASK_RELATIVE, BLOCK_MASK_TOPK, BLOCK_MASK_BAND = 0, 1, 2

_lib = None

_I = ctypes.c_int
_P = ctypes.c_void_p


class AttnFlex(ctypes.Structure):
    """attn_flex_t of include/attn.h (device pointers, NULL = mod off)."""
    _fields_ = [("q_lengths", _P), ("alibi_slopes", _P), ("bias", _P), ("doc_q", _P),
                ("doc_kv", _P), ("bias_B", _I), ("bias_H", _I), ("prefix", _I),
                ("softcap", ctypes.c_float), ("qk_scale", ctypes.c_float),
                ("block_mask", _P), ("block_mask_B", _I)]

BLOCK_EMPTY, BLOCK_PARTIAL, BLOCK_FULL = 0, 1, 2

_SIGS = {
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P]),
    "attn_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P]),
    "attn_fwd_flex": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P,
                           ctypes.POINTER(AttnFlex), _P]),
    "attn_build_block_mask": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, ctypes.POINTER(AttnFlex),
                                   _P]),
    "attn_decode": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "attn_decode_ws": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, ctypes.c_size_t, _P]),
    "attn_decode_static": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "attn_decode_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "attn_bwd_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "attn_block_scores_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "attn_block_scores": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                               ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "attn_block_mask": (_I, [_P, _P, _I, _I, _I, _I, ctypes.c_float, _I, _I, _I, _P]),
    "attn_fwd_block_sparse": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                   _P, _P, _P]),
    "attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                      _P, _P, ctypes.c_size_t, _P]),
    "attn_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P,
                               ctypes.c_size_t, _P]),
    "attn_mask_dump": (_I, [_P, _I, _I, _I, _I, _I, _I, _P]),
    "attn_tile_plan": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_version": (_I, []),
}


def lib() -> ctypes.CDLL:
    """Load libattn_mi355x.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m scaled_dot_product_attn_amd._build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def attn_status_string(status: int) -> str:
    return lib().attn_status_string(status).decode()


def attn_version() -> int:
    return lib().attn_version()


def _check(rc: int, what: str) -> None:
    if rc != ATTN_OK:
        raise RuntimeError(f"{what}: {attn_status_string(rc)} (status {rc})")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _expect(t, shape, name) -> None:
    """Raise ValueError unless tensor t (if given) has exactly this shape.

    The kernels read and write through raw pointers sized from the shape
    arguments, so a tensor of another shape would be read or written past its
    end; the C ABI cannot see tensor sizes, so the binding checks them."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _prefill_shapes(Q, K, V, O=None, LSE=None, k_lengths=None):
    """(B, H, Hkv, Sq, Sk, D) from Q (B, H, Sq, D) and K (B, Hkv, Sk, D),
    with V, O, LSE and k_lengths checked against them."""
    if Q.dim() != 4 or K.dim() != 4:
        raise ValueError("Q and K must be 4-d: (B, H, Sq, D) and (B, Hkv, Sk, D)")
    B, H, Sq, D = Q.shape
    Hkv, Sk = K.shape[1], K.shape[2]
    _expect(K, (B, Hkv, Sk, D), "K")
    _expect(V, (B, Hkv, Sk, D), "V")
    _expect(O, (B, H, Sq, D), "O")
    _expect(LSE, (B, H, Sq), "LSE")
    _expect(k_lengths, (B,), "k_lengths")
    return B, H, Hkv, Sq, Sk, D


def _fwd(name, dtype, O, Q, K, V, LSE, causal, window, input_pos, k_lengths, stream):
    B, H, Hkv, Sq, Sk, D = _prefill_shapes(Q, K, V, O, LSE, k_lengths)
    for t in (O, Q, K, V):
        if t.dtype != dtype:
            raise ValueError(f"{name} takes {dtype} tensors")
    if LSE is not None and LSE.dtype != torch.float32:
        raise ValueError("LSE must be float32")
    if k_lengths is not None and k_lengths.dtype != torch.int32:
        raise ValueError("k_lengths must be int32")
    rc = getattr(lib(), name)(_ptr(O), _ptr(Q), _ptr(K), _ptr(V), _ptr(LSE),
                              B, H, Hkv, Sq, Sk, D, int(bool(causal)), int(window),
                              int(input_pos), _ptr(k_lengths), _stream(stream))
    _check(rc, name)


def attn_fwd(O, Q, K, V, LSE=None, causal=False, window=0, input_pos=0,
             k_lengths=None, stream=None) -> None:
    """bf16 prefill forward into O (and LSE if given); see include/attn.h."""
    _fwd("attn_fwd", torch.bfloat16, O, Q, K, V, LSE, causal, window, input_pos,
         k_lengths, stream)


def attn_fwd_f32(O, Q, K, V, LSE=None, causal=False, window=0, input_pos=0,
                 k_lengths=None, stream=None) -> None:
    """float32 prefill forward into O (and LSE if given); see include/attn.h."""
    _fwd("attn_fwd_f32", torch.float32, O, Q, K, V, LSE, causal, window, input_pos,
         k_lengths, stream)


def attn_fwd_flex(O, Q, K, V, LSE=None, causal=False, window=0, input_pos=0,
                  k_lengths=None, q_lengths=None, prefix=0, softcap=0.0, alibi_slopes=None,
                  bias=None, doc_q=None, doc_kv=None, qk_scale=0.0, block_mask=None,
                  stream=None) -> None:
    """bf16 prefill with the flex mods (see attn_flex_t in include/attn.h).

    ``bias`` float32 (bias_B, bias_H, Sq, Sk) with bias_B in {1, B}, bias_H in
    {1, H}; ``alibi_slopes`` float32 (H,); ``q_lengths`` int32 (B,);
    ``doc_q`` / ``doc_kv`` int32 (B, Sq) / (B, Sk); ``block_mask`` uint8
    (1 or B, ceil(Sq/64), ceil(Sk/64)) of BLOCK_* classes (``build_block_mask``).
    """
    B, H, Hkv, Sq, Sk, D = _prefill_shapes(Q, K, V, O, LSE, k_lengths)
    _expect(q_lengths, (B,), "q_lengths")
    _expect(alibi_slopes, (H,), "alibi_slopes")
    _expect(doc_q, (B, Sq), "doc_q")
    _expect(doc_kv, (B, Sk), "doc_kv")
    if block_mask is not None and (
            block_mask.dtype != torch.uint8 or block_mask.dim() != 3
            or tuple(block_mask.shape[1:]) != (-(-Sq // BLOCK), -(-Sk // BLOCK))
            or block_mask.shape[0] not in (1, B)):
        raise ValueError("block_mask must be uint8 (1 or B, ceil(Sq/64), ceil(Sk/64))")
    for t in (O, Q, K, V):
        if t.dtype != torch.bfloat16:
            raise ValueError("attn_fwd_flex takes bfloat16 tensors")
    for t, dt, name in ((LSE, torch.float32, "LSE"), (k_lengths, torch.int32, "k_lengths"),
                        (q_lengths, torch.int32, "q_lengths"),
                        (alibi_slopes, torch.float32, "alibi_slopes"),
                        (bias, torch.float32, "bias"), (doc_q, torch.int32, "doc_q"),
                        (doc_kv, torch.int32, "doc_kv")):
        if t is not None and t.dtype != dt:
            raise ValueError(f"{name} must be {dt}")
    if bias is not None and (bias.dim() != 4 or tuple(bias.shape[2:]) != (Sq, Sk)
                             or bias.shape[0] not in (1, B) or bias.shape[1] not in (1, H)):
        raise ValueError("bias must be (bias_B, bias_H, Sq, Sk) with bias_B in {1, B}, "
                         "bias_H in {1, H}")
    f = AttnFlex(_ptr(q_lengths), _ptr(alibi_slopes), _ptr(bias), _ptr(doc_q), _ptr(doc_kv),
                 bias.shape[0] if bias is not None else 0,
                 bias.shape[1] if bias is not None else 0,
                 int(prefix), float(softcap), float(qk_scale), _ptr(block_mask),
                 block_mask.shape[0] if block_mask is not None else 0)
    rc = lib().attn_fwd_flex(_ptr(O), _ptr(Q), _ptr(K), _ptr(V), _ptr(LSE), B, H, Hkv, Sq,
                             Sk, D, int(bool(causal)), int(window), int(input_pos),
                             _ptr(k_lengths), ctypes.byref(f), _stream(stream))
    _check(rc, "attn_fwd_flex")


def attn_build_block_mask(block_mask, Sq, Sk, causal=False, window=0, input_pos=0,
                          k_lengths=None, q_lengths=None, prefix=0, doc_q=None, doc_kv=None,
                          stream=None) -> None:
    """BlockMask classes (B, ceil(Sq/64), ceil(Sk/64)) uint8 of the flex mask of
    these arguments into block_mask (see attn_build_block_mask in include/attn.h)."""
    if block_mask.dtype != torch.uint8 or block_mask.dim() != 3:
        raise ValueError("block_mask must be uint8 (B, ceil(Sq/64), ceil(Sk/64))")
    B = block_mask.shape[0]
    _expect(block_mask, (B, -(-Sq // BLOCK), -(-Sk // BLOCK)), "block_mask")
    _expect(k_lengths, (B,), "k_lengths")
    _expect(q_lengths, (B,), "q_lengths")
    _expect(doc_q, (B, Sq), "doc_q")
    _expect(doc_kv, (B, Sk), "doc_kv")
    for t, name in ((k_lengths, "k_lengths"), (q_lengths, "q_lengths"), (doc_q, "doc_q"),
                    (doc_kv, "doc_kv")):
        if t is not None and t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    f = AttnFlex(_ptr(q_lengths), None, None, _ptr(doc_q), _ptr(doc_kv), 0, 0, int(prefix),
                 0.0, 0.0, None, 0)
    rc = lib().attn_build_block_mask(_ptr(block_mask), B, int(Sq), int(Sk), int(bool(causal)),
                                     int(window), int(input_pos), _ptr(k_lengths),
                                     ctypes.byref(f), _stream(stream))
    _check(rc, "attn_build_block_mask")


def build_block_mask(Sq, Sk, B=1, causal=False, window=0, input_pos=0, k_lengths=None,
                     q_lengths=None, prefix=0, doc_q=None, doc_kv=None, device=None):
    """Allocating form of attn_build_block_mask: returns the uint8 BlockMask."""
    if doc_q is not None:
        B = doc_q.shape[0]
        device = device or doc_q.device
    out = torch.empty(B, -(-Sq // BLOCK), -(-Sk // BLOCK), dtype=torch.uint8,
                      device=device or "cuda")
    attn_build_block_mask(out, Sq, Sk, causal, window, input_pos, k_lengths, q_lengths,
                          prefix, doc_q, doc_kv)
    return out


def attn_block_scores_workspace_bytes(B: int, Hkv: int, Sk: int, D: int) -> int:
    return lib().attn_block_scores_workspace_bytes(B, Hkv, Sk, D)


def attn_block_scores(base, rescue, Q, K, kind=0, low=0.5, high=0.9, workspace=None,
                      stream=None) -> None:
    """Block scores (B, H, ceil(Sq/64), ceil(Sk/64)) float32 into base (and rescue)."""
    B, H, Hkv, Sq, Sk, D = _prefill_shapes(Q, K, K)
    _expect(base, (B, H, -(-Sq // BLOCK), -(-Sk // BLOCK)), "base")
    _expect(rescue, (B, H, -(-Sq // BLOCK), -(-Sk // BLOCK)), "rescue")
    for t in (Q, K):
        if t.dtype != torch.bfloat16:
            raise ValueError("attn_block_scores takes bfloat16 Q and K")
    for t in (base, rescue):
        if t is not None and t.dtype != torch.float32:
            raise ValueError("block scores are float32")
    ws = _ptr(workspace) if workspace is not None else None
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().attn_block_scores(_ptr(base), _ptr(rescue), _ptr(Q), _ptr(K), B, H, Hkv, Sq,
                                 Sk, D, int(kind), float(low), float(high), ws, nbytes,
                                 _stream(stream))
    _check(rc, "attn_block_scores")


def attn_block_mask(keep, scores=None, mode=0, alpha=1.0, k=0, diagonal=0, accumulate=False,
                    stream=None) -> None:
    """Block mask rows (..., nqb, nkb) uint8 from block scores of the same shape."""
    if keep.dtype != torch.uint8:
        raise ValueError("keep must be uint8")
    nqb, nkb = keep.shape[-2], keep.shape[-1]
    rows = keep.numel() // nkb
    if scores is not None and (scores.dtype != torch.float32 or scores.shape != keep.shape):
        raise ValueError("scores must be float32 with keep's shape")
    rc = lib().attn_block_mask(_ptr(keep), _ptr(scores), rows, nqb, nkb, int(mode),
                               float(alpha), int(k), int(diagonal), int(bool(accumulate)),
                               _stream(stream))
    _check(rc, "attn_block_mask")


def attn_fwd_block_sparse(O, Q, K, V, keep, LSE=None, causal=False, window=0, input_pos=0,
                          k_lengths=None, stream=None) -> None:
    """bf16 prefill on the kept 64 x 64 blocks of keep (B, H, nqb, nkb) uint8."""
    B, H, Hkv, Sq, Sk, D = _prefill_shapes(Q, K, V, O, LSE, k_lengths)
    for t in (O, Q, K, V):
        if t.dtype != torch.bfloat16:
            raise ValueError("attn_fwd_block_sparse takes bfloat16 tensors")
    if keep.dtype != torch.uint8 or tuple(keep.shape) != (B, H, -(-Sq // BLOCK), -(-Sk // BLOCK)):
        raise ValueError("keep must be uint8 (B, H, ceil(Sq/64), ceil(Sk/64))")
    if k_lengths is not None and k_lengths.dtype != torch.int32:
        raise ValueError("k_lengths must be int32")
    rc = lib().attn_fwd_block_sparse(_ptr(O), _ptr(Q), _ptr(K), _ptr(V), _ptr(LSE), B, H, Hkv,
                                      Sq, Sk, D, int(bool(causal)), int(window), int(input_pos),
                                      _ptr(k_lengths), _ptr(keep), _stream(stream))
    _check(rc, "attn_fwd_block_sparse")


def attn_bwd_workspace_bytes(B: int, H: int, Sq: int, D: int) -> int:
    return lib().attn_bwd_workspace_bytes(B, H, Sq, D)


def attn_bwd(dQ, dK, dV, dO, Q, K, V, O, LSE, causal=False, window=0, input_pos=0,
             k_lengths=None, workspace=None, stream=None) -> None:
    """Backward of attn_fwd into dQ, dK, dV (bf16); see include/attn.h."""
    B, H, Hkv, Sq, Sk, D = _prefill_shapes(Q, K, V, O, LSE, k_lengths)
    if LSE is None:
        raise ValueError("attn_bwd needs the forward's LSE")
    _expect(dQ, (B, H, Sq, D), "dQ")
    _expect(dO, (B, H, Sq, D), "dO")
    _expect(dK, (B, Hkv, Sk, D), "dK")
    _expect(dV, (B, Hkv, Sk, D), "dV")
    for t in (dQ, dK, dV, dO, Q, K, V, O):
        if t.dtype != torch.bfloat16:
            raise ValueError("attn_bwd takes bfloat16 tensors")
    if LSE.dtype != torch.float32:
        raise ValueError("LSE must be float32")
    if k_lengths is not None and k_lengths.dtype != torch.int32:
        raise ValueError("k_lengths must be int32")
    ws = _ptr(workspace) if workspace is not None else None
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().attn_bwd(_ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dO), _ptr(Q), _ptr(K), _ptr(V),
                        _ptr(O), _ptr(LSE), B, H, Hkv, Sq, Sk, D, int(bool(causal)),
                        int(window), int(input_pos), _ptr(k_lengths), ws, nbytes,
                        _stream(stream))
    _check(rc, "attn_bwd")


def attn_decode_workspace_bytes(B: int, H: int, n_splits: int, D: int) -> int:
    return lib().attn_decode_workspace_bytes(B, H, n_splits, D)


def _dec_args(O, Q, K, V, lengths):
    if Q.dim() != 3 or K.dim() != 4:
        raise ValueError("decode Q must be (B, H, D) and K (B, Hkv, Smax, D)")
    B, H, D = Q.shape
    Hkv, Smax = K.shape[1], K.shape[2]
    _expect(K, (B, Hkv, Smax, D), "K")
    _expect(V, (B, Hkv, Smax, D), "V")
    _expect(O, (B, H, D), "O")
    _expect(lengths, (B,), "lengths")
    for t in (O, Q, K, V):
        if t.dtype != torch.bfloat16:
            raise ValueError("decode takes bfloat16 tensors")
    if lengths.dtype != torch.int32:
        raise ValueError("lengths must be int32")
    return B, H, Hkv, Smax, D


def attn_decode(O, Q, K, V, lengths, n_splits=8, stream=None) -> None:
    """Split-KV decode into O; the library allocates its scratch stream-ordered."""
    B, H, Hkv, Smax, D = _dec_args(O, Q, K, V, lengths)
    rc = lib().attn_decode(_ptr(O), _ptr(Q), _ptr(K), _ptr(V), _ptr(lengths),
                           int(n_splits), B, H, Hkv, Smax, D, _stream(stream))
    _check(rc, "attn_decode")


def attn_decode_ws(O, Q, K, V, lengths, n_splits, workspace, stream=None) -> None:
    """Split-KV decode using a caller-owned uint8 device workspace."""
    B, H, Hkv, Smax, D = _dec_args(O, Q, K, V, lengths)
    ws = _ptr(workspace) if workspace is not None else None
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().attn_decode_ws(_ptr(O), _ptr(Q), _ptr(K), _ptr(V), _ptr(lengths),
                              int(n_splits), B, H, Hkv, Smax, D, ws, nbytes,
                              _stream(stream))
    _check(rc, "attn_decode_ws")


def attn_decode_static(O, Q, K, V, lengths, n_splits=8, stream=None) -> None:
    """Split-KV decode whose scratch is the library's static per-GPU array
    (no allocation; overlapping calls on one GPU race)."""
    B, H, Hkv, Smax, D = _dec_args(O, Q, K, V, lengths)
    rc = lib().attn_decode_static(_ptr(O), _ptr(Q), _ptr(K), _ptr(V), _ptr(lengths),
                                  int(n_splits), B, H, Hkv, Smax, D, _stream(stream))
    _check(rc, "attn_decode_static")


def attn_decode_paged(O, Q, K_cache, V_cache, block_tables, lengths, n_splits=8,
                      workspace=None, stream=None) -> None:
    """Split-KV decode over a paged (num_blocks, block_size, Hkv, D) cache.

    ``block_tables`` int32 (B, max_blocks), ``lengths`` int32 (B,); with
    ``workspace=None`` the library allocates its scratch stream-ordered.
    """
    if Q.dim() != 3 or K_cache.dim() != 4:
        raise ValueError("Q must be (B, H, D) and K_cache (num_blocks, block_size, Hkv, D)")
    B, H, D = Q.shape
    num_blocks, block_size, Hkv, Dk = K_cache.shape
    if Dk != D or tuple(V_cache.shape) != tuple(K_cache.shape):
        raise ValueError("K_cache / V_cache must be (num_blocks, block_size, Hkv, D)")
    _expect(O, (B, H, D), "O")
    _expect(lengths, (B,), "lengths")
    for t in (O, Q, K_cache, V_cache):
        if t.dtype != torch.bfloat16:
            raise ValueError("decode takes bfloat16 tensors")
    for t in (block_tables, lengths):
        if t.dtype != torch.int32:
            raise ValueError("block_tables and lengths must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be (B, max_blocks)")
    ws = _ptr(workspace) if workspace is not None else None
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().attn_decode_paged(_ptr(O), _ptr(Q), _ptr(K_cache), _ptr(V_cache),
                                 _ptr(block_tables), _ptr(lengths), int(n_splits), B, H,
                                 Hkv, num_blocks, block_size, block_tables.shape[1], D,
                                 ws, nbytes, _stream(stream))
    _check(rc, "attn_decode_paged")


def attn_mask_dump(M, Sq, Sk, causal=False, window=0, input_pos=0, k_len=None,
                   stream=None) -> None:
    """The kernels' own mask predicate into M (uint8 (Sq, Sk))."""
    _expect(M, (Sq, Sk), "M")
    if M.dtype != torch.uint8:
        raise ValueError("M must be uint8")
    rc = lib().attn_mask_dump(_ptr(M), Sq, Sk, int(bool(causal)), int(window),
                              int(input_pos), Sk if k_len is None else int(k_len),
                              _stream(stream))
    _check(rc, "attn_mask_dump")


def fwd_tile_positions(group: int = 1) -> int:
    """Query positions per prefill workgroup for group = H / Hkv: TILE_M
    divided by the query heads it serves (the largest power of two up to 8
    dividing group)."""
    hp = 1
    while hp < 8 and group % (2 * hp) == 0:
        hp *= 2
    return TILE_M // hp


def attn_tile_plan(P, Sq, Sk, causal=False, window=0, input_pos=0, k_len=None, group=1,
                   stream=None) -> None:
    """The prefill kernel's tile plan into P (int8 (ceil(Sq/TP), ceil(Sk/64)),
    TP = fwd_tile_positions(group))."""
    _expect(P, (-(-Sq // fwd_tile_positions(group)), -(-Sk // TILE_N)), "P")
    if P.dtype != torch.int8:
        raise ValueError("P must be int8")
    rc = lib().attn_tile_plan(_ptr(P), Sq, Sk, int(bool(causal)), int(window),
                              int(input_pos), Sk if k_len is None else int(k_len),
                              int(group), _stream(stream))
    _check(rc, "attn_tile_plan")


# ---------------------------------------------------------------------------
# allocating conveniences
# ---------------------------------------------------------------------------

def fwd(q, k, v, causal=False, window=0, input_pos=0, k_lengths=None,
        return_lse=True, stream=None):
    """Allocate O (and LSE) and run the forward matching q's dtype
    (attn_fwd for bfloat16, attn_fwd_f32 for float32)."""
    B, H, Sq, D = q.shape
    O = torch.empty_like(q)
    LSE = torch.empty(B, H, Sq, dtype=torch.float32, device=q.device) if return_lse else None
    fn = attn_fwd if q.dtype == torch.bfloat16 else attn_fwd_f32
    fn(O, q, k, v, LSE, causal, window, input_pos, k_lengths, stream)
    return (O, LSE) if return_lse else O


sdpa = fwd  # the same allocating forward under the scaled-dot-product name


def decode(q, k, v, lengths, n_splits=8, stream=None):
    """Allocate O and run split-KV decode."""
    O = torch.empty_like(q)
    attn_decode(O, q, k, v, lengths, n_splits, stream)
    return O
