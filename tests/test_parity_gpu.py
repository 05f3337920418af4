"""GPU parity: the HIP kernels, called through the C ABI, against the fp64 oracle.

Tolerances: max-abs error <= 2e-2 on bf16 outputs, <= 1e-5 on float32
outputs, LSE within 1e-3; mask dump and tile plan bit-exact.  Inputs are the
seeded generators of ``scaled_dot_product_attn_amd.workloads``; the oracle is
fed the exact values that went to the GPU.
"""

import concurrent.futures as cf
import math
import os
import sys

import numpy as np
import pytest
import torch

import scaled_dot_product_attn_amd as attn
from scaled_dot_product_attn_amd import workloads as wl
from oracle import attn_oracle as ora

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-5
TOL_LSE = 1e-3
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _run_prefill(w, lse=True):
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    kl = None if w.k_lengths is None else w.k_lengths.to(DEV)
    O, L = attn.sdpa(q, k, v, w.causal, w.window, w.input_pos, kl, return_lse=True)
    torch.cuda.synchronize()
    return O, L


def _oracle_workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _oracle_by_heads(fn, B, H):
    """Run an oracle function that takes ``heads=[(b, h), ...]`` over every
    (batch, head) pair, the pairs dealt to a few host threads (NumPy releases
    the GIL in its products and exponentials), and merge the results: each
    call fills only its own pairs and leaves the rest NaN."""
    pairs = [(b, h) for b in range(B) for h in range(H)]
    n = min(_oracle_workers(), len(pairs))
    chunks = [pairs[i::n] for i in range(n)]
    out = None
    with cf.ThreadPoolExecutor(n) as ex:
        for chunk, res in zip(chunks, ex.map(lambda c: fn(heads=c), chunks)):
            if out is None:
                out = tuple(np.full(r.shape, np.nan) for r in res)
            for b, h in chunk:
                for o, r in zip(out, res):
                    o[b, h] = r[b, h]
    return out


def _compare_rows(On, Ln, Or, Lr, tol, what="O"):
    """Every element the oracle computed (not NaN) must match: O within tol
    and finite, LSE within TOL_LSE, -inf exactly where the oracle has it."""
    sel = ~np.isnan(Or)
    assert sel.any()
    assert np.isfinite(On[sel]).all(), f"non-finite {what} where the oracle has a value"
    err = float(np.max(np.abs(On[sel] - Or[sel])))
    assert err <= tol, f"{what} max-abs error {err} > {tol}"
    lsel = ~np.isnan(Lr)
    np.testing.assert_array_equal(np.isneginf(Ln[lsel]), np.isneginf(Lr[lsel]))
    fin = lsel & np.isfinite(Lr)
    if fin.any():
        lerr = np.max(np.abs(Ln[fin] - Lr[fin]))
        assert lerr <= TOL_LSE, f"LSE error {lerr}"
    return err


def _check_prefill(w, O, L, tol, heads=None, rows=None, threads=False):
    kl = None if w.k_lengths is None else w.k_lengths.cpu().numpy()
    q, k, v = _np(w.q), _np(w.k), _np(w.v)
    run = lambda heads=heads: ora.attn_ref(q, k, v, w.causal, w.window, w.input_pos, kl,
                                           heads=heads, rows=rows)
    if threads and heads is None:
        Or, Lr = _oracle_by_heads(run, *w.q.shape[:2])
    else:
        Or, Lr = run()
    return _compare_rows(_np(O), _np(L), Or, Lr, tol)


# ---------------------------------------------------------------------------
# mask predicate and tile plan: bit-exact
# ---------------------------------------------------------------------------

MASK_CASES = [
    (128, 128, 1, 0, 0, 128), (257, 257, 1, 0, 0, 257), (100, 300, 1, 0, 200, 300),
    (300, 300, 1, 64, 0, 300), (192, 1000, 1, 100, 800, 1000), (64, 64, 0, 0, 0, 64),
    (130, 130, 0, 0, 0, 77), (50, 90, 1, 7, -20, 90), (333, 333, 1, 1, 0, 333),
    (129, 700, 1, 0, 600, 650), (64, 64, 1, 0, 0, 0), (200, 64, 1, 3, 100, 64),
    (256, 256, 1, 300, 0, 256), (77, 5000, 1, 129, 4900, 4950),
]


@pytest.mark.parametrize("Sq,Sk,causal,window,ip,kl", MASK_CASES)
def test_mask_dump_bitexact(Sq, Sk, causal, window, ip, kl):
    M = torch.empty(Sq, Sk, dtype=torch.uint8, device=DEV)
    attn.attn_mask_dump(M, Sq, Sk, causal, window, ip, kl)
    want = ora.allowed_mask(Sq, Sk, bool(causal), window, ip, kl)
    np.testing.assert_array_equal(M.cpu().numpy().astype(bool), want)


@pytest.mark.parametrize("group", [1, 4, 8])
@pytest.mark.parametrize("Sq,Sk,causal,window,ip,kl", MASK_CASES + [
    (4096, 4096, 1, 0, 0, 4096), (2048, 16384, 1, 4096, 14336, 16384), (4096, 4096, 0, 0, 0, 4096)])
def test_tile_plan_bitexact(Sq, Sk, causal, window, ip, kl, group):
    tp = attn.fwd_tile_positions(group)
    nqt, nkt = -(-Sq // tp), -(-Sk // attn.TILE_N)
    P = torch.empty(nqt, nkt, dtype=torch.int8, device=DEV)
    attn.attn_tile_plan(P, Sq, Sk, causal, window, ip, kl, group)
    want = ora.tile_plan_ref(Sq, Sk, bool(causal), window, ip, kl, tp, attn.TILE_N)
    np.testing.assert_array_equal(P.cpu().numpy(), want)


# ---------------------------------------------------------------------------
# prefill, bf16
# ---------------------------------------------------------------------------

BF16_CASES = [
    # B, H, Hkv, Sq, Sk, D, causal, window, input_pos, k_lengths
    (1, 4, 1, 256, 256, 128, True, 0, 0, None),
    (2, 4, 2, 257, 257, 128, True, 0, 0, None),
    (1, 2, 2, 300, 300, 128, False, 0, 0, None),
    (1, 4, 4, 100, 400, 128, True, 0, 300, None),
    (1, 8, 2, 384, 1000, 128, True, 128, 616, None),
    (2, 4, 1, 200, 333, 128, True, 0, 133, [333, 250]),
    (2, 2, 1, 130, 190, 128, False, 0, 0, [190, 1]),
    (1, 4, 2, 256, 256, 64, True, 0, 0, None),
    (1, 2, 1, 65, 129, 64, True, 33, 64, None),
    (1, 2, 2, 1, 1, 128, True, 0, 0, None),
    (1, 2, 2, 7, 3, 128, False, 0, 0, None),
    (1, 3, 3, 128, 128, 128, True, 1, 0, None),
    (1, 2, 1, 96, 96, 128, True, 0, -40, None),           # leading rows see nothing
    (1, 2, 1, 64, 256, 128, True, 16, 300, [200]),         # window past k_len: empty rows
    (1, 8, 1, 512, 512, 128, True, 0, 0, None),           # MQA
    (3, 4, 2, 150, 200, 128, True, 0, 60, [-7, 10**6, 120]),  # key lengths clamped to [0, Sk]
    # 516 work items: the persistent schedule (two or more items per CU on a
    # 256-CU GPU), with 4 items past the last multiple of 8
    (1, 172, 43, 600, 600, 64, True, 0, 0, None),
    (2, 86, 43, 700, 500, 64, False, 0, 0, [500, 321]),
]


@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"c{int(c[6])}w{c[7]}p{c[8]}")
def test_prefill_bf16_parity(case):
    B, H, Hkv, Sq, Sk, D, causal, window, ip, kl = case
    _say(f"prefill bf16 {case}")
    w = wl.prefill_random(B, H, Hkv, Sq, Sk, D, torch.bfloat16, seed=7, causal=causal,
                          window=window, input_pos=ip, k_lengths=kl)
    O, L = _run_prefill(w)
    _check_prefill(w, O, L, TOL_BF16)


def test_prefill_bf16_no_lse_matches():
    w = wl.prefill_random(1, 4, 2, 200, 200, 128, torch.bfloat16, seed=8, causal=True)
    O1, _ = _run_prefill(w)
    O2 = attn.sdpa(w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), True, return_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)


def test_prefill_sk_zero_gives_zero_and_neg_inf():
    q = torch.randn(1, 2, 70, 128, device=DEV).bfloat16()
    k = torch.empty(1, 1, 0, 128, device=DEV, dtype=torch.bfloat16)
    O, L = attn.sdpa(q, k, k, False)
    torch.cuda.synchronize()
    assert torch.all(O == 0) and torch.all(torch.isneginf(L))


def test_identity_v_exposes_probabilities():
    # V = I (Sk = D): O = P, so the zero pattern of O is exactly the mask.
    Sq = Sk = D = 128
    for causal, window, ip in [(True, 0, 0), (True, 37, 0), (False, 0, 0)]:
        w = wl.prefill_random(1, 2, 1, Sq, Sk, D, torch.bfloat16, seed=9, causal=causal,
                              window=window, input_pos=ip)
        w.v = torch.eye(Sk, D).bfloat16()[None, None]
        O, L = _run_prefill(w)
        P = O.float().cpu().numpy()[0]
        ok = ora.allowed_mask(Sq, Sk, causal, window, ip)
        for h in range(2):
            np.testing.assert_array_equal(P[h] != 0, ok)
            np.testing.assert_allclose(P[h].sum(axis=1), 1.0, atol=2e-2)
        _check_prefill(w, O, L, TOL_BF16)


def test_nan_poison_outside_valid_keys():
    # K/V past k_lengths (and past the causal frontier) hold NaN: never read.
    B, H, Hkv, Sq, Sk, D = 2, 4, 2, 200, 512, 128
    kls = [300, 137]
    w = wl.prefill_random(B, H, Hkv, Sq, Sk, D, torch.bfloat16, seed=10, causal=True,
                          input_pos=100, k_lengths=kls)
    O_clean, L_clean = _run_prefill(w)
    for b, n in enumerate(kls):
        w.k[b, :, n:] = float("nan")
        w.v[b, :, n:] = float("nan")
    w.k[:, :, 100 + Sq:] = float("nan")   # beyond every query's position
    w.v[:, :, 100 + Sq:] = float("nan")
    O, L = _run_prefill(w)
    assert torch.isfinite(O.float()).all()
    assert torch.equal(O, O_clean) and torch.equal(L, L_clean)


def test_prefill_deterministic_and_stream():
    w = wl.prefill_random(2, 8, 2, 333, 333, 128, torch.bfloat16, seed=11, causal=True)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    O1, L1 = attn.sdpa(q, k, v, True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        O2, L2 = attn.sdpa(q, k, v, True)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_gqa_equals_repeated_heads_on_gpu():
    w = wl.prefill_random(1, 8, 2, 256, 256, 128, torch.bfloat16, seed=12, causal=True)
    O, L = _run_prefill(w)
    wd = wl.Prefill("dense", w.q, w.k.repeat_interleave(4, 1), w.v.repeat_interleave(4, 1), True)
    Od, Ld = _run_prefill(wd)
    assert torch.equal(O, Od) and torch.equal(L, Ld)


# ---------------------------------------------------------------------------
# prefill, float32
# ---------------------------------------------------------------------------

F32_CASES = [
    (1, 4, 4, 128, 128, 64, True, 0, 0, None),            # the tiny fp32 workload's shape
    (2, 4, 2, 130, 200, 128, True, 0, 70, [200, 99]),
    (1, 2, 1, 77, 77, 64, False, 0, 0, None),
    (1, 2, 2, 90, 300, 128, True, 50, 210, None),
]


# ---------------------------------------------------------------------------
# scores that rise from tile to tile
# ---------------------------------------------------------------------------

def _rising(w, step, every=1):
    """All-ones queries and keys constant within each 64-key tile, so that the
    scaled score rises by ``step`` (natural units) from one tile to the next:
    in every ``every``-th KV head and its query heads (the others keep their
    random values).  Past a rise of ~7.6 per tile the kernels' optimistic
    softmax steps fail (a P above 2^16) and the item is walked again with
    exact steps; past ~89 the exponentials overflow."""
    B, H, Sq, D = w.q.shape
    Hkv, Sk = w.k.shape[1], w.k.shape[2]
    G = H // Hkv
    a = (torch.arange(Sk) // 64).float() * (step / math.sqrt(D))
    for g in range(0, Hkv, every):
        w.k[:, g] = a[:, None].expand(Sk, D).to(w.k.dtype)
        w.q[:, g * G:(g + 1) * G] = 1.0
    return w


# (B, H, Hkv, Sq, Sk, D, causal, window, input_pos, step, every)
RISING_CASES = [
    (1, 4, 2, 256, 256, 128, True, 0, 0, 12.0, 1),
    (1, 4, 2, 300, 300, 128, False, 0, 0, 100.0, 1),      # exponentials overflow
    (2, 8, 2, 333, 333, 64, True, 100, 0, 10.0, 2),       # window; rising and random heads
    (1, 8, 1, 200, 456, 128, True, 0, 256, 3.0, 1),       # P x 2^4.3 per tile: fails late
    (1, 8, 8, 130, 390, 128, False, 0, 0, 9.0, 3),
]


@pytest.mark.parametrize("case", RISING_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"s{c[9]}")
def test_prefill_rising_scores(case):
    B, H, Hkv, Sq, Sk, D, causal, window, ip, step, every = case
    _say(f"prefill rising scores {case}")
    w = _rising(wl.prefill_random(B, H, Hkv, Sq, Sk, D, torch.bfloat16, seed=13, causal=causal,
                                  window=window, input_pos=ip), step, every)
    O, L = _run_prefill(w)
    assert torch.isfinite(O.float()).all()
    _check_prefill(w, O, L, TOL_BF16)


def test_prefill_rising_scores_persistent():
    # 512 work items, two per workgroup on a 256-CU GPU: an item that fails is
    # walked again after the next item has started; every other KV head rises
    _say("prefill rising scores, persistent schedule")
    B, H, Hkv, S, D = 1, 64, 64, 2048, 64
    w = _rising(wl.prefill_random(B, H, Hkv, S, S, D, torch.bfloat16, seed=14, causal=True),
                20.0, 2)
    O, L = _run_prefill(w)
    assert torch.isfinite(O.float()).all()
    rows = sorted(set(range(0, 70)) | set(range(S // 2 - 40, S // 2 + 40)) |
                  set(range(S - 70, S)))
    _check_prefill(w, O, L, TOL_BF16, rows=rows, threads=True)


def test_flex_rising_scores():
    # the flex instantiations (documents; bias and soft-cap) and the BlockMask one
    B, H, Hkv, S, D = 2, 8, 2, 300, 128
    w = _rising(_flex_inputs(B, H, Hkv, S, S, D, seed=15), 12.0)
    docs = _docs(B, S, 3, 16)
    g = torch.Generator().manual_seed(17)
    kw = dict(causal=True, window=0, input_pos=0, k_lengths=None)
    for mods in (dict(doc_q=docs, doc_kv=docs),
                 dict(bias=torch.randn(B, 1, S, S, generator=g), softcap=400.0)):
        _say(f"flex rising scores {sorted(mods)}")
        O, L = _run_flex(w, **kw, **mods)
        assert torch.isfinite(O.float()).all()
        _check_flex(w, O, L, **kw, **mods)
    bm = _gpu_block_mask(B, S, S, dict(doc_q=docs, doc_kv=docs), kw)
    O1, L1 = _run_flex(w, **kw, doc_q=docs, doc_kv=docs, block_mask=bm)
    _check_flex(w, O1, L1, **kw, doc_q=docs, doc_kv=docs)


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "x".join(map(str, c[:6])))
def test_prefill_f32_parity(case):
    B, H, Hkv, Sq, Sk, D, causal, window, ip, kl = case
    _say(f"prefill f32 {case}")
    w = wl.prefill_random(B, H, Hkv, Sq, Sk, D, torch.float32, seed=13, causal=causal,
                          window=window, input_pos=ip, k_lengths=kl)
    O, L = _run_prefill(w)
    _check_prefill(w, O, L, TOL_F32)


def test_tiny_f32_workload():
    _say("workload tiny_f32")
    w = wl.make("tiny_f32")
    O, L = _run_prefill(w)
    _check_prefill(w, O, L, TOL_F32)


# ---------------------------------------------------------------------------
# full-size workloads: every output element against the oracle
# ---------------------------------------------------------------------------

def _sample_rows(Sq, rng, n=48):
    fixed = [0, 1, 63, 64, 127, 128, Sq // 2, Sq - 129, Sq - 2, Sq - 1]
    extra = rng.choice(Sq, size=n, replace=False).tolist()
    return np.unique(np.clip(fixed + extra, 0, Sq - 1))


@pytest.mark.parametrize("name", ["gqa_causal", "window_offset", "image_clustered"])
def test_full_size_workload_every_element(name):
    # the launch bench.py times (persistent grid, every XCD slot), every
    # (batch, head) and every row of O and LSE against the fp64 oracle
    _say(f"workload {name}")
    w = wl.make(name)
    O, L = _run_prefill(w)
    err = _check_prefill(w, O, L, TOL_BF16, threads=True)
    _say(f"  {name}: max-abs error {err:.3e} over every element")


# ---------------------------------------------------------------------------
# split-KV decode
# ---------------------------------------------------------------------------

def _check_decode(w, O, tol=TOL_BF16, batches=None):
    Or, _ = ora.decode_ref(_np(w.q), _np(w.k), _np(w.v), w.lengths.cpu().numpy(),
                           batches=batches)
    On = _np(O)
    sel = ~np.isnan(Or)
    err = np.max(np.abs(On[sel] - Or[sel]))
    assert err <= tol, f"decode max-abs error {err}"
    return err


DEC_CASES = [
    # B, H, Hkv, D, smin, smax, n_splits
    (4, 8, 2, 128, 1, 300, 8),
    (3, 4, 4, 128, 60, 70, 3),
    (5, 16, 2, 128, 100, 2000, 1),
    (2, 8, 1, 64, 1, 500, 4),
    (6, 32, 8, 128, 512, 4096, 8),
    (2, 4, 4, 64, 64, 64, 64),
    (3, 16, 1, 128, 200, 900, 8),   # 16 heads per KV head: four head chunks
    (2, 4, 2, 128, 1, 3000, 100),   # more slices than a wave has lanes, most empty
    (300, 2, 1, 64, 1, 200, 4),     # more sequences than the longest-first ranking covers
]


@pytest.mark.parametrize("case", DEC_CASES, ids=lambda c: "x".join(map(str, c)))
def test_decode_parity(case):
    B, H, Hkv, D, smin, smax, ns = case
    _say(f"decode {case}")
    w = wl.decode_random(B, H, Hkv, D, smin, smax, ns, seed=21)
    w.q, w.k, w.v, w.lengths = (t.to(DEV) for t in (w.q, w.k, w.v, w.lengths))
    O = attn.decode(w.q, w.k, w.v, w.lengths, ns)
    torch.cuda.synchronize()
    _check_decode(w, O)


def test_decode_edge_lengths_and_poison():
    B, H, Hkv, D, Smax = 6, 8, 2, 128, 256
    w = wl.decode_random(B, H, Hkv, D, 1, Smax, 8, seed=22, pad_value=float("nan"))
    w.lengths = torch.tensor([0, 1, 63, 64, 65, 256], dtype=torch.int32)
    g = torch.Generator().manual_seed(3)
    for b, n in enumerate(w.lengths.tolist()):
        w.k[b] = float("nan")
        w.v[b] = float("nan")
        w.k[b, :, :n] = torch.randn(Hkv, n, D, generator=g).bfloat16()
        w.v[b, :, :n] = torch.randn(Hkv, n, D, generator=g).bfloat16()
    w.q, w.k, w.v, w.lengths = (t.to(DEV) for t in (w.q, w.k, w.v, w.lengths))
    for ns in (1, 2, 8, 64):
        O = attn.decode(w.q, w.k, w.v, w.lengths, ns)
        torch.cuda.synchronize()
        assert torch.isfinite(O.float()).all()
        assert torch.all(O[0] == 0)          # zero length -> zero output
        _check_decode(w, O)


def test_decode_lengths_clamped_to_cache():
    # lengths outside [0, Smax] are clamped on the device: -5 attends to nothing,
    # 10**6 to the whole cache
    B, H, Hkv, D, Smax = 4, 8, 2, 128, 200
    w = wl.decode_random(B, H, Hkv, D, 1, Smax, 8, seed=25)
    w.lengths = torch.tensor([-5, 10**6, Smax, 0], dtype=torch.int32)
    w.q, w.k, w.v, w.lengths = (t.to(DEV) for t in (w.q, w.k, w.v, w.lengths))
    for ns in (1, 8):
        O = attn.decode(w.q, w.k, w.v, w.lengths, ns)
        torch.cuda.synchronize()
        assert torch.all(O[0] == 0) and torch.all(O[3] == 0)
        _check_decode(w, O)


def test_decode_splits_invariant_and_ws():
    w = wl.decode_random(8, 16, 4, 128, 10, 3000, 8, seed=23)
    w.q, w.k, w.v, w.lengths = (t.to(DEV) for t in (w.q, w.k, w.v, w.lengths))
    outs = [attn.decode(w.q, w.k, w.v, w.lengths, ns) for ns in (1, 2, 3, 8, 64)]
    nb = attn.attn_decode_workspace_bytes(8, 16, 8, 128)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    O_ws = torch.empty_like(w.q)
    attn.attn_decode_ws(O_ws, w.q, w.k, w.v, w.lengths, 8, ws)
    torch.cuda.synchronize()
    assert torch.equal(O_ws, outs[3])
    for O in outs:
        assert (O.float() - outs[0].float()).abs().max().item() <= TOL_BF16
        _check_decode(w, O)


def test_decode_matches_single_query_prefill():
    w = wl.decode_random(4, 8, 2, 128, 1, 700, 8, seed=24)
    w.q, w.k, w.v, w.lengths = (t.to(DEV) for t in (w.q, w.k, w.v, w.lengths))
    O = attn.decode(w.q, w.k, w.v, w.lengths, 8)
    for b, n in enumerate(w.lengths.tolist()):
        Op, _ = attn.sdpa(w.q[b][None, :, None].contiguous(), w.k[b][None].contiguous(),
                          w.v[b][None].contiguous(), True, 0, n - 1)
        torch.cuda.synchronize()
        assert (Op[0, :, 0].float() - O[b].float()).abs().max().item() <= TOL_BF16


def test_decode_full_size_workload_every_sequence():
    _say("workload decode_split")
    w = wl.make("decode_split", device=DEV)
    O = torch.empty_like(w.q)
    ws = torch.empty(attn.attn_decode_workspace_bytes(*w.q.shape[:2], w.n_splits,
                                                      w.q.shape[2]),
                     dtype=torch.uint8, device=DEV)
    attn.attn_decode_ws(O, w.q, w.k, w.v, w.lengths, w.n_splits, ws)   # as bench.py runs it
    torch.cuda.synchronize()
    On = _np(O)
    assert np.isfinite(On).all()
    lengths = w.lengths.cpu().tolist()
    err = 0.0
    for b, n in enumerate(lengths):
        # the sequence's valid keys only (the padding is never attended)
        Or, _ = ora.decode_ref(_np(w.q[b:b + 1]), _np(w.k[b:b + 1, :, :n]),
                               _np(w.v[b:b + 1, :, :n]), np.array([n]))
        err = max(err, float(np.max(np.abs(On[b:b + 1] - Or))))
    assert err <= TOL_BF16, f"decode max-abs error {err}"
    _say(f"  decode_split: max-abs error {err:.3e} over all {len(lengths)} sequences")


# ---------------------------------------------------------------------------
# paged-KV decode
# ---------------------------------------------------------------------------

def _to_dev_paged(w):
    for f in ("q", "k_cache", "v_cache", "block_tables", "lengths"):
        setattr(w, f, getattr(w, f).to(DEV))
    return w


def _check_paged(w, O, tol=TOL_BF16):
    Or, _ = ora.decode_paged_ref(_np(w.q), _np(w.k_cache), _np(w.v_cache),
                                 w.block_tables.cpu().numpy(), w.lengths.cpu().numpy())
    err = np.max(np.abs(_np(O) - Or))
    assert err <= tol, f"paged decode max-abs error {err}"
    return err


PAGED_CASES = [
    # B, H, Hkv, D, smin, smax, block_size, n_splits
    (4, 8, 2, 128, 1, 300, 16, 8),
    (3, 4, 4, 128, 60, 70, 8, 3),
    (5, 16, 2, 128, 100, 2000, 32, 1),
    (2, 8, 1, 64, 1, 500, 8, 4),
    (6, 32, 8, 128, 512, 4096, 16, 8),
    (2, 4, 4, 64, 64, 64, 1, 64),
    (3, 8, 2, 128, 1, 1000, 64, 8),
    (2, 16, 2, 128, 1, 700, 16, 8),      # eight query heads per KV head
    (2, 8, 2, 128, 1, 300, 2, 4),        # blocks smaller than a wave's keys
    (300, 2, 1, 64, 1, 200, 16, 4),      # more sequences than the longest-first ranking covers
    (2, 8, 2, 64, 1, 300, 4, 4),
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=lambda c: "x".join(map(str, c)))
def test_decode_paged_parity(case):
    B, H, Hkv, D, smin, smax, bs, ns = case
    _say(f"paged decode {case}")
    w = _to_dev_paged(wl.decode_paged(B, H, Hkv, D, smin, smax, bs, ns, seed=31,
                                      spare_blocks=5))
    O = torch.empty_like(w.q)
    attn.attn_decode_paged(O, w.q, w.k_cache, w.v_cache, w.block_tables, w.lengths, ns)
    torch.cuda.synchronize()
    _check_paged(w, O)


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_decode_paged_equals_contiguous_bitwise(bs):
    # Same draws in both layouts: the two kernels do the same arithmetic in the
    # same order, so the outputs must be identical.
    B, H, Hkv, D, smin, smax, ns = 6, 16, 4, 128, 1, 3000, 8
    c = wl.decode_random(B, H, Hkv, D, smin, smax, ns, seed=32)
    p = _to_dev_paged(wl.decode_paged(B, H, Hkv, D, smin, smax, bs, ns, seed=32))
    Oc = attn.decode(c.q.to(DEV), c.k.to(DEV), c.v.to(DEV), c.lengths.to(DEV), ns)
    Op = torch.empty_like(p.q)
    attn.attn_decode_paged(Op, p.q, p.k_cache, p.v_cache, p.block_tables, p.lengths, ns)
    torch.cuda.synchronize()
    assert torch.equal(Op, Oc)


def test_decode_paged_poison_and_edge_lengths():
    B, H, Hkv, D, bs = 6, 8, 2, 128, 16
    # every sequence holds 250 tokens: the last of its 16 blocks has 6 NaN slots
    w = wl.decode_paged(B, H, Hkv, D, 250, 250, bs, 8, seed=33, pad_value=float("nan"),
                        spare_blocks=4)
    # block 0 becomes a NaN spare that padded keys point at; shift every table entry
    nan_block = torch.full((1,) + tuple(w.k_cache.shape[1:]), float("nan"), dtype=torch.bfloat16)
    w.k_cache = torch.cat([nan_block, w.k_cache])
    w.v_cache = torch.cat([nan_block, w.v_cache])
    w.block_tables = torch.where(w.block_tables >= 0, w.block_tables + 1, w.block_tables)
    _to_dev_paged(w)
    written = w.lengths.clone()
    for lens in ([0, 1, 15, 16, 17, 250], [250, 0, 0, 33, 200, 1]):
        # keep each length within the tokens the workload wrote for it
        w.lengths = torch.minimum(torch.tensor(lens, dtype=torch.int32, device=DEV), written)
        for ns in (1, 2, 8, 64):
            O = torch.empty_like(w.q)
            attn.attn_decode_paged(O, w.q, w.k_cache, w.v_cache, w.block_tables, w.lengths, ns)
            torch.cuda.synchronize()
            assert torch.isfinite(O.float()).all()
            for b, n in enumerate(w.lengths.tolist()):
                if n == 0:
                    assert torch.all(O[b] == 0)
            _check_paged(w, O)


def test_decode_paged_workspace_matches_allocating():
    w = _to_dev_paged(wl.decode_paged(5, 16, 4, 128, 10, 3000, 16, 8, seed=34))
    O1 = torch.empty_like(w.q)
    attn.attn_decode_paged(O1, w.q, w.k_cache, w.v_cache, w.block_tables, w.lengths, 8)
    nb = attn.attn_decode_workspace_bytes(5, 16, 8, 128)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    O2 = torch.empty_like(w.q)
    attn.attn_decode_paged(O2, w.q, w.k_cache, w.v_cache, w.block_tables, w.lengths, 8,
                           workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)
    _check_paged(w, O1)


def test_decode_paged_full_size_workload_every_sequence():
    _say("workload decode_paged")
    w = wl.make("decode_paged", device=DEV)
    O = torch.empty_like(w.q)
    ws = torch.empty(attn.attn_decode_workspace_bytes(*w.q.shape[:2], w.n_splits,
                                                      w.q.shape[2]),
                     dtype=torch.uint8, device=DEV)
    attn.attn_decode_paged(O, w.q, w.k_cache, w.v_cache, w.block_tables, w.lengths,
                           w.n_splits, workspace=ws)   # as bench.py runs it
    torch.cuda.synchronize()
    On = _np(O)
    assert np.isfinite(On).all()
    lengths = w.lengths.cpu().tolist()
    bs = w.k_cache.shape[1]
    err = 0.0
    for b, n in enumerate(lengths):
        # only the sequence's own blocks go to the host, in table order, so
        # the oracle's table for them is 0, 1, 2, ...
        nb = (n + bs - 1) // bs
        blocks = w.block_tables[b, :nb].long()
        Or, _ = ora.decode_paged_ref(_np(w.q[b:b + 1]), _np(w.k_cache[blocks]),
                                     _np(w.v_cache[blocks]), np.arange(nb)[None],
                                     np.array([n]))
        err = max(err, float(np.max(np.abs(On[b:b + 1] - Or))))
    assert err <= TOL_BF16, f"paged decode max-abs error {err}"
    _say(f"  decode_paged: max-abs error {err:.3e} over all {len(lengths)} sequences")


# ---------------------------------------------------------------------------
# flex variants
# ---------------------------------------------------------------------------

def _flex_inputs(B, H, Hkv, Sq, Sk, D, seed, qscale=1.0):
    w = wl.prefill_random(B, H, Hkv, Sq, Sk, D, torch.bfloat16, seed=seed)
    if qscale != 1.0:
        w.q = (w.q.float() * qscale).bfloat16()
    return w


def _run_flex(w, causal=True, window=0, input_pos=0, k_lengths=None, **mods):
    dev = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in mods.items()}
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    O = torch.empty_like(q)
    L = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    kl = None if k_lengths is None else torch.tensor(k_lengths, dtype=torch.int32, device=DEV)
    attn.attn_fwd_flex(O, q, k, v, L, causal, window, input_pos, kl, **dev)
    torch.cuda.synchronize()
    return O, L


def _check_flex(w, O, L, causal=True, window=0, input_pos=0, k_lengths=None, heads=None,
                rows=None, threads=False, **mods):
    np_mods = {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in mods.items()}
    if "qk_scale" in np_mods:  # the oracle's name for qk_scale
        np_mods["scale"] = np_mods.pop("qk_scale")
    q, k, v = _np(w.q), _np(w.k), _np(w.v)
    run = lambda heads=heads: ora.flex_ref(q, k, v, causal, window, input_pos, k_lengths,
                                           heads=heads, rows=rows, **np_mods)
    if threads and heads is None:
        Or, Lr = _oracle_by_heads(run, *w.q.shape[:2])
    else:
        Or, Lr = run()
    return _compare_rows(_np(O), _np(L), Or, Lr, TOL_BF16, "flex O")


def _docs(B, S, n_docs, seed):
    g = torch.Generator().manual_seed(seed)
    out = torch.empty(B, S, dtype=torch.int32)
    for b in range(B):
        cuts = torch.sort(torch.randperm(S - 1, generator=g)[:n_docs - 1] + 1).values.tolist()
        edges = [0] + cuts + [S]
        for d, (a, c) in enumerate(zip(edges, edges[1:])):
            out[b, a:c] = d
    return out


FLEX_CASES = {
    "softcap": dict(shape=(2, 8, 2, 257, 257, 128), qscale=4.0, mods=dict(softcap=20.0)),
    "softcap_d64": dict(shape=(1, 4, 4, 300, 300, 64), qscale=4.0, mods=dict(softcap=5.0)),
    # a cap above 60 / log2(e) (no fixed softmax reference) with ALiBi
    "softcap_large_alibi": dict(shape=(1, 4, 2, 300, 300, 128), qscale=6.0,
                                mods=dict(softcap=50.0, alibi=True)),
    "alibi_offset": dict(shape=(1, 8, 2, 200, 456, 128), causal=True, input_pos=256,
                         mods=dict(alibi=True)),
    "bias_full": dict(shape=(2, 4, 2, 257, 300, 128), causal=False, mods=dict(bias=(2, 4))),
    "bias_broadcast": dict(shape=(2, 4, 2, 257, 257, 128), mods=dict(bias=(1, 1))),
    "bias_heads": dict(shape=(2, 4, 1, 130, 190, 64), causal=False, mods=dict(bias=(1, 4))),
    "document": dict(shape=(2, 8, 2, 600, 600, 128), mods=dict(docs=5)),
    "document_noncausal": dict(shape=(1, 4, 2, 300, 300, 128), causal=False, mods=dict(docs=3)),
    "prefix_lm": dict(shape=(2, 4, 2, 300, 300, 128), mods=dict(prefix=100)),
    "prefix_long": dict(shape=(1, 4, 1, 520, 520, 128), mods=dict(prefix=400)),
    "q_lengths": dict(shape=(2, 4, 2, 600, 600, 128), mods=dict(q_lengths=[517, 37])),
    "qk_scale": dict(shape=(1, 4, 2, 200, 200, 128), mods=dict(qk_scale=0.05)),
    # PrefixMask | sliding window: rows past the prefix see two key intervals
    "prefix_window_gap": dict(shape=(2, 8, 2, 600, 600, 128), window=128,
                              mods=dict(prefix=100)),
    "prefix_window_merged": dict(shape=(1, 4, 1, 300, 300, 64), window=200,
                                 mods=dict(prefix=150)),
    "prefix_window_g8": dict(shape=(1, 16, 2, 333, 333, 128), window=64,
                             mods=dict(prefix=70, q_lengths=[300])),
    "prefix_window_offset": dict(shape=(2, 4, 2, 200, 500, 128), window=96, input_pos=300,
                                 k_lengths=[500, 420], mods=dict(prefix=70, docs=3)),
    # the mask-extension instantiation with the bias tile and every score mod
    "prefix_window_everything": dict(shape=(2, 8, 2, 330, 330, 128), window=100, input_pos=20,
                                     k_lengths=[330, 290], qscale=2.0,
                                     mods=dict(prefix=50, softcap=15.0, alibi=True,
                                               bias=(2, 1), docs=3, q_lengths=[300, 330])),
    "prefix_window_d64_g1": dict(shape=(1, 4, 4, 300, 300, 64), window=40,
                                 mods=dict(prefix=90, softcap=5.0)),
    "everything": dict(shape=(2, 8, 2, 300, 330, 128), input_pos=30, k_lengths=[330, 250],
                       qscale=2.0,
                       mods=dict(softcap=15.0, alibi=True, bias=(2, 1), docs=4, prefix=40,
                                 q_lengths=[290, 300])),
}


def _build_mods(case, w, seed):
    B, H, Hkv, Sq, Sk, D = case["shape"]
    g = torch.Generator().manual_seed(seed)
    mods = {}
    for k, v in case["mods"].items():
        if k == "alibi":
            mods["alibi_slopes"] = -torch.rand(H, generator=g, dtype=torch.float32) * 0.1
        elif k == "bias":
            mods["bias"] = torch.randn(v + (Sq, Sk), generator=g, dtype=torch.float32)
        elif k == "docs":
            docs = _docs(B, max(Sq, Sk), v, seed)
            mods["doc_q"] = docs[:, :Sq].contiguous()
            mods["doc_kv"] = docs[:, :Sk].contiguous()
        elif k == "q_lengths":
            mods["q_lengths"] = torch.tensor(v, dtype=torch.int32)
        else:
            mods[k] = v
    return mods


@pytest.mark.parametrize("name", list(FLEX_CASES))
def test_flex_parity(name):
    case = FLEX_CASES[name]
    _say(f"flex {name} {case['shape']}")
    w = _flex_inputs(*case["shape"], seed=60, qscale=case.get("qscale", 1.0))
    mods = _build_mods(case, w, 61)
    kw = dict(causal=case.get("causal", True), window=case.get("window", 0),
              input_pos=case.get("input_pos", 0), k_lengths=case.get("k_lengths"))
    O, L = _run_flex(w, **kw, **mods)
    assert torch.isfinite(O.float()).all()
    _check_flex(w, O, L, **kw, **mods)


# BlockMask cases: (B, H, Hkv, Sq, Sk, D, causal, window, input_pos, k_lengths,
# q_lengths, prefix, documents per sequence, one mask for every batch)
BLOCK_MASK_CASES = {
    "docs_g4": (2, 8, 2, 700, 700, 128, True, 0, 0, None, None, 0, 9, False),
    "docs_g8": (1, 16, 2, 520, 520, 128, True, 0, 0, None, None, 0, 6, False),
    "docs_g1_lengths_d64": (2, 4, 4, 600, 600, 64, True, 0, 0, [600, 455], [590, 600], 0, 5,
                            False),
    "docs_noncausal_g2": (1, 4, 2, 300, 300, 128, False, 0, 0, None, None, 0, 4, False),
    "docs_window_prefix": (1, 8, 2, 640, 640, 128, True, 160, 0, None, None, 64, 4, False),
    "docs_offset": (2, 8, 2, 256, 512, 128, True, 0, 256, [512, 400], None, 0, 5, False),
    "docs_shared": (2, 8, 2, 400, 400, 128, True, 0, 0, None, None, 0, 7, True),
}


def _block_mask_case(name):
    (B, H, Hkv, Sq, Sk, D, causal, window, ip, kl, ql, prefix, nd, shared) = \
        BLOCK_MASK_CASES[name]
    w = _flex_inputs(B, H, Hkv, Sq, Sk, D, seed=64)
    docs = _docs(1 if shared else B, ip + Sq if ip + Sq > Sk else Sk, nd, 65)
    if shared:
        docs = docs.expand(B, -1).contiguous()
    # one id vector per sequence: queries take the ids at their absolute positions
    mods = dict(doc_q=docs[:, ip:ip + Sq].contiguous(), doc_kv=docs[:, :Sk].contiguous())
    if prefix:
        mods["prefix"] = prefix
    if ql is not None:
        mods["q_lengths"] = torch.tensor(ql, dtype=torch.int32)
    kw = dict(causal=causal, window=window, input_pos=ip, k_lengths=kl)
    return w, mods, kw, shared


def _oracle_block_mask(B, Sq, Sk, mods, kw):
    out = []
    for b in range(B):
        ok = ora.flex_mask(Sq, Sk, kw["causal"], kw["window"], kw["input_pos"],
                           None if kw["k_lengths"] is None else kw["k_lengths"][b],
                           None if "q_lengths" not in mods else int(mods["q_lengths"][b]),
                           mods.get("prefix", 0), mods["doc_q"][b].numpy(),
                           mods["doc_kv"][b].numpy())
        out.append(ora.block_mask_ref(ok))
    return np.stack(out)


def _gpu_block_mask(B, Sq, Sk, mods, kw):
    kl = None if kw["k_lengths"] is None else torch.tensor(kw["k_lengths"], dtype=torch.int32,
                                                          device=DEV)
    ql = mods["q_lengths"].to(DEV) if "q_lengths" in mods else None
    bm = torch.full((B, -(-Sq // 64), -(-Sk // 64)), 255, dtype=torch.uint8, device=DEV)
    attn.attn_build_block_mask(bm, Sq, Sk, kw["causal"], kw["window"], kw["input_pos"], kl, ql,
                               mods.get("prefix", 0), mods["doc_q"].to(DEV),
                               mods["doc_kv"].to(DEV))
    torch.cuda.synchronize()
    return bm


@pytest.mark.parametrize("name", list(BLOCK_MASK_CASES))
def test_build_block_mask_bitexact(name):
    _say(f"build_block_mask {name}")
    w, mods, kw, _ = _block_mask_case(name)
    shape = (w.q.shape[0], w.q.shape[2], w.k.shape[2])
    bm = _gpu_block_mask(*shape, mods, kw)
    ref = _oracle_block_mask(*shape, mods, kw)
    np.testing.assert_array_equal(bm.cpu().numpy(), ref)
    assert (ref == 0).any() and (ref == 2).any()


def test_flex_block_mask_with_score_mods():
    # BlockMask + bias tile + soft-cap + ALiBi (the BIAS + XM instantiation)
    _say("flex block_mask with bias, soft-cap, ALiBi")
    B, H, Hkv, S, D = 2, 8, 2, 330, 128
    w = _flex_inputs(B, H, Hkv, S, S, D, seed=67, qscale=2.0)
    docs = _docs(B, S, 5, 68)
    g = torch.Generator().manual_seed(69)
    mods = dict(doc_q=docs, doc_kv=docs, softcap=15.0,
                alibi_slopes=-torch.rand(H, generator=g) * 0.1,
                bias=torch.randn(B, 1, S, S, generator=g))
    kw = dict(causal=True, window=0, input_pos=0, k_lengths=None)
    bm = _gpu_block_mask(B, S, S, dict(doc_q=docs, doc_kv=docs), kw)
    O, L = _run_flex(w, **kw, **mods, block_mask=bm)
    _check_flex(w, O, L, **kw, **mods)
    O0, L0 = _run_flex(w, **kw, **mods)
    assert torch.equal(O, O0) and torch.equal(L, L0)


@pytest.mark.parametrize("name", list(BLOCK_MASK_CASES))
def test_flex_block_mask_parity(name):
    _say(f"flex block_mask {name}")
    w, mods, kw, shared = _block_mask_case(name)
    bm = _gpu_block_mask(w.q.shape[0], w.q.shape[2], w.k.shape[2], mods, kw)
    if shared:
        assert torch.equal(bm[0], bm[1])
        bm = bm[:1].contiguous()
    O, L = _run_flex(w, **kw, **mods, block_mask=bm)
    assert torch.isfinite(O.float()).all()
    _check_flex(w, O, L, **kw, **mods)
    # the skipped tiles are those every row of the tile masks away: the
    # result is the one without the block mask, bit for bit
    O0, L0 = _run_flex(w, **kw, **mods)
    assert torch.equal(O, O0) and torch.equal(L, L0)
    # a coarser mask (FULL taken as PARTIAL) gives the same result
    O1, L1 = _run_flex(w, **kw, **mods, block_mask=torch.clamp(bm, max=1))
    assert torch.equal(O, O1) and torch.equal(L, L1)


def test_build_block_mask_full_size():
    # the causal GQA shape cut into documents: every block of both sequences
    _say("build_block_mask gqa_causal-size, 16 documents")
    B, S = 2, 4096
    docs = _docs(B, S, 16, 66)
    mods = dict(doc_q=docs, doc_kv=docs)
    kw = dict(causal=True, window=0, input_pos=0, k_lengths=None)
    bm = _gpu_block_mask(B, S, S, mods, kw)
    np.testing.assert_array_equal(bm.cpu().numpy(), _oracle_block_mask(B, S, S, mods, kw))


def test_flex_without_mods_matches_plain():
    w = _flex_inputs(2, 8, 2, 300, 300, 128, seed=62)
    O, L = _run_flex(w, causal=True)
    Op, Lp = _run_prefill(wl.Prefill("p", w.q, w.k, w.v, True))
    assert (O.float() - Op.float()).abs().max().item() <= 2 * TOL_BF16 / 4
    assert (L - Lp).abs().max().item() <= 1e-4
    _check_flex(w, O, L, causal=True)


def test_flex_full_size_every_element():
    # the causal GQA shape with soft-capping and ALiBi, every element
    _say("flex gqa_causal-size softcap + alibi")
    w = wl.make("gqa_causal")
    g = torch.Generator().manual_seed(63)
    slopes = -torch.rand(32, generator=g) * 0.01
    O, L = _run_flex(w, causal=True, softcap=30.0, alibi_slopes=slopes)
    err = _check_flex(w, O, L, causal=True, threads=True, softcap=30.0, alibi_slopes=slopes)
    _say(f"  max-abs error {err:.3e} over every element")


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def _bwd_run(w, seed=80):
    g = torch.Generator().manual_seed(seed)
    dO = torch.randn(w.q.shape, generator=g).bfloat16()
    q, k, v, do = (t.to(DEV) for t in (w.q, w.k, w.v, dO))
    kl = None if w.k_lengths is None else w.k_lengths.to(DEV)
    O = torch.empty_like(q)
    L = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    attn.attn_fwd(O, q, k, v, L, w.causal, w.window, w.input_pos, kl)
    dQ, dK, dV = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    attn.attn_bwd(dQ, dK, dV, do, q, k, v, O, L, w.causal, w.window, w.input_pos, kl)
    torch.cuda.synchronize()
    return dO, dQ, dK, dV


def _bwd_envelopes(q, k, v, dO, causal, window, input_pos, kl, heads):
    """Per-element magnitude envelopes of the three gradients: each output
    element's sum of the absolute values of the terms that make it up, plus
    the perturbations the kernels' roundings feed into those terms (written
    from the oracle's own steps: mask, scores, softmax).

      envV = P^T |dO|
      A    = P * (|dP| + |delta| + rowsum(|dO| * (|O| + P |V|)))
      envQ = scale * A |K|,   envK = scale * A^T |Q|

    A bounds |dS| and, scaled by 2^-8, how far dS moves when delta is taken
    from the bf16-rounded forward O (rounding and P's own bf16 rounding inside
    it); see the tolerance derivation in the design notes."""
    B, H, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = H // Hkv
    scale = 1.0 / math.sqrt(D)
    envQ = np.full(q.shape, np.nan)
    envK = np.zeros(k.shape)
    envV = np.zeros(v.shape)
    for b, h in heads:
        g = h // G
        ok = ora.allowed_mask(Sq, Sk, causal, window, input_pos,
                              None if kl is None else int(kl[b]))
        P, _, _ = ora.softmax_stats(ora.apply_mask(ora.scores(q[b, h], k[b, g], scale), ok))
        dP = dO[b, h] @ v[b, g].T
        delta = (dP * P).sum(axis=1, keepdims=True)
        O = P @ v[b, g]
        OV = P @ np.abs(v[b, g])
        rounding = (np.abs(dO[b, h]) * (np.abs(O) + OV)).sum(axis=1, keepdims=True)
        A = P * (np.abs(dP) + np.abs(delta) + rounding)
        envV[b, g] += P.T @ np.abs(dO[b, h])
        envQ[b, h] = scale * (A @ np.abs(k[b, g]))
        envK[b, g] += scale * (A.T @ np.abs(q[b, h]))
    return envQ, envK, envV


# Per-element backward bound: |got - ref| <= BWD_ENV * env + BWD_REL * |ref|
# + BWD_ABS (env from _bwd_envelopes; bf16 operands P and dS and bf16 outputs).
BWD_ENV = 2.0 ** -6
BWD_REL = 2.0 ** -8
BWD_ABS = 1e-6


def _bwd_check(w, dO, dQ, dK, dV, heads=None):
    kl = None if w.k_lengths is None else w.k_lengths.cpu().numpy()
    q, k, v, do = _np(w.q), _np(w.k), _np(w.v), _np(dO)
    B, H = w.q.shape[:2]
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    rQ, rK, rV = ora.attn_bwd_ref(q, k, v, do, w.causal, w.window, w.input_pos, kl,
                                  heads=pairs)
    eQ, eK, eV = _bwd_envelopes(q, k, v, do, w.causal, w.window, w.input_pos, kl, pairs)
    G = H // w.k.shape[1]
    groups = {(b, h // G) for b, h in pairs}
    errs = {}
    for name, got, ref, env in (("dQ", dQ, rQ, eQ), ("dK", dK, rK, eK), ("dV", dV, rV, eV)):
        g = _np(got)
        if name == "dQ":
            sel = ~np.isnan(ref)
        else:
            # every query head of a group is in `pairs`, so its sums are whole
            sel = np.zeros(ref.shape, dtype=bool)
            for b, gg in groups:
                sel[b, gg] = True
        assert np.isfinite(g[sel]).all(), f"non-finite {name}"
        diff = np.abs(g[sel] - ref[sel])
        bound = BWD_ENV * env[sel] + BWD_REL * np.abs(ref[sel]) + BWD_ABS
        worst = int(np.argmax(diff / bound))
        errs[name] = (float(diff.max()), float(diff[worst] / bound[worst]))
        assert diff[worst] <= bound[worst], (
            f"{name}: error {diff[worst]:.3e} above its bound {bound[worst]:.3e} "
            f"(|ref| {abs(ref[sel][worst]):.3e}, envelope {env[sel][worst]:.3e})")
    return errs


BWD_CASES = [
    # B, H, Hkv, Sq, Sk, D, causal, window, input_pos, k_lengths
    (1, 4, 2, 128, 128, 128, True, 0, 0, None),
    (2, 4, 1, 257, 257, 128, True, 0, 0, None),
    (1, 2, 2, 300, 300, 128, False, 0, 0, None),
    (1, 8, 2, 200, 456, 128, True, 128, 256, [456]),
    (2, 4, 2, 130, 190, 64, True, 0, 60, [190, 100]),
    (1, 4, 4, 96, 96, 64, False, 0, 0, None),
    (1, 2, 1, 64, 256, 128, True, 16, 300, [200]),
    (1, 4, 2, 33, 700, 128, False, 0, 0, [650]),
    # one partial key tile (Sk < 64) and fewer than 64 query rows at D = 128
    (1, 2, 1, 45, 50, 128, True, 0, 5, None),
    # eight query heads per KV head, a ragged tail on both sides
    (1, 8, 1, 200, 333, 128, True, 0, 133, None),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"-c{int(c[6])}w{c[7]}p{c[8]}")
def test_bwd_parity(case):
    B, H, Hkv, Sq, Sk, D, causal, window, ip, kl = case
    _say(f"bwd {case}")
    w = wl.prefill_random(B, H, Hkv, Sq, Sk, D, torch.bfloat16, seed=81, causal=causal,
                          window=window, input_pos=ip, k_lengths=kl)
    dO, dQ, dK, dV = _bwd_run(w)
    for t in (dQ, dK, dV):
        assert torch.isfinite(t.float()).all()
    errs = _bwd_check(w, dO, dQ, dK, dV)
    _say("  " + ", ".join(f"{k} max {e:.2e} ({r:.2f} of bound)" for k, (e, r) in errs.items()))


def test_bwd_keys_nobody_sees_get_zero():
    w = wl.prefill_random(1, 4, 2, 100, 300, 128, torch.bfloat16, seed=82, causal=True,
                          k_lengths=[200])
    _, dQ, dK, dV = _bwd_run(w)
    # keys >= 200 are past k_lengths, keys >= 100 are past every causal row
    assert torch.all(dK[:, :, 100:] == 0) and torch.all(dV[:, :, 100:] == 0)


def test_bwd_full_size_two_kv_groups():
    # the causal GQA workload: every query head of KV head 0 of batch 0 and of
    # KV head 7 of batch 1, per element against the bound
    _say("bwd gqa_causal, KV groups (0, 0) and (1, 7)")
    w = wl.make("gqa_causal")
    dO, dQ, dK, dV = _bwd_run(w)
    heads = [(0, h) for h in range(4)] + [(1, h) for h in range(28, 32)]
    errs = _bwd_check(w, dO, dQ, dK, dV, heads=heads)
    _say("  " + ", ".join(f"{k} max {e:.2e} ({r:.2f} of bound)" for k, (e, r) in errs.items()))


# ---------------------------------------------------------------------------
# block-sparse prefill: estimators, block masks, attention on kept blocks
# ---------------------------------------------------------------------------

def _nb(n):
    return -(-n // attn.BLOCK)


@pytest.mark.parametrize("shape", [(1, 4, 2, 200, 300, 128), (2, 2, 2, 64, 130, 64),
                                   (1, 8, 1, 256, 1000, 128)])
def test_block_scores_parity(shape):
    B, H, Hkv, Sq, Sk, D = shape
    _say(f"block scores {shape}")
    w = wl.prefill_random(B, H, Hkv, Sq, Sk, D, torch.bfloat16, seed=95)
    q, k = w.q.to(DEV), w.k.to(DEV)
    base = torch.empty(B, H, _nb(Sq), _nb(Sk), device=DEV)
    resc = torch.empty_like(base)
    mm = torch.empty_like(base)
    attn.attn_block_scores(base, resc, q, k, attn.BLOCK_SCORES_RBS)
    attn.attn_block_scores(mm, None, q, k, attn.BLOCK_SCORES_MINMAX)
    torch.cuda.synchronize()
    rb, rr = ora.rbs_block_scores_ref(_np(w.q), _np(w.k), attn.BLOCK)
    rm = ora.minmax_block_scores_ref(_np(w.q), _np(w.k), attn.BLOCK)
    for name, got, ref in (("base", base, rb), ("rescue", resc, rr), ("minmax", mm, rm)):
        err = np.max(np.abs(_np(got) - ref) / np.maximum(1.0, np.abs(ref)))
        assert err <= 1e-4, f"{name} relative error {err}"


def test_block_masks_bitexact():
    g = torch.Generator().manual_seed(96)
    B, H, nqb, nkb = 2, 3, 5, 37
    s = torch.randn(B, H, nqb, nkb, generator=g)
    s[0, 0, 0, 3] = s[0, 0, 0, 7] = s[0, 0, 0].max() + 1.0   # a tie at the top
    sd = s.to(DEV)
    keep = torch.zeros(B, H, nqb, nkb, dtype=torch.uint8, device=DEV)
    sn = s.numpy()
    for alpha in (0.22, 0.18, 1.0):
        attn.attn_block_mask(keep, sd, attn.BLOCK_MASK_RELATIVE, alpha=alpha)
        torch.cuda.synchronize()
        # the keep decision in the kernel's precision (float32), as the oracle
        # takes it with dtype=float32
        np.testing.assert_array_equal(keep.cpu().numpy().astype(bool),
                                      ora.relative_block_mask_ref(sn, alpha, np.float32))
    for kk in (0, 1, 5, 37):
        attn.attn_block_mask(keep, sd, attn.BLOCK_MASK_TOPK, k=kk)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(keep.cpu().numpy().astype(bool),
                                      ora.top_k_block_mask_ref(sn, kk))
    # the recipe's union: relative | relative | band
    attn.attn_block_mask(keep, sd, attn.BLOCK_MASK_RELATIVE, alpha=0.22)
    attn.attn_block_mask(keep, -sd, attn.BLOCK_MASK_RELATIVE, alpha=0.18, accumulate=True)
    attn.attn_block_mask(keep, None, attn.BLOCK_MASK_BAND, diagonal=2, accumulate=True)
    torch.cuda.synchronize()
    want = (ora.relative_block_mask_ref(sn, 0.22, np.float32)
            | ora.relative_block_mask_ref(-sn, 0.18, np.float32)
            | ora.band_block_mask_ref(nqb, nkb, 2)[None, None])
    np.testing.assert_array_equal(keep.cpu().numpy().astype(bool), want)


SPARSE_CASES = [
    # B, H, Hkv, Sq, Sk, D, causal, window, input_pos, k_lengths, density
    (1, 4, 2, 512, 512, 128, True, 0, 0, None, 0.3),
    (2, 4, 1, 300, 700, 128, False, 0, 0, [700, 450], 0.25),
    (1, 8, 2, 257, 257, 64, True, 0, 0, None, 0.5),
    (1, 4, 4, 384, 1024, 128, True, 256, 640, None, 0.4),
]


@pytest.mark.parametrize("case", SPARSE_CASES, ids=lambda c: "x".join(map(str, c[:6])))
def test_block_sparse_fwd_parity(case):
    B, H, Hkv, Sq, Sk, D, causal, window, ip, kl, dens = case
    _say(f"block-sparse fwd {case}")
    w = wl.prefill_random(B, H, Hkv, Sq, Sk, D, torch.bfloat16, seed=97, causal=causal,
                          window=window, input_pos=ip, k_lengths=kl)
    g = torch.Generator().manual_seed(98)
    keep = (torch.rand(B, H, _nb(Sq), _nb(Sk), generator=g) < dens).to(torch.uint8)
    keep[0, 0, 1] = 0                     # one row block keeps nothing
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    O = torch.empty_like(q)
    L = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    kld = None if kl is None else w.k_lengths.to(DEV)
    attn.attn_fwd_block_sparse(O, q, k, v, keep.to(DEV), L, causal, window, ip, kld)
    torch.cuda.synchronize()
    Or, Lr = ora.block_sparse_attn_ref(_np(w.q), _np(w.k), _np(w.v), keep.numpy(), attn.BLOCK,
                                       causal, window, ip, None if kl is None else kl)
    err = np.max(np.abs(_np(O) - Or))
    assert err <= TOL_BF16, f"O max-abs error {err}"
    Ln = _np(L)
    np.testing.assert_array_equal(np.isneginf(Ln), np.isneginf(Lr))
    fin = np.isfinite(Lr)
    assert np.max(np.abs(Ln[fin] - Lr[fin])) <= TOL_LSE
    assert torch.all(O[0, 0, 64:128] == 0)


def test_block_sparse_all_kept_equals_dense_bitwise():
    w = wl.prefill_random(1, 8, 2, 600, 600, 128, torch.bfloat16, seed=99, causal=True)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    keep = torch.ones(1, 8, _nb(600), _nb(600), dtype=torch.uint8, device=DEV)
    O = torch.empty_like(q)
    attn.attn_fwd_block_sparse(O, q, k, v, keep, None, True)
    Od = attn.sdpa(q, k, v, True, return_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(O, Od)


def test_block_sparse_rising_scores():
    # the block-sparse kernel's optimistic softmax steps fail on scores that
    # rise from tile to tile: the item is walked again with exact steps
    B, H, Hkv, S, D = 1, 8, 2, 600, 128
    w = _rising(wl.prefill_random(B, H, Hkv, S, S, D, torch.bfloat16, seed=100, causal=True),
                12.0, 1)
    g = torch.Generator().manual_seed(101)
    keep = (torch.rand(B, H, _nb(S), _nb(S), generator=g) < 0.6).to(torch.uint8)
    q, k, v = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV)
    O = torch.empty_like(q)
    L = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    attn.attn_fwd_block_sparse(O, q, k, v, keep.to(DEV), L, True)
    torch.cuda.synchronize()
    Or, Lr = ora.block_sparse_attn_ref(_np(w.q), _np(w.k), _np(w.v), keep.numpy(), attn.BLOCK,
                                       True, 0, 0, None)
    sel = ~np.isnan(Or)
    assert np.isfinite(_np(O)[sel]).all()
    err = np.max(np.abs(_np(O)[sel] - Or[sel]))
    assert err <= TOL_BF16, f"O max-abs error {err}"
    Ln = _np(L)
    np.testing.assert_array_equal(np.isneginf(Ln), np.isneginf(Lr))
    fin = np.isfinite(Lr)
    assert np.max(np.abs(Ln[fin] - Lr[fin])) <= TOL_LSE


def test_rbs_pipeline_on_image_workload():
    _say("RBS pipeline on image_clustered")
    w = wl.make("image_clustered", device=DEV)
    B, H, S, D = w.q.shape
    nb = _nb(S)
    base = torch.empty(B, H, nb, nb, device=DEV)
    resc = torch.empty_like(base)
    attn.attn_block_scores(base, resc, w.q, w.k, attn.BLOCK_SCORES_RBS)
    keep = torch.empty(B, H, nb, nb, dtype=torch.uint8, device=DEV)
    attn.attn_block_mask(keep, base, attn.BLOCK_MASK_RELATIVE, alpha=0.22)
    attn.attn_block_mask(keep, resc, attn.BLOCK_MASK_RELATIVE, alpha=0.18, accumulate=True)
    attn.attn_block_mask(keep, None, attn.BLOCK_MASK_BAND, diagonal=1, accumulate=True)
    O = torch.empty_like(w.q)
    L = torch.empty(B, H, S, device=DEV)
    attn.attn_fwd_block_sparse(O, w.q, w.k, w.v, keep, L, False)
    torch.cuda.synchronize()
    _say(f"  kept density {keep.float().mean().item():.3f}")
    heads = [(0, 0), (0, 17)]
    rows = _sample_rows(S, np.random.default_rng(100))
    rb, rr = ora.rbs_block_scores_ref(_np(w.q[:, :1]), _np(w.k[:, :1]), attn.BLOCK)
    assert np.max(np.abs(_np(base[:, :1]) - rb) / np.maximum(1, np.abs(rb))) <= 1e-4
    assert np.max(np.abs(_np(resc[:, :1]) - rr) / np.maximum(1, np.abs(rr))) <= 1e-4
    # the min/max box bound at the full size too (one head against the oracle)
    mm = torch.empty_like(base)
    attn.attn_block_scores(mm, None, w.q, w.k, attn.BLOCK_SCORES_MINMAX)
    torch.cuda.synchronize()
    rm = ora.minmax_block_scores_ref(_np(w.q[:, 17:18]), _np(w.k[:, 17:18]), attn.BLOCK)
    assert np.max(np.abs(_np(mm[:, 17:18]) - rm) / np.maximum(1, np.abs(rm))) <= 1e-4
    Or, Lr = ora.block_sparse_attn_ref(_np(w.q), _np(w.k), _np(w.v), keep.cpu().numpy(),
                                       attn.BLOCK, heads=heads, rows=rows)
    sel = ~np.isnan(Lr)
    err = np.max(np.abs(_np(O)[sel] - Or[sel]))
    assert err <= TOL_BF16, err
