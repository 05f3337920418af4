"""Pins of the fp64 oracle against what the pages and mathematics fix.

None of these compare the oracle with itself through a retyped formula: each
check comes from a hand-worked example (tests/golden/), a closed form, an
invariant the pages state, an independent route (pure-Python / mpmath brute
force, torch's own SDPA in float64), or a special case with a known answer.
``test_planted_mistakes`` plants plausible bugs in the oracle and checks that
at least one pin catches each.
"""

import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

from oracle import attn_oracle as ora

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _num(x):
    """Golden fixtures spell irrational entries as short expressions."""
    if x is None:
        return -math.inf
    if isinstance(x, (int, float)):
        return float(x)
    e = math.e
    table = {
        "2ln3": 2 * math.log(3.0), "ln4": math.log(4.0), "ln(e+1)": math.log(e + 1),
        "4e/(e+1)": 4 * e / (e + 1), "4/(e+1)": 4 / (e + 1), "8e/(e+1)": 8 * e / (e + 1),
    }
    return table[x]


# ---------------------------------------------------------------------------
# masks
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", _load("masks.json")["cases"], ids=lambda c: c["name"])
def test_mask_golden(case):
    m = ora.additive_mask(case["seq_len"], case["offset"], case["window"])
    want = np.array([[_num(x) for x in row] for row in case["mask"]])
    assert m.shape == (1, 1, case["seq_len"], case["offset"] + case["seq_len"])
    np.testing.assert_array_equal(m[0, 0], want)


@pytest.mark.parametrize("seq_len,offset", [(1, 0), (7, 0), (5, 3), (16, 100)])
def test_mask_shape_values_lower_triangular(seq_len, offset):
    m = ora.additive_mask(seq_len, offset)
    assert m.shape == (1, 1, seq_len, offset + seq_len)
    assert set(np.unique(m[0, 0]).tolist()) <= {0.0, -math.inf}
    if offset == 0:
        np.testing.assert_array_equal(m[0, 0] == 0, np.tri(seq_len, dtype=bool))


def _row_count_closed_form(p, kl, causal, window):
    hi = min(p, kl - 1) if causal else kl - 1
    lo = max(0, p - window + 1) if window > 0 else 0
    return max(0, hi - lo + 1)


@pytest.mark.parametrize("Sq,Sk,causal,window,ip,kl", [
    (33, 33, True, 0, 0, 33), (20, 50, True, 7, 30, 50), (20, 50, True, 7, 30, 41),
    (9, 9, False, 0, 0, 5), (40, 64, True, 1, 24, 64), (16, 16, True, 100, 0, 16),
    (12, 30, True, 5, -3, 30), (12, 30, True, 0, 40, 30), (8, 8, True, 4, 0, 0),
])
def test_mask_row_counts(Sq, Sk, causal, window, ip, kl):
    ok = ora.allowed_mask(Sq, Sk, causal, window, ip, kl)
    for i in range(Sq):
        n = int(ok[i].sum())
        assert n == _row_count_closed_form(ip + i, kl, causal, window)
        if window > 0:
            assert n <= window
        if ok[i].any():  # allowed keys form one contiguous run
            js = np.nonzero(ok[i])[0]
            assert js[-1] - js[0] + 1 == len(js)


def test_window_equals_tylo_form():
    # Tylo's SlidingWindowMask(w) attends q - w <= kv <= q: our window w + 1.
    for w in range(0, 6):
        ok = ora.allowed_mask(12, 20, True, w + 1, 8, 20)
        q = 8 + np.arange(12)[:, None]
        kv = np.arange(20)[None, :]
        np.testing.assert_array_equal(ok, (q - w <= kv) & (kv <= q))


def test_window_requires_causal():
    with pytest.raises(ValueError):
        ora.allowed_mask(4, 4, causal=False, window=2)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def _closed_form_inputs():
    g = _load("closed_form.json")
    q = np.array([[_num(x) for x in r] for r in g["q"]])
    k = np.array([[_num(x) for x in r] for r in g["k"]])
    v = np.array([[_num(x) for x in r] for r in g["v"]])
    return g, q, k, v


@pytest.mark.parametrize("mode", ["noncausal", "causal"])
def test_closed_form_attention(mode):
    g, q, k, v = _closed_form_inputs()
    O, LSE = ora.attn_ref(q[None, None], k[None, None], v[None, None],
                          causal=(mode == "causal"))
    want_o = np.array([[_num(x) for x in r] for r in g[mode]["O"]])
    want_l = np.array([_num(x) for x in g[mode]["LSE"]])
    np.testing.assert_allclose(O[0, 0], want_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(LSE[0, 0], want_l, rtol=0, atol=1e-13)


def test_closed_form_gqa_two_heads_share_kv():
    g, q, k, v = _closed_form_inputs()
    Q = np.stack([q, q[::-1]])[None]            # H = 2 query heads
    O, LSE = ora.attn_ref(Q, k[None, None], v[None, None], causal=False)
    want = np.array([[_num(x) for x in r] for r in g["noncausal"]["O"]])
    np.testing.assert_allclose(O[0, 0], want, atol=1e-13)
    np.testing.assert_allclose(O[0, 1], want[::-1], atol=1e-13)


def test_closed_form_decode():
    g, q, k, v = _closed_form_inputs()
    Q = np.stack([q[1], q[1]])[:, None, :]       # (B=2, H=1, D)
    K = np.stack([k, k])[:, None]                # (B=2, Hkv=1, Smax=2, D)
    V = np.stack([v, v])[:, None]
    lengths = np.array(g["decode"]["lengths"])
    want_o = np.array([[_num(x) for x in r] for r in g["decode"]["O"]])
    want_l = np.array([_num(x) for x in g["decode"]["LSE"]])
    for fn in (lambda: ora.decode_ref(Q, K, V, lengths),
               lambda: ora.decode_split_ref(Q, K, V, lengths, n_splits=2, tile_n=1)):
        O, LSE = fn()
        np.testing.assert_allclose(O[:, 0], want_o, atol=1e-13)
        np.testing.assert_allclose(LSE[:, 0], want_l, atol=1e-13)


# ---------------------------------------------------------------------------
# brute force (pure Python, mpmath at 50 digits)
# ---------------------------------------------------------------------------

def _brute(Q, K, V, causal, window, ip, k_lengths):
    """Attention by explicit loops: for every query, sum exp(score) over the
    keys the masks allow, weights = exp(score) / sum, no max subtraction."""
    mpmath.mp.dps = 50
    B, H, Sq, D = Q.shape
    Hkv, Sk = K.shape[1], K.shape[2]
    G = H // Hkv
    O = np.zeros((B, H, Sq, V.shape[3]))
    L = np.zeros((B, H, Sq))
    for b in range(B):
        kl = Sk if k_lengths is None else min(max(int(k_lengths[b]), 0), Sk)
        for h in range(H):
            kvh = h // G
            for i in range(Sq):
                pos = ip + i
                keys = [j for j in range(Sk)
                        if j < kl and (not causal or j <= pos)
                        and (window <= 0 or pos - j < window)]
                if not keys:
                    L[b, h, i] = -math.inf
                    continue
                sc = {j: mpmath.mpf(mpmath.fsum(mpmath.mpf(float(Q[b, h, i, d])) * mpmath.mpf(float(K[b, kvh, j, d]))
                                                for d in range(D))) / mpmath.sqrt(D)
                      for j in keys}
                w = {j: mpmath.exp(sc[j]) for j in keys}
                tot = mpmath.fsum(w.values())
                for d in range(V.shape[3]):
                    O[b, h, i, d] = float(mpmath.fsum(w[j] * mpmath.mpf(float(V[b, kvh, j, d]))
                                                      for j in keys) / tot)
                L[b, h, i] = float(mpmath.log(tot))
    return O, L


BRUTE_CASES = [
    dict(B=1, H=2, Hkv=1, Sq=5, Sk=5, D=4, causal=True, window=0, ip=0, kl=None),
    dict(B=2, H=4, Hkv=2, Sq=3, Sk=9, D=8, causal=True, window=4, ip=6, kl=[9, 8]),
    dict(B=1, H=3, Hkv=3, Sq=6, Sk=7, D=3, causal=False, window=0, ip=0, kl=[5]),
    dict(B=2, H=2, Hkv=1, Sq=4, Sk=6, D=5, causal=True, window=0, ip=-2, kl=[6, 0]),
]


@pytest.mark.parametrize("c", BRUTE_CASES, ids=lambda c: f"S{c['Sq']}x{c['Sk']}w{c['window']}")
def test_bruteforce_mpmath(c):
    rng = np.random.default_rng(11)
    Q = rng.standard_normal((c["B"], c["H"], c["Sq"], c["D"]))
    K = rng.standard_normal((c["B"], c["Hkv"], c["Sk"], c["D"]))
    V = rng.standard_normal((c["B"], c["Hkv"], c["Sk"], c["D"]))
    O, LSE = ora.attn_ref(Q, K, V, c["causal"], c["window"], c["ip"], c["kl"])
    Ob, Lb = _brute(Q, K, V, c["causal"], c["window"], c["ip"], c["kl"])
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(LSE), np.isinf(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(LSE[fin], Lb[fin], rtol=0, atol=1e-12)
    # rows with nothing allowed: zero output (reading for empty rows)
    assert np.all(O[~fin] == 0.0)


def test_decode_bruteforce():
    rng = np.random.default_rng(12)
    B, H, Hkv, S, D = 3, 4, 2, 9, 6
    Q = rng.standard_normal((B, H, D))
    K = rng.standard_normal((B, Hkv, S, D))
    V = rng.standard_normal((B, Hkv, S, D))
    lengths = np.array([9, 1, 4])
    O, LSE = ora.decode_ref(Q, K, V, lengths)
    for b in range(B):
        Ob, Lb = _brute(Q[b][None, :, None], K[b][None], V[b][None], False, 0, 0, [lengths[b]])
        np.testing.assert_allclose(O[b], Ob[0, :, 0], atol=1e-12)
        np.testing.assert_allclose(LSE[b], Lb[0, :, 0], atol=1e-12)


# ---------------------------------------------------------------------------
# library cross-check: torch SDPA in float64 on CPU
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,H,Hkv,Sq,Sk,D,causal,window,ip", [
    (1, 4, 4, 128, 128, 64, True, 0, 0),
    (2, 8, 2, 64, 96, 32, True, 0, 32),
    (1, 4, 1, 48, 80, 16, True, 20, 32),
    (1, 2, 2, 64, 64, 32, False, 0, 0),
])
def test_against_torch_sdpa_fp64(B, H, Hkv, Sq, Sk, D, causal, window, ip):
    gen = torch.Generator().manual_seed(3)
    q = torch.randn(B, H, Sq, D, generator=gen, dtype=torch.float64)
    k = torch.randn(B, Hkv, Sk, D, generator=gen, dtype=torch.float64)
    v = torch.randn(B, Hkv, Sk, D, generator=gen, dtype=torch.float64)
    i = torch.arange(Sq)[:, None] + ip
    j = torch.arange(Sk)[None, :]
    m = torch.ones(Sq, Sk, dtype=torch.bool)
    if causal:
        m &= j <= i
    if window:
        m &= j > i - window
    G = H // Hkv
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(G, 1), v.repeat_interleave(G, 1), attn_mask=m)
    O, _ = ora.attn_ref(q.numpy(), k.numpy(), v.numpy(), causal, window, ip)
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# invariants and special cases
# ---------------------------------------------------------------------------

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_gqa_equals_repeated_kv_heads():
    Q, K, V = _rand((2, 8, 17, 16), 1), _rand((2, 2, 23, 16), 2), _rand((2, 2, 23, 16), 3)
    O, L = ora.attn_ref(Q, K, V, True, 5, 6, [23, 11])
    Od, Ld = ora.attn_ref(Q, np.repeat(K, 4, axis=1), np.repeat(V, 4, axis=1), True, 5, 6, [23, 11])
    np.testing.assert_allclose(O, Od, atol=1e-14)
    np.testing.assert_allclose(L, Ld, atol=1e-14)


def test_constant_v_gives_constant_output():
    Q, K = _rand((1, 2, 20, 8), 4), _rand((1, 2, 20, 8), 5)
    V = np.broadcast_to(np.arange(8.0) - 3.5, (1, 2, 20, 8))
    O, _ = ora.attn_ref(Q, K, V, True, 6, 0)
    np.testing.assert_allclose(O, V[:, :, :20], atol=1e-13)


def test_zero_query_uniform_weights():
    Sq, Sk, W, ip = 10, 30, 7, 15
    Q = np.zeros((1, 1, Sq, 8))
    K, V = _rand((1, 1, Sk, 8), 6), _rand((1, 1, Sk, 8), 7)
    O, L = ora.attn_ref(Q, K, V, True, W, ip)
    for i in range(Sq):
        p = ip + i
        js = list(range(max(0, p - W + 1), min(p, Sk - 1) + 1))
        np.testing.assert_allclose(O[0, 0, i], V[0, 0, js].mean(axis=0), atol=1e-13)
        np.testing.assert_allclose(L[0, 0, i], math.log(len(js)), atol=1e-13)


def test_single_allowed_key():
    Q, K, V = _rand((1, 2, 6, 8), 8), _rand((1, 2, 12, 8), 9), _rand((1, 2, 12, 8), 10)
    O, L = ora.attn_ref(Q, K, V, True, 1, 3)          # window 1: only key p
    for h in range(2):
        for i in range(6):
            j = 3 + i
            np.testing.assert_allclose(O[0, h, i], V[0, h, j], atol=1e-14)
            np.testing.assert_allclose(L[0, h, i], Q[0, h, i] @ K[0, h, j] / math.sqrt(8), atol=1e-13)


def test_identity_v_exposes_probabilities():
    # With V = I (Sk == D) the output rows are the softmax probabilities.
    Sk = D = 16
    Q, K = _rand((1, 1, 16, D), 11), _rand((1, 1, Sk, D), 12)
    V = np.eye(Sk)[None, None]
    for causal, W, ip in [(True, 0, 0), (True, 5, 0), (False, 0, 0)]:
        P, L = ora.attn_ref(Q, K, V, causal, W, ip)
        ok = ora.allowed_mask(16, Sk, causal, W, ip)
        assert np.all(P[0, 0] >= 0)
        np.testing.assert_allclose(P[0, 0].sum(axis=1), 1.0, atol=1e-14)
        assert np.all(P[0, 0][~ok] == 0.0)
        # LSE is the log of the plain (unshifted) exponential sum
        s = Q[0, 0] @ K[0, 0].T / math.sqrt(D)
        want = np.log(np.where(ok, np.exp(s), 0.0).sum(axis=1))
        np.testing.assert_allclose(L[0, 0], want, atol=1e-13)


def test_k_lengths_equal_truncation():
    Q, K, V = _rand((2, 2, 9, 8), 13), _rand((2, 2, 20, 8), 14), _rand((2, 2, 20, 8), 15)
    O, L = ora.attn_ref(Q, K, V, False, 0, 0, [20, 7])
    Ot, Lt = ora.attn_ref(Q[1:], K[1:, :, :7], V[1:, :, :7])
    np.testing.assert_allclose(O[1:], Ot, atol=1e-14)
    np.testing.assert_allclose(L[1:], Lt, atol=1e-14)


def test_decode_equals_single_query_prefill():
    rng = np.random.default_rng(16)
    B, H, Hkv, S, D = 4, 8, 2, 40, 16
    Q = rng.standard_normal((B, H, D))
    K, V = rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    lengths = np.array([40, 1, 17, 33])
    O, L = ora.decode_ref(Q, K, V, lengths)
    for b in range(B):
        n = int(lengths[b])
        Op, Lp = ora.attn_ref(Q[b][None, :, None], K[b][None], V[b][None], True, 0, n - 1)
        np.testing.assert_allclose(O[b], Op[0, :, 0], atol=1e-13)
        np.testing.assert_allclose(L[b], Lp[0, :, 0], atol=1e-13)


@pytest.mark.parametrize("n_splits", [1, 2, 3, 8, 64])
def test_decode_split_merge_invariant(n_splits):
    rng = np.random.default_rng(17)
    B, H, Hkv, S, D = 3, 4, 2, 300, 8
    Q = rng.standard_normal((B, H, D))
    K, V = rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    lengths = np.array([300, 65, 0])
    O, L = ora.decode_ref(Q, K, V, lengths)
    Os, Ls = ora.decode_split_ref(Q, K, V, lengths, n_splits, tile_n=64)
    np.testing.assert_allclose(Os, O, atol=1e-13)
    np.testing.assert_allclose(Ls[:2], L[:2], atol=1e-13)
    assert np.all(Os[2] == 0) and np.all(np.isneginf(Ls[2]))


def test_split_bounds_cover_once():
    for n in [0, 1, 63, 64, 65, 512, 32768, 1000]:
        for ns in [1, 3, 8]:
            b = ora.split_bounds(n, ns, 64)
            assert len(b) == ns
            covered = [j for lo, hi in b for j in range(lo, hi)]
            assert covered == list(range(n))
            assert all(lo % 64 == 0 for lo, hi in b if hi > lo)


@pytest.mark.parametrize("case", _load("tile_plans.json")["cases"], ids=lambda c: c["name"])
def test_tile_plan_golden(case):
    plan = ora.tile_plan_ref(case["Sq"], case["Sk"], case["causal"], case["window"],
                             case["input_pos"], case["k_len"], case["tile_m"], case["tile_n"])
    np.testing.assert_array_equal(plan, np.array(case["plan"], dtype=np.int8))


def test_allowed_pairs_closed_forms():
    # causal square: S(S+1)/2; window W on a long enough history: Sq*W.
    assert ora.allowed_pairs(4096, 4096, True, 0, 0, 4096) == 4096 * 4097 // 2
    assert ora.allowed_pairs(2048, 16384, True, 4096, 14336, 16384) == 2048 * 4096
    assert ora.allowed_pairs(64, 64, False, 0, 0, 64) == 64 * 64


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin above
# ---------------------------------------------------------------------------

def _pins_pass():
    checks = [
        lambda: [test_mask_golden(c) for c in _load("masks.json")["cases"]],
        lambda: [test_closed_form_attention(m) for m in ("noncausal", "causal")],
        test_closed_form_gqa_two_heads_share_kv,
        test_closed_form_decode,
        lambda: test_bruteforce_mpmath(BRUTE_CASES[1]),
        test_zero_query_uniform_weights,
        test_single_allowed_key,
        lambda: test_decode_split_merge_invariant(3),
        lambda: [test_tile_plan_golden(c) for c in _load("tile_plans.json")["cases"]],
    ]
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError, TypeError):
            return False
    return True


def _mutant_scale(q, k, scale):
    return (q @ k.T) / q.shape[1]


def _mutant_transposed_scores(q, k, scale):
    return scale * (k @ q.T)


def _mutant_no_normalise(s):
    P, M, L = ORIG_SOFTMAX(s)
    return P * np.maximum(L, 1e-300)[:, None], M, L


def _mutant_lse_no_max(M, L):
    out = np.full(M.shape, -np.inf)
    ok = L > 0
    out[ok] = np.log(L[ok])
    return out


def _mutant_combine_transposed(P, v):
    return P.T @ v


ORIG_SOFTMAX = ora.softmax_stats


def _mutant_allowed_window_tylo(Sq, Sk, causal=False, window=0, input_pos=0, k_len=None):
    return ORIG_ALLOWED(Sq, Sk, causal, window + 1 if window > 0 else 0, input_pos, k_len)


def _mutant_allowed_strict_causal(Sq, Sk, causal=False, window=0, input_pos=0, k_len=None):
    ok = ORIG_ALLOWED(Sq, Sk, causal, window, input_pos, k_len)
    if causal:
        i = np.arange(Sq)[:, None] + input_pos
        ok &= np.arange(Sk)[None, :] < i
    return ok


def _mutant_allowed_ignore_klen(Sq, Sk, causal=False, window=0, input_pos=0, k_len=None):
    return ORIG_ALLOWED(Sq, Sk, causal, window, input_pos, None)


ORIG_ALLOWED = ora.allowed_mask


@pytest.mark.parametrize("target,mutant", [
    ("scores", _mutant_scale),
    ("scores", _mutant_transposed_scores),
    ("softmax_stats", _mutant_no_normalise),
    ("lse_from_stats", _mutant_lse_no_max),
    ("combine", _mutant_combine_transposed),
    ("allowed_mask", _mutant_allowed_window_tylo),
    ("allowed_mask", _mutant_allowed_strict_causal),
    ("allowed_mask", _mutant_allowed_ignore_klen),
])
def test_planted_mistakes(monkeypatch, target, mutant):
    assert _pins_pass()
    monkeypatch.setattr(ora, target, mutant)
    assert not _pins_pass(), f"no pin caught the planted mistake in {target}"


def test_planted_gqa_mapping_mistake(monkeypatch):
    # Query head h reading KV head h % Hkv instead of h // G must be caught.
    real = ora.attn_ref

    def mutant(Q, K, V, *a, **kw):
        Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
        H, Hkv = Q.shape[1], K.shape[1]
        outs = [real(Q[:, h:h + 1], K[:, h % Hkv:h % Hkv + 1], V[:, h % Hkv:h % Hkv + 1], *a, **kw)
                for h in range(H)]
        return (np.concatenate([o for o, _ in outs], axis=1),
                np.concatenate([l for _, l in outs], axis=1))

    monkeypatch.setattr(ora, "attn_ref", mutant)
    with pytest.raises(AssertionError):
        test_bruteforce_mpmath(BRUTE_CASES[1])


# ---------------------------------------------------------------------------
# paged KV cache
# ---------------------------------------------------------------------------

def _scatter_to_pages(K, V, lengths, bs, rng, spare_blocks=3):
    """Write a contiguous (B, Hkv, S, D) cache into shuffled physical blocks.

    Written independently of the oracle's gather: blocks are dealt to the
    sequences from a random permutation, unused blocks and table slots hold
    poison (NaN rows, table entry -1 / out of range).
    """
    B, Hkv, S, D = K.shape
    nblk = [-(-int(n) // bs) for n in lengths]
    maxb = max(max(nblk), 1) + 1
    total = sum(nblk) + spare_blocks
    perm = rng.permutation(total)
    Kc = np.full((total, bs, Hkv, D), np.nan)
    Vc = np.full((total, bs, Hkv, D), np.nan)
    table = np.full((B, maxb), -1, dtype=np.int64)
    table[:, -1] = 10 ** 9
    nxt = 0
    for b in range(B):
        for i in range(nblk[b]):
            phys = int(perm[nxt]); nxt += 1
            table[b, i] = phys
            for slot in range(bs):
                t = i * bs + slot
                if t < lengths[b]:
                    for g in range(Hkv):
                        Kc[phys, slot, g] = K[b, g, t]
                        Vc[phys, slot, g] = V[b, g, t]
    return Kc, Vc, table


@pytest.mark.parametrize("bs", [1, 8, 16, 32])
def test_paged_decode_equals_contiguous(bs):
    # vllm_mlx.attention: (num_blocks, block_size, num_kv_heads, head_size)
    # cache + block tables must give exactly the contiguous decode.
    rng = np.random.default_rng(30 + bs)
    B, H, Hkv, S, D = 4, 8, 2, 70, 16
    Q = rng.standard_normal((B, H, D))
    K, V = rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    lengths = np.array([70, 1, 33, 0])
    Kc, Vc, table = _scatter_to_pages(K, V, lengths, bs, rng)
    O, L = ora.decode_ref(Q, K, V, lengths)
    Op, Lp = ora.decode_paged_ref(Q, Kc, Vc, table, lengths)
    np.testing.assert_array_equal(Op, O)
    np.testing.assert_array_equal(Lp, L)
    assert np.all(np.isfinite(Op))


def test_paged_length_clamped_to_table_capacity():
    rng = np.random.default_rng(41)
    B, H, Hkv, S, D, bs = 2, 2, 1, 32, 8, 8
    Q = rng.standard_normal((B, H, D))
    K, V = rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    Kc = K[0].transpose(1, 0, 2).reshape(S // bs, bs, Hkv, D)
    Vc = V[0].transpose(1, 0, 2).reshape(S // bs, bs, Hkv, D)
    table = np.array([[0, 1, 2, 3], [0, 1, 2, 3]])
    Op, Lp = ora.decode_paged_ref(Q, Kc, Vc, table, np.array([10 ** 6, -5]))
    O, L = ora.decode_ref(Q[:1], K[:1], V[:1], np.array([S]))
    np.testing.assert_array_equal(Op[:1], O)
    assert np.all(Op[1] == 0) and np.all(np.isneginf(Lp[1]))


def test_planted_paged_gather_mistake(monkeypatch):
    # block and slot swapped, or the wrong KV head, must be caught.
    def swapped(cache, table_row, n, g):
        cache = np.asarray(cache)
        bs = cache.shape[1]
        t = np.arange(n)
        return np.asarray(cache[np.asarray(table_row)[t % bs], t // bs, g], dtype=np.float64)

    def head0(cache, table_row, n, g):
        return ORIG_GATHER(cache, table_row, n, 0)

    for mutant in (swapped, head0):
        monkeypatch.setattr(ora, "gather_paged", mutant)
        with pytest.raises((AssertionError, IndexError)):
            test_paged_decode_equals_contiguous(16)


ORIG_GATHER = ora.gather_paged


# ---------------------------------------------------------------------------
# flex variants (score mods and mask mods)
# ---------------------------------------------------------------------------

def _flex_case(seed, B=2, H=4, Hkv=2, Sq=12, Sk=15, D=8):
    rng = np.random.default_rng(seed)
    return (rng, rng.standard_normal((B, H, Sq, D)), rng.standard_normal((B, Hkv, Sk, D)),
            rng.standard_normal((B, Hkv, Sk, D)))


@pytest.mark.parametrize("causal,window,ip,kl", [(False, 0, 0, None), (True, 0, 0, None),
                                                 (True, 4, 3, [15, 9]), (True, 0, -2, [6, 15])])
def test_flex_without_mods_is_plain_attention(causal, window, ip, kl):
    _, Q, K, V = _flex_case(50)
    O, L = ora.flex_ref(Q, K, V, causal, window, ip, kl)
    Or, Lr = ora.attn_ref(Q, K, V, causal, window, ip, kl)
    np.testing.assert_array_equal(O, Or)
    np.testing.assert_array_equal(L, Lr)


def _torch_sdpa_additive(Q, K, V, add):
    """torch's own SDPA in float64 with a float additive mask (B or 1, H, Sq, Sk)."""
    H, Hkv = Q.shape[1], K.shape[1]
    rep = H // Hkv
    q, k, v = (torch.from_numpy(x) for x in (Q, K, V))
    k = k.repeat_interleave(rep, dim=1)
    v = v.repeat_interleave(rep, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=torch.from_numpy(add)).numpy()


@pytest.mark.parametrize("bias_shape", [(1, 1), (2, 1), (1, 4), (2, 4)])
def test_flex_bias_alibi_document_prefix_vs_torch_sdpa(bias_shape):
    rng, Q, K, V = _flex_case(51)
    B, H, Sq, D = Q.shape
    Sk = K.shape[2]
    ip, prefix = 3, 5
    bias = rng.standard_normal(bias_shape + (Sq, Sk))
    slopes = -np.array([0.5, 0.25, 0.125, 0.0625])
    doc_q = np.array([[0] * 6 + [1] * 6, [0] * 12])
    doc_kv = np.array([[0] * 9 + [1] * 6, [0] * 10 + [2] * 5])
    kl, ql = [15, 11], [12, 9]
    O, L = ora.flex_ref(Q, K, V, True, 0, ip, kl, ql, prefix, 0.0, slopes, bias, doc_q, doc_kv)
    # the additive mask, written out pair by pair
    add = np.zeros((B, H, Sq, Sk))
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                for j in range(Sk):
                    p = ip + i
                    ok = (j <= p or j < prefix) and j < kl[b] and i < ql[b] \
                        and doc_q[b][i] == doc_kv[b][j]
                    add[b, h, i, j] = (bias[b % bias_shape[0], h % bias_shape[1], i, j]
                                       + slopes[h] * (p - j)) if ok else -np.inf
    Ot = _torch_sdpa_additive(Q, K, V, add)
    has = np.isfinite(add).any(axis=3)
    np.testing.assert_allclose(O[has], Ot[has], atol=1e-12)
    assert np.all(O[~has] == 0) and np.all(np.isneginf(L[~has]))
    sc = np.einsum("bhid,bhjd->bhij", Q, np.repeat(K, 2, axis=1)) / math.sqrt(D)
    tot = np.where(np.isfinite(add), np.exp(sc + np.where(np.isfinite(add), add, 0.0)), 0.0)
    lse_t = np.log(tot.sum(axis=3)[has])
    np.testing.assert_allclose(L[has], lse_t, atol=1e-12)


def test_alibi_closed_form_geometric_weights():
    # Q = 0 makes every score slope*(p - j); with V = identity, O row p is the
    # probability vector x^(p-j) / sum_{t<=p} x^t, x = e^slope (causal).
    S = D = 16
    slope = -0.3
    Q = np.zeros((1, 1, S, D))
    K = np.random.default_rng(52).standard_normal((1, 1, S, D))
    V = np.eye(S)[None, None]
    O, L = ora.flex_ref(Q, K, V, True, alibi_slopes=[slope])
    x = math.exp(slope)
    for p in range(S):
        want = np.array([x ** (p - j) if j <= p else 0.0 for j in range(S)])
        want /= (1 - x ** (p + 1)) / (1 - x)
        np.testing.assert_allclose(O[0, 0, p], want, atol=1e-14)
        assert abs(L[0, 0, p] - math.log((1 - x ** (p + 1)) / (1 - x))) < 1e-13


def test_softcap_bruteforce_mpmath():
    # brute force at 40 digits: scaled score, plus bias and ALiBi, then the cap
    rng, Q, K, V = _flex_case(53, B=1, H=2, Hkv=1, Sq=4, Sk=6, D=3)
    Q *= 3.0   # large scores so the cap bites
    cap, ip = 1.5, 2
    bias = rng.standard_normal((1, 2, 4, 6))
    slopes = [-0.7, 0.4]
    O, L = ora.flex_ref(Q, K, V, True, 0, ip, softcap=cap, alibi_slopes=slopes, bias=bias)
    mpmath.mp.dps = 40
    for h in range(2):
        for i in range(4):
            p = ip + i
            w = []
            for j in range(p + 1):
                s = mpmath.mpf(0)
                for d in range(3):
                    s += mpmath.mpf(Q[0, h, i, d]) * mpmath.mpf(K[0, 0, j, d])
                s = s / mpmath.sqrt(3) + mpmath.mpf(bias[0, h, i, j]) + slopes[h] * (p - j)
                w.append(mpmath.exp(cap * mpmath.tanh(s / cap)))
            tot = mpmath.fsum(w)
            for d in range(3):
                o = mpmath.fsum(w[j] * mpmath.mpf(V[0, 0, j, d]) for j in range(p + 1)) / tot
                assert abs(float(o) - O[0, h, i, d]) < 1e-13
            assert abs(float(mpmath.log(tot)) - L[0, h, i]) < 1e-13


def test_softcap_limits():
    _, Q, K, V = _flex_case(54)
    O, _ = ora.flex_ref(Q, K, V, True, softcap=1e7)
    Or, _ = ora.attn_ref(Q, K, V, True)
    np.testing.assert_allclose(O, Or, atol=1e-9)
    # a tiny cap squeezes every score to ~0: uniform weights over allowed keys
    O, L = ora.flex_ref(Q, K, V, True, softcap=1e-9)
    G = Q.shape[1] // K.shape[1]
    for i in range(Q.shape[2]):
        for h in range(Q.shape[1]):
            np.testing.assert_allclose(O[:, h, i], V[:, h // G, :i + 1].mean(axis=1), atol=1e-9)
            np.testing.assert_allclose(L[:, h, i], math.log(i + 1), atol=1e-9)


def test_prefix_lm_decomposes():
    # prefix_lm(len) = Causal | Prefix(len): rows inside the prefix see the whole
    # prefix (bidirectional), later rows are plain causal rows.
    _, Q, K, V = _flex_case(55, Sq=14, Sk=14)
    n = 6
    O, L = ora.flex_ref(Q, K, V, True, prefix=n)
    Oa, La = ora.attn_ref(Q, K, V, False, 0, 0, [n, n])
    Oc, Lc = ora.attn_ref(Q, K, V, True)
    np.testing.assert_array_equal(O[:, :, :n], Oa[:, :, :n])
    np.testing.assert_array_equal(O[:, :, n:], Oc[:, :, n:])
    np.testing.assert_array_equal(L[:, :, n:], Lc[:, :, n:])


def test_document_mask_block_diagonal_equals_separate_sequences():
    _, Q, K, V = _flex_case(56, B=1, Sq=13, Sk=13)
    bounds = [0, 4, 9, 13]
    doc = np.repeat(np.arange(3), np.diff(bounds))[None]
    O, L = ora.flex_ref(Q, K, V, True, doc_q=doc, doc_kv=doc)
    for a, b in zip(bounds, bounds[1:]):
        Od, Ld = ora.attn_ref(Q[:, :, a:b], K[:, :, a:b], V[:, :, a:b], True)
        np.testing.assert_allclose(O[:, :, a:b], Od, atol=1e-14)
        np.testing.assert_allclose(L[:, :, a:b], Ld, atol=1e-14)


def test_q_lengths_rows_attend_to_nothing():
    _, Q, K, V = _flex_case(57)
    O, L = ora.flex_ref(Q, K, V, True, q_lengths=[5, 12])
    Or, Lr = ora.attn_ref(Q, K, V, True)
    np.testing.assert_array_equal(O[0, :, :5], Or[0, :, :5])
    assert np.all(O[0, :, 5:] == 0) and np.all(np.isneginf(L[0, :, 5:]))
    np.testing.assert_array_equal(O[1], Or[1])


def test_prefix_or_window_rows_hand_worked():
    # PrefixMask(2) | sliding window of 3 keys (causal): row i sees keys
    # {0, 1} and {i-2 .. i}; from row 5 on these are two separate intervals
    ok = ora.flex_mask(10, 10, True, 3, 0, prefix=2)
    want = [{0, 1}, {0, 1}, {0, 1, 2}, {0, 1, 2, 3}, {0, 1, 2, 3, 4}, {0, 1, 3, 4, 5},
            {0, 1, 4, 5, 6}, {0, 1, 5, 6, 7}, {0, 1, 6, 7, 8}, {0, 1, 7, 8, 9}]
    for i, keys in enumerate(want):
        assert set(np.flatnonzero(ok[i])) == keys, i
    # with input_pos = -3 the window part of rows 0..2 is empty, the prefix stays
    ok = ora.flex_mask(6, 6, True, 3, -3, prefix=2)
    assert [set(np.flatnonzero(r)) for r in ok] == [{0, 1}, {0, 1}, {0, 1}, {0, 1},
                                                   {0, 1}, {0, 1, 2}]


def test_prefix_or_window_attention_is_attention_over_the_two_intervals():
    _, Q, K, V = _flex_case(58, Sq=12, Sk=12)
    O, L = ora.flex_ref(Q, K, V, True, 3, prefix=2)
    keys = [0, 1, 7, 8, 9]  # row 9: the prefix and the window's three keys
    Og, Lg = ora.attn_ref(Q[:, :, 9:10], K[:, :, keys], V[:, :, keys], False)
    np.testing.assert_allclose(O[:, :, 9:10], Og, atol=1e-14)
    np.testing.assert_allclose(L[:, :, 9:10], Lg, atol=1e-14)


def _block_mask_pins_pass():
    try:
        # two documents of 128 under a causal mask, 64 x 64 blocks
        doc = np.repeat([0, 1], 128)
        got = ora.block_mask_ref(ora.flex_mask(256, 256, True, doc_q=doc, doc_kv=doc))
        assert got.tolist() == [[1, 0, 0, 0], [2, 1, 0, 0], [0, 0, 1, 0], [0, 0, 2, 1]]
        # ragged last blocks are classed on the pairs that exist
        got = ora.block_mask_ref(ora.flex_mask(100, 100, True))
        assert got.tolist() == [[1, 0], [2, 1]]
        # key lengths and shifted queries
        got = ora.block_mask_ref(ora.flex_mask(64, 128, False, k_len=100))
        assert got.tolist() == [[2, 1]]
        got = ora.block_mask_ref(ora.flex_mask(64, 192, True, input_pos=128))
        assert got.tolist() == [[2, 2, 1]]
        # unequal tile sizes, worked by hand: rows {0,1},{2,3}; keys {0,1,2},{3,4}
        got = ora.block_mask_ref(ora.flex_mask(4, 5, True), tile_m=2, tile_n=3)
        assert got.shape == (2, 2) and got.tolist() == [[1, 0], [2, 1]]
        # a batch axis is carried through
        ok = np.stack([ora.flex_mask(4, 5, True), np.ones((4, 5), bool)])
        assert ora.block_mask_ref(ok, 2, 3).tolist() == [[[1, 0], [2, 1]], [[2, 2], [2, 2]]]
    except AssertionError:
        return False
    return True


def test_block_mask_closed_forms():
    assert _block_mask_pins_pass()


ORIG_BLOCK_MASK = ora.block_mask_ref


def _mut_bm_classes_swapped(ok, tile_m=64, tile_n=64):
    c = ORIG_BLOCK_MASK(ok, tile_m, tile_n)
    return np.where(c == 1, 2, np.where(c == 2, 1, 0)).astype(np.uint8)


def _mut_bm_tiles_swapped(ok, tile_m=64, tile_n=64):
    return ORIG_BLOCK_MASK(ok, tile_n, tile_m)


def _mut_bm_padded(ok, tile_m=64, tile_n=64):
    ok = np.asarray(ok, bool)
    Sq, Sk = ok.shape[-2:]
    pad = np.zeros(ok.shape[:-2] + (-(-Sq // tile_m) * tile_m, -(-Sk // tile_n) * tile_n), bool)
    pad[..., :Sq, :Sk] = ok
    return ORIG_BLOCK_MASK(pad, tile_m, tile_n)


@pytest.mark.parametrize("mutant", [_mut_bm_classes_swapped, _mut_bm_tiles_swapped,
                                    _mut_bm_padded])
def test_planted_block_mask_mistakes(monkeypatch, mutant):
    assert _block_mask_pins_pass()
    monkeypatch.setattr(ora, "block_mask_ref", mutant)
    assert not _block_mask_pins_pass()


def _flex_pins_pass():
    checks = [
        lambda: test_flex_bias_alibi_document_prefix_vs_torch_sdpa((2, 4)),
        test_alibi_closed_form_geometric_weights,
        test_softcap_bruteforce_mpmath,
        test_prefix_lm_decomposes,
        test_document_mask_block_diagonal_equals_separate_sequences,
        test_q_lengths_rows_attend_to_nothing,
        test_prefix_or_window_rows_hand_worked,
        test_prefix_or_window_attention_is_attention_over_the_two_intervals,
    ]
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError, TypeError):
            return False
    return True


ORIG_SCORE_MODS = ora.score_mods
ORIG_FLEX_MASK = ora.flex_mask


def _mut_alibi_sign(s, rows, input_pos, bias=None, alibi_slope=None, softcap=0.0):
    return ORIG_SCORE_MODS(s, rows, input_pos, bias,
                           None if alibi_slope is None else -alibi_slope, softcap)


def _mut_alibi_local_positions(s, rows, input_pos, bias=None, alibi_slope=None, softcap=0.0):
    return ORIG_SCORE_MODS(s, rows, 0, bias, alibi_slope, softcap)


def _mut_softcap_first(s, rows, input_pos, bias=None, alibi_slope=None, softcap=0.0):
    out = softcap * np.tanh(s / softcap) if softcap else s
    return ORIG_SCORE_MODS(out, rows, input_pos, bias, alibi_slope, 0.0)


def _mut_bias_transposed(s, rows, input_pos, bias=None, alibi_slope=None, softcap=0.0):
    if bias is not None:
        bias = np.asarray(bias)
        n = min(bias.shape)
        bias = bias.copy()
        bias[:n, :n] = bias[:n, :n].T
    return ORIG_SCORE_MODS(s, rows, input_pos, bias, alibi_slope, softcap)


def _mut_prefix_and(Sq, Sk, causal=False, window=0, input_pos=0, k_len=None, q_len=None,
                    prefix=0, doc_q=None, doc_kv=None):
    ok = ORIG_FLEX_MASK(Sq, Sk, causal, window, input_pos, k_len, q_len, 0, doc_q, doc_kv)
    if prefix > 0:
        ok &= np.arange(Sk)[None, :] < prefix
    return ok


def _mut_qlen_ignored(Sq, Sk, causal=False, window=0, input_pos=0, k_len=None, q_len=None,
                      prefix=0, doc_q=None, doc_kv=None):
    return ORIG_FLEX_MASK(Sq, Sk, causal, window, input_pos, k_len, None, prefix, doc_q, doc_kv)


def _mut_doc_shifted(Sq, Sk, causal=False, window=0, input_pos=0, k_len=None, q_len=None,
                     prefix=0, doc_q=None, doc_kv=None):
    if doc_q is not None:
        doc_q = np.roll(np.asarray(doc_q), 1)
    return ORIG_FLEX_MASK(Sq, Sk, causal, window, input_pos, k_len, q_len, prefix, doc_q, doc_kv)


def _mut_prefix_dropped_with_window(Sq, Sk, causal=False, window=0, input_pos=0, k_len=None,
                                    q_len=None, prefix=0, doc_q=None, doc_kv=None):
    return ORIG_FLEX_MASK(Sq, Sk, causal, window, input_pos, k_len, q_len,
                          0 if window > 0 else prefix, doc_q, doc_kv)


@pytest.mark.parametrize("target,mutant", [
    ("flex_mask", _mut_prefix_dropped_with_window),
    ("score_mods", _mut_alibi_sign),
    ("score_mods", _mut_alibi_local_positions),
    ("score_mods", _mut_softcap_first),
    ("score_mods", _mut_bias_transposed),
    ("flex_mask", _mut_prefix_and),
    ("flex_mask", _mut_qlen_ignored),
    ("flex_mask", _mut_doc_shifted),
])
def test_planted_flex_mistakes(monkeypatch, target, mutant):
    assert _flex_pins_pass()
    monkeypatch.setattr(ora, target, mutant)
    assert not _flex_pins_pass(), f"no pin caught the planted mistake in {target}"


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def _loss(Q, K, V, dO, **kw):
    O, _ = ora.attn_ref(Q, K, V, **kw)
    return float(np.sum(np.where(np.isnan(O), 0.0, O) * dO))


@pytest.mark.parametrize("kw", [dict(causal=False), dict(causal=True),
                                dict(causal=True, window=3, input_pos=2, k_lengths=[7, 5])],
                         ids=["full", "causal", "window_offset_klen"])
def test_bwd_matches_central_differences(kw):
    # d/dx of sum(dO * O(Q, K, V)) by central differences of the forward oracle
    rng = np.random.default_rng(70)
    B, H, Hkv, Sq, Sk, D = 2, 4, 2, 5, 7, 3
    Q = rng.standard_normal((B, H, Sq, D))
    K = rng.standard_normal((B, Hkv, Sk, D))
    V = rng.standard_normal((B, Hkv, Sk, D))
    dO = rng.standard_normal((B, H, Sq, D))
    dQ, dK, dV = ora.attn_bwd_ref(Q, K, V, dO, **kw)
    eps = 1e-6
    for X, G in ((Q, dQ), (K, dK), (V, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            x0 = X[idx]
            X[idx] = x0 + eps
            lp = _loss(Q, K, V, dO, **kw)
            X[idx] = x0 - eps
            lm = _loss(Q, K, V, dO, **kw)
            X[idx] = x0
            num[idx] = (lp - lm) / (2 * eps)
        G = np.where(np.isnan(G), 0.0, G)
        np.testing.assert_allclose(G, num, atol=1e-7)


def test_bwd_matches_torch_autograd():
    rng = np.random.default_rng(71)
    B, H, Hkv, S, D = 2, 8, 2, 33, 16
    Q = rng.standard_normal((B, H, S, D))
    K = rng.standard_normal((B, Hkv, S, D))
    V = rng.standard_normal((B, Hkv, S, D))
    dO = rng.standard_normal((B, H, S, D))
    dQ, dK, dV = ora.attn_bwd_ref(Q, K, V, dO, causal=True)
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(H // Hkv, dim=1), v.repeat_interleave(H // Hkv, dim=1),
        is_causal=True)
    o.backward(torch.from_numpy(dO))
    np.testing.assert_allclose(dQ, q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK, k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV, v.grad.numpy(), atol=1e-12)


def test_bwd_special_cases():
    rng = np.random.default_rng(72)
    B, H, S, D = 1, 2, 6, 4
    Q = rng.standard_normal((B, H, S, D))
    K = rng.standard_normal((B, H, S, D))
    V = rng.standard_normal((B, H, S, D))
    dO = rng.standard_normal((B, H, S, D))
    # constant V: O does not depend on Q or K at all
    Vc = np.ones_like(V) * 0.7
    dQ, dK, dV = ora.attn_bwd_ref(Q, K, Vc, dO, causal=True)
    np.testing.assert_allclose(dQ, 0.0, atol=1e-14)
    np.testing.assert_allclose(dK, 0.0, atol=1e-14)
    # dV columns sum to the dO columns (each row of P sums to one)
    np.testing.assert_allclose(dV.sum(axis=2), dO.sum(axis=2), atol=1e-12)
    # a row whose only key is itself (window 1): O = V_i exactly, so dV_i = dO_i
    # and no gradient reaches Q or K
    dQ, dK, dV = ora.attn_bwd_ref(Q, K, V, dO, causal=True, window=1)
    np.testing.assert_allclose(dV, dO, atol=1e-14)
    np.testing.assert_allclose(dQ, 0.0, atol=1e-14)
    np.testing.assert_allclose(dK, 0.0, atol=1e-14)


def test_planted_bwd_mistakes(monkeypatch):
    def no_rowsum(P, dP):
        return P * dP

    def transposed(P, dP):
        return (P * (dP - (dP * P).sum(axis=1, keepdims=True))).T.T * 1.0001

    for mutant in (no_rowsum, transposed):
        monkeypatch.setattr(ora, "softmax_backward", mutant)
        with pytest.raises(AssertionError):
            test_bwd_matches_central_differences(dict(causal=True))
    monkeypatch.undo()
    real = ora.scores
    monkeypatch.setattr(ora, "scores", lambda q, k, scale: real(q, k, 1.0))
    with pytest.raises(AssertionError):
        test_bwd_matches_torch_autograd()


# ---------------------------------------------------------------------------
# block-sparse prefill: estimators, block masks, masked attention
# ---------------------------------------------------------------------------

def test_key_block_stats_bruteforce():
    rng = np.random.default_rng(90)
    k = rng.standard_normal((11, 3))
    c, r, lo, hi = ora.key_block_stats(k, 4)
    assert c.shape == (3, 3)
    for b, rows in enumerate([k[0:4], k[4:8], k[8:11]]):
        for d in range(3):
            assert abs(c[b, d] - math.fsum(rows[:, d]) / len(rows)) < 1e-15
            assert lo[b, d] == min(rows[:, d]) and hi[b, d] == max(rows[:, d])
        assert abs(r[b] - max(math.dist(x, c[b]) for x in rows)) < 1e-14


def test_radius_weights_hand_worked():
    # quantiles of [1..5]: median 3, 90th percentile 4.6 (linear interpolation)
    np.testing.assert_allclose(ora.radius_weights(np.array([1., 2., 3., 4., 5.])),
                               [0, 0, 0, 0.625, 1], atol=1e-15)
    # equal quantiles: only blocks strictly wider than r_low get the bound
    np.testing.assert_array_equal(ora.radius_weights(np.array([2., 2., 2., 2.])), [0, 0, 0, 0])
    np.testing.assert_array_equal(ora.radius_weights(np.array([1., 2., 2., 2., 2.]), 0.5, 0.6),
                                  [0, 0, 0, 0, 0])


def _exact_block_scores(Q, K, bs):
    """lse over a query block's tokens of the true max_k q.k/sqrt(D) in the key block."""
    B, H, Sq, D = Q.shape
    Hkv, Sk = K.shape[1], K.shape[2]
    nq, nk = -(-Sq // bs), -(-Sk // bs)
    out = np.empty((B, H, nq, nk))
    for b in range(B):
        for h in range(H):
            s = Q[b, h] @ K[b, h // (H // Hkv)].T / math.sqrt(D)
            for a in range(nq):
                for c in range(nk):
                    m = s[a * bs:(a + 1) * bs, c * bs:(c + 1) * bs].max(axis=1)
                    out[b, h, a, c] = math.log(math.fsum(math.exp(x) for x in m))
    return out


def test_rbs_scores_mpmath_and_bounds():
    rng = np.random.default_rng(91)
    B, H, Hkv, Sq, Sk, D, bs = 1, 2, 1, 6, 9, 3, 4
    Q = rng.standard_normal((B, H, Sq, D))
    K = rng.standard_normal((B, Hkv, Sk, D))
    base, rescue = ora.rbs_block_scores_ref(Q, K, bs)
    c, r, _, _ = ora.key_block_stats(K[0, 0], bs)
    beta = ora.radius_weights(r)
    mpmath.mp.dps = 30
    for h in range(H):
        for a in range(2):
            for blk in range(3):
                tb, tr = [], []
                for i in range(a * bs, min((a + 1) * bs, Sq)):
                    q = [mpmath.mpf(x) for x in Q[0, h, i]]
                    qc = mpmath.fsum(q[d] * mpmath.mpf(c[blk, d]) for d in range(D))
                    qn = mpmath.sqrt(mpmath.fsum(x * x for x in q))
                    tb.append(mpmath.exp(qc / mpmath.sqrt(D)))
                    tr.append(mpmath.exp((qc + qn * mpmath.mpf(r[blk] * beta[blk])) / mpmath.sqrt(D)))
                assert abs(float(mpmath.log(mpmath.fsum(tb))) - base[0, h, a, blk]) < 1e-12
                assert abs(float(mpmath.log(mpmath.fsum(tr))) - rescue[0, h, a, blk]) < 1e-12
    assert np.all(rescue >= base - 1e-12)
    # with the full radius (beta = 1) the rescue score bounds the true block score
    exact = _exact_block_scores(Q, K, bs)
    full = beta == 1
    assert full.any()
    assert np.all(rescue[..., full] >= exact[..., full] - 1e-12)


def test_minmax_scores_bound_and_single_key_blocks():
    rng = np.random.default_rng(92)
    Q = rng.standard_normal((1, 2, 10, 4))
    K = rng.standard_normal((1, 2, 13, 4))
    mm = ora.minmax_block_scores_ref(Q, K, 4)
    assert np.all(mm >= _exact_block_scores(Q, K, 4) - 1e-12)
    # one key per block: the box is a point, the bound is exact
    np.testing.assert_allclose(ora.minmax_block_scores_ref(Q, K, 1),
                               _exact_block_scores(Q, K, 1), atol=1e-12)


def test_relative_and_topk_masks_hand_worked():
    s = np.array([[0.0, -1.0, -2.0, -1.5], [3.0, 1.0, 3.0, 2.0]])
    # ln 0.22 = -1.514: keep scores >= max - 1.514
    np.testing.assert_array_equal(ora.relative_block_mask_ref(s, 0.22),
                                  [[True, True, False, True], [True, False, True, True]])
    np.testing.assert_array_equal(ora.top_k_block_mask_ref(s, 2),
                                  [[True, True, False, False], [True, False, True, False]])
    np.testing.assert_array_equal(ora.top_k_block_mask_ref(np.ones((1, 4)), 2),
                                  [[True, True, False, False]])
    np.testing.assert_array_equal(ora.band_block_mask_ref(3, 4, 1),
                                  [[1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0]])


def test_relative_mask_decision_precision():
    # ln 0.18 = -1.71479842809..., which float32 rounds down to
    # -1.71479845047; a score at exactly that float32 value sits below the
    # exact threshold (dropped in float64) and on the float32 threshold (kept
    # when the decision is taken in float32, as a float32 kernel takes it)
    t32 = np.float32(math.log(0.18))
    assert float(t32) < math.log(0.18)
    s = np.array([[0.0, t32, np.float32(-1.8), np.float32(-1.7)]], dtype=np.float32)
    np.testing.assert_array_equal(ora.relative_block_mask_ref(s, 0.18),
                                  [[True, False, False, True]])
    np.testing.assert_array_equal(ora.relative_block_mask_ref(s, 0.18, np.float32),
                                  [[True, True, False, True]])


def test_block_sparse_attention_vs_torch_and_special_cases():
    rng = np.random.default_rng(93)
    B, H, Hkv, S, D, bs = 1, 4, 2, 20, 8, 4
    Q = rng.standard_normal((B, H, S, D))
    K = rng.standard_normal((B, Hkv, S, D))
    V = rng.standard_normal((B, Hkv, S, D))
    nb = S // bs
    keep = rng.random((B, H, nb, nb)) < 0.5
    keep[:, :, np.arange(nb), np.arange(nb)] = True        # diagonal kept
    keep[0, 1, 2] = False                                  # a row block with no key
    O, L = ora.block_sparse_attn_ref(Q, K, V, keep, bs, causal=True)
    tok = np.repeat(np.repeat(keep, bs, axis=2), bs, axis=3)
    ok = tok & np.tril(np.ones((S, S), dtype=bool))
    qt, kt, vt = (torch.from_numpy(x) for x in (Q, np.repeat(K, 2, axis=1), np.repeat(V, 2, axis=1)))
    Ot = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(ok)).numpy()
    has = ok.any(axis=3)
    np.testing.assert_allclose(O[has], Ot[has], atol=1e-12)
    assert np.all(O[~has] == 0) and np.all(np.isneginf(L[~has]))
    assert (~has[0, 1, 8:12]).all()
    # keeping every block is plain attention
    Oa, La = ora.block_sparse_attn_ref(Q, K, V, np.ones_like(keep), bs, causal=True)
    Or, Lr = ora.attn_ref(Q, K, V, True)
    np.testing.assert_array_equal(Oa, Or)


def _bs_pins_pass():
    checks = [test_key_block_stats_bruteforce, test_radius_weights_hand_worked,
              test_rbs_scores_mpmath_and_bounds, test_minmax_scores_bound_and_single_key_blocks,
              test_relative_and_topk_masks_hand_worked,
              test_block_sparse_attention_vs_torch_and_special_cases]
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError, TypeError):
            return False
    return True


ORIG_STATS = ora.key_block_stats
ORIG_RW = ora.radius_weights
ORIG_REL = ora.relative_block_mask_ref
ORIG_TOPK = ora.top_k_block_mask_ref


def _mut_stats_sum(k, bs):
    c, r, lo, hi = ORIG_STATS(k, bs)
    return c * bs, r, lo, hi


def _mut_stats_min_radius(k, bs):
    k = np.asarray(k, dtype=np.float64)
    c, r, lo, hi = ORIG_STATS(k, bs)
    r = np.array([np.sqrt(((k[b * bs:(b + 1) * bs] - c[b]) ** 2).sum(axis=1)).min()
                  for b in range(len(r))])
    return c, r, lo, hi


def _mut_rw_swapped(r, low=0.5, high=0.9):
    return ORIG_RW(r, high, low)


def _mut_rel_alpha(scores, alpha):
    s = np.asarray(scores, dtype=np.float64)
    return s >= s.max(axis=-1, keepdims=True) + alpha


def _mut_topk_ties(scores, k):
    s = np.asarray(scores, dtype=np.float64)
    return ORIG_TOPK(s[..., ::-1], k)[..., ::-1]


@pytest.mark.parametrize("target,mutant", [
    ("key_block_stats", _mut_stats_sum),
    ("key_block_stats", _mut_stats_min_radius),
    ("radius_weights", _mut_rw_swapped),
    ("relative_block_mask_ref", _mut_rel_alpha),
    ("top_k_block_mask_ref", _mut_topk_ties),
])
def test_planted_block_sparse_mistakes(monkeypatch, target, mutant):
    assert _bs_pins_pass()
    monkeypatch.setattr(ora, target, mutant)
    assert not _bs_pins_pass(), f"no pin caught the planted mistake in {target}"


def test_planted_block_sparse_attention_mistake(monkeypatch):
    real = ora.block_sparse_attn_ref

    def transposed(Q, K, V, keep, *a, **kw):
        return real(Q, K, V, np.swapaxes(np.asarray(keep), -1, -2), *a, **kw)

    monkeypatch.setattr(ora, "block_sparse_attn_ref", transposed)
    with pytest.raises(AssertionError):
        test_block_sparse_attention_vs_torch_and_special_cases()
