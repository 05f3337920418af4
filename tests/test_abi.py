"""CPU checks of the C ABI and host logic (no GPU needed).

* the library loads and exports every entry point include/attn.h declares;
* argument validation returns the documented status codes before any HIP call;
* the kernels' mask geometry and tile classifier, compiled for the host,
  agree bit-exactly with the oracle's brute-force mask and tile plan.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import scaled_dot_product_attn_amd as attn
from scaled_dot_product_attn_amd import _build
from oracle import attn_oracle as ora

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.LIB_PATH):
        _build.build()
    return attn.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\*]+\s+\**)+\**(attn_\w+)\s*\(", text, re.M)))


def test_header_declares_expected_entry_points():
    names = _declared()
    for n in ("attn_fwd", "attn_fwd_f32", "attn_decode", "attn_decode_ws",
              "attn_decode_workspace_bytes", "attn_decode_paged", "attn_fwd_flex",
              "attn_bwd", "attn_bwd_workspace_bytes", "attn_block_scores",
              "attn_block_scores_workspace_bytes", "attn_block_mask", "attn_fwd_block_sparse",
              "attn_decode_static", "attn_mask_dump", "attn_build_block_mask",
              "attn_tile_plan",
              "attn_status_string", "attn_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", attn.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, re.M))
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_version_and_status_strings(lib):
    assert attn.attn_version() == 10000
    assert attn.attn_status_string(0) == "ok"
    assert "invalid" in attn.attn_status_string(1)
    assert "unsupported" in attn.attn_status_string(2)
    assert "HIP" in attn.attn_status_string(3)
    assert attn.attn_status_string(99) == "unknown status"


def _fwd(lib, fn="attn_fwd", O=1, Q=1, K=1, V=1, B=1, H=4, Hkv=2, Sq=8, Sk=8,
         D=128, causal=1, window=0, ip=0):
    return getattr(lib, fn)(O, Q, K, V, None, B, H, Hkv, Sq, Sk, D, causal, window,
                            ip, None, None)


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_f32"])
def test_fwd_argument_errors(lib, fn):
    assert _fwd(lib, fn, H=3, Hkv=2) == attn.ATTN_EINVAL
    assert _fwd(lib, fn, Hkv=0) == attn.ATTN_EINVAL
    assert _fwd(lib, fn, B=0) == attn.ATTN_EINVAL
    assert _fwd(lib, fn, Sq=-1) == attn.ATTN_EINVAL
    assert _fwd(lib, fn, causal=0, window=4) == attn.ATTN_EINVAL
    assert _fwd(lib, fn, causal=2) == attn.ATTN_EINVAL
    assert _fwd(lib, fn, D=96) == attn.ATTN_EUNSUPPORTED
    assert _fwd(lib, fn, D=256) == attn.ATTN_EUNSUPPORTED
    assert _fwd(lib, fn, O=None) == attn.ATTN_EINVAL
    assert _fwd(lib, fn, K=None) == attn.ATTN_EINVAL
    assert _fwd(lib, fn, Sq=2**31 - 10) == attn.ATTN_EUNSUPPORTED
    # nothing to do: returns before touching the device
    assert _fwd(lib, fn, Sq=0, O=None, Q=None) == attn.ATTN_OK


def test_fwd_flex_argument_errors(lib):
    def flex(f=None, causal=1, window=0, B=1, H=4, Sq=8, Sk=8, D=128):
        return lib.attn_fwd_flex(1, 1, 1, 1, None, B, H, 2, Sq, Sk, D, causal, window, 0,
                                 None, None if f is None else ctypes.byref(f), None)
    assert flex(H=3) == attn.ATTN_EINVAL
    assert flex(D=96) == attn.ATTN_EUNSUPPORTED
    assert flex(causal=0, window=3) == attn.ATTN_EINVAL
    assert flex(attn.AttnFlex(softcap=-1.0)) == attn.ATTN_EINVAL
    assert flex(attn.AttnFlex(qk_scale=-0.5)) == attn.ATTN_EINVAL
    assert flex(attn.AttnFlex(prefix=-1)) == attn.ATTN_EINVAL
    # a prefix beside a window is accepted (a row then sees two key intervals):
    # with Sq = 0 the call returns before touching the device
    assert flex(attn.AttnFlex(prefix=4), window=2, Sq=0) == attn.ATTN_OK
    assert flex(attn.AttnFlex(block_mask=8, block_mask_B=3), B=2) == attn.ATTN_EINVAL
    assert flex(attn.AttnFlex(block_mask=8, block_mask_B=0)) == attn.ATTN_EINVAL
    assert flex(attn.AttnFlex(block_mask=8, block_mask_B=1), Sk=64 * 2048 + 1) == \
        attn.ATTN_EUNSUPPORTED
    assert flex(attn.AttnFlex(bias=8, bias_B=3, bias_H=1), B=2) == attn.ATTN_EINVAL
    assert flex(attn.AttnFlex(bias=8, bias_B=1, bias_H=2)) == attn.ATTN_EINVAL
    assert flex(attn.AttnFlex(bias=8, bias_B=1, bias_H=1), Sq=40000, Sk=40000) == \
        attn.ATTN_EUNSUPPORTED
    assert flex(attn.AttnFlex(doc_q=8)) == attn.ATTN_EINVAL
    assert flex(attn.AttnFlex(doc_kv=8)) == attn.ATTN_EINVAL
    assert flex(Sq=0) == attn.ATTN_OK


def test_build_block_mask_argument_errors(lib):
    def bm(out=8, B=1, Sq=8, Sk=8, causal=1, window=0, f=None):
        return lib.attn_build_block_mask(out, B, Sq, Sk, causal, window, 0, None,
                                         None if f is None else ctypes.byref(f), None)
    assert bm(B=0) == attn.ATTN_EINVAL
    assert bm(Sq=-1) == attn.ATTN_EINVAL
    assert bm(causal=2) == attn.ATTN_EINVAL
    assert bm(causal=0, window=3) == attn.ATTN_EINVAL
    assert bm(window=-1) == attn.ATTN_EINVAL
    assert bm(f=attn.AttnFlex(prefix=-1)) == attn.ATTN_EINVAL
    assert bm(f=attn.AttnFlex(doc_q=8)) == attn.ATTN_EINVAL
    assert bm(Sk=64 * 2048 + 1) == attn.ATTN_EUNSUPPORTED
    assert bm(out=None) == attn.ATTN_EINVAL
    # nothing to do: returns before touching the device
    assert bm(out=None, Sq=0) == attn.ATTN_OK
    assert bm(out=None, Sk=0) == attn.ATTN_OK


def test_bwd_argument_errors(lib):
    def bwd(dQ=1, dK=1, dV=1, dO=1, L=1, H=4, Hkv=2, Sq=8, Sk=8, D=128, causal=1, window=0,
            ws=256, nbytes=1 << 20):
        return lib.attn_bwd(dQ, dK, dV, dO, 1, 1, 1, 1, L, 1, H, Hkv, Sq, Sk, D, causal,
                            window, 0, None, ws, nbytes, None)
    assert bwd(H=3) == attn.ATTN_EINVAL
    assert bwd(D=96) == attn.ATTN_EUNSUPPORTED
    # a head's Q / dO rows past the 32-bit byte offsets of the staging loads
    assert bwd(H=2, Hkv=2, Sq=(1 << 31) // (128 * 4), Sk=8) == attn.ATTN_EUNSUPPORTED
    assert bwd(causal=0, window=2) == attn.ATTN_EINVAL
    for k in ("dQ", "dK", "dV", "dO", "L"):
        assert bwd(**{k: None}) == attn.ATTN_EINVAL, k
    need = lib.attn_bwd_workspace_bytes(1, 4, 8, 128)
    assert need == 2 * 256
    assert bwd(nbytes=need - 1) == attn.ATTN_EINVAL
    assert bwd(ws=260, nbytes=need) == attn.ATTN_EINVAL
    assert lib.attn_bwd_workspace_bytes(0, 4, 8, 128) == 0
    assert bwd(Sq=0, Sk=0) == attn.ATTN_OK


def test_block_sparse_argument_errors(lib):
    def sc(kind=0, low=0.5, high=0.9, H=4, Hkv=2, Sq=64, Sk=64, D=128, base=1):
        return lib.attn_block_scores(base, None, 1, 1, 1, H, Hkv, Sq, Sk, D, kind, low, high,
                                     256, 1 << 30, None)
    assert sc(kind=2) == attn.ATTN_EINVAL
    assert sc(low=1.5) == attn.ATTN_EINVAL
    assert sc(H=3) == attn.ATTN_EINVAL
    assert sc(D=96) == attn.ATTN_EUNSUPPORTED
    assert sc(Sk=64 * 4097) == attn.ATTN_EUNSUPPORTED
    assert sc(base=None) == attn.ATTN_EINVAL
    assert lib.attn_block_scores_workspace_bytes(1, 2, 64, 128) > 0
    assert lib.attn_block_scores_workspace_bytes(1, 2, 64, 80) == 0

    def mk(keep=1, scores=1, rows=4, mode=0, alpha=0.5, k=1):
        return lib.attn_block_mask(keep, scores, rows, 2, 8, mode, alpha, k, 1, 0, None)
    assert mk(keep=None) == attn.ATTN_EINVAL
    assert mk(mode=3) == attn.ATTN_EINVAL
    assert mk(alpha=0.0) == attn.ATTN_EINVAL
    assert mk(alpha=1.5) == attn.ATTN_EINVAL
    assert mk(mode=1, k=-1) == attn.ATTN_EINVAL
    assert mk(scores=None) == attn.ATTN_EINVAL
    assert mk(rows=0) == attn.ATTN_OK

    def sp(keep=1, Sk=64, causal=1, window=0):
        return lib.attn_fwd_block_sparse(1, 1, 1, 1, None, 1, 4, 2, 64, Sk, 128, causal,
                                         window, 0, None, keep, None)
    assert sp(keep=None) == attn.ATTN_EINVAL
    assert sp(causal=0, window=3) == attn.ATTN_EINVAL
    assert sp(Sk=64 * 2049) == attn.ATTN_EUNSUPPORTED


def test_decode_argument_errors(lib):
    def dec(O=1, Q=1, K=1, V=1, L=1, ns=8, B=2, H=8, Hkv=2, S=64, D=128):
        return lib.attn_decode(O, Q, K, V, L, ns, B, H, Hkv, S, D, None)
    assert dec(ns=0) == attn.ATTN_EINVAL
    assert dec(H=6, Hkv=4) == attn.ATTN_EINVAL
    assert dec(S=0) == attn.ATTN_EINVAL
    assert dec(L=None) == attn.ATTN_EINVAL
    assert dec(D=80) == attn.ATTN_EUNSUPPORTED
    ws_need = lib.attn_decode_workspace_bytes(2, 8, 8, 128)
    assert ws_need == 2 * 8 * 8 * 128 * 4 + 512
    # too small or misaligned workspace: rejected before any launch
    assert lib.attn_decode_ws(1, 1, 1, 1, 1, 8, 2, 8, 2, 64, 128, 256, ws_need - 1,
                              None) == attn.ATTN_EINVAL
    assert lib.attn_decode_ws(1, 1, 1, 1, 1, 8, 2, 8, 2, 64, 128, 260, ws_need,
                              None) == attn.ATTN_EINVAL
    assert lib.attn_decode_workspace_bytes(0, 8, 8, 128) == 0
    assert lib.attn_decode_workspace_bytes(2, 8, 8, 96) == 0


def test_decode_static_argument_errors(lib):
    # the argument checks of attn_decode, and sizes past the static scratch
    # refused before any HIP call (the array's address is not looked up)
    def dec(O=1, Q=1, K=1, V=1, L=1, ns=8, B=2, H=8, Hkv=2, S=64, D=128):
        return lib.attn_decode_static(O, Q, K, V, L, ns, B, H, Hkv, S, D, None)
    assert dec(ns=0) == attn.ATTN_EINVAL
    assert dec(H=6, Hkv=4) == attn.ATTN_EINVAL
    assert dec(L=None) == attn.ATTN_EINVAL
    assert dec(D=80) == attn.ATTN_EUNSUPPORTED
    limit = attn.DECODE_STATIC_SCRATCH_BYTES
    # the largest batch that fits at H = 32, n_splits = 8, D = 128, and one more
    per_seq = lib.attn_decode_workspace_bytes(1, 32, 8, 128)
    B = limit // per_seq
    while lib.attn_decode_workspace_bytes(B, 32, 8, 128) > limit:
        B -= 1
    assert lib.attn_decode_workspace_bytes(B + 1, 32, 8, 128) > limit
    assert dec(B=B + 1, H=32, Hkv=8) == attn.ATTN_EUNSUPPORTED
    assert dec(B=4096, H=32, Hkv=8) == attn.ATTN_EUNSUPPORTED


def test_decode_paged_argument_errors(lib):
    def dec(O=1, Q=1, K=1, V=1, T=1, L=1, ns=8, B=2, H=8, Hkv=2, nb=16, bs=16, mb=4,
            D=128, ws=256, nbytes=1 << 20):
        return lib.attn_decode_paged(O, Q, K, V, T, L, ns, B, H, Hkv, nb, bs, mb, D, ws,
                                     nbytes, None)
    assert dec(ns=0) == attn.ATTN_EINVAL
    assert dec(H=6, Hkv=4) == attn.ATTN_EINVAL
    assert dec(nb=0) == attn.ATTN_EINVAL
    assert dec(mb=0) == attn.ATTN_EINVAL
    assert dec(bs=0) == attn.ATTN_EINVAL
    assert dec(bs=12) == attn.ATTN_EINVAL          # not a power of two
    assert dec(bs=2048) == attn.ATTN_EUNSUPPORTED
    assert dec(mb=2 ** 30, bs=16) == attn.ATTN_EUNSUPPORTED
    assert dec(T=None) == attn.ATTN_EINVAL
    assert dec(L=None) == attn.ATTN_EINVAL
    assert dec(D=96) == attn.ATTN_EUNSUPPORTED
    need = lib.attn_decode_workspace_bytes(2, 8, 8, 128)
    assert dec(nbytes=need - 1) == attn.ATTN_EINVAL
    assert dec(ws=260, nbytes=need) == attn.ATTN_EINVAL


def test_debug_export_argument_errors(lib):
    assert lib.attn_mask_dump(None, 4, 4, 0, 2, 0, 4, None) == attn.ATTN_EINVAL
    assert lib.attn_mask_dump(None, 4, 4, 1, 0, 0, 4, None) == attn.ATTN_EINVAL
    assert lib.attn_mask_dump(None, 0, 4, 1, 0, 0, 4, None) == attn.ATTN_OK
    assert lib.attn_tile_plan(None, 4, 4, 1, 0, 0, 4, 1, None) == attn.ATTN_EINVAL
    assert lib.attn_tile_plan(None, 0, 0, 1, 0, 0, 0, 1, None) == attn.ATTN_OK
    assert lib.attn_tile_plan(1, 4, 4, 1, 0, 0, 4, 0, None) == attn.ATTN_EINVAL


@pytest.fixture(scope="module")
def plan_check(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("host") / "plan_check")
    subprocess.run([_build.HIPCC, "-O1", "-std=c++17",
                    "-I", os.path.join(ROOT, "scaled_dot_product_attn_amd", "csrc"),
                    os.path.join(ROOT, "tests", "host", "plan_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Sq = int(rng.integers(1, 300))
        Sk = int(rng.integers(0, 400))
        causal = int(rng.integers(0, 2))
        window = int(rng.choice([0, 0, 1, 2, 5, 64, 100, 500])) if causal else 0
        ip = int(rng.integers(-100, 500))
        kl = int(rng.integers(-5, Sk + 6))
        tm, tn = [(128, 64), (64, 32), (16, 16), (7, 5)][int(rng.integers(0, 4))]
        # a prefix (prefix_lm) only with causal masking and no window
        prefix = int(rng.choice([0, 0, 1, 7, 100, 300])) if causal and window == 0 else 0
        cases.append((Sq, Sk, causal, window, ip, kl, tm, tn, prefix))
    return cases


def _plan_from_mask(ok, Sq, Sk, tm, tn):
    """Empty / partial / full per tile, by brute force over the element mask."""
    nqt, nkt = -(-Sq // tm), -(-Sk // tn)
    pad = np.zeros((Sq, nkt * tn), dtype=bool)
    pad[:, :Sk] = ok
    plan = np.empty((nqt, nkt), dtype=np.int8)
    for qt in range(nqt):
        for kt in range(nkt):
            blk = pad[qt * tm:(qt + 1) * tm, kt * tn:(kt + 1) * tn]
            plan[qt, kt] = ora.TILE_EMPTY if not blk.any() else (
                ora.TILE_FULL if blk.all() else ora.TILE_PARTIAL)
    return plan


def test_host_geometry_matches_oracle(plan_check):
    cases = _random_cases(400, 1) + [
        (4096, 4096, 1, 0, 0, 4096, 128, 64, 0), (2048, 16384, 1, 4096, 14336, 16384, 128, 64, 0),
        (256, 256, 1, 0, 0, 256, 128, 64, 0), (256, 256, 1, 64, 0, 256, 128, 64, 0),
        (100, 100, 0, 0, 0, 100, 64, 64, 0), (10, 0, 0, 0, 0, 0, 128, 64, 0),
        (300, 300, 1, 0, 0, 300, 256, 64, 100), (300, 300, 1, 0, -50, 250, 256, 64, 400),
    ]
    inp = "\n".join(" ".join(map(str, c)) for c in cases) + "\n"
    out = subprocess.run([plan_check], input=inp, capture_output=True, text=True,
                         check=True).stdout.split("\n")
    pos = 0
    for (Sq, Sk, causal, window, ip, kl, tm, tn, prefix) in cases:
        _, nqt, nkt = out[pos].split()
        pos += 1
        plan = np.array([[int(ch) for ch in out[pos + r]] for r in range(int(nqt))],
                        dtype=np.int8).reshape(int(nqt), int(nkt))
        pos += int(nqt)
        case = (Sq, Sk, causal, window, ip, kl, tm, tn, prefix)
        mask = ora.flex_mask(Sq, Sk, bool(causal), window, ip, kl, prefix=prefix)
        if prefix == 0:
            want = ora.tile_plan_ref(Sq, Sk, bool(causal), window, ip, kl, tm, tn)
        else:
            want = _plan_from_mask(mask, Sq, Sk, tm, tn)
        np.testing.assert_array_equal(plan, want, err_msg=str(case))
        assert out[pos] == f"rows {Sq}"
        pos += 1
        rows = np.array([list(map(int, out[pos + i].split())) for i in range(Sq)])
        pos += Sq
        j = np.arange(Sk)[None, :]
        got = (j >= rows[:, :1]) & (j < rows[:, 1:])
        np.testing.assert_array_equal(got, mask, err_msg=str(case))
