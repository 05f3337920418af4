"""CPU checks of the Python binding's argument checks (no GPU needed).

The kernels address every tensor through a raw pointer and the sizes passed
with it, so the binding must refuse a tensor whose shape does not match those
sizes before it reaches the library.  The tensors here live on the CPU: a
shape error must come first (ValueError naming the shape); tensors of the
right shapes get as far as the device check ("must live on the GPU").
"""

import os
import subprocess
import sys

import pytest
import torch

import scaled_dot_product_attn_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

bf = torch.bfloat16
f32 = torch.float32
i32 = torch.int32


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


B, H, HKV, SQ, SK, D = 2, 8, 2, 16, 24, 64


def prefill(**over):
    t = dict(O=z(B, H, SQ, D), Q=z(B, H, SQ, D), K=z(B, HKV, SK, D), V=z(B, HKV, SK, D),
             LSE=z(B, H, SQ, dtype=f32), k_lengths=z(B, dtype=i32))
    t.update(over)
    return t


PREFILL_BAD = {
    "O": z(B, H, SQ + 1, D),
    "V": z(B, HKV, SK - 1, D),
    "K": z(B + 1, HKV, SK, D),
    "LSE": z(B, H, SQ + 1, dtype=f32),
    "k_lengths": z(B + 1, dtype=i32),
}


def _shape_error(fn):
    with pytest.raises(ValueError, match="shape|4-d|must be \\("):
        fn()


def _device_error(fn):
    with pytest.raises(ValueError, match="GPU"):
        fn()


@pytest.mark.parametrize("bad", list(PREFILL_BAD))
@pytest.mark.parametrize("entry", ["attn_fwd", "attn_fwd_flex", "attn_fwd_block_sparse"])
def test_prefill_shape_mismatch_refused(entry, bad):
    t = prefill(**{bad: PREFILL_BAD[bad]})
    keep = z(B, H, 1, 1, dtype=torch.uint8)
    if entry == "attn_fwd":
        fn = lambda: attn.attn_fwd(t["O"], t["Q"], t["K"], t["V"], t["LSE"], True,
                                   k_lengths=t["k_lengths"])
    elif entry == "attn_fwd_flex":
        fn = lambda: attn.attn_fwd_flex(t["O"], t["Q"], t["K"], t["V"], t["LSE"], True,
                                        k_lengths=t["k_lengths"])
    else:
        fn = lambda: attn.attn_fwd_block_sparse(t["O"], t["Q"], t["K"], t["V"], keep, t["LSE"],
                                                True, k_lengths=t["k_lengths"])
    _shape_error(fn)


def test_prefill_right_shapes_reach_the_device_check():
    t = prefill()
    _device_error(lambda: attn.attn_fwd(t["O"], t["Q"], t["K"], t["V"], t["LSE"], True,
                                        k_lengths=t["k_lengths"]))
    f = {k: v.float() if v.dtype == bf else v for k, v in t.items()}
    _device_error(lambda: attn.attn_fwd_f32(f["O"], f["Q"], f["K"], f["V"], f["LSE"], True))


@pytest.mark.parametrize("mod,bad", [
    ("q_lengths", z(B + 1, dtype=i32)), ("alibi_slopes", z(H - 1, dtype=f32)),
    ("doc_q", z(B, SQ + 1, dtype=i32)), ("doc_kv", z(B, SK - 1, dtype=i32)),
    ("bias", z(1, 1, SQ, SK + 1, dtype=f32)), ("bias", z(3, 1, SQ, SK, dtype=f32)),
    ("bias", z(1, 3, SQ, SK, dtype=f32))])
def test_flex_mod_shape_mismatch_refused(mod, bad):
    t = prefill()
    kw = {mod: bad}
    if mod == "doc_q":
        kw["doc_kv"] = z(B, SK, dtype=i32)
    if mod == "doc_kv":
        kw["doc_q"] = z(B, SQ, dtype=i32)
    with pytest.raises(ValueError, match="shape|bias must be"):
        attn.attn_fwd_flex(t["O"], t["Q"], t["K"], t["V"], t["LSE"], True, **kw)


@pytest.mark.parametrize("bad", ["dQ", "dK", "dV", "dO", "O", "LSE"])
def test_bwd_shape_mismatch_refused(bad):
    t = prefill()
    g = dict(dQ=z(B, H, SQ, D), dK=z(B, HKV, SK, D), dV=z(B, HKV, SK, D), dO=z(B, H, SQ, D),
             O=t["O"], LSE=t["LSE"])
    wrong = {"dQ": z(B, H, SQ, D + 1), "dK": z(B, HKV, SK + 1, D), "dV": z(B, 1, SK, D),
             "dO": z(B, H, SQ - 1, D), "O": z(B, H + 1, SQ, D), "LSE": z(B, H, 1, dtype=f32)}
    g[bad] = wrong[bad]
    _shape_error(lambda: attn.attn_bwd(g["dQ"], g["dK"], g["dV"], g["dO"], t["Q"], t["K"],
                                       t["V"], g["O"], g["LSE"], True))
    with pytest.raises(ValueError, match="LSE"):
        attn.attn_bwd(z(B, H, SQ, D), z(B, HKV, SK, D), z(B, HKV, SK, D), z(B, H, SQ, D),
                      t["Q"], t["K"], t["V"], t["O"], None, True)


def decode_args(**over):
    t = dict(O=z(B, H, D), Q=z(B, H, D), K=z(B, HKV, 100, D), V=z(B, HKV, 100, D),
             lengths=z(B, dtype=i32))
    t.update(over)
    return t


@pytest.mark.parametrize("entry", ["attn_decode", "attn_decode_ws", "attn_decode_static"])
@pytest.mark.parametrize("bad,val", [("O", z(B, H + 1, D)), ("V", z(B, HKV, 99, D)),
                                     ("K", z(B, HKV, 100, D + 1)),
                                     ("lengths", z(B + 3, dtype=i32))])
def test_decode_shape_mismatch_refused(entry, bad, val):
    t = decode_args(**{bad: val})
    args = (t["O"], t["Q"], t["K"], t["V"], t["lengths"], 8)
    if entry == "attn_decode_ws":
        fn = lambda: attn.attn_decode_ws(*args, z(4096, dtype=torch.uint8))
    else:
        fn = lambda: getattr(attn, entry)(*args)
    _shape_error(fn)


def test_decode_right_shapes_reach_the_device_check():
    t = decode_args()
    _device_error(lambda: attn.attn_decode(t["O"], t["Q"], t["K"], t["V"], t["lengths"], 8))


@pytest.mark.parametrize("bad,val", [("O", z(B, H, D + 2)), ("lengths", z(B - 1, dtype=i32))])
def test_paged_decode_shape_mismatch_refused(bad, val):
    t = dict(O=z(B, H, D), Q=z(B, H, D), K=z(10, 16, HKV, D), V=z(10, 16, HKV, D),
             T=z(B, 4, dtype=i32), L=z(B, dtype=i32))
    t[bad if bad != "lengths" else "L"] = val
    _shape_error(lambda: attn.attn_decode_paged(t["O"], t["Q"], t["K"], t["V"], t["T"], t["L"]))


def test_block_scores_and_debug_exports_shape_mismatch_refused():
    q, k = z(B, H, 130, D), z(B, HKV, 200, D)
    _shape_error(lambda: attn.attn_block_scores(z(B, H, 3, 3, dtype=f32), None, q, k))
    _shape_error(lambda: attn.attn_block_scores(z(B, H, 3, 4, dtype=f32),
                                                z(B, H, 2, 4, dtype=f32), q, k))
    _shape_error(lambda: attn.attn_mask_dump(z(10, 11, dtype=torch.uint8), 10, 12))
    _shape_error(lambda: attn.attn_tile_plan(z(1, 2, dtype=torch.int8), 300, 100))


def test_fwd_is_the_allocating_forward():
    assert attn.sdpa is attn.fwd
    _device_error(lambda: attn.fwd(z(B, H, SQ, D), z(B, HKV, SK, D), z(B, HKV, SK, D), True))


def _run_logged(env_value):
    code = ("import scaled_dot_product_attn_amd as a; l = a.lib(); "
            "print(l.attn_fwd(1, 1, 1, 1, None, 1, 3, 2, 8, 8, 128, 1, 0, 0, None, None))")
    env = dict(os.environ)
    env.pop("ATTN_LOG", None)
    if env_value is not None:
        env["ATTN_LOG"] = env_value
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_launch_log_only_when_asked():
    on = _run_logged("1")
    assert on.returncode == 0 and on.stdout.strip() == str(attn.ATTN_EINVAL)
    assert "[attn] attn_fwd B=1 H=3 Hkv=2 Sq=8 Sk=8 D=128" in on.stderr
    assert "-> invalid argument" in on.stderr
    for value in (None, "0"):
        off = _run_logged(value)
        assert off.returncode == 0 and "[attn]" not in off.stderr


@pytest.mark.parametrize("group,tp", [(1, 256), (2, 128), (3, 256), (4, 64), (6, 128),
                                      (8, 32), (16, 32)])
def test_tile_positions_per_group(group, tp):
    # query positions per prefill workgroup: its 256 rows over the largest
    # power of two up to 8 dividing the group
    assert attn.fwd_tile_positions(group) == tp
