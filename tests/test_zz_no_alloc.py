"""GPU check of attn_decode_static, the decode entry point that allocates
nothing: its slice partials live in the library's static per-GPU scratch.

It must give exactly what attn_decode_ws (caller-owned workspace, same
kernels) gives, call after call: two calls in a row, the second with a smaller
input, and the oracle agrees with both to the bf16 bound.
"""

import sys

import numpy as np
import pytest
import torch

import scaled_dot_product_attn_amd as attn
from scaled_dot_product_attn_amd import workloads as wl
from oracle import attn_oracle as ora

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL_BF16 = 2e-2


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _one_call(B, H, Hkv, D, smin, smax, ns, seed):
    print(f"decode_static B={B} H={H} Hkv={Hkv} D={D} len=[{smin},{smax}] n_splits={ns}",
          flush=True)
    sys.stdout.flush()
    w = wl.decode_random(B, H, Hkv, D, smin, smax, ns, seed=seed)
    q, k, v, lens = (t.to(DEV) for t in (w.q, w.k, w.v, w.lengths))
    O_static = torch.empty_like(q)
    attn.attn_decode_static(O_static, q, k, v, lens, ns)
    ws = torch.empty(max(1, attn.attn_decode_workspace_bytes(B, H, ns, D)), dtype=torch.uint8,
                     device=DEV)
    O_ws = torch.empty_like(q)
    attn.attn_decode_ws(O_ws, q, k, v, lens, ns, ws)
    torch.cuda.synchronize()
    # the same kernels in the same order: identical bits
    assert torch.equal(O_static, O_ws)
    Or, _ = ora.decode_ref(_np(w.q), _np(w.k), _np(w.v), w.lengths.numpy())
    err = float(np.max(np.abs(_np(O_static) - Or)))
    assert err <= TOL_BF16, f"decode_static max-abs error {err}"
    return O_static


def test_decode_static_matches_workspace_entry_point_twice():
    # a larger call first, then a smaller one over the partials it left
    _one_call(24, 32, 8, 128, 512, 6000, 8, seed=41)
    _one_call(3, 8, 2, 64, 1, 300, 4, seed=42)


def test_decode_static_single_slice_and_size_limit():
    _one_call(2, 4, 4, 128, 1, 200, 1, seed=43)   # one slice: no scratch used
    # more partials than the static scratch holds: refused before any launch
    B, H, ns, D = 4096, 32, 8, 128
    assert attn.attn_decode_workspace_bytes(B, H, ns, D) > attn.DECODE_STATIC_SCRATCH_BYTES
    q = torch.zeros(B, H, D, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(B, 8, 1, D, dtype=torch.bfloat16, device=DEV)
    lens = torch.ones(B, dtype=torch.int32, device=DEV)
    with pytest.raises(RuntimeError, match="unsupported"):
        attn.attn_decode_static(torch.empty_like(q), q, kv, kv, lens, ns)
