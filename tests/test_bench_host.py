"""CPU checks of bench.py's work accounting against the oracle's mask."""

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import attn_oracle as ora  # noqa: E402


@pytest.mark.parametrize("Sq,Sk,causal,window,ip,kl", [
    (300, 300, True, 0, 0, 300), (128, 1000, True, 100, 872, 1000), (64, 64, False, 0, 0, 40),
    (90, 200, True, 7, -30, 150), (50, 50, True, 0, 60, 50),
])
def test_allowed_pairs_matches_oracle_mask(Sq, Sk, causal, window, ip, kl):
    assert bench.allowed_pairs(Sq, Sk, causal, window, ip, kl) == \
        ora.allowed_pairs(Sq, Sk, causal, window, ip, kl)


def test_workload_flops_closed_forms():
    # causal square: S(S+1)/2 pairs per head; window: Sq*W; full: Sq*Sk.
    assert bench.allowed_pairs(4096, 4096, True, 0, 0, 4096) * 64 * 512 == 274945015808
    assert bench.allowed_pairs(2048, 16384, True, 4096, 14336, 16384) * 32 * 512 == 137438953472
    assert bench.allowed_pairs(4096, 4096, False, 0, 0, 4096) * 32 * 512 == 274877906944


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_timing_stats_median_and_min():
    assert bench.timing_stats([3.0, 1.0, 2.0]) == {"mean": 2.0, "median": 2.0, "min": 1.0}
    assert bench.timing_stats([4.0, 1.0, 2.0, 3.0]) == {"mean": 2.5, "median": 2.5, "min": 1.0}


def test_document_flops_matches_oracle_mask():
    import torch
    from scaled_dot_product_attn_amd import workloads as wl
    doc = wl.document_ids(2, 300, 5, seed=3)
    pairs = sum(int(ora.flex_mask(300, 300, True, doc_q=doc[b].numpy(),
                                  doc_kv=doc[b].numpy()).sum()) for b in range(2))
    assert bench.document_flops(doc, 3, 64) == 4 * 64 * 3 * pairs
    # one document is plain causal attention
    one = torch.zeros(1, 100, dtype=torch.int32)
    assert bench.document_flops(one, 1, 1) == 4 * 100 * 101 // 2


def test_document_ids_recipe():
    from scaled_dot_product_attn_amd import workloads as wl
    doc = wl.document_ids(2, 4096, 16, seed=9)
    for row in doc.tolist():
        assert row[0] == 0 and row[-1] == 15
        assert all(b - a in (0, 1) for a, b in zip(row, row[1:]))


def test_timing_event_flag_is_the_device_scope_release():
    # the bench's timing events are recorded with a device-scope release; the
    # flag's value must be the runtime header's hipEventReleaseToDevice
    import re
    hdr = "/opt/rocm/include/hip/hip_runtime_api.h"
    if not os.path.exists(hdr):
        pytest.skip("no HIP headers")
    m = re.search(r"#define\s+hipEventReleaseToDevice\s+(0x[0-9a-fA-F]+)", open(hdr).read())
    assert m and int(m.group(1), 16) == bench.DeviceEvent.RELEASE_TO_DEVICE
