"""The allocation-free top-k entry point (logits_argmax_topk_noalloc) against the workspace one.

Both entry points are called through the C ABI on the same logits.  The allocation-free one
keeps its candidates in the library's per-device array, which holds whatever the previous call
left, so it is called twice in a row, the second time on a smaller input, and each result must
equal logits_argmax_topk's bit for bit (indices and values).  A request past the array's size is
rejected on the host, before anything is launched.
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

W4_ERR_WORKSPACE = -4


@pytest.fixture(scope="module")
def w4():
    import int4_weight_only_group_amd as w4
    return w4


def _logits(m, v, seed):
    import torch
    rng = synth.rng(seed, synth.W_TEST, 77, synth.T_X)
    host = (rng.standard_normal((m, v), dtype=np.float32) * np.float32(0.9)).astype(np.float32)
    return torch.from_numpy(host).to("cuda")


def _both(w4, logits, k):
    import torch
    m = logits.shape[0]
    ws = torch.empty(max(16, w4.topk_workspace_bytes(m, logits.shape[1], k)), dtype=torch.uint8, device="cuda")
    i_ref, v_ref = w4.logits_argmax_topk(logits, k, workspace=ws)
    idx = torch.full((m, k), -1, dtype=torch.int32, device="cuda")
    val = torch.full((m, k), float("nan"), dtype=torch.float32, device="cuda")
    w4.logits_argmax_topk_noalloc(logits, k, idx=idx, val=val)
    torch.cuda.synchronize()
    return (i_ref.cpu().numpy(), v_ref.cpu().numpy()), (idx.cpu().numpy(), val.cpu().numpy())


@pytest.mark.parametrize("first,second", [
    ((8, 262144, 64, 1), (1, 151936, 40, 2)),   # Gemma-shaped head rows, then the Qwen2.5-3B head
    ((4, 151936, 40, 3), (2, 70001, 17, 4)),    # then a ragged, shorter row with fewer keys
    ((3, 4096, 64, 5), (1, 1000, 5, 6)),         # rows short enough to take one pass only
])
def test_noalloc_matches_workspace_entry_point_twice(w4, first, second):
    for m, v, k, seed in (first, second):
        logits = _logits(m, v, seed)
        (i_ref, v_ref), (i_na, v_na) = _both(w4, logits, k)
        assert np.array_equal(i_na, i_ref), (m, v, k)
        assert np.array_equal(v_na.view(np.uint32), v_ref.view(np.uint32)), (m, v, k)


def test_noalloc_rejects_requests_past_its_array(w4):
    import torch
    lib = w4.lib()
    # 129 rows of top-64 over 262144 logits need 129 * 64 * 64 * 8 bytes > 4 MiB
    m, v, k = 129, 262144, 64
    need = w4.topk_workspace_bytes(m, v, k)
    assert need > 4 << 20
    logits = torch.empty((1, 16), dtype=torch.float32, device="cuda")  # never read: rejected first
    idx = torch.empty((1, 16), dtype=torch.int32, device="cuda")
    st = lib.logits_argmax_topk_noalloc(logits.data_ptr(), v, m, v, k, idx.data_ptr(), idx.data_ptr(),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == W4_ERR_WORKSPACE
    # 128 such rows fit exactly
    assert w4.topk_workspace_bytes(128, v, k) == 4 << 20
