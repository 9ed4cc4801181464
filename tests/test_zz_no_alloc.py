"""The pooled mask builder without a workspace (static scratch), through the
C ABI, against the workspace form on the same inputs: masks bit for bit, on
two calls in a row, the second on a smaller input than the first, so that
the second runs on scratch the first left behind."""
import numpy as np
import pytest
import torch

import block_sparse_attention_flashattention_amd as bsa
import synth
from _gpu_util import DEV, dev, note, shape_of

pytestmark = pytest.mark.gpu


def _both(w, x, mode, param):
    s = shape_of(w)
    q, k = dev(x["q"]), dev(x["k"])
    n = w.B * w.H * w.nQ * w.nK
    ws = torch.empty(bsa.bsa_pooled_workspace_bytes(s), dtype=torch.uint8, device=DEV)
    m_ws = torch.full((n,), 7, dtype=torch.uint8, device=DEV)
    bsa.bsa_build_mask_pooled(s, q, k, w.scale, mode, param, m_ws, ws)
    del ws
    m_na = torch.full((n,), 9, dtype=torch.uint8, device=DEV)
    bsa.bsa_build_mask_pooled_noalloc(s, q, k, w.scale, mode, param, m_na)
    torch.cuda.synchronize()
    return m_ws.cpu().numpy(), m_na.cpu().numpy()


def test_pooled_noalloc_matches_workspace_form_twice():
    big = synth.workload("wan13b_480p")                       # 37.7 MB of scratch
    small = synth.Workload("pooled_small", 2, 3, 128, 5, 12, 17, 64, 64, "bf16", "pooled", 610,
                           True)
    cases = [(big, 1, big.pooled_param), (small, 3, 0.5), (small, 0, 4.0)]
    for w, mode, param in cases:
        note(f"no-alloc pooled: {w.name} mode {mode} param {param}")
        x = synth.make_qkv(w)
        a, b = _both(w, x, mode, param)
        assert set(np.unique(a)) <= {0, 1}
        np.testing.assert_array_equal(b, a)
        note(f"  {int(a.sum())} of {a.size} tiles kept, identical")
