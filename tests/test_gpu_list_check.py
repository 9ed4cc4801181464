"""GPU side of the debug check of block lists, through the C ABI.

The device check must reach the same result (row and rule) as the host
check on the same lists, and with BSA_CHECK=1 the calls that consume lists
must refuse malformed ones before launching anything. Every list used here
stays inside its buffers (entries out of range point past the last key
block, never below the first), so no kernel reads outside its inputs even if
a check were to let a list through.
"""
import os

import numpy as np
import pytest
import torch

import block_sparse_attention_flashattention_amd as bsa
from _gpu_util import DEV, dev, note

pytestmark = pytest.mark.gpu


def _lists(rows):
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    kv = np.array([c for r in rows for c in r] or [0], dtype=np.int32)
    return rp, kv


def _check_result(s, rp, kv, shared, asc, on_device):
    try:
        if on_device:
            bsa.bsa_check_block_lists(s, shared, dev(rp), dev(kv), 0, asc, kv_len=int(rp[-1]))
        else:
            bsa.bsa_check_block_lists(s, shared, rp, kv, 0, asc, kv_len=int(rp[-1]))
        return ""
    except bsa.BsaError as e:
        return e.detail


def test_device_check_agrees_with_host_check():
    r = np.random.default_rng(9)
    s = bsa.shape(2, 3, 128, 5, 9, 13, 64)           # nQ = nK = 10, ragged last block
    R, nK = 2 * 3 * s.nQ, s.nK
    n_bad = 0
    for trial in range(60):
        rows = [sorted(r.choice(nK, size=r.integers(0, nK + 1), replace=False).tolist())
                for _ in range(R)]
        kind = trial % 4
        if kind == 1:
            rows[r.integers(R)] += [nK + int(r.integers(0, 3))]      # past the last block
        elif kind == 2:
            row = rows[r.integers(R)]
            if row:
                row.append(row[0])                                  # a repeat
        elif kind == 3:
            row = rows[r.integers(R)]
            r.shuffle(row)                                          # order only
        rp, kv = _lists(rows)
        for asc in (False, True):
            host_v = _check_result(s, rp, kv, 0, asc, False)
            dev_v = _check_result(s, rp, kv, 0, asc, True)
            assert host_v == dev_v, (trial, asc, host_v, dev_v)
            n_bad += bool(host_v)
    note(f"device and host checks agree on 120 list sets ({n_bad} malformed)")
    assert n_bad > 20


def test_bsa_check_env_refuses_malformed_lists():
    s = bsa.shape(1, 2, 128, 3, 9, 13, 128)          # N = 351: nQ = 3, nK = 6
    g = torch.Generator().manual_seed(3)
    q, k, v = (torch.randn(1, s.N, 2, 128, generator=g).to(torch.bfloat16).to(DEV)
               for _ in range(3))
    rows_ok = [[0, 1, 2], [1, 2, 3, 4], [3, 4, 5]]
    rows_bad = [[0, 1, 2], [1, 2, 6], [3, 4, 5]]       # block 6 does not exist
    old = os.environ.get("BSA_CHECK")
    os.environ["BSA_CHECK"] = "1"
    try:
        rp, kv = (dev(a) for a in _lists(rows_ok))
        o = torch.zeros_like(q)
        bsa.bsa_sparse_attn_fwd(s, q, k, v, o, None, rp, kv, 1)
        torch.cuda.synchronize()
        assert o.abs().sum().item() > 0
        rp, kv = (dev(a) for a in _lists(rows_bad))
        o = torch.zeros_like(q)
        with pytest.raises(bsa.BsaError) as e:
            bsa.bsa_sparse_attn_fwd(s, q, k, v, o, None, rp, kv, 1)
        assert e.value.status == 1 and "row 1: rule 4" in e.value.detail
        torch.cuda.synchronize()
        assert o.abs().sum().item() == 0                 # nothing was launched
        # the visiting-order call needs ascending input
        rp, kv = (dev(a) for a in _lists([[0, 2, 1], [1, 2], [3]]))
        out = torch.empty_like(kv)
        with pytest.raises(bsa.BsaError) as e:
            bsa.bsa_order_block_lists(s, bsa.ORDER_RADIAL, rp, 1, kv, out)
        assert "row 0: rule 6" in e.value.detail
    finally:
        if old is None:
            del os.environ["BSA_CHECK"]
        else:
            os.environ["BSA_CHECK"] = old
