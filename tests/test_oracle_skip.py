"""Pins for the oracle's carried skip mask over denoising steps (CPU only)."""
import numpy as np
import pytest

import oracle
import synth


def small_workload():
    # a few frames of a small video grid, ragged last blocks (N = 5*6*7 = 210)
    return synth.Workload("skip_small", 1, 2, 32, 5, 6, 7, 16, 16, "bf16", "skip",
                          77, True, tau=2.0, steps=4)


def test_infinite_threshold_never_marks_and_equals_dense(oracle_lib):
    w = small_workload()
    x = synth.make_qkv(w, step=0)
    skip = np.zeros((w.B, w.H, w.nQ, w.nK), np.uint8)
    o, lse, gap, new = oracle.skip_step(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, skip, np.inf)
    assert not new.any()
    ones = np.ones((w.nQ, w.nK), np.uint8)
    o2, lse2, _ = oracle.attention(x["q"], x["k"], x["v"], w.Bq, w.Bk, w.scale, ones, 0)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


@pytest.mark.parametrize("order", [oracle.ORDER_ASCENDING, oracle.ORDER_RADIAL])
def test_skip_set_grows_monotonically_and_rows_never_empty(oracle_lib, order):
    w = small_workload()
    v = synth.make_qkv(w, step=0, want=("v",))["v"]
    skip = np.zeros((w.B, w.H, w.nQ, w.nK), np.uint8)
    total = []
    for s in range(w.steps):
        qk = synth.make_step_qk(w, s)
        _, _, gap, new = oracle.skip_step(qk["q"], qk["k"], v, w.Bq, w.Bk, w.scale, skip, w.tau,
                                          order=order)
        assert np.all(new >= skip)                       # monotone OR
        assert np.all((1 - new).sum(axis=-1) >= 1)       # never an empty row
        # the first visited tile of each row has gap +inf and is never marked
        eff = (1 - skip).reshape(-1, w.nK)
        row_ptr = np.concatenate([[0], np.cumsum(eff.sum(axis=1))]).astype(np.int32)
        kv = np.concatenate([np.nonzero(e)[0] for e in eff]).astype(np.int32)
        first = oracle.order_lists(row_ptr, kv, w.N, w.Bq, w.Bk, order)[row_ptr[:-1]]
        assert np.all(gap[np.arange(gap.shape[0]), first] == np.inf)
        skip = new
        total.append(int(skip.sum()))
    assert total[-1] > 0


def _run_steps(w, v, skip, steps, order):
    """Advance the carried skip set over the given denoising steps; returns the
    final set and each step's (o, lse) as computed."""
    outs = []
    for s in steps:
        qk = synth.make_step_qk(w, s)
        o, lse, _, skip = oracle.skip_step(qk["q"], qk["k"], v, w.Bq, w.Bk, w.scale, skip, w.tau,
                                           order=order)
        outs.append((o, lse))
    return skip, outs


@pytest.mark.parametrize("order", [oracle.ORDER_ASCENDING, oracle.ORDER_RADIAL])
def test_skip_set_save_and_restore_resumes_exactly(oracle_lib, tmp_path, order):
    """LiteAttention summary page, section 六: the skip mask persists across
    denoising steps. The carried set is the whole state of the carry, so ten
    steps in one run equal five steps, the set written to disk and read back,
    then the other five: same sets, same outputs, bit for bit."""
    w = small_workload().with_(steps=10, tau=1.0)
    v = synth.make_qkv(w, step=0, want=("v",))["v"]
    zero = np.zeros((w.B, w.H, w.nQ, w.nK), np.uint8)
    full, outs_full = _run_steps(w, v, zero, range(10), order)
    half, outs_a = _run_steps(w, v, zero, range(5), order)
    path = tmp_path / "skip.npy"
    np.save(path, half)
    restored = np.load(path)                     # allow_pickle defaults to False
    assert restored.dtype == np.uint8 and np.array_equal(restored, half)
    resumed, outs_b = _run_steps(w, v, restored, range(5, 10), order)
    np.testing.assert_array_equal(resumed, full)
    for (o1, l1), (o2, l2) in zip(outs_full, outs_a + outs_b):
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)
    assert full.sum() > half.sum() > 0          # the set grew in both halves
