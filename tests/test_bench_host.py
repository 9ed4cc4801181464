"""Host logic of bench.py that needs no GPU: the CPU baseline's row sample,
the counter-record keys and the trace summary's split of dispatches."""
import argparse
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
import synth  # noqa: E402


def test_stratified_rows_cover_every_stratum():
    """720p: 40 heads x 591 row blocks (ragged last), frames of 3,600 tokens."""
    BH, nQ, N, bq, F = 40, 591, 75600, 128, 3600
    rows = bench.stratified_rows(BH, nQ, 20, N, bq, F, np.random.default_rng(1))
    heads, a = rows // nQ, rows % nQ
    assert len(np.unique(rows)) == len(rows)
    straddle = {x for x in range(nQ) if (x * bq) // F != (min(N, (x + 1) * bq) - 1) // F}
    for h in range(BH):
        mine = set(a[heads == h].tolist())
        assert len(mine) == 20 and 0 in mine and nQ - 1 in mine
        assert len(mine & straddle) >= 5
    assert np.all(np.diff(rows) > 0)


def test_stratified_rows_small_heads_take_everything():
    rows = bench.stratified_rows(2, 3, 20, 300, 128, 100, np.random.default_rng(0))
    assert rows.tolist() == [0, 1, 2, 3, 4, 5]


def test_counter_record_keys_name_what_changes_the_lists():
    ns = argparse.Namespace(tau_schedule=None, order="radial", share_after=None,
                            pooled_mode=3, pooled_param=0.5, token_order="choose",
                            pyramid=None)
    assert bench.variant_key(ns, synth.workload("wan13b_480p")) == \
        "wan13b_480p:mode=3:param=0.5:order=choose"
    ns = argparse.Namespace(tau_schedule=None, order="radial", share_after=None,
                            pooled_mode=None, pooled_param=None, token_order=None, pyramid=None)
    assert bench.variant_key(ns, synth.workload("skip_carry_480p")) == \
        "skip_carry_480p:tau=10.0:order=radial"
    assert bench.variant_key(ns, synth.workload("wan14b_720p")) == "wan14b_720p"


def test_pyramid_flops_count_the_keys_of_each_level():
    """The forward's flop count of pyramid lists equals 4 d |R_a| times the
    pooled keys that the level mask gives each row (a level-l block of len
    tokens holds len / 2^l of them), at 1 to 4 levels and a ragged last block."""
    import oracle
    B, H, N, bq, bk, d = 1, 2, 296, 64, 64, 128
    nQ, nK = -(-N // bq), -(-N // bk)
    rng = np.random.default_rng(5)
    for L in (1, 2, 3, 4):
        mask = rng.integers(0, L + 1, size=(B, H, nQ, nK)).astype(np.uint8)
        rp, kv, qm = oracle.compact_pyramid(mask, B, H, nQ, nK, N, bk, L, nQ * nK)
        rb, _ = oracle.pyramid_regions(N, bk, L)
        got = bench.pyramid_flops(rp, kv, qm, N, bq, bk, d, nQ, rb)
        want = 0
        for h in range(H):
            for a in range(nQ):
                ra = min(N, (a + 1) * bq) - a * bq
                for c in range(nK):
                    m = int(mask[0, h, a, c])
                    if m:
                        want += 4 * d * ra * ((min(N, (c + 1) * bk) - c * bk) >> (m - 1))
        assert got == want, (L, got, want)
