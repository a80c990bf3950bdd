"""Grouping cadence over a denoising trajectory (host-only C-ABI calls and the
PermutationCache helper; no GPU).

The pages state the cadence: grouping only during the first quarter of the
denoising steps, each permutation reused across four adjacent steps (paper
digest, clustering-rationale paragraph and limitations; news article,
"V-Smooth"; insight article, "Value Is the Error Source Earlier Methods
Underestimated").  The reading pinned here: step s regroups when
s < 0.25 * T and s % 4 == 0; every later step keeps the latest permutation.
"""
import pytest

import bit_attention_video_vc_amd as vc
from bit_attention_video_vc_amd import binding as bd


def _due_steps(T, reuse=4, fraction=0.25):
    return [s for s in range(T) if vc.group_due(s, T, reuse, fraction)]


def test_pages_cadence_on_common_trajectories():
    # first quarter of 40 steps is steps 0..9; of 50 steps 0..12 (12 < 12.5)
    assert _due_steps(40) == [0, 4, 8]
    assert _due_steps(50) == [0, 4, 8, 12]
    assert _due_steps(4) == [0]
    assert _due_steps(1) == [0]
    assert vc.group_count(40) == 3 and vc.group_count(50) == 4


@pytest.mark.parametrize("T,reuse,frac", [(40, 4, 0.25), (50, 4, 0.25), (7, 2, 0.5), (30, 1, 0.25),
                                          (9, 4, 1.0), (13, 3, 0.3)])
def test_cadence_invariants(T, reuse, frac):
    due = _due_steps(T, reuse, frac)
    assert due[0] == 0
    assert len(due) == vc.group_count(T, reuse, frac)
    for s in range(T):
        src = vc.group_source(s, T, reuse, frac)
        assert src in due and src <= s
        # the latest regrouping step at or before s
        assert src == max(d for d in due if d <= s)
        if s < frac * T:
            assert s - src < reuse
    # every regrouping step lies in the window, spaced by `reuse`
    assert all(d < frac * T for d in due)
    assert all(b - a == reuse for a, b in zip(due, due[1:]))


def test_fraction_one_reuse_one_regroups_every_step():
    assert _due_steps(6, 1, 1.0) == list(range(6))


@pytest.mark.parametrize("args", [(0, 0, 4, 0.25), (-1, 10, 4, 0.25), (10, 10, 4, 0.25), (0, 10, 0, 0.25),
                                  (0, 10, 4, 0.0), (0, 10, 4, 1.5), (0, 10, 4, float("nan"))])
def test_invalid_arguments(args):
    L = vc.lib()
    assert L.vc_group_due(*args) == -1
    assert L.vc_group_source(*args) == -1


def test_amortized_share_from_the_pages_overhead():
    # with the pages' +30% per grouping step, the cadence spreads it to
    # 0.30 * count / T of the trajectory's attention time
    for T in (40, 50):
        share = 0.30 * vc.group_count(T) / T
        assert 0.015 < share < 0.03


def test_permutation_cache_regroups_on_cadence_only():
    calls = []

    def fake_group(V, k, iters):
        calls.append((V, k, iters))
        return (("perm", V), None, None)

    T = 40
    cache = vc.PermutationCache(T, k=8, iters=3, group_fn=fake_group)
    got = {}
    for s in range(T):
        for layer in ("L0", "L1"):
            got[(layer, s)] = cache.perm(layer, s, (layer, s))
    assert cache.group_calls == 2 * 3
    assert [c[0] for c in calls] == [(l, s) for s in (0, 4, 8) for l in ("L0", "L1")]
    assert all(c[1:] == (8, 3) for c in calls)
    for s in range(T):
        src = vc.group_source(s, T)
        assert got[("L1", s)] == ("perm", ("L1", src))


def test_permutation_cache_rejects_a_missing_source():
    cache = vc.PermutationCache(40, group_fn=lambda V, k, it: (V, None, None))
    with pytest.raises(bd.VcError):
        cache.perm("L0", 5, "v")          # step 5 needs step 4's permutation, never computed
    cache.perm("L0", 0, "v0")
    with pytest.raises(bd.VcError):
        cache.perm("L0", 6, "v6")         # still only step 0's permutation
