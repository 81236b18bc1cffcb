"""The panel schedule of the blocked Cholesky steps, as a model of its rules.

The potrf steps of the damped inverse (the K-FAC page's Cholesky-based
inverse paragraph) apply each finished panel p to the rows below it in one
of three ways: a trailing update that covers every row below step k (run
only every second or third step where the trailing matrix is large, several
panels at once), the row workgroups of step k applying the panels their row
still lacks, and, in a step without a trailing update, workgroups that bring
row k + 1 up to date.  This model follows the rules the host applies in
`kfac_damped_inverse` (thresholds of 1024 and 8192 trailing blocks: two- and
three-panel updates where V is formed beside potrf, four and eight panels
otherwise, where the next row is brought up to date each step) and checks the
invariant the kernels rely on: when row k is factored it has received every
panel p < k exactly once, and the row workgroups never apply more than three.
"""
import random

import pytest

PASS2_TILES, PASS3_TILES, MAX_DEPTH = 1024, 8192, 3
DEEP_PASS2, DEEP_PASS3 = 4, 8   # update depths where the next row is brought up to date by the step before


def syrk_tiles(nb, k):
    t = nb - k - 1
    return t * (t + 1) // 2 if k >= 1 and t > 0 else 0


def schedule_violation(nbs, fused):
    nbmax = max(nbs)
    applied = [[[] for _ in range(nb)] for nb in nbs]
    last_pass, next_done = 0, False
    for k in range(nbmax):
        plo = last_pass
        rplo = k - 1 if next_done else last_pass
        if k - rplo > MAX_DEPTH:
            return f"step {k}: row applies {k - rplo} panels"
        for m, nb in enumerate(nbs):
            if k < nb:
                applied[m][k] += list(range(rplo, k))
                if sorted(applied[m][k]) != list(range(k)):
                    return f"row {k} of matrix {m} (nb {nb}) holds panels {sorted(applied[m][k])}"
        trail = sum(syrk_tiles(nb, k) for nb in nbs)
        if fused:
            depth = 3 if trail >= PASS3_TILES else 2 if trail >= PASS2_TILES else 1
        else:
            depth = DEEP_PASS3 if trail >= PASS3_TILES else DEEP_PASS2 if trail >= PASS2_TILES else 1
        if k - last_pass >= depth or trail == 0:
            last_pass = k
        else:
            trail = 0
        next_done = (not fused) and trail == 0 and k > plo and k + 1 < nbmax
        if trail > 0:
            for m, nb in enumerate(nbs):
                for i in range(k + 1, nb):
                    applied[m][i] += list(range(plo, k))
        if next_done:
            for m, nb in enumerate(nbs):
                if k + 1 < nb:
                    applied[m][k + 1] += list(range(plo, k))
    return None


WORKLOADS = {
    "stress16": [72] * 8 + [36] * 8 + [64] * 5 + [32] * 5 + [8] * 6,
    "encoder12": [64] * 24 + [48] * 12 + [16] * 60,
    "mlp4": [16, 32, 32, 16, 32, 32, 16, 1],
}


@pytest.mark.parametrize("name", sorted(WORKLOADS))
@pytest.mark.parametrize("fused", [False, True])
def test_schedule_workloads(name, fused):
    assert schedule_violation(WORKLOADS[name], fused) is None


def test_schedule_random_batches():
    rng = random.Random(7)
    for _ in range(300):
        nbs = [rng.randint(1, 80) for _ in range(rng.randint(1, 12))]
        for fused in (False, True):
            assert schedule_violation(nbs, fused) is None, nbs


def test_schedule_model_catches_a_skipped_panel():
    """The checker itself: a schedule whose next-row update starts one panel
    late leaves a panel out, and the check says so."""
    def broken(nbs):
        nbmax = max(nbs)
        applied = [[[] for _ in range(nb)] for nb in nbs]
        last_pass, next_done = 0, False
        for k in range(nbmax):
            plo = last_pass
            rplo = k - 1 if next_done else last_pass
            for m, nb in enumerate(nbs):
                if k < nb:
                    applied[m][k] += list(range(rplo, k))
                    if sorted(applied[m][k]) != list(range(k)):
                        return "missing"
            trail = sum(syrk_tiles(nb, k) for nb in nbs)
            depth = 3 if trail >= PASS3_TILES else 2 if trail >= PASS2_TILES else 1
            if k - last_pass >= depth or trail == 0:
                last_pass = k
            else:
                trail = 0
            next_done = trail == 0 and k > plo and k + 1 < nbmax
            if trail > 0:
                for m, nb in enumerate(nbs):
                    for i in range(k + 1, nb):
                        applied[m][i] += list(range(plo, k))
            if next_done:
                for m, nb in enumerate(nbs):
                    if k + 1 < nb:
                        applied[m][k + 1] += list(range(plo + 1, k))   # the mistake
        return None
    assert broken(WORKLOADS["stress16"]) == "missing"
