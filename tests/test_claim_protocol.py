"""CPU model of the claiming protocol of the one-matrix kernels
(weight_only_quantized_wq_amd/csrc/wq_claim.hpp, used by
gemm_verify_matrix_kernel and gemm_i8_matrix_kernel).

The model follows the device rules step by step, with random wave speeds
and with device atomics that land after a random delay, so that two claims
in flight can land swapped:
  * units are claimed in order from a workgroup counter; the waves whose
    static first unit exists start without a claim, and every wave claims
    (and resolves) its next unit before it finishes the current one;
  * a workgroup's local blocks 0 and 1 are blockIdx.x and blockIdx.x + G;
    halfway through local block j >= 1 (unit ups // 2) local block j + 1 is
    claimed from the launch counter (2 G + n), but only once block j's own
    number is known; a block past the matrix hands the same mark on;
  * a unit of local block j writes slot j % R once block j - R has been
    added up; the block's last unit adds it up and frees the slot.
It checks that every (block, unit) is processed exactly once, that no slot
is overwritten before it is added up, and that no schedule deadlocks.  With
the claim made before the block's own number is known (the first version),
the model strands blocks, as the GPU did.
"""
import random

import pytest


def run_model(nb, grid, ups, ordered=True, waves=8, ring=2, lmax=64, seed=0, max_steps=3_000_000):
    rnd = random.Random(seed)
    per = -(-nb // grid)
    cap = min(2 * per + 2, lmax)
    counter = [0]
    processed, stored = {}, {}
    wgs = []
    for w in range(grid):
        first = min(ups, waves)
        wg = {"gblk": [-1] * lmax, "uctr": first, "cnt": [0] * ring, "freed": [r - ring for r in range(ring)],
              "part": [[None] * ups for _ in range(ring)], "pending": []}
        wg["gblk"][0] = w
        wg["gblk"][1] = w + grid
        wg["waves"] = [{"cur": (0, v, w) if v < first else None, "state": "init"} for v in range(waves)]
        wgs.append(wg)

    def land_atomics(wg):
        for a in list(wg["pending"]):
            a[0] -= 1
            if a[0] <= 0:
                wg["gblk"][a[1]] = 2 * grid + counter[0]
                counter[0] += 1
                wg["pending"].remove(a)

    active = [(wg, wv) for wg in wgs for wv in wg["waves"]]
    steps = 0
    while active:
        steps += 1
        if steps > max_steps:
            raise RuntimeError("deadlock")
        k = rnd.randrange(len(active))
        wg, wv = active[k]
        land_atomics(wg)
        st = wv["state"]
        if st == "exit":
            active[k] = active[-1]
            active.pop()
            continue
        if st in ("init", "claimnext"):
            if st == "init" and wv["cur"] is not None:
                wv["state"] = "claimnext"
                continue
            i = wg["uctr"]
            wg["uctr"] += 1
            jl, u = divmod(i, ups)
            wv["first_claim"] = st == "init"
            if jl >= cap:
                wv["pend"] = None
                wv["state"] = "resolved"
                continue
            wv["pend"] = (jl, u)
            if not ordered and jl >= 1 and u == ups // 2 and jl + 1 < cap:
                wg["pending"].append([rnd.randint(0, 20), jl + 1])
            wv["state"] = "waitblk"
        elif st == "waitblk":
            jl, u = wv["pend"]
            gb = wg["gblk"][jl]
            if gb < 0:
                continue
            if ordered and jl >= 1 and u == ups // 2 and jl + 1 < cap:
                if gb < nb:
                    wg["pending"].append([rnd.randint(0, 20), jl + 1])
                else:
                    wg["gblk"][jl + 1] = nb
            wv["pend"] = (jl, u, gb) if gb < nb else None
            wv["state"] = "resolved"
        elif st == "resolved":
            c = wv["pend"]
            if wv["first_claim"]:
                if c is None:
                    wv["state"] = "exit"
                else:
                    wv["cur"] = c
                    wv["state"] = "claimnext"
                continue
            wv["nxt"] = c
            wv["state"] = "work"
            wv["timer"] = rnd.randint(1, 6) * (4 if rnd.random() < 0.1 else 1)
        elif st == "work":
            wv["timer"] -= 1
            if wv["timer"] <= 0:
                wv["state"] = "waitslot"
        elif st == "waitslot":
            jl, u, gb = wv["cur"]
            sl = jl % ring
            if wg["freed"][sl] != jl - ring:
                continue
            assert wg["part"][sl][u] is None, "slot overwritten before it was added up"
            wg["part"][sl][u] = gb
            processed[(gb, u)] = processed.get((gb, u), 0) + 1
            done = wg["cnt"][sl]
            wg["cnt"][sl] += 1
            if done == ups - 1:
                assert all(p == gb for p in wg["part"][sl]), "units of two blocks in one slot"
                stored[gb] = stored.get(gb, 0) + 1
                wg["part"][sl] = [None] * ups
                wg["cnt"][sl] = 0
                wg["freed"][sl] = jl
            if wv["nxt"] is None:
                wv["state"] = "exit"
            else:
                wv["cur"], wv["nxt"] = wv["nxt"], None
                wv["state"] = "claimnext"
    missing = sorted(set(range(nb)) - set(stored))
    return missing, stored, processed


# (blocks, workgroups, units per block): one block per workgroup, a few
# more blocks than workgroups, many more; one unit per block up to 16
CASES = [(448, 64, 8), (1002, 64, 8), (64, 64, 8), (80, 64, 8), (5, 5, 8), (1, 1, 1), (37, 37, 3),
         (250, 64, 16), (250, 64, 4), (150, 64, 1), (400, 64, 1), (2, 2, 16), (75, 64, 5), (100, 16, 7)]


@pytest.mark.parametrize("nb,grid,ups", CASES)
def test_claim_protocol_covers_every_unit_once(nb, grid, ups):
    for seed in range(4):
        missing, stored, processed = run_model(nb, grid, ups, seed=seed)
        assert not missing, (seed, missing[:5])
        assert all(c == 1 for c in stored.values())
        assert all(processed.get((b, u)) == 1 for b in range(nb) for u in range(ups))


def test_unordered_claims_strand_blocks():
    """The first version claimed the next block without waiting for the
    current one's number: claims that land swapped then strand a block or
    leave a wave waiting for a slot no one frees (the spin bound ends it)."""
    bad = 0
    for seed in range(16):
        try:
            missing, _, _ = run_model(150, 64, 1, ordered=False, seed=seed, max_steps=300_000)
            bad += bool(missing)
        except RuntimeError:
            bad += 1
    assert bad > 0
