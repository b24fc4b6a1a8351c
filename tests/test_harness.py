"""CPU tests of the invariance harness, with negative controls: mock backends that
are not batch-invariant in the ways the M-0002 record ("How it works") names --
a reduction split chosen from the batch size, dependence on batch position, run-to-run
nondeterminism -- must each be reported, with the first differing (request, row,
element); an invariant mock must come out clean."""
import numpy as np
import pytest

from invariant_deterministic_amd import harness

P, K, N = 24, 512, 16


@pytest.fixture(scope="module")
def data():
    rng = np.random.default_rng(7)
    A = rng.standard_normal((P, 2, K)).astype(np.float32)  # each request: 2 rows (tokens)
    W = rng.standard_normal((N, K)).astype(np.float32)
    return A, W


def matmul_split(rows, W, splits):
    """fp32 row products with K cut into `splits` contiguous parts summed in order."""
    parts = np.array_split(np.arange(K), splits)
    out = np.zeros((rows.shape[0], W.shape[0]), np.float32)
    for p in parts:
        out = (out + (rows[:, p] @ W[:, p].T).astype(np.float32)).astype(np.float32)
    return out


def backend_from(A, W, splits_of_m):
    def backend(reqs, variant):
        rows = np.concatenate([A[r] for r in reqs])
        out = matmul_split(rows, W, splits_of_m(len(rows)))
        return [out[2 * i:2 * i + 2] for i in range(len(reqs))]
    return backend


def test_invariant_backend_is_clean(data):
    A, W = data
    calls = harness.plan(range(P), [1, 3, 8, 24], repeats=10, seed=1)
    rep = harness.run(backend_from(A, W, lambda m: 4), calls)
    assert rep.invariant, rep.summary()
    assert rep.identical_pct == 100.0 and rep.max_distinct == 1
    assert all(v >= 10 for v in rep.observations.values())
    assert rep.rows_total > 0


def test_split_from_batch_size_is_caught(data):
    """A backend that picks the K-split count from M (1 part for a lone request, 8 once the
    call has 16 rows or more) gives other bits in large batches: the harness reports it and
    names the first differing element, which must really differ."""
    A, W = data
    calls = harness.plan(range(P), [1, 3, 8, 24], repeats=2, seed=2)
    backend = backend_from(A, W, lambda m: 1 if m < 16 else 8)
    rep = harness.run(backend, calls)
    assert not rep.invariant
    assert rep.max_distinct == 2
    assert rep.identical_pct < 100.0
    fd = rep.first_diff
    assert fd is not None and "B=8" in fd["call"]  # B = 1 and 3 have < 16 rows: same bits
    r, row, e = fd["request"], fd["row"], fd["element"]
    alone = matmul_split(A[r], W, 1)
    assert alone.reshape(2, -1)[row, e] == fd["reference"]
    assert fd["got"] != fd["reference"]
    # the element named is the first difference: re-run that call and compare the row
    call = next(c for c in calls if c.label == fd["call"])
    got = backend(list(call.ids), None)[list(call.ids).index(r)]
    assert got[row, e] == fd["got"]
    assert got[row, :e].tobytes() == alone[row, :e].tobytes()
    assert (got[:row] == alone[:row]).all()


def test_first_difference_is_exact():
    """A mock that flips one known element when the batch has exactly 3 requests."""
    base = {r: np.arange(6, dtype=np.uint16).reshape(2, 3) + 10 * r for r in range(5)}

    def backend(reqs, variant):
        outs = [base[r].copy() for r in reqs]
        if len(reqs) == 3:
            outs[1][1, 2] ^= 0x8000
        return outs

    calls = [harness.Call((r,), None, f"alone {r}") for r in range(5)]
    calls += [harness.Call((0, 4, 2), None, "trio"), harness.Call((1, 2), None, "pair")]
    rep = harness.run(backend, calls)
    assert rep.first_diff == dict(call="trio", request=4, row=1, element=2, reference=int(base[4][1, 2]),
                                  got=int(base[4][1, 2] ^ 0x8000), rows_differing=1)
    assert rep.distinct[4] == 2 and rep.distinct[0] == 1 and rep.distinct[2] == 1
    assert rep.rows_total == 10 and rep.rows_identical == 9


def test_position_dependence_is_caught(data):
    """Output that leaks from the previous request in the batch (as a shared, racy buffer would)."""
    A, W = data

    def backend(reqs, variant):
        outs = [matmul_split(A[r], W, 4) for r in reqs]
        for i in range(1, len(outs)):
            outs[i] = outs[i] + np.float32(1e-7) * outs[i - 1]
        return outs

    rep = harness.run(backend, harness.plan(range(P), [2, 5], repeats=1, seed=3))
    assert not rep.invariant and rep.first_diff["call"].startswith("B=2")


def test_run_to_run_nondeterminism_is_counted(data):
    """Same input, same output: a backend whose bits change from run to run is reported
    through the distinct-output count even when only lone requests are run."""
    A, W = data
    state = {"n": 0}

    def backend(reqs, variant):
        state["n"] += 1
        return [matmul_split(A[r], W, 1 + state["n"] % 3) for r in reqs]

    rep = harness.run(backend, harness.plan(range(4), [], repeats=10, seed=4))
    assert rep.max_distinct > 1 and not rep.invariant


def test_variants_and_outside_reference():
    """Variant labels reach the backend; a supplied reference that differs counts as a distinct output."""
    seen = []

    def backend(reqs, variant):
        seen.append(variant)
        return [np.full((1, 4), r, np.int32) for r in reqs]

    calls = harness.plan([0, 1], [2], repeats=1, batch_repeats=1, variants=("whole", "chunked"))
    rep = harness.run(backend, calls)
    assert rep.invariant and set(seen) == {"whole", "chunked"}
    rep = harness.run(backend, calls, reference={0: np.full((1, 4), 9, np.int32)})
    assert not rep.invariant and rep.distinct[0] == 2 and rep.first_diff["request"] == 0
