"""Invariance harness: run a pool of requests through a backend alone, batched,
permuted and repeated, and report per request how many distinct outputs it
produced and where the first difference from its reference run lies.

What it checks follows the pages.  The "Receipts" page ("Same input, same
output") runs one request many times and counts the distinct answers; its
opening paragraph asks that a request's output not depend on the other users
sharing the batch, the prompt cache or run-ahead.  The M-0002 record ("How it
works") names the cause of differences: a reduction order that depends on the
load, e.g. a split count chosen from the batch size.

The harness holds no arithmetic of the forward path.  A backend is a callable
``backend(requests, variant) -> list of numpy arrays`` that runs the given
requests together in one call (in the order given) and returns each request's
output, first axis = the request's rows (tokens).  ``variant`` is an opaque
label of how the call is made (e.g. a prefill chunk size); requests are run
with variant None unless a plan says otherwise.  The harness composes the
calls, hashes output bytes and compares them.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Any, Callable, Hashable, Optional, Sequence

import numpy as np

__all__ = ["Call", "Report", "plan", "run"]


@dataclass(frozen=True)
class Call:
    """One backend call: the request ids it runs together, in this order, and a variant label."""
    ids: tuple
    variant: Hashable = None
    label: str = ""


@dataclass
class Report:
    """Outcome of a harness run.

    distinct[r]       -- number of distinct output hashes of request r over all calls
    observations[r]   -- how many calls produced an output for request r
    rows_identical    -- rows bit-identical to the request's reference run, over all rows seen
    rows_total        -- rows seen (reference runs excluded)
    first_diff        -- the first (in call order) output that differs from its reference:
                         call label, request, row, flat element index within the row, and the
                         two values; None when every output matched
    """
    distinct: dict = field(default_factory=dict)
    observations: dict = field(default_factory=dict)
    rows_identical: int = 0
    rows_total: int = 0
    calls: int = 0
    first_diff: Optional[dict] = None

    @property
    def identical_pct(self) -> float:
        return 100.0 * self.rows_identical / self.rows_total if self.rows_total else 100.0

    @property
    def max_distinct(self) -> int:
        return max(self.distinct.values()) if self.distinct else 0

    @property
    def invariant(self) -> bool:
        return self.first_diff is None and self.max_distinct <= 1

    def summary(self) -> str:
        s = (f"{len(self.distinct)} requests, {self.calls} calls, {self.rows_total} rows compared: "
             f"{self.identical_pct:.4f}% rows identical, distinct outputs per request max "
             f"{self.max_distinct}")
        if self.first_diff is not None:
            s += f"; first difference {self.first_diff}"
        return s


def plan(pool: Sequence[Hashable], batch_sizes: Sequence[int], repeats: int = 10, batch_repeats: int = 2,
         seed: int = 0, alone: bool = True, variants: Sequence[Hashable] = (None,)) -> list:
    """The standard composition set over a request pool.

    - every request alone, ``repeats`` times (the "same input, same output" runs);
    - for each batch size B: a random subset of B requests in random order, the same
      subset reversed and rotated by one, each ``batch_repeats`` times; B larger than
      the pool is clipped to the pool;
    - each call once per variant label in ``variants``.
    The first alone call of a request (first variant) is its reference.
    """
    rng = np.random.default_rng(seed)
    pool = list(pool)
    calls = []
    for v in variants:
        if alone:
            for rep in range(repeats):
                for r in pool:
                    calls.append(Call((r,), v, f"alone {r!r} rep {rep} variant {v!r}"))
        for B in batch_sizes:
            B = min(int(B), len(pool))
            idx = [pool[i] for i in rng.permutation(len(pool))[:B]]
            orders = {"random": idx, "reversed": idx[::-1], "rotated": idx[1:] + idx[:1]}
            for name, ids in orders.items():
                if B == 1 and name != "random":
                    continue
                for rep in range(batch_repeats):
                    calls.append(Call(tuple(ids), v, f"B={B} {name} rep {rep} variant {v!r}"))
    return calls


def _first_difference(ref: np.ndarray, got: np.ndarray):
    if ref.shape != got.shape or ref.dtype != got.dtype:
        return {"shape": (ref.shape, got.shape), "dtype": (str(ref.dtype), str(got.dtype))}
    rb = np.ascontiguousarray(ref).reshape(ref.shape[0], -1) if ref.ndim else ref.reshape(1, 1)
    gb = np.ascontiguousarray(got).reshape(got.shape[0], -1) if got.ndim else got.reshape(1, 1)
    rv = rb.view(np.uint8).reshape(rb.shape[0], -1)
    gv = gb.view(np.uint8).reshape(gb.shape[0], -1)
    bad_rows = np.nonzero((rv != gv).any(axis=1))[0]
    row = int(bad_rows[0])
    eb = (rb[row].view(np.uint8).reshape(rb.shape[1], -1) != gb[row].view(np.uint8).reshape(gb.shape[1], -1))
    elem = int(np.nonzero(eb.any(axis=1))[0][0])
    return {"row": row, "element": elem, "reference": rb[row, elem].item(), "got": gb[row, elem].item(),
            "rows_differing": int(len(bad_rows))}


def run(backend: Callable[[list, Any], list], calls: Sequence[Call],
        request_of: Callable[[Hashable], Any] = lambda r: r,
        reference: Optional[dict] = None, log: Optional[Callable[[str], None]] = None) -> Report:
    """Run ``calls`` in order and compare every output with its request's reference.

    ``request_of(id)`` turns a pool id into what the backend takes.  The reference of a
    request is ``reference[id]`` when given, else its first output in call order.
    """
    rep = Report()
    refs = dict(reference or {})
    hashes: dict = {}
    for call in calls:
        if log is not None:
            log(call.label or repr(call.ids))
        outs = backend([request_of(r) for r in call.ids], call.variant)
        if len(outs) != len(call.ids):
            raise ValueError(f"backend returned {len(outs)} outputs for {len(call.ids)} requests")
        rep.calls += 1
        for r, out in zip(call.ids, outs):
            out = np.asarray(out)
            hashes.setdefault(r, set()).add(hashlib.sha256(np.ascontiguousarray(out).tobytes()).hexdigest())
            rep.observations[r] = rep.observations.get(r, 0) + 1
            if r not in refs:
                refs[r] = out.copy()
                continue
            ref = refs[r]
            n_rows = out.shape[0] if out.ndim else 1
            rep.rows_total += n_rows
            if ref.shape == out.shape and ref.dtype == out.dtype:
                a = np.ascontiguousarray(ref).reshape(n_rows, -1).view(np.uint8)
                b = np.ascontiguousarray(out).reshape(n_rows, -1).view(np.uint8)
                same = ~(a != b).any(axis=1)
                rep.rows_identical += int(same.sum())
                if not same.all() and rep.first_diff is None:
                    rep.first_diff = dict(call=call.label, request=r, **_first_difference(ref, out))
            elif rep.first_diff is None:
                rep.first_diff = dict(call=call.label, request=r, **_first_difference(ref, out))
    # a reference supplied from outside counts as one more distinct output if it differs
    for r, ref in (reference or {}).items():
        if r in hashes:
            hashes[r].add(hashlib.sha256(np.ascontiguousarray(np.asarray(ref)).tobytes()).hexdigest())
    rep.distinct = {r: len(h) for r, h in hashes.items()}
    return rep
