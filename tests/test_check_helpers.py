"""CPU tests of the GPU tests' own checkers: the plan-validity check and the
exact top-k check against a kernel's own logits must accept a correct
result and reject each plausible mistake (wrong order inside a segment,
shifted offsets, a stray row, a tie broken the wrong way)."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from _gpu_common import check_plan_valid, check_topk_own_logits, order_keys


def _random_plan(T=300, E=40, k=5, pad=7, seed=0):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts = O.expert_counts(idx, E)
    offs = O.padded_offsets(counts, pad)
    cap = O.rows_capacity(T, E, k, pad)
    tok_row, row_src = O.assign_slots(idx, offs, E, cap)
    return idx, counts, offs, tok_row, row_src, E, pad


def test_plan_check_accepts_oracle_plan():
    for seed in range(3):
        check_plan_valid(*_random_plan(seed=seed))
    # pad 1 and a single expert
    check_plan_valid(*_random_plan(T=50, E=1, k=1, pad=1))


def test_plan_check_rejects_mistakes():
    idx, counts, offs, tok_row, row_src, E, pad = _random_plan()
    # two tokens of one expert exchanged (order inside the segment)
    e = int(idx[0, 0])
    ts, js = np.nonzero(idx == e)
    bad = tok_row.copy()
    bad[ts[0], js[0]], bad[ts[1], js[1]] = tok_row[ts[1], js[1]], \
        tok_row[ts[0], js[0]]
    with pytest.raises(AssertionError):
        check_plan_valid(idx, counts, offs, bad, row_src, E, pad)
    # offsets without padding
    raw = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    with pytest.raises(AssertionError):
        check_plan_valid(idx, counts, raw, tok_row, row_src, E, pad)
    # a padding row claiming a token
    rs = row_src.copy()
    rs[np.nonzero(rs < 0)[0][0]] = 0
    with pytest.raises(AssertionError):
        check_plan_valid(idx, counts, offs, tok_row, rs, E, pad)
    # counts off by one
    c2 = counts.copy()
    c2[0] += 1
    with pytest.raises(AssertionError):
        check_plan_valid(idx, c2, offs, tok_row, row_src, E, pad)


def test_order_keys_rank_like_floats():
    v = np.array([-np.inf, -3.5, -1e-30, -0.0, 0.0, 1e-30, 2.0, np.inf],
                 dtype=np.float32)
    key = order_keys(v)
    assert (np.diff(key) > 0).all()


def test_topk_check_exact_ties_and_order():
    # float32 logits with exact ties: the lower expert index ranks first
    l = np.array([[1.0, 3.0, 3.0, -2.0, 0.5, 3.0],
                  [0.0, -0.0, 0.25, 0.25, -1.0, 7.0]], dtype=np.float32)
    k = 4
    idx, w = O.select_topk(l.astype(np.float64), k)
    check_topk_own_logits(idx, w, l, k)
    # -0.0 ranks below +0.0 in the kernel's key: row 1 picks 5, 2, 3, then
    # +0.0 (expert 0) before -0.0 (expert 1)
    assert list(idx[1]) == [5, 2, 3, 0]
    swapped = idx.copy()
    swapped[0, [0, 1]] = swapped[0, [1, 0]]      # tie broken upward
    with pytest.raises(AssertionError):
        check_topk_own_logits(swapped, w, l, k)
    w_bad = w.copy()
    w_bad[0, 0] += 1e-5
    with pytest.raises(AssertionError):
        check_topk_own_logits(idx, w_bad, l, k)
