"""The mask checker of the GPU parity tests, on hand-built oracle rows (CPU).

A library row may differ from the oracle's only by taking a decision the oracle
flags as near its boundary the other way (the theta guard on a query or key block,
the tau cut of the cumulative mass, a tie of compressed logits at the cut).  These
cases build such rows with the oracle's own predictor and check that the checker
accepts exactly the alternatives and rejects any other change, forced blocks
included.
"""

import dataclasses

import numpy as np

from oracle import predict as OP

import _ref as R


def make_ref(logits, simq, simk, p):
    rows = [OP.predict_row(i, logits[i], simq[i], simk, p) for i in range(logits.shape[0])]
    return {"mask": np.array([r for r, _ in rows]), "info": [inf for _, inf in rows],
            "logits": logits, "simq": simq, "simk": simk}


def base_params(**kw):
    p = OP.MaskParams(N=8 * 16, block_q=16, block_k=16, tau=0.9, theta=0.5, sink_front=16)
    return dataclasses.replace(p, **kw)


def test_identical_row_is_admissible_and_other_rows_are_not():
    rng = np.random.default_rng(0)
    p = base_params()
    logits = rng.normal(0, 3, size=(8, 8))
    ref = make_ref(logits, np.full(8, 0.9), np.full(8, 0.9), p)
    for i in range(8):
        assert R.admissible_row(ref["mask"][i], i, ref, p)[0]
        if not ref["info"][i]["border"]:
            got = ref["mask"][i].copy()
            j = int(np.argmin(np.where(got, np.inf, logits[i])))  # a dropped block
            got[j] = True
            assert not R.admissible_row(got, i, ref, p)[0]
    # the sink block (block 0) must be kept
    got = ref["mask"][3].copy()
    got[0] = False
    assert not R.admissible_row(got, 3, ref, p)[0]


def test_key_block_near_theta_may_flip_only_its_own_consequences():
    p = base_params(tau=0.5)
    logits = np.tile(np.array([0.0, 5.0, 4.0, 1.0, 0.5, 0.2, 0.1, -1.0]), (8, 1))
    simk = np.full(8, 0.9)
    simk[6] = 0.5 + 4e-6  # within 1e-5 of theta: block 6 may be read as forced
    ref = make_ref(logits, np.full(8, 0.9), simk, p)
    i = 2
    assert "theta" in ref["info"][i]["border"]
    alt_simk = simk.copy()
    alt_simk[6] = 0.5 - 4e-6
    alt, _ = OP.predict_row(i, logits[i], 0.9, alt_simk, p)
    assert not np.array_equal(alt, ref["mask"][i]) and alt[6]
    assert R.admissible_row(alt, i, ref, p)[0]
    wrong = alt.copy()
    wrong[7] = True  # an unrelated block
    assert not R.admissible_row(wrong, i, ref, p)[0]
    no_sink = ref["mask"][i].copy()
    no_sink[0] = False
    assert not R.admissible_row(no_sink, i, ref, p)[0]


def test_query_block_near_theta_may_be_read_as_a_full_row():
    p = base_params(tau=0.5)
    logits = np.tile(np.array([0.0, 5.0, 4.0, 1.0, 0.5, 0.2, 0.1, -1.0]), (8, 1))
    simq = np.full(8, 0.9)
    simq[4] = 0.5 - 3e-6
    ref = make_ref(logits, simq, np.full(8, 0.9), p)
    assert ref["mask"][4].all()  # forced full row in the oracle
    alt, _ = OP.predict_row(4, logits[4], 0.5 + 3e-6, np.full(8, 0.9), p)
    assert not alt.all()
    assert R.admissible_row(alt, 4, ref, p)[0]
    half = alt.copy()
    half[7] = True
    assert not R.admissible_row(half, 4, ref, p)[0]


def test_tau_cut_within_band_moves_by_one_block_only():
    p = base_params(theta=None, sink_front=0, tau=0.75)
    # candidates 0..7 with probabilities 0.5, 0.25, 0.125, ... : the mass before the
    # third block is exactly 0.75; put tau 3e-6 above it
    pr = np.array([0.5, 0.25, 0.125, 0.0625, 0.03125, 0.015625, 0.0078125, 0.0078125])
    logits = np.tile(np.log(pr), (8, 1))
    p = dataclasses.replace(p, tau=0.75 + 3e-6)
    ref = make_ref(logits, np.full(8, 0.9), np.full(8, 0.9), p)
    row = ref["mask"][0]
    assert "tau" in ref["info"][0]["border"] and row.sum() == 3
    fewer = row.copy()
    fewer[2] = False
    assert R.admissible_row(fewer, 0, ref, p)[0]
    two_fewer = fewer.copy()
    two_fewer[1] = False
    assert not R.admissible_row(two_fewer, 0, ref, p)[0]
    more = row.copy()
    more[3] = True
    assert not R.admissible_row(more, 0, ref, p)[0]


def test_tied_logits_at_the_cut_may_swap():
    p = base_params(theta=None, sink_front=0, tau=None, sparsity=0.5)  # keep 4 of 8
    logits = np.tile(np.array([3.0, 2.5, 2.0, 1.00002, 1.0, -1.0, -2.0, -3.0]), (8, 1))
    ref = make_ref(logits, np.full(8, 0.9), np.full(8, 0.9), p)
    row = ref["mask"][5]
    assert "tie" in ref["info"][5]["border"] and row[3] and not row[4]
    swapped = row.copy()
    swapped[3], swapped[4] = False, True
    assert R.admissible_row(swapped, 5, ref, p)[0]
    far = row.copy()
    far[2], far[5] = False, True  # not tied
    assert not R.admissible_row(far, 5, ref, p)[0]
