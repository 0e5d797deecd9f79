"""CPU tests of the protocol selector's cost model (host logic): wire bytes of each encoding, the
non-negative least-squares fit, the choice and its crossover, and the committed table measured on the GPU."""
import math
import os

import numpy as np
import pytest

from tensor_all_reduce_amd import selector as sel


def test_wire_bytes_and_blocks():
    assert sel.wire_bytes("ll", 4096) == 8192                      # 4 payload + 4 epoch bytes per slot
    assert sel.wire_bytes("flag512", 1024) == 1024 + 4             # one flag word per 512-element block
    assert sel.wire_bytes("flag2048", 1 << 20) == (1 << 20) + 4 * 256
    assert sel.blocks("flag8192", 1 << 20) == 64
    assert sel.blocks("ll", 1 << 20) == (1 << 20) // 4 // sel.LL_BLOCK_SLOTS
    with pytest.raises(ValueError):
        sel.flag_block("ll")


def synthetic(coefs, sizes=(1 << 12, 1 << 14, 1 << 16, 1 << 18, 1 << 20, 1 << 22, 1 << 24), ranks=(2, 4, 8)):
    rows = []
    for enc, (a, b, c, d, e) in coefs.items():
        for S in sizes:
            for R in ranks:
                rows.append((enc, S, R, max(a + b * R, d + (c * R + e) * sel.wire_bytes(enc, S))))
    return rows


# (a, b, c, d, e): floor a + b R, transfer d + (c R + e) wire; each branch binds on part of the sizes above,
# and the transfer branch at several R (so that c and e are both determined)
COEFS = {"ll": (7.5, 0.25, 9.0e-7, 2.0, 2.0e-7), "flag512": (6.0, 0.25, 2.3e-6, 1.0, 3.0e-6),
         "flag2048": (6.5, 0.2, 2.2e-6, 1.5, 2.0e-6), "flag8192": (8.0, 0.3, 2.0e-6, 2.5, 0.0)}


def test_fit_recovers_exact_coefficients():
    costs = sel.fit(synthetic(COEFS))
    for enc, want in COEFS.items():
        for g, w in zip(costs[enc].coef, want):
            assert g == pytest.approx(w, rel=1e-4, abs=1e-9), (enc, costs[enc].coef)


def test_fit_is_non_negative():
    rows = [("ll", S, R, 100.0 - S * 1e-5) for S in (1 << 10, 1 << 14, 1 << 18, 1 << 20) for R in (2, 8)]
    c = sel.fit(rows)["ll"].coef
    assert all(v >= 0 for v in c)


def test_choice_and_crossover_match_the_closed_form():
    costs = {e: sel.EncodingCost(e, c) for e, c in COEFS.items()}
    assert sel.select(costs, 1 << 10, 8) == "flag512"   # small: the lowest floor decides
    assert sel.select(costs, 1 << 26, 8) == "ll"        # large: the cheapest byte decides
    # ll against flag512 at R = 8: ll still sits on its floor 7.5 + 0.25 R = 9.5 where flag512's transfer
    # time 1 + (2.3e-6 R + 3e-6) S (1 + 4/1024) reaches it, so that is where the choice flips
    a_l, b_l, c_l, d_l, e_l = COEFS["ll"]
    a_f, b_f, c_f, d_f, e_f = COEFS["flag512"]
    R = 8
    S_eq = (a_l + b_l * R - d_f) / ((c_f * R + e_f) * (1 + 4 / 1024))
    assert d_l + (c_l * R + e_l) * 2 * S_eq < a_l + b_l * R  # (ll on its floor there)
    two = {"ll", "flag512"}
    below, above = int(S_eq * 0.95) // 2 * 2, int(S_eq * 1.05) // 2 * 2
    assert sel.select(costs, below, R, allowed=two) == "flag512"
    assert sel.select(costs, above, R, allowed=two) == "ll"
    steps = sel.crossover(costs, R)
    assert steps[0][1] == "flag512" and steps[-1][1] == "ll"
    assert [S for S, _ in steps] == sorted(S for S, _ in steps)


def test_ties_take_the_listed_order():
    same = {e: sel.EncodingCost(e, (5.0, 0.0, 0.0, 0.0, 0.0)) for e in sel.ENCODINGS}
    assert sel.select(same, 1 << 20, 4) == sel.ENCODINGS[0]
    with pytest.raises(ValueError):
        sel.select(same, 1 << 20, 4, allowed=set())


def test_save_load_round_trip(tmp_path):
    costs = {e: sel.EncodingCost(e, c) for e, c in COEFS.items()}
    p = os.path.join(tmp_path, "t.json")
    sel.save(p, costs, [("ll", 1024, 2, 7.5)], "cmd", "machine")
    back = sel.load(p)
    assert {e: c.coef for e, c in back.items()} == {e: tuple(c) for e, c in COEFS.items()}


def test_four_coefficient_table_loads_without_the_per_rank_term(tmp_path):
    import json
    p = os.path.join(tmp_path, "old.json")
    json.dump({"coefficients": {"ll": [7.5, 0.25, 9.0e-7, 2.0]}, "measured": []}, open(p, "w"))
    assert sel.load(p)["ll"].coef == (7.5, 0.25, 9.0e-7, 2.0, 0.0)


def test_per_rank_term_separates_message_size_from_rank_count():
    """With e > 0 the transfer time of one R and twice the bytes exceeds that of twice R and the same
    bytes (the per-rank term doubles in the first case only); with e = 0 the two are equal."""
    with_e = sel.EncodingCost("flag512", (0.0, 0.0, 1.0e-6, 0.0, 4.0e-6))
    no_e = sel.EncodingCost("flag512", (0.0, 0.0, 1.0e-6, 0.0, 0.0))
    S = 1 << 24
    assert with_e.predict(2 * S, 2) > with_e.predict(S, 4)
    assert no_e.predict(2 * S, 2) == pytest.approx(no_e.predict(S, 4), rel=1e-3)


@pytest.mark.skipif(not os.path.exists(sel.DEFAULT_TABLE), reason="no measured table committed")
def test_committed_table_chooses_well_on_its_own_measurements():
    """On the latencies measured on the GPU, the fitted model's choice costs little against the fastest
    encoding measured at each point."""
    import json
    doc = json.load(open(sel.DEFAULT_TABLE))
    costs = sel.load()
    by = {}
    for enc, S, R, t in doc["measured"]:
        by.setdefault((S, R), {})[enc] = t
    regrets = []
    for (S, R), meas in by.items():
        choice = sel.select(costs, S, R, allowed=set(meas))
        regrets.append(meas[choice] / min(meas.values()) - 1.0)
    assert len(regrets) >= 10
    assert max(regrets) <= 0.10 and float(np.mean(regrets)) <= 0.01, regrets


def test_committed_choice_on_the_slot_workload():
    """The measured table picks flag words for the 8-rank [128, 8192] bf16 workload (2 MiB per rank): the
    flag receiver reads half the bytes and the sender's fences are amortized over large spans. For two
    ranks and small messages, where the fixed cost of the flag read and fence is not paid back, it picks
    the 8-byte slots."""
    costs = sel.load()
    assert sel.select(costs, 2 << 20, 8).startswith("flag")
    assert sel.select(costs, 16 << 10, 2) == "ll"


def test_self_sync_reduce_refuses_epochs_its_inbox_already_carries():
    """The inbox starts zero-filled, so epoch 0 would pass every readiness check before anything was sent;
    the receive side refuses it (and anything that is not a 32-bit epoch word)."""
    from tensor_all_reduce_amd.flash_allreduce import SelfSyncReduce
    for bad in (0, -1, 1 << 32):
        with pytest.raises(ValueError):
            SelfSyncReduce._check_epoch(bad)
    SelfSyncReduce._check_epoch(1)
    SelfSyncReduce._check_epoch((1 << 32) - 1)


def test_regret_scores_a_table_on_latencies_it_was_not_fitted_to():
    """regret(): hand-built latencies where the closed-form choice is known.  Two points, four encodings; at
    the first the table's choice is the fastest (0% loss), at the second it picks an encoding 25% slower
    than the fastest.  Points where an encoding is missing are skipped."""
    costs = {e: sel.EncodingCost(e, c) for e, c in (("ll", (1.0, 0, 0, 0, 0)), ("flag512", (2.0, 0, 0, 0, 0)),
                                                    ("flag2048", (3.0, 0, 0, 0, 0)), ("flag8192", (4.0, 0, 0, 0, 0)))}
    rows = [("ll", 1024, 2, 10.0), ("flag512", 1024, 2, 12.0), ("flag2048", 1024, 2, 13.0), ("flag8192", 1024, 2, 14.0),
            ("ll", 4096, 8, 20.0), ("flag512", 4096, 8, 16.0), ("flag2048", 4096, 8, 17.0), ("flag8192", 4096, 8, 18.0),
            ("ll", 8192, 8, 5.0)]
    r = sel.regret(costs, rows)
    assert r == {"points": 2, "fastest": 1, "mean_pct": 12.5, "max_pct": 25.0}
    assert sel.regret(costs, rows[-1:]) == {"points": 0, "fastest": 0, "mean_pct": None, "max_pct": None}


@pytest.mark.skipif(not os.path.exists(sel.DEFAULT_TABLE), reason="no measured table committed")
def test_regret_of_the_committed_table_on_its_own_measurements():
    """The committed table scored by regret() on the latencies stored with it: the same bound as the test
    above, computed by the function the benchmark uses on fresh measurements."""
    import json
    doc = json.load(open(sel.DEFAULT_TABLE))
    r = sel.regret(sel.load(), [tuple(x) for x in doc["measured"]])
    assert r["points"] >= 10 and r["max_pct"] <= 10.0 and r["mean_pct"] <= 1.0, r
