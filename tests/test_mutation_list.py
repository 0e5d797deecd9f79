"""The oracle's mutation check (``tests/mutation_check.py``) stays in step with the oracle's source: every
listed mistake still applies to exactly one place, and one of them, run end to end, is caught by the pins.
The whole check (every mutant, about a minute on 8 cores) is run by hand: ``python tests/mutation_check.py``."""
import mutation_check as mc


def test_every_mutant_applies_once():
    with open(mc.SRC) as fh:
        text = fh.read()
    names = [m[0] for m in mc.MUTANTS]
    assert len(set(names)) == len(names)
    for name, old, new in mc.MUTANTS:
        assert old != new, name
        assert text.count(old) == 1, name
    assert set(mc.EQUIVALENT) <= set(names)


def test_one_mutant_is_caught():
    name, old, new = next(m for m in mc.MUTANTS if m[0] == "reduce: descending fold")
    _, killed, why = mc.run_one(name, old, new, timeout=300)
    assert killed, why
