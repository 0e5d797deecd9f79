"""The kernel mutation check (``tests/kernel_mutation_check.py``) stays in step with the HIP sources: every
listed mistake still applies to exactly one place, and names the GPU test files that exist."""
import os

import kernel_mutation_check as kmc


def test_every_kernel_mutant_applies_once():
    names = [m[0] for m in kmc.MUTANTS]
    assert len(set(names)) == len(names)
    assert len({kmc.slug(n) for n in names}) == len(names)
    for name, src, old, new, tests in kmc.MUTANTS:
        with open(os.path.join(kmc.CSRC, src)) as fh:
            text = fh.read()
        assert old != new, name
        assert text.count(old) == 1, name
        assert tests and all(os.path.exists(os.path.join(kmc.ROOT, "tests", t)) for t in tests), name
