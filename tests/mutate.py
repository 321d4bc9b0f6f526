"""Source-level mutants of an oracle module, for planted-mistake tests.

``mutant(module, edits)`` returns a fresh module object built from the
module's own source with each (old, new) text edit applied; every ``old``
must occur exactly once, so a mutation site that the source no longer has
fails loudly instead of silently testing the unmutated code.  Runs on the CPU
only; nothing here touches the GPU path.
"""
from __future__ import annotations

import inspect
import itertools
import sys
import types

_ids = itertools.count()


def mutant(module, edits):
    src = inspect.getsource(module)
    for old, new in edits:
        n = src.count(old)
        if n != 1:
            raise AssertionError(f"mutation site occurs {n} times in {module.__name__}: {old!r}")
        src = src.replace(old, new)
    name = f"{module.__name__}__mutant{next(_ids)}"
    mod = types.ModuleType(name)
    mod.__file__ = module.__file__
    mod.__package__ = module.__package__
    sys.modules[name] = mod  # dataclasses look the defining module up while the class is built
    try:
        exec(compile(src, f"<mutant of {module.__name__}>", "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod
