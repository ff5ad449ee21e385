"""Planted-mistake helper: builds a copy of an oracle module with one textual
change, on the CPU, so tests can show that the pins catch that mistake."""
from __future__ import annotations

import os
import types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def mutant(modname: str, old: str, new: str):
    path = os.path.join(ROOT, "oracle", modname + ".py")
    with open(path) as f:
        src = f.read()
    assert old in src, f"mutation anchor not found in oracle/{modname}.py: {old!r}"
    m = types.ModuleType(f"oracle._mutant_{modname}")
    m.__package__ = "oracle"
    m.__file__ = path
    exec(compile(src.replace(old, new, 1), path, "exec"), m.__dict__)
    return m


def caught(pins, mod) -> bool:
    """True if at least one pin fails (assertion or error) on the module."""
    for pin in pins:
        try:
            pin(mod)
        except Exception:
            return True
    return False
