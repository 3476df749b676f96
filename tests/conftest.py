"""Shared pytest setup: the `gpu` marker, golden-file parsing and the oracle fixture."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def parse_number(tok: str) -> float:
    """'m' or 'mpe' meaning m * 2^e, exact in fp64."""
    if "p" in tok:
        m, e = tok.split("p")
        return float(m) * 2.0 ** int(e)
    return float(tok)


def load_golden(name: str) -> list[dict]:
    """Parse a golden file into cases: {'name': ..., key: [tokens...]}; '#' starts a comment."""
    cases: list[dict] = []
    cur: dict | None = None
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("case "):
                cur = {"name": line[5:].strip()}
                cases.append(cur)
                continue
            key, val = line.split(":", 1)
            if cur is None:
                cur = {"name": "_"}
                cases.append(cur)
            cur[key.strip()] = val.split()
    return cases


@pytest.fixture(scope="session")
def oracle():
    from oracle import oracle as o
    o.build(force=False)
    return o


@pytest.fixture(scope="session")
def bruteforce():
    from oracle import bruteforce as b
    return b


def f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)
