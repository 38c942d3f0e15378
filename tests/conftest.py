import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def golden_path(name):
    return os.path.join(GOLDEN, name)


def read_golden_lines(name):
    with open(golden_path(name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


def read_golden_blocks(name):
    """Parse 'block NAME scale_bits=0x..' / 'w: ...' / 'codes: ...' triples."""
    lines = read_golden_lines(name)
    out = []
    for i in range(0, len(lines), 3):
        head, wl, cl = lines[i:i + 3]
        _, bname, sb = head.split()
        scale_bits = int(sb.split("=")[1], 16)
        w = [float(v) for v in wl.split(":", 1)[1].split()]
        codes = [int(v, 16) for v in cl.split(":", 1)[1].split()]
        out.append((bname, scale_bits, w, codes))
    return out
