"""Readers for the text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            yield [f.strip() for f in line.split("|")]


def hexes(field):
    return [int(t, 16) for t in field.split()]


def ints(field):
    return [int(t) for t in field.split()]
