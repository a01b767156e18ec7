"""Readers for the text fixtures under tests/golden/ (no arithmetic of the product)."""
import os
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_table(name):
    """Rows of 'key value' pairs; '#' starts a comment."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out.append((int(k, 16), v))
    return out


def e2m1_table():
    """code -> Fraction (exact), from the OCP MX FP4 table."""
    return {k: Fraction(v.lstrip("-")) * (-1 if v.startswith("-") else 1) for k, v in read_table("e2m1_values.txt")}


def e2m1_sign_table():
    """code -> True if the value is negative (includes -0)."""
    return {k: v.startswith("-") for k, v in read_table("e2m1_values.txt")}
