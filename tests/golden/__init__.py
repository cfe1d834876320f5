"""Hand-derived fixtures (text) and the reader for their ``key = values`` lines."""

import os

HERE = os.path.dirname(os.path.abspath(__file__))


def read_fixture(name):
    """List of (key, [tokens]) in file order; '#' starts a comment."""
    out = []
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, val = line.partition("=")
            out.append((key.strip(), val.split()))
    return out


def num(tok):
    return int(tok, 16) if tok.lower().startswith(("0x", "-0x")) else float(tok)
