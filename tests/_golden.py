"""Reader for the text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows(name):
    """Non-comment lines of a fixture, split on whitespace."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


def keyed(name):
    """Fixture lines as {first field: [remaining fields], ...} (last wins)."""
    d = {}
    for r in rows(name):
        d.setdefault(r[0], []).append(r[1:])
    return d
