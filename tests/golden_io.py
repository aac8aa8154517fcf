"""Reader for the small text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_fixture(name):
    """key -> list of tokens, for 'key v1 v2 ...' lines; '#' lines are comments."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            out.setdefault(k, []).append(v)
    return out
