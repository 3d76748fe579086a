"""Parity statistics recorded by the GPU tests (flagged and ambiguous
acceptance counts, near-tie selections, errors of sampled units). conftest.py
prints them in pytest's terminal summary, so the test log keeps them whatever
output capture is in effect."""
STATS = []


def record(test, **fields):
    STATS.append((test, fields))


def lines():
    out = []
    for test, fields in STATS:
        body = ", ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}" for k, v in fields.items())
        out.append(f"{test}: {body}")
    return out
