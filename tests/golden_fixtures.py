"""Reader for the text fixtures under tests/golden/.

Each fixture is `key: value value ...` lines plus `#` comment lines that name
the page and section the values come from.  Values are returned as lists of
strings; `nums(key)` converts them to floats or ints.
"""
import os

_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


class Fixture(dict):
    def nums(self, key, kind=float):
        return [kind(v) for v in self[key]]

    def num(self, key, kind=float):
        (v,) = self.nums(key, kind)
        return v


def load(name: str) -> Fixture:
    fx = Fixture()
    with open(os.path.join(_DIR, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(":")
            fx[key.strip()] = rest.split()
    return fx
