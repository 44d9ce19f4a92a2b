"""Reader for the small text fixtures in this folder.

Each fixture holds values printed on the pages, with the citation in its
header comment.  Lines are ``key v1 v2 ...``; repeated keys accumulate.
"""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name):
    out = {}
    with open(os.path.join(HERE, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            nums = [float(x) if "." in x else int(x) for x in vals]
            out.setdefault(key, []).append(nums)
    return out
