"""Search fp16 (a, amax) pairs whose MSD pre-rounding value is an exact tie.

Reproduces the inputs stored in msd_tie_vectors.json.  It evaluates the
expansion of one element in numpy float32 only to FIND candidates; the test
that consumes the vectors re-proves every tie in exact rational arithmetic
(tests/exact_fp32.py) and never trusts this search's arithmetic.

usage: python tests/golden/find_tie_vectors.py
"""
import json

import numpy as np


def main(seed=7, per_level=4):
    f1, f2 = np.float32(7.49), np.float32(14.98)
    allh = np.arange(0x0001, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    rng = np.random.default_rng(seed)
    found = {1: [], 2: [], 3: []}
    for amax in rng.choice(allh[allh > 1e-3], 12000, replace=False):
        a = allh[allh <= amax]
        a = np.concatenate([a, -a])
        t1 = (f1 * a) / np.float32(amax)
        t2 = (t1 - np.rint(t1)) * f2
        t3 = (t2 - np.rint(t2)) * f2
        for lvl, t in ((1, t1), (2, t2), (3, t3)):
            fl = np.floor(np.abs(t))
            idx = np.nonzero((np.abs(t) - fl == 0.5) & (fl % 2 == 0))[0]
            if len(idx) and len(found[lvl]) < per_level:
                i = idx[0]
                found[lvl].append({"a": "%#06x" % int(np.float16(a[i]).view(np.uint16)),
                                   "amax": "%#06x" % int(np.float16(amax).view(np.uint16)),
                                   "tie_level": lvl, "t": float(t[i])})
        if all(len(v) >= per_level for v in found.values()):
            break
    print(json.dumps([v for lvl in (1, 2, 3) for v in found[lvl]], indent=1))


if __name__ == "__main__":
    main()


def find_order_vectors(seed=5, count=6):
    """Pairs where (7.49*a)/amax and (a/amax)*7.49 give different levels."""
    f1, f2 = np.float32(7.49), np.float32(14.98)
    allh = np.arange(0x0001, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    rng = np.random.default_rng(seed)
    out = []

    def levels(t1):
        a1 = np.rint(t1); t2 = (t1 - a1) * f2
        a2 = np.rint(t2); t3 = (t2 - a2) * f2
        return a1, a2, np.rint(t3)

    for amax in rng.choice(allh[allh > 1e-3], 4000, replace=False):
        a = allh[allh <= amax]
        la = levels((f1 * a) / np.float32(amax))
        lb = levels((a / np.float32(amax)) * f1)
        diff = np.nonzero((la[0] != lb[0]) | (la[1] != lb[1]) | (la[2] != lb[2]))[0]
        if len(diff):
            i = diff[0]
            out.append({"a": "%#06x" % int(np.float16(a[i]).view(np.uint16)),
                        "amax": "%#06x" % int(np.float16(amax).view(np.uint16))})
        if len(out) >= count:
            break
    print(json.dumps(out, indent=1))
