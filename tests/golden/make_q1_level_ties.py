"""Write tests/golden/q1_level_ties.json: 1Q grid levels whose exact power of
two lies close to a binary32 rounding midpoint, with the oracle's levels.

TurboAdam package page, 1Q: a block's levels lie on a logarithmic grid
between two fp16 log2 endpoints.  A level is 2^x for a double x, rounded
once to binary32; where 2^x lies within a few double ulps of a midpoint
between two binary32 values, a double exp2 with a one-ulp error can round
to the wrong side, so these are the inputs that tell an exact level from a
double exp2 rounded again.

Input selection only: seeded random (lo, hi, bits, k) over every finite fp16
endpoint pair in [-149, 128], screened with numpy's 64-bit-significand
exp2 (long double) for a relative distance to the nearest midpoint below
2^-47; one seeded pass over the widths 2, 4 and 8, a second over 3 and 6.
Every stored level comes from oracle.q1_levels; the tests check each one
against a 60-digit decimal power.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "q1_level_ties.json")
SEED = 20260
SEED_3_6 = 20261
ROUNDS = 32
BATCH = 1 << 22
LIMIT = 2.0 ** -47


def screen(rng, pool, widths):
    a = rng.choice(pool, BATCH).view(np.float16).astype(np.float64)
    b = rng.choice(pool, BATCH).view(np.float16).astype(np.float64)
    lo, hi = np.minimum(a, b), np.maximum(a, b)
    bits = rng.choice(np.array(widths), BATCH)
    L = (1 << bits).astype(np.float64)
    k = np.floor(rng.random(BATCH) * (L - 1)) + 1
    x = lo + ((hi - lo) * (k - 1)) / (L - 2)
    y = np.exp2(x.astype(np.longdouble))
    with np.errstate(over="ignore"):
        f = y.astype(np.float32)
        up = np.nextafter(f, np.float32(np.inf)).astype(np.longdouble)
    dn = np.nextafter(f, np.float32(0)).astype(np.longdouble)
    fd = f.astype(np.longdouble)
    with np.errstate(invalid="ignore"):
        d = np.minimum(np.abs(y - (fd + up) / 2), np.abs(y - (fd + dn) / 2)) / y
    keep = np.nonzero(np.isfinite(d) & (d < LIMIT))[0]
    return [(float(np.log2(d[i])), np.float16(lo[i]), np.float16(hi[i]), int(bits[i]), int(k[i])) for i in keep]


def main():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = codes.view(np.float16).astype(np.float64)
    pool = codes[np.isfinite(vals) & (vals >= -149) & (vals <= 128)]
    found = {}
    for seed, widths in ((SEED, [2, 4, 8]), (SEED_3_6, [3, 6])):
        rng = np.random.Generator(np.random.PCG64(seed))
        for _ in range(ROUNDS):
            for log2d, lo, hi, bits, k in screen(rng, pool, widths):
                lo16 = int(np.array([lo]).view(np.uint16)[0])
                hi16 = int(np.array([hi]).view(np.uint16)[0])
                found.setdefault((lo16, hi16, bits, k), log2d)
    rows = []
    for (lo16, hi16, bits, k), log2d in sorted(found.items(), key=lambda kv: kv[1]):
        lev = oracle.q1_levels(lo16, hi16, bits)
        rows.append({"lo16": f"{lo16:04x}", "hi16": f"{hi16:04x}", "bits": bits, "k": k,
                     "level_hex": f"{int(lev[k:k + 1].view(np.uint32)[0]):08x}",
                     "log2_rel_distance": round(log2d, 3)})
    with open(OUT, "w") as f:
        json.dump({"source": "TurboAdam package page, 1Q (logarithmic grid levels)",
                   "recipe": " ".join(__doc__.split("\n\n")[2].split()),
                   "seed": SEED, "seed_3_6": SEED_3_6, "samples": 2 * ROUNDS * BATCH, "rows": rows}, f,
                  indent=1)
    print(OUT, len(rows))


if __name__ == "__main__":
    main()
