"""Write tests/golden/adversarial_groups.npz.

Groups of values on which shortcuts of the symmetric rule give different
codes from the IEEE float32 quotient the rule prescribes:

* "recip": fl32(x * fl32(1/scale)) rounds to another integer than
  fl32(x / scale);
* "f64":   the float64 quotient x / scale rounds to another integer.

The search uses plain NumPy; the stored expected codes and scales come from
oracle.codec only.  Run from the repository root:
    python tests/golden/make_adversarial.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from oracle import codec  # noqa: E402


def mine(bits, group, kind, want, seed):
    rng = np.random.default_rng(seed)
    qmax = (1 << (bits - 1)) - 1
    found = []
    rounds = 0
    while len(found) < want and rounds < 400:
        rounds += 1
        x = rng.standard_normal((200_000, group), dtype=np.float32)
        x = x.astype(np.float16).astype(np.float32) if kind == "f16" else x
        m = np.max(np.abs(x), axis=1)
        s = (m / np.float32(qmax)).astype(np.float32)
        q = (x / s[:, None]).astype(np.float32)
        c_true = np.clip(np.rint(q), -qmax, qmax)
        r = (np.float32(1.0) / s).astype(np.float32)
        c_recip = np.clip(np.rint((x * r[:, None]).astype(np.float32)),
                          -qmax, qmax)
        c_f64 = np.clip(np.rint(x.astype(np.float64) /
                                s[:, None].astype(np.float64)), -qmax, qmax)
        bad = np.nonzero(np.any(c_true != c_recip, axis=1) |
                         np.any(c_true != c_f64, axis=1))[0]
        for i in bad[: want - len(found)]:
            found.append(x[i].copy())
    return found


def main():
    xs, bits_l, dt = [], [], []
    for bits in (8, 4, 3, 2):
        for group, kind in ((128, "f32"), (32, "f32"), (64, "f16")):
            got = mine(bits, group, kind, 6, seed=1000 * bits + group)
            for x in got:
                pad = np.zeros(128, np.float32)
                pad[:group] = x
                xs.append(pad)
                bits_l.append(bits)
                dt.append(group)
    xs = np.stack(xs)
    bits_a = np.array(bits_l, np.int32)
    glen = np.array(dt, np.int32)
    codes = np.zeros(xs.shape, np.int8)
    scales = np.zeros(len(xs), np.float32)
    for i in range(len(xs)):
        c, s = codec.quantize_group(xs[i, :glen[i]], int(bits_a[i]))
        codes[i, :glen[i]] = c
        scales[i] = s
    np.savez(os.path.join(HERE, "adversarial_groups.npz"), x=xs, bits=bits_a,
             group_len=glen, codes=codes, scales=scales)
    print(f"{len(xs)} groups written")


if __name__ == "__main__":
    main()
