"""Writes closed_forms.json: small attention and unmask cases whose exact
answers follow from closed forms, evaluated in 50-digit mpmath.

The pages print no worked numerical example for either operation, so these
fixtures are derived from the mathematics of the definitions instead:
* two visible keys: the softmax weights are logistic(s1 - s2);
* a constant logit row of size V: confidence 1/V, argmax id 0;
* one spike Delta above a constant row: confidence 1/(1 + (V-1) e^-Delta);
* two equal spikes: confidence 1/(2 + (V-2) e^-Delta), argmax the lower id.

This script uses mpmath only; it imports neither the oracle nor the HIP
library.  Run:  python tests/golden/make_golden.py
"""
import json
import os

import mpmath as mp

mp.mp.dps = 50


def f(x):
    return float(x)


def two_key_case(q, k1, k2, v1, v2, scale):
    s1 = scale * sum(mp.mpf(a) * b for a, b in zip(q, k1))
    s2 = scale * sum(mp.mpf(a) * b for a, b in zip(q, k2))
    w1 = 1 / (1 + mp.e ** (s2 - s1))
    w2 = 1 - w1
    out = [w1 * a + w2 * b for a, b in zip(v1, v2)]
    lse = mp.log(mp.e ** s1 + mp.e ** s2)
    return dict(q=q, k1=k1, k2=k2, v1=v1, v2=v2, scale=scale, w1=f(w1), out=[f(o) for o in out],
                lse=f(lse))


def main():
    cases = {
        "attention_two_keys": [
            # P=1 prefix row (k1, v1) and L=1 block row (k2, v2); one query.
            two_key_case([1.0, 0.0], [2.0, 0.0], [0.0, 0.0], [1.0, 0.0], [0.0, 1.0], 1.0),
            two_key_case([0.5, -1.0, 2.0], [1.0, 1.0, 1.0], [-1.0, 0.5, 0.25],
                         [3.0, -2.0, 0.5], [-1.0, 4.0, 2.0], 0.5),
        ],
        "unmask_rows": [],
    }
    V = 1000
    cases["unmask_rows"].append(dict(kind="constant", V=V, value=0.75, argmax=0,
                                     conf=f(mp.mpf(1) / V)))
    for delta, pos in [(2.0, 17), (8.0, 999), (0.5, 0)]:
        c = 1 / (1 + (V - 1) * mp.e ** (-mp.mpf(delta)))
        cases["unmask_rows"].append(dict(kind="spike", V=V, base=-1.0, delta=delta, pos=pos,
                                         argmax=pos, conf=f(c)))
    for delta, p1, p2 in [(3.0, 40, 7), (1.0, 500, 501)]:
        c = 1 / (2 + (V - 2) * mp.e ** (-mp.mpf(delta)))
        cases["unmask_rows"].append(dict(kind="two_spikes", V=V, base=0.0, delta=delta,
                                         pos=[p1, p2], argmax=min(p1, p2), conf=f(c)))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "closed_forms.json")
    with open(path, "w") as fh:
        json.dump(cases, fh, indent=1)
        fh.write("\n")


if __name__ == "__main__":
    main()
