"""Hand derivation of the LAMB worked examples in 40-digit decimal arithmetic.

Writes lamb_worked.json.  This is an independent derivation of a few-element
case step by step (it does not call the oracle); the JSON keeps every
intermediate so that a reader can check each number by eye.

Method: LAMB (You et al. 2020), the optimizer named in the LAMB row of the
MegaScale study guide, ch.2 §2.2 (paper §3.1) technique table.  Hyper-parameters
as in the layer workloads: lr 1e-3, beta1 0.9, beta2 0.999, eps 1e-6, wd 0.01.
"""
import decimal
import json
import os
from decimal import Decimal as D

decimal.getcontext().prec = 40
B1, B2, EPS, LR, WD = D("0.9"), D("0.999"), D("1e-6"), D("1e-3"), D("0.01")


def step(w, g, m, v, t):
    m = [B1 * a + (1 - B1) * b for a, b in zip(m, g)]
    v = [B2 * a + (1 - B2) * b * b for a, b in zip(v, g)]
    mh = [a / (1 - B1 ** t) for a in m]
    vh = [a / (1 - B2 ** t) for a in v]
    u = [a / (b.sqrt() + EPS) + WD * c for a, b, c in zip(mh, vh, w)]
    wn = sum(a * a for a in w).sqrt()
    un = sum(a * a for a in u).sqrt()
    r = wn / un if (wn > 0 and un > 0) else D(1)
    w_new = [a - LR * r * b for a, b in zip(w, u)]
    return dict(m=m, v=v, m_hat=mh, v_hat=vh, u=u, w_norm=wn, u_norm=un, ratio=r, w=w_new)


def s(x):
    return [str(a) for a in x] if isinstance(x, list) else str(x)


def main():
    cases = []
    w0, g1 = [D(3), D(4)], [D("0.5"), D("-0.25")]
    z = [D(0), D(0)]
    r1 = step(w0, g1, z, z, 1)
    g2 = [D("-0.5"), D("0.5")]
    r2 = step(r1["w"], g2, r1["m"], r1["v"], 2)
    cases.append(dict(name="two_steps", w0=s(w0), grads=[s(g1), s(g2)],
                      steps=[{k: s(v) for k, v in r1.items()}, {k: s(v) for k, v in r2.items()}]))
    g = [D(1), D(-1)]
    r0 = step(z, g, z, z, 1)
    cases.append(dict(name="zero_weight_norm", w0=s(z), grads=[s(g)],
                      steps=[{k: s(v) for k, v in r0.items()}]))
    doc = dict(source="LAMB (You et al. 2020) as named by the MegaScale study guide, "
                      "ch.2 sec.2.2 technique table, LAMB row; derived in 40-digit decimal",
               hparams=dict(lr="1e-3", beta1="0.9", beta2="0.999", eps="1e-6", weight_decay="0.01"),
               cases=cases)
    with open(os.path.join(os.path.dirname(__file__), "lamb_worked.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
