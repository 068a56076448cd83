"""Writes adamw_order.json: single AdamW elements whose result bits depend on
the order of operations, evaluated exactly as the page's code writes them.

Source: "ZeRO and FSDP sharding" (tirogla.com), section Code, the AdamW step.
Its three update lines, read with Rust's rules (binary32 arithmetic, `*` and
`/` of equal precedence and left-associative, one rounding per operation, no
fused multiply-add), fix one bit pattern per element:

  m <- b1*m + (1-b1)*g                          = fl(fl(b1 m) + fl(omb1 g))
  v <- b2*v + (1-b2)*g*g                        = fl(fl(b2 v) + fl(fl(omb2 g) g))
  w <- w*(1 - lr*wd) - lr/bc1*m/(sqrt(v)/bc2 + eps)
                      = fl(fl(w decay) - fl(fl(a m) / fl(fl(sqrt(v) / bc2) + eps)))

with bc1 = 1 - b1^t and bc2 = sqrt(1 - b2^t) (the same section), the powers
taken as running binary32 products (the repository's reading of `powi`),
omb = fl(1 - b), a = fl(lr / bc1) and decay = fl(1 - fl(lr wd)): the page
writes `lr / bc1` and `1.0 - lr * wd` inside the element expression, and
these are the same binary32 values for every element.

Each case is chosen so that at least one alternative association that a
careless implementation might use gives different bits:

  v_assoc      (1-b2) * (g*g)            instead of ((1-b2)*g)*g
  u_assoc      (lr/bc1) * (m / den)      instead of ((lr/bc1)*m) / den
  den_recip    sqrt(v) * (1/bc2)         instead of sqrt(v) / bc2
  den_sqrt     sqrt(v / (bc2*bc2))       instead of sqrt(v) / bc2

The evaluation uses tests/f32exact.py (exact rationals, one IEEE rounding per
operation); it calls neither the oracle nor the library.  Run from the
repository root:  python tests/golden/make_adamw_order.py
"""
from __future__ import annotations

import json
import os
import random
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import f32exact as F  # noqa: E402

ONE = F.from_decimal("1")

# (lr, b1, b2, eps, wd) as decimal literals: the page's toy, the GPT-scale
# optimizer of "ZeRO: Three Ledgers" (lr 3e-4, betas 0.9 / 0.95, wd 0.1, eps
# of the page's code) and two sets that make eps and the betas matter more.
HYPERS = [
    ("0.01", "0.9", "0.95", "1e-8", "0.1"),
    ("3e-4", "0.9", "0.95", "1e-8", "0.1"),
    ("1e-3", "0.8", "0.99", "5e-4", "0.5"),
    ("2e-3", "0.5", "0.9", "1e-6", "2.0"),
]

ALTS = ("v_assoc", "u_assoc", "den_recip", "den_sqrt")


def scalars(t, lr, b1, b2, wd):
    p1 = p2 = ONE
    for _ in range(t):
        p1 = F.mul(p1, b1)
        p2 = F.mul(p2, b2)
    bc1 = F.sub(ONE, p1)
    bc2 = F.sqrt(F.sub(ONE, p2))
    return dict(omb1=F.sub(ONE, b1), omb2=F.sub(ONE, b2), bc1=bc1, bc2=bc2,
                a=F.div(lr, bc1), decay=F.sub(ONE, F.mul(lr, wd)))


def element(w, m, v, g, h, s, alt=None):
    """One AdamW element; alt selects one wrong association."""
    m1 = F.add(F.mul(h["b1"], m), F.mul(s["omb1"], g))
    if alt == "v_assoc":
        v_inc = F.mul(s["omb2"], F.mul(g, g))
    else:
        v_inc = F.mul(F.mul(s["omb2"], g), g)
    v1 = F.add(F.mul(h["b2"], v), v_inc)
    if alt == "den_recip":
        scaled = F.mul(F.sqrt(v1), F.div(ONE, s["bc2"]))
    elif alt == "den_sqrt":
        scaled = F.sqrt(F.div(v1, F.mul(s["bc2"], s["bc2"])))
    else:
        scaled = F.div(F.sqrt(v1), s["bc2"])
    den = F.add(scaled, h["eps"])
    if alt == "u_assoc":
        u = F.mul(s["a"], F.div(m1, den))
    else:
        u = F.div(F.mul(s["a"], m1), den)
    w1 = F.sub(F.mul(w, s["decay"]), u)
    return m1, v1, w1


def draw(rng):
    """A state and gradient of the magnitudes a training run has: w ~ 0.02,
    gradients ~ 1e-3 spread over a few decades, moments consistent with them."""
    gs = 1e-3 * 10 ** rng.uniform(-2, 1)
    g = rng.gauss(0, gs)
    m = rng.gauss(0, gs * 0.5)
    v = (gs * rng.uniform(0.05, 2.0)) ** 2
    w = rng.gauss(0, 0.02)
    return [F.encode_float(x) for x in (w, m, v, g)]


def main():
    rng = random.Random(20240611)
    cases = []
    want = {a: 10 for a in ALTS}
    plain = 10
    tries = 0
    while (any(want.values()) or plain) and tries < 200000:
        tries += 1
        hp = HYPERS[rng.randrange(len(HYPERS))]
        t = rng.randint(1, 20)
        lr, b1, b2, eps, wd = (F.from_decimal(x) for x in hp)
        h = dict(b1=b1, b2=b2, eps=eps)
        s = scalars(t, lr, b1, b2, wd)
        w, m, v, g = draw(rng)
        good = element(w, m, v, g, h, s)
        differs = [a for a in ALTS if element(w, m, v, g, h, s, a) != good]
        keep = any(want[a] > 0 for a in differs) or (plain > 0 and not differs)
        if not keep:
            continue
        for a in differs:
            want[a] = max(0, want[a] - 1)
        if not differs:
            plain -= 1
        cases.append(dict(
            hyper=dict(zip(("lr", "b1", "b2", "eps", "wd"), hp)), t=t,
            w=f"{w:08x}", m=f"{m:08x}", v=f"{v:08x}", g=f"{g:08x}",
            expect=dict(m=f"{good[0]:08x}", v=f"{good[1]:08x}", w=f"{good[2]:08x}"),
            alternatives_that_differ=differs))
    assert not any(want.values()) and not plain, (want, plain)
    doc = dict(
        cite="ZeRO and FSDP sharding (tirogla.com), section Code: the AdamW step "
             "(update lines for m, v and w; bias corrections 1 - b1^t, sqrt(1 - b2^t))",
        reading="binary32, one rounding per operation, Rust's left-to-right association; "
                "b^t as running binary32 products; omb = 1 - b, lr/bc1 and 1 - lr*wd in binary32",
        generator="tests/golden/make_adamw_order.py (exact rationals, tests/f32exact.py)",
        fields="bit patterns as hex; hyper as the page's decimal literals, rounded to binary32",
        cases=cases)
    out = os.path.join(HERE, "adamw_order.json")
    with open(out, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"{len(cases)} cases after {tries} draws -> {out}")


if __name__ == "__main__":
    main()
