"""40-digit Decimal brute force of decode attention (TEST INFRASTRUCTURE).

An independent evaluation of the same definition as oracle.reference, for tiny
shapes only: every product, sum and exponential is taken in Python's decimal
module (precision 40) from the exact decimal expansion of each float64 input.
It pins the float64 oracle: the two must agree to about 1e-13.

Definition (decode-long page, "Local attention" and "Final normalise +
store"): out = sum_t exp(x_t - M) v_t / sum_t exp(x_t - M),
x_t = scale * sum_d q_d k_{t,d}, M = max_t x_t.
"""
from __future__ import annotations

from decimal import Decimal, localcontext
from typing import List, Sequence


def attend_decimal(q: Sequence[float], K: Sequence[Sequence[float]],
                   V: Sequence[Sequence[float]], scale: float) -> List[float]:
    """Brute-force softmax(scale * q K^T) V for one query row, rounded to float."""
    with localcontext() as ctx:
        ctx.prec = 40
        sc = Decimal(float(scale))
        qd = [Decimal(float(a)) for a in q]
        xs = []
        for row in K:
            acc = Decimal(0)
            for a, b in zip(qd, row):
                acc += a * Decimal(float(b))
            xs.append(sc * acc)
        if not xs:
            return [0.0] * (len(V[0]) if V else len(q))
        M = max(xs)
        es = [(x - M).exp() for x in xs]
        den = sum(es, Decimal(0))
        d = len(V[0])
        out = []
        for c in range(d):
            num = Decimal(0)
            for e, row in zip(es, V):
                num += e * Decimal(float(row[c]))
            out.append(float(num / den))
        return out
