"""Write tests/golden/tiny_exact.json: exact rational outputs of the HGRN2
recurrence on one tiny hand-chosen input.

The pages print no worked example, so this fixture is produced by the exact
rational oracle (``oracle.exact``) and nothing else.  Run from the repository
root:  python tests/golden/make_golden.py
"""
import json
import os
import sys
from fractions import Fraction as F

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "..", ".."))
from oracle import exact  # noqa: E402

# T = 5 tokens, d_k = 3 decay channels, d_v = 2 value columns.  Gates f are
# rationals in [0, 1] with one exact zero (a full reset of one channel) and one
# exact one (no decay); k = 1 - f as in HGRN2's tied input gate.
f = [[F(1, 2), F(3, 4), F(1, 1)],
     [F(2, 3), F(0, 1), F(1, 5)],
     [F(7, 8), F(1, 3), F(1, 1)],
     [F(1, 4), F(5, 6), F(2, 7)],
     [F(9, 10), F(1, 2), F(3, 5)]]
k = [[1 - x for x in row] for row in f]
q = [[F(1), F(-2), F(1, 3)],
     [F(3, 2), F(1, 4), F(-1)],
     [F(-1, 2), F(2), F(5, 4)],
     [F(2, 3), F(-3, 4), F(1)],
     [F(1, 5), F(1, 2), F(-2)]]
v = [[F(2), F(-1)],
     [F(1, 3), F(4)],
     [F(-3, 2), F(1, 2)],
     [F(5), F(-2, 3)],
     [F(-1, 4), F(3)]]
h0 = [[F(1, 7), F(-2)], [F(0), F(1, 2)], [F(3), F(-1, 9)]]
dy = [[F(1), F(1, 2)],
      [F(-2), F(3)],
      [F(1, 3), F(-1)],
      [F(2), F(2)],
      [F(-1, 2), F(1, 4)]]
dht = [[F(1), F(0)], [F(-1, 2), F(2)], [F(1, 3), F(1)]]

y, ST = exact.forward(q, k, v, f, h0)
dq, dk, dv, df, dh0 = exact.backward(q, k, v, f, dy, h0, dht)
dlogf = [[f[t][c] * df[t][c] for c in range(3)] for t in range(5)]


def enc(m):
    return [[str(x) for x in row] for row in m]


out = {
    "about": "exact rational HGRN2 recurrence; inputs chosen by hand; written by "
             "tests/golden/make_golden.py from oracle.exact",
    "citation": "HGRN2: Gated Linear RNNs with State Expansion (paperlayer.ai summary), "
                "§3.2 (outer-product state, diagonal forget gate, matrix-vector readout); "
                "§2.1 (input gate tied as one minus the forget gate)",
    "f": enc(f), "k": enc(k), "q": enc(q), "v": enc(v), "h0": enc(h0), "dy": enc(dy),
    "dht": enc(dht),
    "y": enc(y), "ht": enc(ST), "dq": enc(dq), "dk": enc(dk), "dv": enc(dv),
    "dlog_f": enc(dlogf), "dh0": enc(dh0),
}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_exact.json")
with open(path, "w") as fh:
    json.dump(out, fh, indent=1)
print("wrote", path)
