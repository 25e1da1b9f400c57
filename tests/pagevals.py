"""Page values from tests/golden as exact fractions, plus the three-token Markov
example of the rayaq.ca page turned into logits (log-probabilities)."""
import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOK = {"a": 0, "b": 1, "c": 2}


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def frac_rows(table):
    return {k: [Fraction(x) for x in v] for k, v in table.items()}


MARKOV = load("markov_3token.json")
ROUNDS = load("markov_rounds.json")
P = frac_rows(MARKOV["target_p"])
Q = frac_rows(MARKOV["draft_q"])
# float64 matrices indexed [previous token, next token]
P_MAT = np.array([[float(x) for x in P[t]] for t in "abc"])
Q_MAT = np.array([[float(x) for x in Q[t]] for t in "abc"])
LOGP = np.log(P_MAT)
LOGQ = np.log(Q_MAT)
