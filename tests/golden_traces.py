"""Parser for tests/golden/commit_traces.txt (hand-worked commit traces)."""
import math
import os
from dataclasses import dataclass, field
from typing import List

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "commit_traces.txt")


@dataclass
class Trace:
    name: str
    V: int
    mask_id: int
    S: int
    T: int
    gamma: float
    logits: np.ndarray = None
    init_tokens: List[int] = None
    init_bits: int = 0
    steps: list = field(default_factory=list)


def _delta(s: str) -> float:
    if s.startswith("ln"):
        return math.log(float(s[2:]))
    return float(s)


def load() -> List[Trace]:
    traces, cur = [], None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = line.split()
            if w[0] == "trace":
                cur = Trace(w[1], int(w[3]), int(w[5]), int(w[7]), int(w[9]), float(w[11]))
                cur.logits = np.zeros((cur.S, cur.V), dtype=np.float32)
            elif w[0] == "row":
                pos, tok = int(w[1]), int(w[2])
                if w[3] == "nan":
                    cur.logits[pos, :] = np.nan
                else:
                    cur.logits[pos, tok] = np.float32(_delta(w[3]))
            elif w[0] == "init":
                i = w.index("bits")
                cur.init_tokens = [int(x) for x in w[1:i]]
                cur.init_bits = int(w[i + 1])
            elif w[0] == "step":
                t = int(w[1])
                com = [] if w[3] == "-" else [int(x) for x in w[3].split(",")]
                i_b = w.index("bits")
                toks = [int(x) for x in w[5:i_b]]
                bits = int(w[i_b + 1])
                n = int(w[i_b + 3])
                cur.steps.append(dict(step=t, commit=com, tokens=toks, bits=bits, n=n))
            elif w[0] == "end":
                traces.append(cur)
                cur = None
    return traces
