"""Parser for the hand-written dequantisation fixtures in this folder."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load_dequant_fixture(name: str):
    meta, rows_bytes, scales, biases, expect = {}, {}, {}, {}, []
    with open(os.path.join(HERE, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] in ("bits", "cols", "group", "rows"):
                meta[tok[0]] = int(tok[1])
            elif tok[0] == "bytes":
                rows_bytes[int(tok[1])] = {int(k): int(v, 16) for k, v in (t.split("=") for t in tok[2:])}
            elif tok[0] in ("scale", "bias"):
                d = scales if tok[0] == "scale" else biases
                d[(int(tok[1]), int(tok[2]))] = (int(tok[3], 16), float(tok[4]))
            elif tok[0] == "expect":
                expect.append((int(tok[1]), int(tok[2]), float(tok[3])))
    bits, cols, group, rows = meta["bits"], meta["cols"], meta["group"], meta["rows"]
    codes = np.zeros((rows, cols * bits // 8), np.uint8)
    for r, d in rows_bytes.items():
        for j, v in d.items():
            codes[r, j] = v
    ng = cols // group
    sc = np.zeros((rows, ng), np.uint16)
    bi = np.zeros((rows, ng), np.uint16)
    sc_val = np.zeros((rows, ng))
    bi_val = np.zeros((rows, ng))
    for (r, g), (b, v) in scales.items():
        sc[r, g], sc_val[r, g] = b, v
    for (r, g), (b, v) in biases.items():
        bi[r, g], bi_val[r, g] = b, v
    return dict(bits=bits, cols=cols, group=group, rows=rows, codes=codes, scales=sc, biases=bi,
                scale_values=sc_val, bias_values=bi_val, expect=expect)
