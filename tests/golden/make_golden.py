"""Write the oracle regression snapshot ``c1_rows.json``.

The pages ("MiniPIC: Flexible Position-Independent Caching in <100LOC") print
no worked numeric example of the attention output, so no fixture here carries
the pages' own numbers. This snapshot holds oracle outputs for a few rows of
the tiny fp32 workload (2 SSep spans of 32 tokens and a 16-token PDep question,
§3.3.1 layout); it calls nothing but ``workload`` and ``oracle``. It guards
the oracle against silent changes: regenerate it only together with a change
to the oracle's arithmetic whose commit message names the passage behind it.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workload  # noqa: E402

ROWS = [0, 1, 31, 32, 47, 63, 64, 79]


def main():
    w = workload.make_config("c1")
    out = oracle.workload_reference(w, 0, rows=np.array(ROWS))
    doc = {
        "workload": "c1 (seed 1): fp32, Hq 4, Hkv 2, d 64, theta 1e4, spans 32+32 SSep + 16 PDep",
        "source": "oracle.workload_reference via tests/golden/make_golden.py",
        "rows": ROWS,
        "out_head0_first8": [[float(x) for x in out[i, 0, :8]] for i in range(len(ROWS))],
        "out_sum_per_row": [float(out[i].sum()) for i in range(len(ROWS))],
    }
    with open(os.path.join(HERE, "c1_rows.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
