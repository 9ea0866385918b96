"""Write workload_counts.json from the oracle alone.

Run from the repository root: ``python tests/golden/make_golden.py``.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    doc = {"written_by": "tests/golden/make_golden.py (calls oracle.partition_index and oracle.pair_counts only)",
           "workloads": {}}
    for num, w in sorted(workloads.WORKLOADS.items()):
        ranks = {}
        for r in range(w.cp_size):
            idx, cu_rows = oracle.partition_index(w.seq_len, w.n_img_array, w.cu_seqlens, w.cp_size, r)
            padded, real = oracle.pair_counts(w.seq_len, w.n_img_array, w.cu_seqlens, w.cp_size, r)
            ranks[str(r)] = {"rows": int(len(idx)), "pads": int((idx < 0).sum()),
                             "pairs_padded": padded, "pairs_real": real,
                             "cu_rows": [int(x) for x in cu_rows]}
        doc["workloads"][str(num)] = {"name": w.name, "seq_len": w.seq_len,
                                      "cu_seqlens": [int(x) for x in w.cu_seqlens],
                                      "n_img": [int(x) for x in w.n_img], "cp_size": w.cp_size,
                                      "ranks": ranks}
    with open(os.path.join(HERE, "workload_counts.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
