"""Turn the parity record the GPU tests write (MLA_PARITY_RECORD=<file>.jsonl, one JSON line per
check) into a markdown table: raw max-abs and RMSE, the scale-normalised figures, the LSE relative
error and the slack left under the per-element bar |gpu - ref| <= 1e-2 + 2^-8 (|ref| + sum p|v|).

    python tests/parity_record_summary.py record.jsonl > summary.md
"""
from __future__ import annotations

import json
import sys


def main(path: str) -> None:
    rows = [json.loads(line) for line in open(path)]
    print("| check | O max-abs | O RMSE | max-abs / max(1, max|O|) | RMSE / max(1, rms O) | LSE rel | per-element slack |")
    print("|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['case']} | {r['maxabs']:.2e} | {r['rmse']:.2e} | {r['maxabs_norm']:.2e} | {r['rmse_norm']:.2e} | "
              f"{r['lse_rel']:.1e} | {-r['elem_excess']:.2e} |")
    print()
    print(f"{len(rows)} checks; largest raw O max-abs {max(r['maxabs'] for r in rows):.3e}; smallest per-element "
          f"slack {min(-r['elem_excess'] for r in rows):.3e}")


if __name__ == "__main__":
    main(sys.argv[1])
