"""Writes tests/golden/bf16_envelope.json: the inherent bf16 envelope of the
end-to-end taps ln_av, z and branch on every bf16 case the GPU parity tests
compare with the oracle (tests/bf16_envelope.py defines the envelope and the
cases).  Calls only the float64 oracle.

    python tests/golden/make_bf16_envelope.py [--jobs N]
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))


def _one(job):
    import bf16_envelope as E
    from edge_workloads import edge_workload
    kind, key, arg = job
    t0 = time.time()
    if kind == "full":
        w, seqs = E.load_full_size_case(key)
        sub = w.sub_batch(seqs)
        env = E.envelope(sub)
        info = {"sequences": seqs, "rows": int(sub.T)}
    else:
        ekind, flags = arg
        w = edge_workload(ekind, **flags)
        env = E.envelope(w)
        info = {"rows": int(w.T)}
    info.update({t: float(env[t]) for t in E.TAPS})
    return key, info, time.time() - t0


def jobs():
    import bf16_envelope as E
    out = [("full", key, None) for key, _, _, _ in E.full_size_cases()]
    for ekind in ("bf16", "bf16_s1"):
        for fname, flags in E.EDGE_FLAGS:
            out.append(("edge", E.edge_key(ekind, fname), (ekind, flags)))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    a = ap.parse_args()
    import bf16_envelope as E
    cases = {}
    with cf.ProcessPoolExecutor(max_workers=a.jobs) as ex:
        for key, info, dt in ex.map(_one, jobs()):
            print(f"{key}: " + ", ".join(f"{t} {info[t]:.4e}" for t in E.TAPS) + f"  ({dt:.1f} s)",
                  flush=True)
            cases[key] = info
    doc = {
        "what": "max |tap_bf16 - tap_exact| / rms(tap_exact) of the float64 oracle with u, v, q, k, "
                "the attention's pointwise weights, z and the branch rounded to bf16 inside it "
                "(tests/bf16_envelope.py); the GPU tests allow this plus "
                f"{E.MARGIN}",
        "generator": "tests/golden/make_bf16_envelope.py",
        "cases": dict(sorted(cases.items())),
    }
    with open(E.ENVELOPE_FILE, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"wrote {E.ENVELOPE_FILE}")


if __name__ == "__main__":
    main()
