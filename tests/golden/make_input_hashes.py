"""Writes input_sha256.json: sha256 of the fp16 bytes each seeded workload
generator produces (the generator-determinism pin).  Calls only workloads.py;
no value here comes from the HIP path or the oracle.

Run from the repository root:  python tests/golden/make_input_hashes.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import workloads  # noqa: E402


def hashes():
    out = {}
    for name, w in workloads.WORKLOADS.items():
        if isinstance(w, workloads.GemmWorkload):
            A, Bt, C = workloads.gemm_inputs(w)
            out[name] = {"A": workloads.sha256(A), "Bt": workloads.sha256(Bt),
                         "C": workloads.sha256(C)}
        else:
            A, B = workloads.trmm_inputs(w)
            out[name] = {"A_cm": workloads.sha256(A), "B_cm": workloads.sha256(B)}
        ri, cj = workloads.sample_indices(w.seed, 8192, 8192)
        out[name]["samples_8192"] = workloads.sha256(ri) + workloads.sha256(cj)[:16]
    for name, w in workloads.TRSM_WORKLOADS.items():
        A, B = workloads.trsm_inputs(w)
        out[name] = {"A_cm": workloads.sha256(A), "B_cm": workloads.sha256(B)}
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_sha256.json")
    with open(path, "w") as f:
        json.dump(hashes(), f, indent=1, sort_keys=True)
    print("wrote", path)
