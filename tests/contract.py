"""Parity checks shared by the tests (test infrastructure).

Floating-point attention outputs are compared with the fp64 oracle
elementwise in allclose form:  |gpu - ref| <= ATOL + RTOL * |ref|  with
ATOL = 2e-3 and RTOL = 1e-2 (bf16 storage, fp32 accumulation).  Because decode
outputs shrink like 1/sqrt(length), that bound alone would let a near-zero
output pass on long contexts, so every comparison also requires the scaled
error  max|gpu - ref| / max|ref|  to stay at or below SCALED (1e-2).
Integer and byte results are compared bit for bit.
"""

import numpy as np

ATOL = 2e-3
RTOL = 1e-2
SCALED = 1e-2


def contract_report(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise AssertionError(f"shape {got.shape} != {ref.shape}")
    err = np.abs(got - ref)
    finite = bool(np.all(np.isfinite(got)))
    bound_ok = bool(np.all(err <= ATOL + RTOL * np.abs(ref))) if finite else False
    max_ref = float(np.max(np.abs(ref))) if ref.size else 0.0
    max_err = float(np.max(err)) if err.size else 0.0
    scaled = max_err / max_ref if max_ref > 0 else max_err
    return {"finite": finite, "bound_ok": bound_ok, "max_err": max_err,
            "max_ref": max_ref, "scaled": scaled,
            "ok": finite and bound_ok and scaled <= SCALED}


def assert_contract(got, ref, what=""):
    rep = contract_report(got, ref)
    if not rep["ok"]:
        raise AssertionError(f"{what}: parity failed {rep}")
    return rep
