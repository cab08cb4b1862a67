"""Helpers shared by the GPU parity tests: device transfer and the tolerance
checks (max abs error on O and LSE; -inf LSE entries must agree exactly and
are left out of the max)."""
import sys

import numpy as np
import torch

TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-5, 1e-5)}
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype):
    """float32 numpy array (already representable in dtype) -> device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        TDT[dtype]).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_o_lse(o, lse, o_ref, lse_ref, dtype, what=""):
    """o, lse: GPU results as float64 numpy; refs from the oracle (NaN =
    not computed)."""
    tol_o, tol_l = TOL[dtype]
    sel = ~np.isnan(lse_ref)
    ninf_ref = np.isneginf(lse_ref) & sel
    ninf = np.isneginf(lse) & sel
    assert np.array_equal(ninf, ninf_ref), f"{what}: -inf LSE rows differ"
    fin = sel & ~ninf_ref
    assert np.all(np.isfinite(lse[fin])), f"{what}: non-finite LSE"
    err_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]), initial=0.0))
    osel = ~np.isnan(o_ref)
    assert np.all(np.isfinite(o[osel])), f"{what}: non-finite O"
    err_o = float(np.max(np.abs(o[osel] - o_ref[osel]), initial=0.0))
    say(f"  {what}: max|dO| = {err_o:.3e} (tol {tol_o}), "
        f"max|dLSE| = {err_l:.3e} (tol {tol_l})")
    assert err_o <= tol_o, f"{what}: O error {err_o} > {tol_o}"
    assert err_l <= tol_l, f"{what}: LSE error {err_l} > {tol_l}"
    return err_o, err_l
