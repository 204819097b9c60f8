"""Agreement measures between a GPU result and the float64 oracle.

Test infrastructure.  The relative L2 measure is the one the cudnn-frontend SwiGLU
sample prints for its forward and gradients (gemm_swiglu_mlp_fusion.py, _demo):
||a - b|| / max(||b||, 1e-9).  The thresholds are this library's acceptance bar:
  * half-precision outputs: rel-L2 <= 1e-2 and |err| <= 2e-2 (|ref| + rms(ref))
    elementwise, rms over the compared set;
  * relu_aux: bit-exact except where |pre-activation| < 1e-3 rms(pre-activation),
    where float32 accumulation order may flip a sign;
  * bgrad (float32): rel-L2 <= 5e-3.
"""
import numpy as np

from .core import unpack_relu_mask

TOL = {
    "half_rel_l2": 1e-2,
    "half_elem": 2e-2,
    "mask_band": 1e-3,
    "bgrad_rel_l2": 5e-3,
}


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-9))


def _rms(x):
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def check_half_output(x, ref, rel_tol=None, elem_tol=None):
    """Tolerance check for an fp16/bf16 output (already decoded to float64)."""
    rel_tol = TOL["half_rel_l2"] if rel_tol is None else rel_tol
    elem_tol = TOL["half_elem"] if elem_tol is None else elem_tol
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        return False, {"error": f"shape {x.shape} != {ref.shape}"}
    if x.size == 0:
        return True, {"rel_l2": 0.0, "max_excess": 0.0}
    err = np.abs(x - ref)
    bound = elem_tol * (np.abs(ref) + _rms(ref))
    rel = rel_l2(x, ref)
    elem_ok = bool(np.all(err <= bound))  # NaN compares False
    excess = float(np.nanmax(err / np.maximum(bound, 1e-300))) if np.isfinite(err).all() else float("inf")
    ok = elem_ok and rel <= rel_tol
    return ok, {"rel_l2": rel, "max_err_over_bound": excess, "n": int(x.size)}


def check_mask(words, p_ref, ld_aux=None, band=None):
    """relu_aux check: bits against (p_ref > 0), exempting |p_ref| < band * rms(p_ref).

    Also requires the unused tail bits of each row's last word to be zero.
    """
    band = TOL["mask_band"] if band is None else band
    words = np.asarray(words, dtype=np.uint32)
    p_ref = np.asarray(p_ref, dtype=np.float64)
    m, n = p_ref.shape
    nw = (n + 31) // 32
    got = unpack_relu_mask(words, n)
    want = p_ref > 0.0
    exempt = np.abs(p_ref) < band * _rms(p_ref)
    bad = (got != want) & ~exempt
    tail_ok = True
    if n % 32:
        tail_bits = words[:, nw - 1] >> np.uint32(n % 32)
        tail_ok = bool(np.all(tail_bits == 0))
    info = {
        "mismatch": int(bad.sum()),
        "differ_in_band": int(((got != want) & exempt).sum()),
        "exempt": int(exempt.sum()),
        "tail_ok": tail_ok,
    }
    return (info["mismatch"] == 0 and tail_ok), info


def check_bgrad(x, ref, rel_tol=None):
    rel_tol = TOL["bgrad_rel_l2"] if rel_tol is None else rel_tol
    rel = rel_l2(x, ref)
    return rel <= rel_tol, {"rel_l2": rel}
