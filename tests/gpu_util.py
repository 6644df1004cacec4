"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import pytest
import torch

from synth import bf16_bits_from_f32, from_storage

# Tolerances.  Floats: max-abs 2e-2 for bf16 storage (bf16 in, fp32
# accumulate) and 1e-5 for fp32 storage, on m, c, lse, O, Z and S; in addition
# the relative Frobenius error of O and S must stay below 1e-2 (bf16) / 1e-6
# (fp32), because O and S are small (a max-abs bound alone would accept 0).
ATOL = {"bf16": 2e-2, "f32": 1e-5}
RELF = {"bf16": 1e-2, "f32": 1e-6}
# Integers are exact except: argmax where the oracle's top-2 logit gap is below
# 1e-3 * max(1, |m|) (near-ties), and renoise where |c - tau| < 1e-3.
TIE_GAP = 1e-3
TAU_BAND = 1e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def dev(a):
    import uniform_state_discrete_amd as dg
    return dg.to_device(a)


def f64(t):
    """device tensor -> float64 numpy"""
    return t.float().cpu().numpy().astype(np.float64)


def stored(x, dtype):
    """float array -> stored form (uint16 bf16 bits or float32)"""
    x = np.asarray(x, np.float32)
    return bf16_bits_from_f32(x) if dtype == "bf16" else x


def as_f64(a, dtype):
    return from_storage(a, dtype).astype(np.float64)


def close(name, got, ref, atol, relf=None, bf16_ulp=False):
    """max |got - ref| <= atol (elementwise bound max(atol, one bf16 ulp of
    |ref|) when bf16_ulp: for a bf16-stored tensor above 2.56 in magnitude a
    single rounding step exceeds 2e-2), plus an optional relative Frobenius
    bound."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    diff = np.abs(got - ref)
    bound = np.maximum(atol, np.abs(ref) * 2.0 ** -7) if bf16_ulp else atol
    err = float(diff.max()) if got.size else 0.0
    worst = float((diff / bound).max()) if got.size else 0.0
    fro = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)) if got.size else 0.0
    say(f"{name}: max-abs {err:.3e} (tol {atol:.1e}{' or 1 ulp' if bf16_ulp else ''}) rel-fro {fro:.3e}" +
        (f" (tol {relf:.1e})" if relf else ""))
    assert worst <= 1.0, f"{name}: max-abs {err} exceeds the bound (worst ratio {worst:.3f})"
    if relf is not None:
        assert fro <= relf, f"{name}: rel-fro {fro} > {relf}"
    return err, fro


def close_rel(name, got, ref, ulps_rel):
    """max-abs bound scaled by the tensor's magnitude (for intermediates)."""
    ref = np.asarray(ref, np.float64)
    return close(name, got, ref, ulps_rel * max(1.0, float(np.abs(ref).max())))


def argmax_match(name, got, ref, gap, m):
    got = np.asarray(got).reshape(-1)
    ref = np.asarray(ref).reshape(-1)
    tie = np.asarray(gap).reshape(-1) < TIE_GAP * np.maximum(1.0, np.abs(np.asarray(m).reshape(-1)))
    bad = (got != ref) & ~tie
    say(f"{name}: {int(bad.sum())} mismatches, {int(tie.sum())} near-ties excluded of {got.size}")
    assert not bad.any(), f"{name}: argmax mismatch at {np.nonzero(bad)[0][:10]}"
    return int(tie.sum())


def renoise_match(name, got_x, got_mask, ref_x, ref_mask, ref_c, tau, extra_excl=None):
    got_x = np.asarray(got_x).reshape(-1)
    ref_x = np.asarray(ref_x).reshape(-1)
    got_mask = np.asarray(got_mask).reshape(-1)
    ref_mask = np.asarray(ref_mask).reshape(-1)
    band = np.abs(np.asarray(ref_c).reshape(-1) - float(np.float32(tau))) < TAU_BAND
    if extra_excl is not None:
        band = band | np.asarray(extra_excl).reshape(-1)
    bad_m = (got_mask != ref_mask) & ~band
    bad_x = (got_x != ref_x) & ~band
    say(f"{name}: mask mismatches {int(bad_m.sum())}, token mismatches {int(bad_x.sum())}, "
        f"excluded {int(band.sum())} of {got_x.size}, renoised {int(ref_mask.sum())}")
    assert not bad_m.any() and not bad_x.any(), f"{name}: renoise mismatch"
    return int(band.sum())
