"""Parity rules between the HIP path and the fp64 oracle (test helper).

Rules (decision-boundary flags come from the oracle):
* codes: identical wherever the rotated coordinate y_i is farther than 1e-6
  from every threshold; at flagged coordinates only an adjacent level may
  differ; all code mismatches together stay below 1e-6 of the entries (a
  rate over the whole parity session; single calls allow Poisson noise);
* sign bits: compared on keys whose codes all match; for a key with a
  permitted code difference the oracle recomputes the residual stage from the
  GPU's codes.  Identical wherever |(S r)_j| / ||k|| > 1e-6; mismatches below
  1e-6 of the entries;
* half norms: bit-identical except within 1e-6 (relative) of a half-precision
  rounding midpoint, where one ulp is allowed;
* logits: |delta| <= 1e-4 ||q|| ||k|| when both scorers read the same record.
"""

import math

import numpy as np

import oracle as O

# Session totals: the "< 1e-6 of all entries" rule is a rate, enforced over
# every entry the parity suite compares (test_zz_parity_rates.py); each call
# only rejects counts far above that rate (a Poisson 3-sigma allowance).
TOTALS = {"code_mismatch": 0, "code_entries": 0, "sign_mismatch": 0, "sign_entries": 0}


def _rate_ok(count, entries, rate=1e-6):
    mu = rate * entries
    return count <= mu + 3.0 * math.sqrt(mu) + 1.0


def check_encode(cb, keys, gpu_codes, gpu_signs, gpu_nu16, gpu_rho16):
    """keys [n, d] (exact values), GPU outputs unpacked with the oracle's unpack."""
    ref = O.encode(cb, keys)
    n, d = ref.codes.shape
    gc = gpu_codes.reshape(n, d).astype(np.int16)
    rc = ref.codes.astype(np.int16)
    diff = gc != rc
    bad_unflagged = diff & ~ref.code_flag
    assert not bad_unflagged.any(), f"{int(bad_unflagged.sum())} unflagged code mismatches at {np.argwhere(bad_unflagged)[:5].tolist()}"
    assert np.all(np.abs(gc - rc)[diff] <= 1), "flagged code mismatch beyond an adjacent level"
    assert _rate_ok(int(diff.sum()), diff.size), f"{int(diff.sum())} code mismatches in {diff.size}"
    key_mis = diff.any(axis=1)
    sref = ref
    if key_mis.any():
        # recompute the residual stage from the GPU's codes for those keys
        re = O.encode(cb, keys[key_mis], codes=gpu_codes.reshape(n, d)[key_mis])
        sref = O.EncodeResult(**{f: getattr(ref, f).copy() if isinstance(getattr(ref, f), np.ndarray) else getattr(ref, f)
                                 for f in ref.__dataclass_fields__})
        for f in ("signs", "rho", "rho16", "p", "sign_flag", "rho16_flag"):
            getattr(sref, f)[key_mis] = getattr(re, f)
    gs = gpu_signs.reshape(n, -1)
    sd = gs != sref.signs
    bad = sd & ~sref.sign_flag
    assert not bad.any(), f"{int(bad.sum())} unflagged sign mismatches at {np.argwhere(bad)[:5].tolist()}"
    assert _rate_ok(int(sd.sum()), sd.size), f"{int(sd.sum())} sign mismatches in {sd.size}"
    for name, g16, r16, flag in (("nu", gpu_nu16, sref.nu16, sref.nu16_flag),
                                 ("rho", gpu_rho16, sref.rho16, sref.rho16_flag)):
        gb = g16.reshape(n).view(np.uint16).astype(np.int32)
        rb = r16.view(np.uint16).astype(np.int32)
        nd = gb != rb
        assert not (nd & ~flag).any(), f"{name}: {int((nd & ~flag).sum())} unflagged half mismatches, e.g. idx {np.argwhere(nd & ~flag)[:5].ravel().tolist()} gpu {g16.reshape(n)[nd & ~flag][:5]} ref {r16[nd & ~flag][:5]}"
        assert np.all(np.abs(gb - rb)[nd] <= 1), f"{name}: flagged half mismatch beyond one ulp"
    TOTALS["code_mismatch"] += int(diff.sum())
    TOTALS["code_entries"] += int(diff.size)
    TOTALS["sign_mismatch"] += int(sd.sum())
    TOTALS["sign_entries"] += int(sd.size)
    return dict(code_mismatch=int(diff.sum()), sign_mismatch=int(sd.sum()),
                code_flagged=int(ref.code_flag.sum()), sign_flagged=int(sref.sign_flag.sum()))


def check_logits(gpu, ref, q, keys_norm):
    """gpu/ref [G, Qg, N]; q [G, Qg, d]; keys_norm [G, N] fp64 norms of the original keys."""
    tol = 1e-4 * np.linalg.norm(np.asarray(q, np.float64), axis=-1)[:, :, None] * keys_norm[:, None, :]
    err = np.abs(np.asarray(gpu, np.float64) - ref)
    worst = np.max(err / np.maximum(tol, 1e-300)) if err.size else 0.0
    assert np.all(err <= tol), f"logit mismatch: worst |delta|/tol = {worst:.3g}"
    return float(worst)


def check_values(cb, values, gpu_codes, gpu_nu16):
    """Value records (MSE-only): the code and half-norm rules above."""
    ref = O.encode_values(cb, values)
    n, d = ref.codes.shape
    gc = np.asarray(gpu_codes).reshape(n, d).astype(np.int16)
    rc = ref.codes.astype(np.int16)
    diff = gc != rc
    bad = diff & ~ref.code_flag
    assert not bad.any(), f"{int(bad.sum())} unflagged value-code mismatches at {np.argwhere(bad)[:5].tolist()}"
    assert np.all(np.abs(gc - rc)[diff] <= 1), "flagged value-code mismatch beyond an adjacent level"
    assert _rate_ok(int(diff.sum()), diff.size), f"{int(diff.sum())} value-code mismatches in {diff.size}"
    gb = np.asarray(gpu_nu16).reshape(n).view(np.uint16).astype(np.int32)
    rb = ref.nu16.view(np.uint16).astype(np.int32)
    nd = gb != rb
    assert not (nd & ~ref.nu16_flag).any(), "value norm: unflagged half mismatch"
    assert np.all(np.abs(gb - rb)[nd] <= 1), "value norm: flagged half mismatch beyond one ulp"
    TOTALS["code_mismatch"] += int(diff.sum())
    TOTALS["code_entries"] += int(diff.size)
    return ref


def attention_tolerance(vhat, extra=0.0):
    """Bound for |out_gpu - out_oracle| per element when both use the same
    logits: the weights carry fp32 exponentials (relative error ~1e-6) and the
    sums fp32 rounding, so every output element is within 5e-5 of the largest
    decoded value norm of its group (plus `extra`, a relative bound on the
    softmax weights when the logits themselves differ)."""
    vmax = np.max(np.linalg.norm(vhat, axis=-1), axis=-1)          # [G]
    return ((5e-5 + extra) * vmax)[:, None, None]
