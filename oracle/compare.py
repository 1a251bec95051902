"""Comparator for bf16 / fp16 / fp32 outputs against an fp64 reference.

Test infrastructure.  Reports, over one whole output tensor:

* ``nmse``     = sum((y - r)^2) / sum(r^2) in fp64 (the pages' parity gate is
                 NMSE <= 5e-4 against the CPU oracle -- page 2, PR
                 "head_dim=128 decode arm", section "Correctness"; the pages do
                 not define NMSE, this is the plain reading);
* ``max_abs``  = max |y - r|;
* ``bitwise``  = percentage of elements whose bits equal the reference
                 rounded to the output type (round to nearest, ties to even);
* ``n_big``    = count of |r| where the output type's half-ULP alone exceeds a
                 1e-2 max-abs bound (bf16: |r| >= 4; fp16: |r| >= 32).  The
                 max-abs bar applies to the other elements; these pass when
                 they are the correctly rounded value up to a small
                 arithmetic error: within 0.5 + 1/16 ULP of the reference
                 (the plain reading of a max-abs bound on bf16 outputs that
                 rounding alone can break);
* ``worst``    = flat index of the largest |y - r|;
* ``max_rel``  = max |y - r| / |r| over the elements with r != 0;
* ``max_ulps`` = max |y - r| in ULPs of the output type at r (0.5 at most for
                 a correctly rounded output).

``self_test`` repeats the pages' comparator self-test (page 3, PR
"head_dim-128 arm for the warp-split-KV decode kernel", comparator self-test
paragraph): a 1-ULP change in 3 of 2048 elements (offsets 5, 1024, 2047) must
move bitwise agreement from 100% to 2045/2048 = 99.8535%.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

NMSE_TOL = 5e-4
MAX_ABS_TOL = 1e-2
# |y - r| allowed on the n_big elements, in ULPs of the output type at r:
# the half-ULP of a correct rounding plus 1/16 ULP of arithmetic error.
BIG_ULPS_TOL = 0.5 + 1.0 / 16.0


def bf16_bits_to_f64(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round fp64 to the nearest bf16 (ties to even) in one rounding step.

    bf16 keeps 8 significant bits: with x = m * 2^e, 0.5 <= |m| < 1, the
    result is rint(m * 256) / 256 * 2^e (numpy's rint rounds ties to even).
    Normal-range values only; zeros, infinities and NaN are passed through.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(m * 256.0) / 256.0, e)
    f = r.astype(np.float32)          # exact: r has 8 significant bits
    return (f.view(np.uint32) >> 16).astype(np.uint16)


@dataclass
class Report:
    nmse: float
    max_abs: float
    bitwise: float
    n_big: int
    worst: int
    n: int
    max_abs_small: float = 0.0   # max |y - r| over |r| below the n_big threshold
    big_ulps: float = 0.0        # max |y - r| in output-type ULPs of r over the n_big elements
    max_rel: float = 0.0         # max |y - r| / |r| over the elements with r != 0
    max_ulps: float = 0.0        # max |y - r| in output-type ULPs of r over all elements
                                 # (a correctly rounded output has at most 0.5)

    def ok(self, nmse_tol=NMSE_TOL, max_abs_tol=MAX_ABS_TOL) -> bool:
        """NMSE and max-abs bars.  Where the output type's rounding alone can
        exceed the max-abs bar (the n_big elements), the element passes if it
        is the correctly rounded value up to a small arithmetic error (within
        BIG_ULPS_TOL ULPs of the reference) instead: such an exceedance is
        quantization-bound, not an arithmetic error."""
        return bool(np.isfinite(self.nmse) and self.nmse <= nmse_tol
                    and self.max_abs_small <= max_abs_tol and self.big_ulps <= BIG_ULPS_TOL)

    def __str__(self):
        return (f"nmse={self.nmse:.3e} max_abs={self.max_abs:.3e} max_abs_small={self.max_abs_small:.3e} "
                f"max_rel={self.max_rel:.3e} "
                f"max_ulps={self.max_ulps:.3f} bitwise={self.bitwise:.4f}% n_big={self.n_big} "
                f"worst={self.worst} n={self.n}" + (f" big_ulps={self.big_ulps:.3f}" if self.n_big else ""))


# |r| at and above which the half-ULP of the output type alone exceeds the
# 1e-2 max-abs bound: bf16 (2^-9 relative) from 4, binary16 (2^-11) from 32.
_BIG = {"bf16": 4.0, "f16": 32.0, "f32": float("inf")}


def compare(y_bits, ref) -> Report:
    """``y_bits``: the output under test -- bf16 bit patterns (uint16), or a
    numpy float16 / float32 array.  ``ref``: fp64 values, or an output of the
    same kind.  ``bitwise`` compares with the reference rounded to the
    output's type (round to nearest, ties to even; numpy's own conversion for
    float16 / float32)."""
    y_arr = np.asarray(y_bits)
    kind = {np.dtype(np.float16): "f16", np.dtype(np.float32): "f32"}.get(y_arr.dtype, "bf16")
    ref = np.asarray(ref)
    if kind == "bf16":
        y_bits = np.asarray(y_arr, dtype=np.uint16).ravel()
        if ref.dtype == np.uint16:
            r_bits = ref.ravel()
            r = bf16_bits_to_f64(r_bits)
        else:
            r = ref.astype(np.float64).ravel()
            r_bits = f64_to_bf16_bits(r)
        y = bf16_bits_to_f64(y_bits)
    else:
        y_bits = y_arr.ravel()
        y = y_bits.astype(np.float64)
        r = ref.astype(np.float64).ravel()
        r_bits = r.astype(y_arr.dtype)
        uint = np.uint16 if kind == "f16" else np.uint32
        y_bits, r_bits = y_bits.view(uint), r_bits.view(uint)
    if r.shape != y.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {r.shape}")
    n = y.size
    if n == 0:
        return Report(0.0, 0.0, 100.0, 0, -1, 0)
    is_big = np.abs(r) >= _BIG[kind]
    big = int(np.sum(is_big))
    d = y - r
    den = float(np.sum(r * r))
    num = float(np.sum(d * d))
    nmse = num / den if den > 0 else (0.0 if num == 0 else float("inf"))
    ad = np.abs(d)
    if not np.all(np.isfinite(ad)):
        worst = int(np.argmax(~np.isfinite(ad)))
        return Report(float("inf"), float("inf"), float(np.mean(y_bits == r_bits) * 100), big, worst, n,
                      float("inf"), float("inf"))
    worst = int(np.argmax(ad))
    small = float(ad[~is_big].max()) if big < n else 0.0
    # ULP of the output type at |r|: 2^(e - mantissa bits), |r| = m 2^e,
    # 0.5 <= m < 1 (at r = 0: the type's smallest subnormal, so any nonzero
    # y counts as far off)
    mant, emin = {"bf16": (8, -125), "f16": (11, -13), "f32": (24, -125)}[kind]
    _, e = np.frexp(r)
    ulp = np.ldexp(1.0, np.maximum(e, emin) - mant)
    per = ad / ulp
    ulps = float(np.max(per[is_big])) if big else 0.0
    nz = r != 0
    rel = float(np.max(ad[nz] / np.abs(r[nz]))) if np.any(nz) else 0.0
    return Report(nmse, float(ad[worst]), float(np.mean(y_bits == r_bits) * 100.0), big, worst, n,
                  small, ulps, rel, float(np.max(per)))


def bump_ulp(bits, offsets, ulps: int = 1) -> np.ndarray:
    """Return a copy of bf16 bits with the given flat offsets moved by ``ulps``
    units in the last place (away from zero)."""
    out = np.array(bits, dtype=np.uint16, copy=True).ravel()
    for o in offsets:
        out[o] = np.uint16(int(out[o]) + ulps)
    return out.reshape(np.shape(bits))


def self_test(reference_bits) -> tuple[Report, Report]:
    """The pages' comparator self-test on a 2048-element bf16 row set.
    Returns (clean report, corrupted report)."""
    ref = np.asarray(reference_bits, dtype=np.uint16).ravel()
    assert ref.size == 2048
    clean = compare(ref, ref)
    bad = compare(bump_ulp(ref, (5, 1024, 2047)), ref)
    return clean, bad
