"""Comparison rules between a GPU result and the oracle.

Bit-exact: integer-valued inputs make every partial sum exact in fp32 and in
fp64, so C must equal the oracle's rounded output bit for bit.

Tolerance (Gaussian inputs). The stated bound is max |C - C_ref| <= 2e-3 *
rms(C_ref). For float32 outputs it is applied literally against the oracle's
fp64 value. A bfloat16 output cannot meet it literally: rounding an exact
value to 8 significant bits alone moves it by up to half a unit in the last
place, about 1.6% of rms(C) at the shapes used here. For bfloat16 outputs the
bound is therefore applied on top of the output format's own half-ulp:
|C - C64| <= 0.5 * ulp_bf16(C64) + 2e-3 * rms(C64), elementwise.
"""
import numpy as np

TOL_REL_RMS = 2e-3


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def half_ulp_bf16(x):
    """Half the spacing of bfloat16 numbers in the binade of |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126.0)
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def check_exact(got_bits, want_bits, what=""):
    g = np.asarray(got_bits)
    w = np.asarray(want_bits)
    assert g.shape == w.shape, f"{what}: shape {g.shape} != {w.shape}"
    gv = g.view(np.uint16) if g.dtype == np.uint16 else g.view(np.uint32)
    wv = w.view(np.uint16) if w.dtype == np.uint16 else w.view(np.uint32)
    bad = np.nonzero(gv != wv)
    n = len(bad[0])
    assert n == 0, (f"{what}: {n} of {g.size} elements differ, first at "
                    f"{tuple(int(b[0]) for b in bad)}: got {gv[bad][0]:#x} want {wv[bad][0]:#x}")


def tolerance_stats(got, C64, c_dtype, rms_ref=None):
    """Returns a dict of error statistics; 'ok' says whether the rule holds."""
    C64 = np.asarray(C64, dtype=np.float64)
    if c_dtype == "bf16":
        gv = bf16_bits_to_f64(got)
    else:
        gv = np.asarray(got, dtype=np.float32).astype(np.float64)
    rms = float(np.sqrt(np.mean(C64 * C64))) if rms_ref is None else float(rms_ref)
    err = np.abs(gv - C64)
    finite = np.isfinite(gv).all()
    if c_dtype == "bf16":
        allow = half_ulp_bf16(C64) + TOL_REL_RMS * rms
    else:
        allow = np.full(C64.shape, TOL_REL_RMS * rms)
    ok = bool(finite and np.all(err <= allow))
    worst = int(np.argmax(err - allow)) if err.size else 0
    return {
        "ok": ok,
        "max_abs_err": float(err.max()) if err.size else 0.0,
        "rms_err_over_rms": float(np.sqrt(np.mean(err * err)) / rms) if err.size and rms > 0 else 0.0,
        "literal_bound": TOL_REL_RMS * rms,
        "worst_index": worst,
        "worst_excess": float((err - allow).flat[worst]) if err.size else 0.0,
        "rms": rms,
    }


def check_tolerance(got, C64, c_dtype, what="", rms_ref=None):
    s = tolerance_stats(got, C64, c_dtype, rms_ref)
    assert s["ok"], f"{what}: tolerance violated: {s}"
    return s
