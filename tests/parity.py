"""Parity criteria between the HIP path and the oracle (shared by the GPU tests).

Tolerances (the workload's accuracy targets, set with the first kernels and unchanged since):
  packing / page placement / code layout   bit-exact (codes read from the GPU bytes at the oracle's
                                            positions; exact-code tiles compare whole records)
  channel scales c and token scales s'      relative error <= 1e-5
  token offsets m'                          |err| <= 1e-5 * max(|m'|, (2^b - 1) |s'|)
  codes                                     mismatch rate <= 1e-4; every mismatch is +-1 and the
                                            oracle's unrounded (z - mn)/s lies within 1e-3 of a
                                            half-integer (both sides round a value computed in
                                            their own precision; fp32 vs fp64)
  decode output                             relative L2 error <= 2e-3 per (sequence, query head)
                                            against the oracle attending over the GPU's own cache
"""
import numpy as np

import oracle

SCALE_RTOL = 1e-5
CODE_MISMATCH_RATE = 1e-4
TIE_BAND = 1e-3
DECODE_REL_L2 = 2e-3


def check_half(q_gpu, c_gpu, sp_gpu, mp_gpu, ref, bits, what=""):
    """Compare one tile half (codes [128,128], scales) with oracle.quantize_tile_debug output.
    s' and m' are [128] (one group per token) or [ng][128] (groups of 128/ng channels)."""
    qmax = (1 << bits) - 1
    c_ref, sp_ref, mp_ref = ref["c"], ref["sp"], ref["mp"]
    rc = np.abs(c_gpu.astype(np.float64) - c_ref) / np.abs(c_ref)
    assert rc.max() <= SCALE_RTOL, f"{what} c rel err {rc.max():.3g}"
    den = np.maximum(np.abs(sp_ref.astype(np.float64)), 1e-30)
    rs = np.abs(sp_gpu.astype(np.float64) - sp_ref) / den
    rs[sp_ref == 0] = np.abs(sp_gpu[sp_ref == 0])
    assert rs.max() <= SCALE_RTOL, f"{what} s' rel err {rs.max():.3g}"
    bound = SCALE_RTOL * np.maximum(np.abs(mp_ref.astype(np.float64)), qmax * np.abs(sp_ref.astype(np.float64)))
    em = np.abs(mp_gpu.astype(np.float64) - mp_ref)
    assert np.all(em <= bound + 1e-30), f"{what} m' err {(em - bound).max():.3g} over bound"
    d = q_gpu.astype(np.int32) - ref["q"].astype(np.int32)
    bad = d != 0
    n_bad = int(bad.sum())
    if n_bad:
        assert np.all(np.abs(d[bad]) == 1), f"{what} code mismatch larger than 1"
        t = ref["tval"][bad]
        dist = np.abs(t - np.floor(t) - 0.5)
        assert np.all(dist <= TIE_BAND), f"{what} mismatch away from a tie: {dist.max():.3g}"
    return n_bad


def assert_code_rate(n_bad, n_codes, what=""):
    """The mismatch-rate criterion over everything a test compared."""
    assert n_bad <= CODE_MISMATCH_RATE * n_codes, f"{what} {n_bad} code mismatches in {n_codes}"


def check_record(rec_gpu, kb, vb, ref_k, ref_v, what="", group=128):
    """Full record check: layout bit-exact, K and V halves within tolerance.  Returns the number of
    code mismatches (each already checked to be a +-1 flip at a near tie)."""
    # Codes are read out of the GPU bytes at the positions the oracle's layout defines, so a
    # misplaced bit shows up as mismatches far beyond the tie criterion below.
    qk, qv, sc = oracle.unpack_record(kb, vb, rec_gpu, group)
    ck, spk, mpk, cv, spv, mpv = oracle.split_scales(sc, group)
    nk = check_half(qk, ck, spk, mpk, ref_k, kb, what + " K")
    nv = check_half(qv, cv, spv, mpv, ref_v, vb, what + " V")
    return nk + nv


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a)
