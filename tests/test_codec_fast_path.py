"""CPU check of the argument behind the device's division-free codes.

The per-vector codec ("Background": Q = round((X - z)/s)) defines a code as
rint(fl(x - z) / s) with an IEEE fp32 division, clamped to [0, 2^b - 1].
The prompt pack kernel computes t = fl(x - z) * r with r the hardware
reciprocal of s (within 1 ulp) and takes rint(t) unless t lies within 2^-13
of a half-integer, where it redoes the code with the division.  This test
emulates that rule with reciprocals perturbed by up to +-2 ulp and checks,
on inputs shaped like the codec's (fp16 values, z = fp16 of the minimum,
s = fp16 of range / (2^b - 1), including sub-resolution ranges, subnormal
scales and exact half-integer quotients), that whenever the rule keeps t
the code equals the IEEE one.  It emulates the device arithmetic in numpy;
the device itself is compared with the oracle in the GPU tests.
"""
import numpy as np

ZONE = 0.5 - 2.0 ** -13


def _inputs(rng, n, qmax):
    f32 = np.float32
    kind = rng.integers(0, 4, n)
    x = rng.standard_normal(n) * rng.choice([1.0, 8.0, 1e-3, 200.0], n)
    z = x - np.abs(rng.standard_normal(n)) * rng.choice([1.0, 3.0, 1e-4], n)
    s = (np.abs(rng.standard_normal(n)) * 4 + (x - z)) / qmax
    # exact half-integer quotients: s a power of two, x - z = (k + 0.5) s
    tie = kind == 0
    k = rng.integers(0, qmax, n)
    s = np.where(tie, 0.25, s)
    z = np.where(tie, 0.0, z)
    x = np.where(tie, (k + 0.5) * 0.25, x)
    # sub-resolution ranges (subnormal fp16 scales)
    tiny = kind == 1
    s = np.where(tiny, s * 1e-6, s)
    x16 = x.astype(np.float16).astype(f32)
    z16 = z.astype(np.float16).astype(f32)
    s16 = s.astype(np.float16).astype(f32)
    s16 = np.where(s16 == 0, f32(2.0 ** -24), s16)  # a zero scale has its own rule (code 0)
    return x16, z16, s16


def test_fast_codes_equal_ieee_codes_outside_the_zone():
    rng = np.random.default_rng(20261202)
    f32 = np.float32
    kept = 0
    for qmax in (255, 15, 3):
        x, z, s = _inputs(rng, 400_000, qmax)
        a = (x - z).astype(f32)
        exact = np.clip(np.rint((a / s).astype(f32)), 0, qmax)
        r0 = (f32(1) / s).astype(f32)
        for ulp in (-2, -1, 0, 1, 2):
            r = (r0.view(np.int32) + np.int32(ulp)).view(f32)
            t = (a * r).astype(f32)
            rt = np.rint(t)
            keep = np.abs(t - rt) < f32(ZONE)
            # the fused form the compiler may use for the test, fl(a r - rt)
            u = (a.astype(np.float64) * r.astype(np.float64) - rt).astype(f32)
            keep_fused = np.abs(u) < f32(ZONE)
            fast = np.clip(rt, 0, qmax)
            assert np.array_equal(fast[keep], exact[keep]), f"qmax {qmax}, {ulp:+d} ulp"
            assert np.array_equal(fast[keep_fused], exact[keep_fused]), f"qmax {qmax}, {ulp:+d} ulp (fused)"
            kept += int(keep.sum())
            # exact ties inside the code range always go to the division (far
            # beyond it fp32 itself has half-integer spacing and both clamp)
            q = (a / s).astype(np.float64)
            tie_rows = (np.abs(q - np.floor(q) - 0.5) == 0) & (q <= qmax + 1)
            assert tie_rows.any()
            assert not np.any(keep & tie_rows)
    assert kept > 0


def test_zone_is_rare_on_gaussian_vectors():
    """On N(0,1) vectors the division is needed for about 2 in 10^4 codes
    (the kernel's cost model)."""
    rng = np.random.default_rng(7)
    f32 = np.float32
    v = rng.standard_normal((20000, 128)).astype(np.float16).astype(f32)
    mn, mx = v.min(axis=1), v.max(axis=1)
    for qmax in (255, 15, 3):
        s = ((mx - mn) / f32(qmax)).astype(np.float16).astype(f32)
        z = mn.astype(np.float16).astype(f32)
        t = ((v - z[:, None]).astype(f32) * (f32(1) / s)[:, None]).astype(f32)
        near = ~(np.abs(t - np.rint(t)) < f32(ZONE))
        assert near.mean() < 1e-3
