"""The elementwise parity bar shared by the GPU tests (not a test module).

Every element of a GPU result, widened to double, must satisfy

    |gpu - oracle| <= 2e-2 * max(1, |oracle|)            (h13, a, y, out, dx, ...)
    |gpu - oracle| <= 2e-2 * max(1, |oracle|, rss)       (dscores, dW13, dW2)

rss is the oracle's root-sum-square of the terms of that element's sum (D terms for dscores, the
expert's rows for dW13 and dW2). Those outputs are long reductions of bf16 operands that the GPU
forms in fp32 in MFMA order while the oracle sums exactly: a stored bf16 operand (y, a, dy, dh13)
that lands one ulp apart on the two sides moves one term by at most 2^-7 of that term, and a sum
whose terms cancel can end near zero while such differences do not. rss is at least the largest
term, so a one-ulp difference in even the largest operand stays under 2e-2 * rss with a factor
2.5 to spare, while a wrong term, sign or index moves the result by the term itself.
"""
import numpy as np

RTOL = 2e-2


def log(*a):
    print(*a, flush=True)


def check(name, got, ref, scale=None, rtol=RTOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), "%s: non-finite values" % name
    if got.size == 0:
        return
    diff = np.abs(got - ref)
    plain = rtol * np.maximum(1.0, np.abs(ref))
    tol = plain if scale is None else np.maximum(plain, rtol * np.asarray(scale, np.float64))
    r_plain = diff / plain
    r = diff / tol
    worst = np.unravel_index(int(np.argmax(r)), r.shape)
    log("  %-8s max |d|/tol %.3f  (vs 2e-2*max(1,|ref|): %.3f, %d over)  exact %.4f  "
        "normwise %.2e  n %d"
        % (name, float(r.max()), float(r_plain.max()), int((r_plain > 1).sum()),
           float((got == ref).mean()), float(diff.max()) / max(1.0, float(np.abs(ref).max())),
           got.size))
    assert (diff <= tol).all(), "%s: %d elements over the bound, worst at %s: gpu %r ref %r tol %r" % (
        name, int((diff > tol).sum()), worst, float(got[worst]), float(ref[worst]),
        float(tol[worst]))
