"""Recompute the polynomial in softplus_f32 (internal.h).

log1p(e) = 2 atanh(s) with s = e / (2 + e), and for e in (0, 1], s is in
(0, 1/3]. softplus_f32 evaluates 2 atanh(s) as s * q(s^2), q a degree-4
polynomial in z = s^2 on [0, 1/9], fitted to g(z) = 2 atanh(sqrt z) / sqrt z
for the least maximum relative error by the Remez exchange (alternation on six
points). Prints the coefficients rounded to float32 (lowest degree first) and
the relative error of the fit.

    python selective_state_update_amd/csrc/fit_softplus.py
"""
import mpmath as mp
import numpy as np

mp.mp.dps = 40
DEG = 4
Z = mp.mpf(1) / 9


def g(z):
    z = mp.mpf(z)
    if z == 0:
        return mp.mpf(2)
    r = mp.sqrt(z)
    return 2 * mp.atanh(r) / r


def remez(deg=DEG, iters=10, grid_n=2000):
    n = deg + 2
    xs = [Z / 2 * (1 - mp.cos(mp.pi * k / (n - 1))) for k in range(n)]
    grid = [Z * k / grid_n for k in range(grid_n + 1)]
    for _ in range(iters):
        A = mp.matrix(n, n)
        rhs = mp.matrix(n, 1)
        for i, x in enumerate(xs):
            for j in range(deg + 1):
                A[i, j] = x ** j
            A[i, deg + 1] = (-1) ** i * g(x)
            rhs[i] = g(x)
        sol = mp.lu_solve(A, rhs)
        c = [sol[j] for j in range(deg + 1)]
        err = [(sum(c[j] * x ** j for j in range(deg + 1)) - g(x)) / g(x) for x in grid]
        ext = [k for k in range(len(grid))
               if k in (0, len(grid) - 1) or (abs(err[k]) >= abs(err[k - 1]) and abs(err[k]) >= abs(err[k + 1]))]
        sel = []
        for k in ext:  # alternating extrema
            if sel and mp.sign(err[k]) == mp.sign(err[sel[-1]]):
                if abs(err[k]) > abs(err[sel[-1]]):
                    sel[-1] = k
            else:
                sel.append(k)
        while len(sel) > n:
            sel.pop(0 if abs(err[sel[0]]) < abs(err[sel[-1]]) else -1)
        if len(sel) == n:
            xs = [grid[k] for k in sel]
    return c, max(abs(e) for e in err)


if __name__ == "__main__":
    coef, maxerr = remez()
    print("coefficients (float32, degree 0 first):", ["%.9e" % np.float32(float(x)) for x in coef])
    print("max relative error of the fit: %.3e (%.3f fp32 ulp)" % (float(maxerr), float(maxerr) / 2 ** -24))
