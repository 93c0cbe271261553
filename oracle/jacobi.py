"""One-sided (Hestenes) Jacobi SVD and the polar factor U V^T for tiny matrices.

Test infrastructure only.  This is the independent route to the polar factor
that both Muon pages name as the target of the orthogonalisation: for
M = U Σ V^T the orthogonalised update is U V^T (the deep-dive page, section
"Newton-Schulz 迭代：为什么不用 SVD"; the DeepSeek-V4 book ch. 6, §2).  It is
slow (O(sweeps · n² · m)) and meant for matrices of a few dozen rows.

Method: repeatedly apply plane rotations to pairs of columns of a working
copy until every pair is orthogonal; the column norms are then the singular
values, the normalised columns are U, and the accumulated rotations are V.
"""

import numpy as np


def jacobi_svd(a, tol=1e-15, max_sweeps=80):
    """Thin SVD of a real matrix: returns (U, s, Vt) with a = U @ diag(s) @ Vt.

    Singular values come back sorted in decreasing order.  Works on float64.
    """
    a = np.array(a, dtype=np.float64)
    flip = a.shape[0] < a.shape[1]
    if flip:
        a = a.T
    m, n = a.shape
    w = a.copy()
    v = np.eye(n)
    for _ in range(max_sweeps):
        rotated = False
        for p in range(n - 1):
            for q in range(p + 1, n):
                wp, wq = w[:, p], w[:, q]
                alpha = float(wp @ wp)
                beta = float(wq @ wq)
                gamma = float(wp @ wq)
                if abs(gamma) <= tol * np.sqrt(alpha * beta) or gamma == 0.0:
                    continue
                rotated = True
                # Rotation angle that zeroes the (p, q) entry of w^T w.
                zeta = (beta - alpha) / (2.0 * gamma)
                t = np.sign(zeta) / (abs(zeta) + np.sqrt(1.0 + zeta * zeta))
                if zeta == 0.0:
                    t = 1.0
                c = 1.0 / np.sqrt(1.0 + t * t)
                s = c * t
                new_p = c * wp - s * wq
                new_q = s * wp + c * wq
                w[:, p], w[:, q] = new_p, new_q
                vp, vq = v[:, p].copy(), v[:, q].copy()
                v[:, p] = c * vp - s * vq
                v[:, q] = s * vp + c * vq
        if not rotated:
            break
    sig = np.sqrt(np.sum(w * w, axis=0))
    order = np.argsort(-sig)
    sig = sig[order]
    w = w[:, order]
    v = v[:, order]
    u = np.zeros_like(w)
    nz = sig > 0
    u[:, nz] = w[:, nz] / sig[nz]
    if flip:
        # a^T = U S V^T  =>  a = V S U^T
        return v, sig, u.T
    return u, sig, v.T


def polar_factor(a):
    """U V^T of a full-rank matrix a (thin factors), via the Jacobi SVD."""
    u, s, vt = jacobi_svd(a)
    if np.any(s == 0):
        raise ValueError("polar_factor: rank-deficient input")
    return u @ vt
