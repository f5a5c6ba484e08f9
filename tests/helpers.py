"""Comparison helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np


def to_np(t):
    """Exact fp64 host copy of a torch tensor (bf16/fp16/fp32 upcast exactly)."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_fro(got, ref):
    d = np.linalg.norm(got - ref)
    n = np.linalg.norm(ref)
    return d / n if n > 0 else d


def band_ok(got, ref, tol):
    """Every singular value of `got` lies in [lo - tol*hi, hi + tol*hi], lo/hi the min/max
    singular value of `ref`."""
    sr = np.linalg.svd(ref, compute_uv=False)
    sg = np.linalg.svd(got, compute_uv=False)
    lo, hi = sr.min(), sr.max()
    return bool(sg.min() >= lo - tol * hi and sg.max() <= hi + tol * hi), (lo, hi, sg.min(), sg.max())


def say(*a):
    print(*a, flush=True)


def bf16_steps(a, b):
    """Number of bf16 representable steps between round_bf16(a) and round_bf16(b) (RNE)."""
    import torch
    def ordered(x):
        bits = torch.tensor(x).to(torch.bfloat16).view(torch.int16).to(torch.int32).numpy()
        mag = bits & 0x7FFF
        return np.where(bits < 0, -mag, mag)
    return np.abs(ordered(a) - ordered(b))


def f16_steps(a, b):
    """Number of fp16 representable steps between round_f16(a) and round_f16(b) (RNE)."""
    def ordered(x):
        bits = np.asarray(x, dtype=np.float16).view(np.int16).astype(np.int32)
        mag = bits & 0x7FFF
        return np.where(bits < 0, -mag, mag)
    return np.abs(ordered(a) - ordered(b))


def w_update_ok(Wg, W_prev, Ug, lr, wd, dtype="bf16"):
    """W after a step equals (1 - lr wd) W_prev - lr U, evaluated on the returned U and rounded
    once to the weight dtype: within one representable step of the exactly rounded value, or
    within the fp32 arithmetic error of the update (for results that nearly cancel)."""
    w_exp = (1.0 - lr * wd) * W_prev - lr * Ug
    slack = 4 * 2.0 ** -24 * (np.abs(W_prev) + lr * np.abs(Ug)) + 1e-30
    if dtype in ("bf16", "f16"):
        steps = bf16_steps(Wg, w_exp) if dtype == "bf16" else f16_steps(Wg, w_exp)
        ok = (steps <= 1) | (np.abs(Wg - w_exp) <= slack)
    else:
        ok = np.abs(Wg - w_exp) <= slack + np.spacing(np.abs(w_exp).astype(np.float32)).astype(np.float64)
    return bool(ok.all()), float(np.mean(~ok))


def gram_singular_range(O):
    """(min, max) singular value of an n x m matrix (n <= m) from the eigenvalues of the n x n
    Gram matrix O O^T in fp64 (much cheaper than an SVD at n x m = 7168 x 18432)."""
    O = np.asarray(O, dtype=np.float64)
    if O.shape[0] > O.shape[1]:
        O = O.T
    ev = np.linalg.eigvalsh(O @ O.T)
    s = np.sqrt(np.clip(ev, 0.0, None))
    return float(s.min()), float(s.max())


def band_ok_gram(got, ref, tol, ref_range=None):
    """band_ok through gram_singular_range; ref_range may carry the reference's precomputed
    (lo, hi)."""
    lo, hi = gram_singular_range(ref) if ref_range is None else ref_range
    gmin, gmax = gram_singular_range(got)
    return bool(gmin >= lo - tol * hi and gmax <= hi + tol * hi), (lo, hi, gmin, gmax)
