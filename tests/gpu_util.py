"""Helpers of the GPU tests: device copies of seeded problems and the
parity comparison.

Tolerance (fp32 1e-5, bf16 inputs with fp32 accumulation 2e-2, both
relative), per tensor and head ([n, heads, head_dim] and [n, heads] arrays;
other arrays as a whole):
  * the relative error ||got - ref||_2 / ||ref||_2 <= rtol, and
  * elementwise |got - ref| <= rtol*|ref| + rtol*rms(ref) + 8*u*mag, where
    rms is over the head's compared elements, u = 2^-24 is the unit roundoff
    of the float32 arithmetic, and mag (from the oracle) is the sum of the
    absolute values of the terms that define the element: a sum whose terms
    cancel (mag >> |ref|) cannot be computed in float32 to better than about
    u*mag, whatever the order of summation.
lse compares as |got - ref| <= rtol*max(1, |ref|), and -inf (empty rows) must
match exactly.
"""
import numpy as np
import torch

RTOL = {"f32": 1e-5, "bf16": 2e-2}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(x, dtype=None, device="cuda"):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device).contiguous()


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


U32 = 2.0 ** -24


def assert_close(got, ref, rtol, name, mag=None, head_axis="auto", extra=None):
    """head_axis: the axis whose entries get their own statistics (default:
    axis 1 of a [n, heads, head_dim] array; None: the whole array).  extra
    (optional, like ref): a further elementwise error bound that the inputs
    themselves set (see the wide-score-range test), added to the elementwise
    bound and, as its L2 norm, to the relative L2 one."""
    g = got if isinstance(got, np.ndarray) else to_np(got)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    if ref.size == 0:
        return
    if head_axis == "auto":
        head_axis = 1 if ref.ndim == 3 else None
    axes = tuple(a for a in range(ref.ndim) if a != head_axis)
    rms = np.sqrt(np.mean(ref ** 2, axis=axes, keepdims=True))
    d2 = np.sqrt(np.sum((g - ref) ** 2, axis=axes))
    r2 = np.sqrt(np.sum(ref ** 2, axis=axes))
    x2 = 0.0 if extra is None else np.sqrt(np.sum(np.asarray(extra, np.float64) ** 2, axis=axes))
    ok = (d2 <= rtol * r2 + x2) | (r2 == 0)  # an all-zero reference is left to the elementwise bound
    assert np.all(ok), f"{name}: relative L2 error {d2 / np.maximum(r2, 1e-300)} > {rtol} (+ {x2})"
    bound = rtol * np.abs(ref) + rtol * rms
    if mag is not None:
        bound = bound + 8 * U32 * np.asarray(mag, np.float64)
    if extra is not None:
        bound = bound + np.asarray(extra, np.float64)
    err = np.abs(g - ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(bound, 1e-300), 0)), ref.shape)
        rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300)
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} outside tolerance; "
                             f"worst at {idx}: got {g[idx]!r} ref {ref[idx]!r} bound {bound[idx]!r}; "
                             f"rel l2 {rel:.3e}")


def bf16_round(x, ties_even=True):
    """fp64 -> the nearest bfloat16 value (8 significant bits), ties to even;
    with ties_even=False, toward zero (truncation: the tests' own check that
    the comparison below tells the two apart)."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    q = np.round(m * 256.0) if ties_even else np.trunc(m * 256.0)
    return np.ldexp(q, e - 8)


def assert_rounded_to_nearest_even(got, ref, mag, name, head_axis="auto"):
    """bf16 outputs are the float32 results rounded to nearest, ties to even.
    Where the oracle's value lies farther from a rounding midpoint than the
    float32 parity bound (1e-5 |r| + 1e-5 rms + 8 u mag), the rounded value is
    decided, and the GPU's must equal the oracle's rounded to nearest even.
    Also checks that such elements are most of the tensor and that truncation
    would differ on a large share of them."""
    g = got if isinstance(got, np.ndarray) else to_np(got)
    ref = np.asarray(ref, np.float64)
    if head_axis == "auto":
        head_axis = 1 if ref.ndim == 3 else None
    axes = tuple(a for a in range(ref.ndim) if a != head_axis)
    rms = np.sqrt(np.mean(ref ** 2, axis=axes, keepdims=True))
    near = bf16_round(ref)
    ulp = np.ldexp(1.0, np.frexp(ref)[1] - 8)
    margin = 1e-5 * np.abs(ref) + 1e-5 * rms + 8 * U32 * np.asarray(mag, np.float64)
    decided = (ref != 0) & (ulp / 2 - np.abs(ref - near) > margin)
    assert decided.mean() > 0.9, (name, decided.mean())
    assert np.mean(bf16_round(ref, ties_even=False)[decided] != near[decided]) > 0.3, name
    bad = decided & (g != near)
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {int(decided.sum())} decided elements "
                           f"differ from round-to-nearest-even")


def assert_lse(got, ref, rtol, name="lse"):
    g = got if isinstance(got, np.ndarray) else to_np(got)
    ref = np.asarray(ref, np.float64)
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(g), ninf), f"{name}: -inf pattern differs"
    f = ~ninf
    err = np.abs(g[f] - ref[f])
    bound = rtol * np.maximum(1.0, np.abs(ref[f]))
    assert np.all(err <= bound), f"{name}: max err {err.max()} vs bound {bound[np.argmax(err)]}"


def device_problem(P, device="cuda"):
    """Device tensors of a Problem: (indptr, indices, Q, K, V, dY, bias)."""
    dt = TDT[P.cfg.dtype]
    return dict(indptr=dev(P.indptr, device=device), indices=dev(P.indices, device=device),
                Q=dev(P.Q, dt, device), K=dev(P.K, dt, device), V=dev(P.V, dt, device),
                dY=dev(P.dY, dt, device),
                bias=dev(P.bias, torch.float32, device) if P.bias is not None else None)
