"""Shared test utilities: the error ratio and conversions (no method arithmetic)."""
import numpy as np
import torch

TOL = 0.008  # relative L2 error ratio, as in the FLA backend pull request's test plan

# Per-unit bar (unit_ratios): every output is held per 64-token chunk (or per
# state) to TOL, except the per-token scalar gradients dbeta and dg.  Each of
# those is a row reduction whose chunk-level value sums the rounding of every
# bf16 intermediate of the chunk (the stored state and state gradient, R,
# Delta, the rounded A the forward returns); the CPU precision model in
# tests/test_precision_model.py reproduces per-chunk dg errors of about 0.014
# from those rounding points alone.  Their units are held to 0.02, still far
# below the error of one wrong token (about 0.1).
UNIT_TOL = {"dbeta": 0.02, "dg": 0.02}


def ratio(x, ref):
    """||x - ref||_2 / ||ref||_2 in fp64 (||x||_2 when ref is all zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    nr = np.linalg.norm(ref.ravel())
    nd = np.linalg.norm((x - ref).ravel())
    if nr == 0.0:
        return float(np.linalg.norm(x.ravel()))
    return float(nd / nr)


def np64(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def to_dev(d, device="cuda"):
    out = {}
    for k, v in d.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


def unit_ratios(x, ref, kind, cu=None, chunk=64):
    """Error ratio of every unit, as [(unit, ratio), ...].

    kind "tok": [B, T, H, ...] token tensors; a unit is one head of one
    64-token chunk of one sequence (batch rows, or the token ranges of
    cu_seqlens with B = 1), unit id (sequence, chunk, head).  kind "state":
    [N, H, ...] state tensors; a unit is one (row, head), unit id (row, head).

    A unit's error is judged against the larger of its own reference norm and
    the norm it would have at the whole reference's RMS value,
    ||ref|| sqrt(size_u / size).  The relative error of a sum of rounded
    terms grows with its cancellation (sum |terms| / |sum|), so a unit whose
    exact values happen to be far below the tensor's typical magnitude (a
    near-zero dbeta of a two-token sequence, say) is held to the absolute
    error the tensor's typical unit is allowed, not to a relative error it
    cannot have; every other unit is held to its own relative error."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    parts = []
    if kind == "state":
        for n in range(ref.shape[0]):
            for h in range(ref.shape[1]):
                parts.append(((n, h), x[n, h], ref[n, h]))
    elif kind == "tok":
        if cu is None:
            spans = [(b, b, 0, ref.shape[1]) for b in range(ref.shape[0])]
        else:
            cu = [int(c) for c in np.asarray(cu).ravel()]
            spans = [(i, 0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
        for seq, b, s, e in spans:
            for c0 in range(s, e, chunk):
                c1 = min(c0 + chunk, e)
                for h in range(ref.shape[2]):
                    parts.append(((seq, (c0 - s) // chunk, h), x[b, c0:c1, h], ref[b, c0:c1, h]))
    else:
        raise ValueError(kind)
    total = np.linalg.norm(ref.ravel())
    size = max(ref.size, 1)
    out = []
    for unit, xu, ru in parts:
        scale = max(np.linalg.norm(ru.ravel()), total * np.sqrt(ru.size / size))
        if scale > 0.0:
            out.append((unit, float(np.linalg.norm((xu - ru).ravel()) / scale)))
    return out


def check(name, x, ref, kind=None, cu=None, tol=TOL):
    """The parity bar: the whole-tensor error ratio and, with `kind`, the
    worst unit's ratio (unit_ratios) are both <= tol, so a wrong region too
    small to move the whole-tensor ratio (one token of a long sequence) still
    fails.
    Prints both; returns the whole-tensor ratio."""
    if x is None or ref is None:
        assert x is None and ref is None, name
        return 0.0
    x = np64(x)
    r = ratio(x, ref)
    worst = None
    extra = ""
    if kind is not None:
        us = unit_ratios(x, ref, kind, cu)
        if us:
            worst = max(us, key=lambda t: t[1])
        if kind == "tok":
            ws = unit_ratios(x, ref, kind, cu, chunk=1 << 40)
            if ws:
                w2 = max(ws, key=lambda t: t[1])
                extra = "  worst sequence %s %.5f" % (w2[0], w2[1])
    print("%s: ratio %.5f%s%s" % (name, r, "" if worst is None else
                                  "  worst unit %s %.5f" % (worst[0], worst[1]), extra), flush=True)
    assert r <= tol, (name, r)
    utol = UNIT_TOL.get(name.split()[0], tol) if tol == TOL else tol
    if worst is not None:
        assert worst[1] <= utol, (name, "unit", worst)
    return r
