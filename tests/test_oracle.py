"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: finite differences,
closed forms of special cases, the delta rule's retrieval property, linearity,
and structural identities (packing, grouped heads, resuming from a state, the
transposed state layout).  The chunked rearrangement is pinned to the token
recurrence for several chunk sizes, including chunk size 1, where A = I and the
chunked form is the recurrence by inspection.
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(1234)


def rand_problem(B, T, Hq, Hv, K, V, rng, varlen=None, gmin=-1.0):
    if varlen is not None:
        B, T = 1, int(sum(varlen))
    q = rng.normal(size=(B, T, Hq, K))
    k = rng.normal(size=(B, T, Hq, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(B, T, Hv, V))
    g = gmin * rng.random(size=(B, T, Hv))
    beta = rng.random(size=(B, T, Hv))
    N = len(varlen) if varlen is not None else B
    h0 = rng.normal(size=(N, Hv, K, V))
    cu = None if varlen is None else np.concatenate([[0], np.cumsum(varlen)]).astype(np.int64)
    return dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=h0, cu_seqlens=cu)


def loss(d, do, dht, scale):
    o, ht = oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale,
                       initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    return float(np.sum(o * do) + np.sum(ht * dht))


FD_CASES = [dict(B=2, T=t) for t in (1, 2, 3, 5, 9)] + [dict(varlen=[4, 5]), dict(varlen=[3, 0, 6])]


@pytest.mark.parametrize("case", FD_CASES, ids=lambda c: str(c))
def test_backward_matches_finite_differences(case):
    rng = np.random.default_rng(7)
    d = rand_problem(case.get("B", 1), case.get("T", 0), 1, 2, 3, 4, rng, varlen=case.get("varlen"))
    scale = 0.6
    o, ht = oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale,
                       initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    do = rng.normal(size=o.shape)
    dht = rng.normal(size=ht.shape)
    grads = oracle.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, do,
                       initial_state=d["initial_state"], dht=dht, cu_seqlens=d["cu_seqlens"])
    names = ["q", "k", "v", "beta", "g", "initial_state"]
    gidx = {"q": 0, "k": 1, "v": 2, "beta": 3, "g": 4, "initial_state": 5}
    eps = 1e-6
    for name in names:
        x = d[name]
        an = grads[gidx[name]]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[idx]
            x[idx] = orig + eps
            lp = loss(d, do, dht, scale)
            x[idx] = orig - eps
            lm = loss(d, do, dht, scale)
            x[idx] = orig
            fd[idx] = (lp - lm) / (2 * eps)
        scl = max(1.0, np.abs(fd).max())
        assert np.abs(fd - an).max() <= 1e-7 * scl, (name, np.abs(fd - an).max())


def test_beta_zero_closed_form():
    """beta = 0 leaves only decay: S_t = e^{G_t} S_0 with G the running sum of g."""
    rng = np.random.default_rng(3)
    B, T, H, K, V = 2, 37, 2, 5, 6
    d = rand_problem(B, T, H, H, K, V, rng)
    d["beta"][:] = 0.0
    scale = 0.4
    q, k, v, g, S0 = d["q"], d["k"], d["v"], d["g"], d["initial_state"]
    o, ht = oracle.fwd(q, k, v, g, d["beta"], scale, initial_state=S0)
    Gc = np.cumsum(g, axis=1)                              # [B,T,H]
    o_ref = scale * np.exp(Gc)[..., None] * np.einsum("bhkv,bthk->bthv", S0, q)
    ht_ref = np.exp(Gc[:, -1])[..., None, None] * S0
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht, ht_ref, rtol=1e-12, atol=1e-12)

    do = rng.normal(size=o.shape)
    dht = rng.normal(size=ht.shape)
    dq, dk, dv, db, dg, dh0 = oracle.bwd(q, k, v, g, d["beta"], scale, do, initial_state=S0, dht=dht)
    eG = np.exp(Gc)
    GL = Gc[:, -1]
    dq_ref = scale * eG[..., None] * np.einsum("bhkv,bthv->bthk", S0, do)
    np.testing.assert_allclose(dq, dq_ref, rtol=1e-11, atol=1e-12)
    assert np.abs(dk).max() == 0.0 and np.abs(dv).max() == 0.0
    # dS_t = e^{G_L - G_t} dht + scale sum_{s >= t} e^{G_s - G_t} q_s do_s^T
    qdo = np.einsum("bshk,bshv->bshkv", q, do) * eG[..., None, None]       # e^{G_s} q_s do_s^T
    tail = np.flip(np.cumsum(np.flip(qdo, axis=1), axis=1), axis=1)        # sum_{s >= t}
    dS = (np.exp(GL)[:, None, :, None, None] * dht[:, None] + scale * tail) / eG[..., None, None]
    e = v - eG[..., None] * np.einsum("bhkv,bthk->bthv", S0, k)
    db_ref = np.einsum("bthk,bthkv,bthv->bth", k, dS, e)
    np.testing.assert_allclose(db, db_ref, rtol=1e-10, atol=1e-11)
    qSdo = np.einsum("bthk,bhkv,bthv->bth", q, S0, do) * eG * scale
    dg_ref = np.flip(np.cumsum(np.flip(qSdo, axis=1), axis=1), axis=1) \
        + (np.exp(GL) * np.einsum("bhkv,bhkv->bh", dht, S0))[:, None, :]
    np.testing.assert_allclose(dg, dg_ref, rtol=1e-10, atol=1e-11)
    dh0_ref = np.exp(GL)[..., None, None] * dht + scale * qdo.sum(axis=1)
    np.testing.assert_allclose(dh0, dh0_ref, rtol=1e-11, atol=1e-12)


def test_scalar_state_closed_form():
    """K = V = 1: s_t = e^{g_t}(1 - beta_t k_t^2) s_{t-1} + beta_t k_t v_t, a
    first-order linear recurrence with the closed form
    s_t = P_t s_0 + sum_{j<=t} (P_t / P_j) b_j,  P_t = prod_{i<=t} a_i."""
    rng = np.random.default_rng(5)
    T = 50
    q = rng.normal(size=(1, T, 1, 1))
    k = rng.uniform(-1, 1, size=(1, T, 1, 1))
    v = rng.normal(size=(1, T, 1, 1))
    g = -0.3 * rng.random(size=(1, T, 1))
    beta = rng.random(size=(1, T, 1))
    s0 = rng.normal(size=(1, 1, 1, 1))
    scale = 1.3
    o, ht = oracle.fwd(q, k, v, g, beta, scale, initial_state=s0)
    a = np.exp(g[0, :, 0]) * (1 - beta[0, :, 0] * k[0, :, 0, 0] ** 2)
    b = beta[0, :, 0] * k[0, :, 0, 0] * v[0, :, 0, 0]
    P = np.cumprod(a)
    s = P * s0.item() + P * np.cumsum(b / P)
    np.testing.assert_allclose(o[0, :, 0, 0], scale * q[0, :, 0, 0] * s, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(ht.item(), s[-1], rtol=1e-9)


def test_retrieval_property():
    """After writing (k_t, v_t), reading the state with k_t returns
    (1 - beta |k|^2) e^{g} S_{t-1}^T k_t + beta |k|^2 v_t; with |k| = 1 and
    beta = 1 it returns exactly v_t (the delta rule's overwrite)."""
    rng = np.random.default_rng(11)
    T, H, K, V = 12, 2, 6, 5
    d = rand_problem(1, T, H, H, K, V, rng)
    k = d["k"] * rng.uniform(0.5, 1.5, size=(1, T, H, 1))     # not unit norm
    o, _ = oracle.fwd(k, k, d["v"], d["g"], d["beta"], 1.0, initial_state=d["initial_state"])
    for t in range(T):
        if t == 0:
            Sprev = d["initial_state"][0]
        else:
            _, hp = oracle.fwd(k[:, :t], k[:, :t], d["v"][:, :t], d["g"][:, :t], d["beta"][:, :t],
                               1.0, initial_state=d["initial_state"])
            Sprev = hp[0]
        for h in range(H):
            kt = k[0, t, h]
            n2 = kt @ kt
            b = d["beta"][0, t, h]
            ref = (1 - b * n2) * np.exp(d["g"][0, t, h]) * (Sprev[h].T @ kt) + b * n2 * d["v"][0, t, h]
            np.testing.assert_allclose(o[0, t, h], ref, rtol=1e-11, atol=1e-12)
    d["beta"][:] = 1.0
    o, _ = oracle.fwd(d["k"], d["k"], d["v"], d["g"], d["beta"], 1.0, initial_state=d["initial_state"])
    np.testing.assert_allclose(o, d["v"], rtol=1e-11, atol=1e-12)


def test_linear_in_values_and_state():
    rng = np.random.default_rng(13)
    d = rand_problem(2, 21, 1, 2, 4, 3, rng)
    v2 = rng.normal(size=d["v"].shape)
    h2 = rng.normal(size=d["initial_state"].shape)
    a, b = 0.7, -1.9
    args = (d["q"], d["k"])
    o1, s1 = oracle.fwd(*args, d["v"], d["g"], d["beta"], 0.5, initial_state=d["initial_state"])
    o2, s2 = oracle.fwd(*args, v2, d["g"], d["beta"], 0.5, initial_state=h2)
    o3, s3 = oracle.fwd(*args, a * d["v"] + b * v2, d["g"], d["beta"], 0.5,
                        initial_state=a * d["initial_state"] + b * h2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s3, a * s1 + b * s2, rtol=1e-11, atol=1e-11)


CHUNK_CASES = [
    dict(B=2, T=9, Hq=1, Hv=2, K=3, V=4, C=c) for c in (1, 2, 3, 64)
] + [
    dict(B=1, T=200, Hq=2, Hv=4, K=8, V=6, C=64),
    dict(varlen=[70, 1, 64, 129], Hq=2, Hv=2, K=5, V=7, C=64),
    dict(varlen=[5, 0, 11], Hq=1, Hv=3, K=4, V=4, C=4),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: str(c))
def test_chunked_form_equals_recurrence(case):
    rng = np.random.default_rng(17)
    d = rand_problem(case.get("B", 1), case.get("T", 0), case["Hq"], case["Hv"], case["K"],
                     case["V"], rng, varlen=case.get("varlen"))
    C = case["C"]
    kw = dict(initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], 0.8)
    o, ht = oracle.fwd(*args, **kw)
    gc, A, oc, h, htc = oracle.chunked_fwd(*args, chunk=C, **kw)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(htc, ht, rtol=1e-10, atol=1e-10)
    if C == 1:
        assert np.all(A == 1.0)        # a 1x1 unit-lower inverse
    do = rng.normal(size=o.shape)
    dht = rng.normal(size=ht.shape)
    r1 = oracle.bwd(*args[:5], 0.8, do, dht=dht, **kw)
    r2 = oracle.chunked_bwd(*args[:5], 0.8, do, chunk=C, dht=dht, **kw)
    for a, b in zip(r1, r2):
        np.testing.assert_allclose(b, a, rtol=1e-10, atol=1e-10)


def test_chunk_stage_tensors():
    """g_cum restarts at every chunk and sequence; A is unit lower triangular and
    inverts I + M; h[0] of each sequence is its initial state."""
    rng = np.random.default_rng(19)
    lens = [70, 3, 64]
    d = rand_problem(1, 0, 1, 2, 5, 3, rng, varlen=lens)
    C = 64
    gc, A, o, h, ht = oracle.chunked_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], 1.0, chunk=C,
                                         initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    cu = d["cu_seqlens"]
    offs = oracle.chunk_offsets(cu, C)
    assert h.shape[0] == offs[-1] == 4
    for n in range(len(lens)):
        np.testing.assert_array_equal(h[offs[n]], d["initial_state"][n])
        for s in range(cu[n], cu[n + 1], C):
            e = min(s + C, cu[n + 1])
            np.testing.assert_allclose(gc[0, s:e], np.cumsum(d["g"][0, s:e], axis=0), rtol=1e-14)
            Cc = e - s
            for hh in range(2):
                Ablk = A[0, s:e, hh, :Cc]
                assert np.allclose(np.triu(Ablk, 1), 0.0) and np.allclose(np.diag(Ablk), 1.0)
                assert np.all(A[0, s:e, hh, Cc:] == 0.0)
                kk = d["k"][0, s:e, 0]
                gam = gc[0, s:e, hh]
                M = np.tril(d["beta"][0, s:e, hh][:, None] * (kk @ kk.T)
                            * np.exp(gam[:, None] - gam[None, :]), -1)
                np.testing.assert_allclose(Ablk @ (np.eye(Cc) + M), np.eye(Cc), atol=1e-12)


def test_varlen_equals_per_sequence_runs():
    rng = np.random.default_rng(23)
    lens = [5, 0, 17, 9]
    d = rand_problem(1, 0, 2, 4, 3, 5, rng, varlen=lens)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], 0.9)
    o, ht = oracle.fwd(*args, initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    do = rng.normal(size=o.shape)
    dht = rng.normal(size=ht.shape)
    gp = oracle.bwd(*args[:5], 0.9, do, initial_state=d["initial_state"], dht=dht,
                    cu_seqlens=d["cu_seqlens"])
    cu = d["cu_seqlens"]
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        sub = [x[:, sl] for x in args[:5]]
        h0 = d["initial_state"][n:n + 1]
        on, hn = oracle.fwd(*sub, 0.9, initial_state=h0)
        np.testing.assert_array_equal(o[:, sl], on)
        np.testing.assert_array_equal(ht[n:n + 1], hn)
        gn = oracle.bwd(*sub, 0.9, do[:, sl], initial_state=h0, dht=dht[n:n + 1])
        for a, b in zip(gp[:5], gn[:5]):
            np.testing.assert_array_equal(a[:, sl], b)
        np.testing.assert_array_equal(gp[5][n:n + 1], gn[5])
        if lens[n] == 0:
            np.testing.assert_array_equal(hn, h0)
            np.testing.assert_array_equal(gn[5], dht[n:n + 1])


def test_grouped_value_heads_equal_repeated_heads():
    rng = np.random.default_rng(29)
    Hq, Hv = 2, 6
    G = Hv // Hq
    d = rand_problem(2, 13, Hq, Hv, 4, 3, rng)
    args = (d["v"], d["g"], d["beta"], 0.7)
    o, ht = oracle.fwd(d["q"], d["k"], *args, initial_state=d["initial_state"])
    qr = np.repeat(d["q"], G, axis=2)
    kr = np.repeat(d["k"], G, axis=2)
    o2, ht2 = oracle.fwd(qr, kr, *args, initial_state=d["initial_state"])
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(ht, ht2)
    do = rng.normal(size=o.shape)
    g1 = oracle.bwd(d["q"], d["k"], *args[:3], 0.7, do, initial_state=d["initial_state"])
    g2 = oracle.bwd(qr, kr, *args[:3], 0.7, do, initial_state=d["initial_state"])
    for i in (0, 1):
        sums = g2[i].reshape(2, 13, Hq, G, 4).sum(axis=3)
        np.testing.assert_allclose(g1[i], sums, rtol=1e-13, atol=1e-14)
    for a, b in zip(g1[2:], g2[2:]):
        np.testing.assert_array_equal(a, b)


def test_resume_from_final_state_is_bitwise():
    rng = np.random.default_rng(31)
    d = rand_problem(1, 150, 1, 2, 4, 5, rng)
    T1 = 67
    full = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    o, ht = oracle.fwd(*full, 0.5, initial_state=d["initial_state"])
    o1, h1 = oracle.fwd(*[x[:, :T1] for x in full], 0.5, initial_state=d["initial_state"])
    o2, h2 = oracle.fwd(*[x[:, T1:] for x in full], 0.5, initial_state=h1)
    np.testing.assert_array_equal(o, np.concatenate([o1, o2], axis=1))
    np.testing.assert_array_equal(ht, h2)
    do = rng.normal(size=o.shape)
    dht = rng.normal(size=ht.shape)
    gf = oracle.bwd(*full, 0.5, do, initial_state=d["initial_state"], dht=dht)
    g2 = oracle.bwd(*[x[:, T1:] for x in full], 0.5, do[:, T1:], initial_state=h1, dht=dht)
    g1 = oracle.bwd(*[x[:, :T1] for x in full], 0.5, do[:, :T1], initial_state=d["initial_state"],
                    dht=g2[5])
    for i in range(5):
        np.testing.assert_array_equal(gf[i], np.concatenate([g1[i], g2[i]], axis=1))
    np.testing.assert_array_equal(gf[5], g1[5])


def test_state_v_first_is_transpose():
    rng = np.random.default_rng(37)
    d = rand_problem(2, 10, 1, 2, 3, 5, rng)
    h0t = np.swapaxes(d["initial_state"], -1, -2).copy()
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], 0.5)
    o, ht = oracle.fwd(*args, initial_state=d["initial_state"])
    o2, ht2 = oracle.fwd(*args, initial_state=h0t, state_v_first=True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(np.swapaxes(ht, -1, -2), ht2)


def test_heads_mask_samples_units():
    rng = np.random.default_rng(41)
    d = rand_problem(2, 20, 2, 4, 3, 3, rng)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], 0.5)
    o, ht = oracle.fwd(*args, initial_state=d["initial_state"])
    o2, ht2 = oracle.fwd(*args, initial_state=d["initial_state"], heads=[2, 3])
    np.testing.assert_array_equal(o[:, :, 2:], o2[:, :, 2:])
    assert np.all(o2[:, :, :2] == 0)
    np.testing.assert_array_equal(ht[:, 2:], ht2[:, 2:])


# ---- use_qk_l2norm: the recurrence on per-(token, head) unit-length q and k ----

def _raw_qk(d, rng):
    """Rows of q and k with lengths spread over [1.5, 6] (not unit length)."""
    for name in ("q", "k"):
        x = d[name]
        x /= np.linalg.norm(x, axis=-1, keepdims=True)
        x *= rng.uniform(1.5, 6.0, size=x.shape[:-1] + (1,))
    return d


def test_l2norm_backward_matches_finite_differences():
    """dq and dk through the normalisation (and every other gradient) against
    central differences of the normalised forward."""
    rng = np.random.default_rng(11)
    d = _raw_qk(rand_problem(1, 0, 1, 2, 3, 4, rng, varlen=[3, 4]), rng)
    scale = 0.7
    o, ht = oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale,
                       initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
                       use_qk_l2norm=True)
    do = rng.normal(size=o.shape)
    dht = rng.normal(size=ht.shape)

    def L():
        o, ht = oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale,
                           initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
                           use_qk_l2norm=True)
        return float(np.sum(o * do) + np.sum(ht * dht))

    grads = oracle.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, do,
                       initial_state=d["initial_state"], dht=dht, cu_seqlens=d["cu_seqlens"],
                       use_qk_l2norm=True)
    eps = 1e-6
    for gi, name in enumerate(["q", "k", "v", "beta", "g", "initial_state"]):
        x = d[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[idx]
            x[idx] = orig + eps
            lp = L()
            x[idx] = orig - eps
            lm = L()
            x[idx] = orig
            fd[idx] = (lp - lm) / (2 * eps)
        scl = max(1.0, np.abs(fd).max())
        assert np.abs(fd - grads[gi]).max() <= 1e-7 * scl, (name, np.abs(fd - grads[gi]).max())


def test_l2norm_scale_invariance():
    """Scaling rows of q and k by positive factors leaves the normalised
    recurrence unchanged (up to eps / |x|^2 < 1e-6) and divides dq, dk by the
    factors; without the option the output changes."""
    rng = np.random.default_rng(12)
    d = _raw_qk(rand_problem(2, 6, 2, 4, 8, 5, rng), rng)
    scale = 0.5
    cq = rng.uniform(1.0, 4.0, size=d["q"].shape[:-1] + (1,))
    ck = rng.uniform(1.0, 4.0, size=d["k"].shape[:-1] + (1,))
    args = (d["v"], d["g"], d["beta"], scale)
    o1, h1 = oracle.fwd(d["q"], d["k"], *args, initial_state=d["initial_state"], use_qk_l2norm=True)
    o2, h2 = oracle.fwd(cq * d["q"], ck * d["k"], *args, initial_state=d["initial_state"],
                        use_qk_l2norm=True)
    assert np.abs(o1 - o2).max() <= 1e-6 * np.abs(o1).max()
    assert np.abs(h1 - h2).max() <= 1e-6 * np.abs(h1).max()
    o3, _ = oracle.fwd(cq * d["q"], ck * d["k"], *args, initial_state=d["initial_state"])
    assert np.abs(o1 - o3).max() > 1e-2 * np.abs(o1).max()
    do = rng.normal(size=o1.shape)
    g1 = oracle.bwd(d["q"], d["k"], *args, do, initial_state=d["initial_state"], use_qk_l2norm=True)
    g2 = oracle.bwd(cq * d["q"], ck * d["k"], *args, do, initial_state=d["initial_state"],
                    use_qk_l2norm=True)
    assert np.abs(g1[0] - cq * g2[0]).max() <= 1e-6 * np.abs(g1[0]).max()
    assert np.abs(g1[1] - ck * g2[1]).max() <= 1e-6 * np.abs(g1[1]).max()
    for i in (2, 3, 4):
        assert np.abs(g1[i] - g2[i]).max() <= 1e-6 * np.abs(g1[i]).max()


def test_l2norm_on_unit_rows_is_the_plain_recurrence():
    """Unit-length rows: the option changes nothing beyond the 1e-6 eps, in
    either direction (dq, dk lose only their component along q, k)."""
    rng = np.random.default_rng(13)
    d = rand_problem(1, 7, 1, 2, 6, 3, rng)
    d["q"] /= np.linalg.norm(d["q"], axis=-1, keepdims=True)
    scale = 0.9
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], scale)
    o1, h1 = oracle.fwd(*args, initial_state=d["initial_state"], use_qk_l2norm=True)
    o0, h0 = oracle.fwd(*args, initial_state=d["initial_state"])
    assert np.abs(o1 - o0).max() <= 2e-6 * np.abs(o0).max()
    assert np.abs(h1 - h0).max() <= 2e-6 * np.abs(h0).max()
    do = rng.normal(size=o0.shape)
    g1 = oracle.bwd(*args, do, initial_state=d["initial_state"], use_qk_l2norm=True)
    g0 = oracle.bwd(*args, do, initial_state=d["initial_state"])
    for x, i in ((d["q"], 0), (d["k"], 1)):
        proj = g0[i] - x * np.sum(x * g0[i], axis=-1, keepdims=True)
        assert np.abs(g1[i] - proj).max() <= 2e-6 * np.abs(g0[i]).max()
    for i in (2, 3, 4, 5):
        assert np.abs(g1[i] - g0[i]).max() <= 2e-6 * np.abs(g0[i]).max()


def test_l2norm_gradient_is_orthogonal_to_the_input():
    """The loss does not change along q or k, so dq . q = dk . k = 0 per row
    (up to the eps term, relative size eps / |x|^2)."""
    rng = np.random.default_rng(14)
    d = _raw_qk(rand_problem(1, 9, 2, 2, 8, 4, rng), rng)
    o, _ = oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], 0.4,
                      initial_state=d["initial_state"], use_qk_l2norm=True)
    do = rng.normal(size=o.shape)
    gr = oracle.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], 0.4, do,
                    initial_state=d["initial_state"], use_qk_l2norm=True)
    for x, dx in ((d["q"], gr[0]), (d["k"], gr[1])):
        dots = np.abs(np.sum(x * dx, axis=-1))
        scl = np.linalg.norm(x, axis=-1) * np.linalg.norm(dx, axis=-1)
        assert np.all(dots <= 1e-6 * scl + 1e-300)
        assert np.all(np.linalg.norm(dx, axis=-1) > 0)


# ---- beta options: sigmoid(beta) and 2 beta (negative eigenvalues allowed) ----

@pytest.mark.parametrize("sig,neg", [(True, False), (False, True), (True, True)])
def test_beta_options_backward_matches_finite_differences(sig, neg):
    rng = np.random.default_rng(21)
    d = rand_problem(1, 0, 1, 2, 3, 4, rng, varlen=[4, 3])
    d["beta"] = rng.normal(size=d["beta"].shape) if sig else d["beta"]  # logits when sig
    scale = 0.8
    opts = dict(beta_sigmoid=sig, neg_eigval=neg)

    def fwd():
        return oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale,
                          initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], **opts)

    o, ht = fwd()
    do = rng.normal(size=o.shape)
    dht = rng.normal(size=ht.shape)

    def L():
        o, ht = fwd()
        return float(np.sum(o * do) + np.sum(ht * dht))

    grads = oracle.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, do,
                       initial_state=d["initial_state"], dht=dht, cu_seqlens=d["cu_seqlens"],
                       **opts)
    eps = 1e-6
    for gi, name in enumerate(["q", "k", "v", "beta", "g", "initial_state"]):
        x = d[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[idx]
            x[idx] = orig + eps
            lp = L()
            x[idx] = orig - eps
            lm = L()
            x[idx] = orig
            fd[idx] = (lp - lm) / (2 * eps)
        scl = max(1.0, np.abs(fd).max())
        assert np.abs(fd - grads[gi]).max() <= 1e-7 * scl, (name, np.abs(fd - grads[gi]).max())


def test_neg_eigval_unit_beta_is_a_householder_reflection():
    """2 beta = 2, g = 0, v = 0 and unit k: the transition is I - 2 k k^T, a
    reflection, so the state's component along k flips sign and the same
    token applied twice restores the state exactly (up to rounding)."""
    rng = np.random.default_rng(22)
    K, V = 6, 4
    k1 = rng.normal(size=K)
    k1 /= np.linalg.norm(k1)
    k = np.tile(k1, (1, 2, 1, 1))                  # the same key twice, [1, 2, 1, K]
    q = rng.normal(size=(1, 2, 1, K))
    v = np.zeros((1, 2, 1, V))
    g = np.zeros((1, 2, 1))
    beta = np.ones((1, 2, 1))
    S0 = rng.normal(size=(1, 1, K, V))
    _, S1 = oracle.fwd(q[:, :1], k[:, :1], v[:, :1], g[:, :1], beta[:, :1], 1.0,
                       initial_state=S0, neg_eigval=True)
    np.testing.assert_allclose(k1 @ S1[0, 0], -(k1 @ S0[0, 0]), rtol=1e-12, atol=1e-12)
    P = np.eye(K) - np.outer(k1, k1)
    np.testing.assert_allclose(P @ S1[0, 0], P @ S0[0, 0], rtol=1e-12, atol=1e-12)
    _, S2 = oracle.fwd(q, k, v, g, beta, 1.0, initial_state=S0, neg_eigval=True)
    np.testing.assert_allclose(S2, S0, rtol=1e-12, atol=1e-12)
    # without the option the same token is a projection: applied twice = once
    _, P1 = oracle.fwd(q[:, :1], k[:, :1], v[:, :1], g[:, :1], beta[:, :1], 1.0, initial_state=S0)
    _, P2 = oracle.fwd(q, k, v, g, beta, 1.0, initial_state=S0)
    np.testing.assert_allclose(P2, P1, rtol=1e-12, atol=1e-12)


def test_beta_sigmoid_limits():
    """Logit 0 with negative eigenvalues gives beta = 1 (exact overwrite: a
    read with the written unit key returns v); a very negative logit gives
    beta -> 0, leaving only the decay."""
    rng = np.random.default_rng(23)
    d = rand_problem(1, 8, 2, 2, 5, 3, rng)
    zero = np.zeros_like(d["beta"])
    o, _ = oracle.fwd(d["k"], d["k"], d["v"], d["g"], zero, 1.0, initial_state=d["initial_state"],
                      beta_sigmoid=True, neg_eigval=True)
    np.testing.assert_allclose(o, d["v"], rtol=1e-11, atol=1e-12)
    o, ht = oracle.fwd(d["q"], d["k"], d["v"], d["g"], zero - 80.0, 0.5,
                       initial_state=d["initial_state"], beta_sigmoid=True)
    Gc = np.cumsum(d["g"], axis=1)
    o_ref = 0.5 * np.exp(Gc)[..., None] * np.einsum("bhkv,bthk->bthv", d["initial_state"], d["q"])
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)


# ---- gate activation: g = -exp(A_log) softplus(x + dt_bias) ----

def test_softplus_matches_library_routines():
    """The oracle's softplus against numpy's log-add-exp and torch's softplus
    (without its linear cut-off) over both tails and the middle."""
    import torch
    z = np.concatenate([np.linspace(-60.0, 60.0, 241), [-745.0, -1e-8, 0.0, 1e-8, 700.0]])
    sp = oracle.softplus(z)
    np.testing.assert_allclose(sp, np.logaddexp(0.0, z), rtol=1e-14, atol=0.0)
    ref = torch.nn.functional.softplus(torch.tensor(z, dtype=torch.float64), beta=1.0,
                                       threshold=1e4).numpy()
    np.testing.assert_allclose(sp, ref, rtol=1e-14, atol=0.0)
    assert np.all(sp >= 0.0)


def test_gate_closed_forms():
    """At x + dt_bias = 0 the log decay is -exp(A_log) ln 2; for large inputs
    softplus(z) -> z, for very negative ones -> e^z; every decay lies in (0, 1]
    and falls as x grows."""
    A_log = np.array([0.0, np.log(2.0), np.log(16.0)])
    dt_bias = np.array([0.0, -0.5, 3.0])
    x = -dt_bias[None, :] * np.ones((1, 3))
    np.testing.assert_allclose(oracle.gate_map(x, A_log, dt_bias),
                               -np.exp(A_log)[None, :] * np.log(2.0), rtol=1e-15)
    big = np.full((1, 3), 50.0) - dt_bias
    np.testing.assert_allclose(oracle.gate_map(big, A_log, dt_bias), -np.exp(A_log)[None, :] * 50.0,
                               rtol=1e-15)
    small = np.full((1, 3), -50.0) - dt_bias
    np.testing.assert_allclose(oracle.gate_map(small, A_log, dt_bias),
                               -np.exp(A_log)[None, :] * np.exp(-50.0), rtol=1e-14)
    xs = np.linspace(-20, 20, 81)[:, None] * np.ones((1, 3))
    g = oracle.gate_map(xs, A_log, dt_bias)
    assert np.all(g < 0.0) and np.all(np.diff(g, axis=0) < 0.0)
    # no dt_bias means a zero bias
    np.testing.assert_array_equal(oracle.gate_map(xs, A_log), oracle.gate_map(xs, A_log, np.zeros(3)))


@pytest.mark.parametrize("chunked", [False, True])
def test_gate_backward_matches_finite_differences(chunked):
    """Central differences of the loss with respect to every gate input x and
    both per-head parameters (and every other input), through the token
    recurrence and through the naive chunked form (chunk 2, ragged)."""
    rng = np.random.default_rng(31)
    d = rand_problem(1, 0, 1, 2, 3, 4, rng, varlen=[4, 3])
    d["g"] = rng.normal(size=d["g"].shape)              # raw gate inputs
    d["A_log"] = np.log(rng.uniform(1.0, 4.0, size=2))
    d["dt_bias"] = rng.normal(size=2)
    scale = 0.7

    def fwd():
        gate = (d["A_log"], d["dt_bias"])
        if chunked:
            r = oracle.chunked_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale, chunk=2,
                                   initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
                                   gate=gate)
            return r[2], r[4]
        return oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale,
                          initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], gate=gate)

    o, ht = fwd()
    do = rng.normal(size=o.shape)
    dht = rng.normal(size=ht.shape)

    def L():
        o, ht = fwd()
        return float(np.sum(o * do) + np.sum(ht * dht))

    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], scale, do)
    kw = dict(initial_state=d["initial_state"], dht=dht, cu_seqlens=d["cu_seqlens"],
              gate=(d["A_log"], d["dt_bias"]))
    grads = oracle.chunked_bwd(*args, chunk=2, **kw) if chunked else oracle.bwd(*args, **kw)
    assert len(grads) == 8
    eps = 1e-6
    names = ["q", "k", "v", "beta", "g", "initial_state", "A_log", "dt_bias"]
    for gi, name in enumerate(names):
        x = d[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[idx]
            x[idx] = orig + eps
            lp = L()
            x[idx] = orig - eps
            lm = L()
            x[idx] = orig
            fd[idx] = (lp - lm) / (2 * eps)
        scl = max(1.0, np.abs(fd).max())
        assert np.abs(fd - grads[gi]).max() <= 1e-7 * scl, (name, np.abs(fd - grads[gi]).max())
