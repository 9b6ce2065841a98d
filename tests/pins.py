"""Pins of the CPU oracle: closed forms and invariants the pages fix.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError when
the oracle disagrees with an independently computed result.  They are run on
the real oracle by ``test_oracle_pins.py`` and on deliberately broken copies of
it by ``test_oracle_mutants.py`` (every planted mistake must fail some pin).

The independent results never call the oracle's arithmetic: they are written
here from the mathematics, with numpy, in float64.
"""
from __future__ import annotations

import numpy as np

RTOL = 1e-12


def _softplus(v):
    return np.logaddexp(0.0, v)          # library routine: log(e^0 + e^v)


def _sigmoid(g):
    return 0.5 * (1.0 + np.tanh(0.5 * g))  # a different path from 1/(1+e^-g)


def _silu(z):
    return z * _sigmoid(z)


def _close(a, b, rtol=RTOL, atol=1e-14, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if not np.allclose(a, b, rtol=rtol, atol=atol):
        err = np.max(np.abs(a - b) / (atol + rtol * np.abs(b)))
        raise AssertionError("%s: mismatch (worst %.3g of tolerance)" % (what, err))


def _rand_problem(rng, batch=2, D=3, N=4, L=24, a_spread=True):
    x = rng.standard_normal((batch, D, L))
    dt = 0.5 * rng.standard_normal((batch, D, L))
    z = rng.standard_normal((batch, D, L))
    B = rng.standard_normal((batch, N, L))
    C = rng.standard_normal((batch, N, L))
    if a_spread:
        A = -rng.uniform(0.2, 3.0, (D, N))
    else:
        A = -np.tile(np.arange(1.0, N + 1.0), (D, 1))
    Dskip = rng.normal(1.0, 0.3, D)
    bias = np.log(np.expm1(rng.uniform(1e-3, 1e-1, D)))
    h0 = rng.standard_normal((batch, D, N))
    return dict(x=x, dt=dt, z=z, B=B, C=C, A=A, Dskip=Dskip, dt_bias=bias, h0=h0)


# --- P1: Theorem 1 (reader's notes, "Main results (verified)"): with N = 1,
# A = -1, B = 1 the selective SSM is the gated RNN h_t = (1-g_t) h_{t-1} + g_t x_t,
# g_t = sigmoid(pre-activation).  Under ZOH, exp(-softplus(g)) = 1 - sigmoid(g) and
# (1 - exp(-softplus(g))) = sigmoid(g), so the identity is exact; under Euler the
# input weight is softplus(g) instead of sigmoid(g).
def pin_theorem1(o):
    rng = np.random.default_rng(101)
    batch, D, L = 2, 3, 40
    g = 2.0 * rng.standard_normal((batch, D, L))
    x = rng.standard_normal((batch, D, L))
    h0 = rng.standard_normal((batch, D, 1))
    ones_bl = np.ones((batch, 1, L))
    A = -np.ones((D, 1))
    for zoh in (True, False):
        y, hf = o.scan(x, g, ones_bl, ones_bl, A, h0=h0, zoh=zoh)
        h = h0[..., 0].copy()
        ref = np.empty_like(x)
        for t in range(L):
            keep = _sigmoid(-g[..., t])                       # 1 - sigmoid(g)
            w = _sigmoid(g[..., t]) if zoh else _softplus(g[..., t])
            h = keep * h + w * x[..., t]
            ref[..., t] = h
        _close(y, ref, what="theorem 1 (%s)" % ("zoh" if zoh else "euler"))
        _close(hf[..., 0], h, what="theorem 1 final state")


# --- P2: the two limits of the step size (same notes, the remark after Theorem 1).
# As Delta goes to 0 the decay exp(Delta A) tends to 1 and the input weight to 0, so
# the state stays where it was and the token is not taken in; as Delta grows the
# decay vanishes and the state becomes the token's own input term, forgetting the past.
def pin_delta_limits(o):
    rng = np.random.default_rng(102)
    p = _rand_problem(rng, L=16)
    # small Delta: dt = -40 -> Delta ~ 4e-18 (with the bias adding at most ~-2)
    dt = np.full_like(p["x"], -40.0)
    y, hf = o.scan(p["x"], dt, p["B"], p["C"], p["A"], Dskip=p["Dskip"], dt_bias=p["dt_bias"], h0=p["h0"])
    _close(hf, p["h0"], rtol=1e-12, what="small delta keeps state")
    ref = np.einsum("bnt,bdn->bdt", p["C"], p["h0"]) + p["Dskip"][None, :, None] * p["x"]
    _close(y, ref, rtol=1e-12, atol=1e-12, what="small delta readout")
    # large Delta: dt = +40, A <= -0.2 -> Abar <= e^-8 ... use A <= -1 for e^-40
    A = -rng.uniform(1.0, 2.0, p["A"].shape)
    dt = np.full_like(p["x"], 40.0)
    zero_bias = np.zeros_like(p["dt_bias"])
    y1, hf1 = o.scan(p["x"], dt, p["B"], p["C"], A, dt_bias=zero_bias, h0=p["h0"])
    delta = _softplus(40.0)
    href = delta * p["B"][:, None, :, -1] * p["x"][:, :, -1, None]      # (b, d, n)
    _close(hf1, href, rtol=1e-12, what="large delta resets state")
    # y_t for t >= 1 must not depend on h0 nor on x_{<t}
    x2 = p["x"].copy()
    x2[..., :-1] = rng.standard_normal(x2[..., :-1].shape)
    y2, _ = o.scan(p["x"], dt, p["B"], p["C"], A, dt_bias=zero_bias, h0=-3.0 * p["h0"])
    _close(y2[..., 1:], y1[..., 1:], rtol=1e-12, atol=1e-12, what="large delta forgets h0")
    y3, _ = o.scan(x2, dt, p["B"], p["C"], A, dt_bias=zero_bias, h0=p["h0"])
    _close(y3[..., -1], y1[..., -1], rtol=1e-12, atol=1e-12, what="large delta forgets past x")
    ref_last = delta * np.einsum("bn,bn->b", p["C"][..., -1], p["B"][..., -1])[:, None] * p["x"][..., -1]
    _close(y1[..., -1], ref_last, rtol=1e-12, what="large delta readout")


# --- P3: with Delta, B, C constant in time the system is time-invariant and the
# scan equals a convolution with kernel K_k = sum_n C_n Bbar_n Abar_n^k (reader's
# notes, "What they did": time variation is what rules out the convolution; the
# ablations run "constant B and C").  Brute force O(L^2), Abar^k = exp(k Delta A).
def pin_lti_convolution(o):
    rng = np.random.default_rng(103)
    batch, D, N, L = 2, 3, 4, 20
    x = rng.standard_normal((batch, D, L))
    z = rng.standard_normal((batch, D, L))
    dtc = 0.5 * rng.standard_normal((batch, D))
    dt = np.repeat(dtc[..., None], L, axis=-1)
    Bc = rng.standard_normal((batch, N))
    Cc = rng.standard_normal((batch, N))
    B = np.repeat(Bc[..., None], L, axis=-1)
    C = np.repeat(Cc[..., None], L, axis=-1)
    A = -rng.uniform(0.1, 2.0, (D, N))
    Dskip = rng.normal(1, 0.3, D)
    bias = rng.normal(-2, 0.5, D)
    h0 = rng.standard_normal((batch, D, N))
    for zoh in (False, True):
        y, hf = o.scan(x, dt, B, C, A, z=z, Dskip=Dskip, dt_bias=bias, h0=h0, zoh=zoh)
        ref = np.zeros_like(x)
        for b in range(batch):
            for d in range(D):
                delta = _softplus(dtc[b, d] + bias[d])
                a = A[d]
                bbar = (np.expm1(delta * a) / a if zoh else delta) * Bc[b]
                K = np.array([np.sum(Cc[b] * bbar * np.exp(k * delta * a)) for k in range(L)])
                for t in range(L):
                    conv = sum(K[k] * x[b, d, t - k] for k in range(t + 1))
                    init = np.sum(Cc[b] * np.exp((t + 1) * delta * a) * h0[b, d])
                    ref[b, d, t] = (conv + init + Dskip[d] * x[b, d, t]) * _silu(z[b, d, t])
        _close(y, ref, rtol=1e-11, atol=1e-13, what="LTI convolution (%s)" % ("zoh" if zoh else "euler"))


# --- P4: the unrolled ("attention view", Mamba-models page) form of the time-varying
# recurrence: y_t = sum_n C_tn [exp(A_n S_t) h0_n + sum_{s<=t} exp(A_n (S_t - S_s)) Bbar_sn x_s]
# + Dskip x_t, gated, with S_t = sum_{j<=t} Delta_j.  O(L^2 N), sums of Delta in the
# exponent instead of the oracle's running product of exps.
def pin_unrolled(o):
    rng = np.random.default_rng(104)
    p = _rand_problem(rng, batch=2, D=3, N=4, L=24)
    for zoh in (False, True):
        y, hf = o.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], z=p["z"], Dskip=p["Dskip"],
                       dt_bias=p["dt_bias"], h0=p["h0"], zoh=zoh)
        batch, D, L = p["x"].shape
        N = p["A"].shape[1]
        ref = np.zeros_like(p["x"])
        href = np.zeros((batch, D, N))
        for b in range(batch):
            for d in range(D):
                delta = _softplus(p["dt"][b, d] + p["dt_bias"][d])         # (L,)
                S = np.cumsum(delta)
                a = p["A"][d]                                              # (N,)
                for t in range(L):
                    acc = 0.0
                    hn = np.exp(a * S[t]) * p["h0"][b, d]
                    for s in range(t + 1):
                        bb = (np.expm1(delta[s] * a) / a) if zoh else delta[s]
                        hn = hn + np.exp(a * (S[t] - S[s])) * bb * p["B"][b, :, s] * p["x"][b, d, s]
                    acc = np.sum(p["C"][b, :, t] * hn)
                    ref[b, d, t] = (acc + p["Dskip"][d] * p["x"][b, d, t]) * _silu(p["z"][b, d, t])
                    if t == L - 1:
                        href[b, d] = hn
        _close(y, ref, rtol=1e-10, atol=1e-12, what="unrolled form (%s)" % ("zoh" if zoh else "euler"))
        _close(hf, href, rtol=1e-10, atol=1e-12, what="unrolled final state")


# --- P5: the N state components are independent recurrences coupled only by the
# readout sum (reader's notes: the state is D x N numbers).  With Dskip = 0 and no
# gate, y(N states) = sum_n y(scan with the single component n).
def pin_state_decomposition(o):
    rng = np.random.default_rng(105)
    p = _rand_problem(rng, N=5, L=18)
    y, hf = o.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], dt_bias=p["dt_bias"], h0=p["h0"])
    acc = np.zeros_like(y)
    for n in range(p["A"].shape[1]):
        yn, hn = o.scan(p["x"], p["dt"], p["B"][:, n:n + 1], p["C"][:, n:n + 1], p["A"][:, n:n + 1],
                        dt_bias=p["dt_bias"], h0=p["h0"][..., n:n + 1])
        acc += yn
        _close(hn[..., 0], hf[..., n], rtol=1e-14, atol=0, what="component state %d" % n)
    _close(y, acc, rtol=1e-12, atol=1e-14, what="sum over state components")


# --- P6: the state is the whole carried context (reader's notes: built from the input,
# kept apart from the parameters): scanning [0, L) equals scanning [0, L1) and then
# [L1, L) from the state reached at L1.
def pin_split_resume(o):
    rng = np.random.default_rng(106)
    p = _rand_problem(rng, L=30)
    kw = dict(z=p["z"], Dskip=p["Dskip"], dt_bias=p["dt_bias"])
    y, hf = o.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], h0=p["h0"], **kw)
    for L1 in (1, 13, 29):
        s1 = slice(0, L1)
        s2 = slice(L1, None)
        ya, ha = o.scan(p["x"][..., s1], p["dt"][..., s1], p["B"][..., s1], p["C"][..., s1], p["A"],
                        h0=p["h0"], z=p["z"][..., s1], Dskip=p["Dskip"], dt_bias=p["dt_bias"])
        yb, hb = o.scan(p["x"][..., s2], p["dt"][..., s2], p["B"][..., s2], p["C"][..., s2], p["A"],
                        h0=ha, z=p["z"][..., s2], Dskip=p["Dskip"], dt_bias=p["dt_bias"])
        _close(np.concatenate([ya, yb], axis=-1), y, rtol=1e-13, atol=1e-15, what="split at %d" % L1)
        _close(hb, hf, rtol=1e-13, atol=1e-15, what="resumed final state")


# --- P7: generation needs one state update per token (tellworld.net summary,
# "Architecture"): T decode steps reproduce the scan over the same T tokens.
def pin_decode_equals_scan(o):
    rng = np.random.default_rng(107)
    p = _rand_problem(rng, L=12)
    for zoh in (False, True):
        y, hf = o.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], z=p["z"], Dskip=p["Dskip"],
                       dt_bias=p["dt_bias"], h0=p["h0"], zoh=zoh)
        st = p["h0"].copy()
        for t in range(p["x"].shape[-1]):
            yt, st = o.state_update(st, p["x"][..., t], p["dt"][..., t], p["B"][..., t], p["C"][..., t],
                                    p["A"], z=p["z"][..., t], Dskip=p["Dskip"], dt_bias=p["dt_bias"], zoh=zoh)
            _close(yt, y[..., t], rtol=1e-13, atol=1e-15, what="decode step %d" % t)
        _close(st, hf, rtol=1e-13, atol=1e-15, what="decode final state")


# --- P8: linearity and the skip/gate special cases.
def pin_linearity_and_gate(o):
    rng = np.random.default_rng(108)
    p = _rand_problem(rng, L=16)
    base = dict(dt_bias=p["dt_bias"], Dskip=p["Dskip"])
    # without a gate, y is linear in (x, h0) jointly for fixed dt
    x2 = rng.standard_normal(p["x"].shape)
    h02 = rng.standard_normal(p["h0"].shape)
    a, b = 0.7, -1.9
    y1, h1 = o.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], h0=p["h0"], **base)
    y2, h2 = o.scan(x2, p["dt"], p["B"], p["C"], p["A"], h0=h02, **base)
    y3, h3 = o.scan(a * p["x"] + b * x2, p["dt"], p["B"], p["C"], p["A"], h0=a * p["h0"] + b * h02, **base)
    _close(y3, a * y1 + b * y2, rtol=1e-11, atol=1e-12, what="linearity in (x, h0)")
    _close(h3, a * h1 + b * h2, rtol=1e-11, atol=1e-12, what="linearity of the state")
    # C = 0: y = Dskip x silu(z)
    zeroC = np.zeros_like(p["C"])
    y, _ = o.scan(p["x"], p["dt"], p["B"], zeroC, p["A"], z=p["z"], h0=p["h0"], **base)
    _close(y, p["Dskip"][None, :, None] * p["x"] * _silu(p["z"]), rtol=1e-13, what="skip and gate with C = 0")
    # z = 0 closes the gate
    y, _ = o.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], z=np.zeros_like(p["z"]), h0=p["h0"], **base)
    assert np.all(y == 0.0), "z = 0 must give y = 0"
    # softplus: N = 1, A = 0 (Abar = 1), B = C = 1, x = 1, one token: y = Delta = softplus(dt + bias)
    v = np.concatenate([np.linspace(-60, 60, 241), [-1e-8, 0.0, 1e-8, 19.99, 20.01, 35.0]])
    nd = v.size
    one = np.ones((1, 1, 1))
    y, _ = o.scan(np.ones((1, nd, 1)), v.reshape(1, nd, 1), one, one, np.zeros((nd, 1)))
    _close(y[0, :, 0], _softplus(v), rtol=1e-14, atol=1e-300, what="softplus")
    try:
        import torch
        ref = torch.nn.functional.softplus(torch.tensor(v, dtype=torch.float64), threshold=100.0).numpy()
        _close(y[0, :, 0], ref, rtol=1e-14, atol=1e-300, what="softplus vs torch")
        zz = np.linspace(-50, 50, 201)
        ys, _ = o.scan(np.ones((1, zz.size, 1)), np.zeros((1, zz.size, 1)), one, np.zeros((1, 1, 1)),
                       np.zeros((zz.size, 1)), z=zz.reshape(1, -1, 1), Dskip=np.ones(zz.size))
        refs = torch.nn.functional.silu(torch.tensor(zz, dtype=torch.float64)).numpy()
        _close(ys[0, :, 0], refs, rtol=1e-14, atol=1e-300, what="silu vs torch")
    except ImportError:  # pragma: no cover - torch is part of the image
        pass
    # dt_bias enters inside the softplus: shifting dt by c and the bias by -c changes nothing
    c = 0.37
    ya, ha = o.scan(p["x"], p["dt"] + c, p["B"], p["C"], p["A"], z=p["z"], Dskip=p["Dskip"],
                    dt_bias=p["dt_bias"] - c, h0=p["h0"])
    yb, hb = o.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], z=p["z"], Dskip=p["Dskip"],
                    dt_bias=p["dt_bias"], h0=p["h0"])
    _close(ya, yb, rtol=1e-12, atol=1e-14, what="bias inside softplus")


# --- P9: channels and batch rows are independent (reader's notes: D x N state, one
# N-vector per channel; B and C shared across the channels of one sequence):
# permuting channels together with their parameters permutes the outputs exactly,
# and permuting batch rows together with their B, C rows does the same.
def pin_permutations(o):
    rng = np.random.default_rng(109)
    p = _rand_problem(rng, batch=3, D=5, N=3, L=10)
    kw = dict(z=p["z"], Dskip=p["Dskip"], dt_bias=p["dt_bias"], h0=p["h0"])
    y, hf = o.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], **kw)
    perm = np.array([3, 0, 4, 1, 2])
    yp, hp = o.scan(p["x"][:, perm], p["dt"][:, perm], p["B"], p["C"], p["A"][perm], z=p["z"][:, perm],
                    Dskip=p["Dskip"][perm], dt_bias=p["dt_bias"][perm], h0=p["h0"][:, perm])
    assert np.array_equal(yp, y[:, perm]) and np.array_equal(hp, hf[:, perm]), "channel permutation"
    bp = np.array([2, 0, 1])
    yb, hb = o.scan(p["x"][bp], p["dt"][bp], p["B"][bp], p["C"][bp], p["A"], z=p["z"][bp],
                    Dskip=p["Dskip"], dt_bias=p["dt_bias"], h0=p["h0"][bp])
    assert np.array_equal(yb, y[bp]) and np.array_equal(hb, hf[bp]), "batch permutation"
    # decode obeys the same permutations
    yd, sd = o.state_update(p["h0"], p["x"][..., 0], p["dt"][..., 0], p["B"][..., 0], p["C"][..., 0], p["A"],
                            z=p["z"][..., 0], Dskip=p["Dskip"], dt_bias=p["dt_bias"])
    ydp, sdp = o.state_update(p["h0"][:, perm], p["x"][:, perm, 0], p["dt"][:, perm, 0], p["B"][..., 0],
                              p["C"][..., 0], p["A"][perm], z=p["z"][:, perm, 0], Dskip=p["Dskip"][perm],
                              dt_bias=p["dt_bias"][perm])
    assert np.array_equal(ydp, yd[:, perm]) and np.array_equal(sdp, sd[:, perm]), "decode permutation"


# --- P10: one decode step against the written-out formula, all terms present, for a
# few hand-chosen values (state keep/reset and the gate at both ends).
def pin_decode_formula(o):
    rng = np.random.default_rng(110)
    batch, D, N = 2, 4, 3
    st = rng.standard_normal((batch, D, N))
    x = rng.standard_normal((batch, D))
    dt = np.array([[-30.0, -1.0, 0.5, 30.0], [0.0, -3.0, 2.0, 10.0]])
    z = np.array([[-40.0, -0.5, 0.0, 3.0], [1.0, 2.0, -2.0, 40.0]])
    B = rng.standard_normal((batch, N))
    C = rng.standard_normal((batch, N))
    A = -rng.uniform(0.5, 2.0, (D, N))
    Dskip = rng.normal(1, 0.3, D)
    bias = rng.normal(0, 0.2, D)
    for zoh in (False, True):
        y, s1 = o.state_update(st, x, dt, B, C, A, z=z, Dskip=Dskip, dt_bias=bias, zoh=zoh)
        delta = _softplus(dt + bias[None])                             # (b, d)
        abar = np.exp(delta[..., None] * A[None])                      # (b, d, n)
        if zoh:
            bbar = np.expm1(delta[..., None] * A[None]) / A[None]
        else:
            bbar = np.broadcast_to(delta[..., None], abar.shape)
        sref = abar * st + bbar * B[:, None, :] * x[..., None]
        yref = (np.einsum("bdn,bn->bd", sref, C) + Dskip[None] * x) * _silu(z)
        _close(s1, sref, rtol=1e-13, atol=1e-15, what="decode state formula")
        _close(y, yref, rtol=1e-12, atol=1e-14, what="decode output formula")


# --- Backward pass.  Training differentiates the scan, recomputing the state in
# the backward pass (reader's notes, "What they did", Selective SSM item).  The
# oracle's gradients are pinned without re-deriving them: by central finite
# differences of the oracle's own forward scan (which the pins above fix), and by
# exact identities that follow from the scan being linear in some inputs.

def _loss_and_inputs(rng, zoh, tiny_a=False, zero_a=False):
    p = _rand_problem(rng, batch=2, D=3, N=4, L=9)
    if tiny_a:
        # Delta ~ 2-3 and |A| <= 2.5e-4: |Delta A| < 1e-3 (the series branch), with the
        # ZOH term of dA (order Delta^2) comparable to the decay term
        p["dt"] += 2.5
        p["A"][:, 1] = -rng.uniform(1e-4, 2.5e-4, 3)
    if zero_a:
        p["A"][0, 2] = 0.0
    dy = rng.standard_normal(p["x"].shape)
    dhf = rng.standard_normal(p["h0"].shape)
    return p, dy, dhf


_GRAD_OF = {"x": "dx", "dt": "ddt", "z": "dz", "B": "dB", "C": "dC", "A": "dA", "Dskip": "dDskip",
            "dt_bias": "ddt_bias", "h0": "dh0"}


def _fd_check(o, p, dy, dhf, zoh, what):
    def loss(q):
        y, hf = o.scan(q["x"], q["dt"], q["B"], q["C"], q["A"], z=q["z"], Dskip=q["Dskip"], dt_bias=q["dt_bias"],
                       h0=q["h0"], zoh=zoh)
        return float(np.sum(dy * y) + np.sum(dhf * hf))

    g = o.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], dy, z=p["z"], Dskip=p["Dskip"],
                   dt_bias=p["dt_bias"], h0=p["h0"], dh_final=dhf, zoh=zoh)
    for name, gname in _GRAD_OF.items():
        base = p[name]
        fd = np.empty_like(base)
        for idx in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[idx]))
            q = dict(p)
            q[name] = base.copy()
            q[name][idx] = base[idx] + eps
            lp = loss(q)
            q[name][idx] = base[idx] - eps
            lm = loss(q)
            fd[idx] = (lp - lm) / (2.0 * eps)
        _close(g[gname], fd, rtol=1e-6, atol=1e-7, what="%s: d/d%s vs finite differences" % (what, name))


# B1: every gradient against central finite differences of the forward scan,
# both discretisations, with gate, skip, bias, h0 and a final-state gradient.
def pin_bwd_finite_differences(o):
    rng = np.random.default_rng(120)
    for zoh in (False, True):
        p, dy, dhf = _loss_and_inputs(rng, zoh)
        _fd_check(o, p, dy, dhf, zoh, "zoh" if zoh else "euler")


# B2: the ZOH coefficient's derivative in A near A = 0 (series branch) and at A = 0.
def pin_bwd_zoh_small_a(o):
    rng = np.random.default_rng(121)
    p, dy, dhf = _loss_and_inputs(rng, True, tiny_a=True, zero_a=True)
    _fd_check(o, p, dy, dhf, True, "zoh small A")


# B3: exact identities.  Without a gate, (y, h_final) is linear in (x, h0)
# jointly for fixed dt, so <dy, y> + <dhf, h_final> = <dx, x> + <dh0, h0>.  With
# h0 = 0, (y - Dskip x, h_final) is linear in B; y - Dskip x is linear in C; and
# y depends on Dskip only through Dskip x.
def pin_bwd_linear_identities(o):
    rng = np.random.default_rng(122)
    for zoh in (False, True):
        p = _rand_problem(rng, batch=2, D=5, N=3, L=17)
        dy = rng.standard_normal(p["x"].shape)
        dhf = rng.standard_normal(p["h0"].shape)
        kw = dict(Dskip=p["Dskip"], dt_bias=p["dt_bias"], zoh=zoh)
        y, hf = o.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], h0=p["h0"], **kw)
        g = o.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], dy, h0=p["h0"], dh_final=dhf, **kw)
        lhs = np.sum(dy * y) + np.sum(dhf * hf)
        _close(np.sum(g["dx"] * p["x"]) + np.sum(g["dh0"] * p["h0"]), lhs, rtol=1e-12, what="adjoint in (x, h0)")
        skip_part = p["Dskip"][None, :, None] * p["x"]
        _close(np.sum(g["dDskip"] * p["Dskip"]), np.sum(dy * skip_part), rtol=1e-12, what="adjoint in Dskip")
        y0, hf0 = o.scan(p["x"], p["dt"], p["B"], p["C"], p["A"], **kw)
        g0 = o.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], dy, dh_final=dhf, **kw)
        _close(np.sum(g0["dB"] * p["B"]), np.sum(dy * (y0 - skip_part)) + np.sum(dhf * hf0), rtol=1e-12,
               what="adjoint in B")
        _close(np.sum(g0["dC"] * p["C"]), np.sum(dy * (y0 - skip_part)), rtol=1e-12, what="adjoint in C")


# B4: an empty sequence passes dh_final straight to dh0 and has no other gradient;
# a single token with a huge dt forgets h0 (dh0 -> 0) while dx stays finite.
def pin_bwd_edges(o):
    rng = np.random.default_rng(123)
    p = _rand_problem(rng, batch=2, D=3, N=4, L=0)
    dhf = rng.standard_normal(p["h0"].shape)
    g = o.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], np.zeros(p["x"].shape), z=p["z"], h0=p["h0"],
                   dh_final=dhf)
    _close(g["dh0"], dhf, rtol=0, atol=0, what="empty sequence dh0")
    assert not np.any(g["dA"]) and not np.any(g["dDskip"]) and not np.any(g["ddt_bias"]), "empty sequence"
    p = _rand_problem(rng, batch=1, D=2, N=3, L=1)
    p["dt"][:] = 40.0
    p["A"] = -1.0 - np.abs(p["A"])        # Delta A <= -40: Abar < 5e-18
    g = o.scan_bwd(p["x"], p["dt"], p["B"], p["C"], p["A"], np.ones(p["x"].shape), h0=p["h0"])
    assert np.all(np.abs(g["dh0"]) < 1e-15) and np.all(np.isfinite(g["dx"])), "large Delta forgets h0"


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_zoh_small_a, pin_bwd_linear_identities, pin_bwd_edges]

ALL_PINS = [pin_theorem1, pin_delta_limits, pin_lti_convolution, pin_unrolled,
            pin_state_decomposition, pin_split_resume, pin_decode_equals_scan,
            pin_linearity_and_gate, pin_permutations, pin_decode_formula] + BWD_PINS
