"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError on failure, so the
same pins run against the real oracle (tests/test_oracle_pins.py) and against
builds with one planted mistake each (tests/test_oracle_mutants.py), which must
each fail at least one pin.

What pins what:
  - decode: printed tables (tests/golden) for bf16 and E2M1, exhaustive
    16 codes x 255 scales, the nibble-order reading, quantize->decode identity;
  - quantizer: grid values round-trip over scales 0..252, hand-worked ties,
    saturation, sign-of-zero and clamp cases, byte equality with the input
    generator's independent numpy quantizer, fake-quant decode/idempotence/
    error bound, and MXFP4-vs-fake-quant layer equality;
  - backward: central finite differences of the loss sum(dy * y), torch
    float64 autograd of an independent implementation of the layer, the zero
    router gradient at E = 1, exact linearity in dy, bf16-vs-double entry;
  - route: brute force (an independent k-pass argmax over numpy logits),
    constructed exact ties, all-zero router, sum of weights, k=1, the k=2
    closed form, shift invariance, k=E full softmax;
  - permute: inverse identity, histogram prefix, equality with a stable sort;
  - experts + combine: E=1,k=1 reduces to the textbook dense SwiGLU FFN (numpy
    matmuls, non-square H != I so a transposed operand shows), in bf16 and in
    MXFP4 (decoded independently from the golden E2M1 table), identical
    experts, k=E mixture, per-token independence, linearity in W_down,
    silu(0)=0, and a whole layer worked by hand;
  - packed MXFP4 order: hand-worked piece and scale positions
    (tests/golden/mxfp4_packed_positions.txt) and pack/unpack inverse both
    ways, unpack being an independent address-order walk.
"""
from __future__ import annotations

import math
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------- fixtures


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def golden_e2m1():
    return {int(c): float(v) for c, v in _golden_rows("e2m1_codes.txt")}


def golden_hand_layer():
    return {r[0]: [float(v) for v in r[1:]] for r in _golden_rows("hand_layer_h2_i2_e3_k2.txt")}


def _bf16(a):
    return synth.bf16_from_f32(np.asarray(a, np.float32))


def _rand_layer(seed, T, H, E, k, I, wfmt=0, w_std=0.05):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((T, H)))
    wr = _bf16(rng.standard_normal((E, H)) * w_std)
    gu = rng.standard_normal((E, 2 * I, H)) * w_std
    dn = rng.standard_normal((E, H, I)) * w_std
    if wfmt == 0:
        w = synth.Weights(0, _bf16(gu), _bf16(dn))
    else:
        q = [synth.mxfp4_quantize(gu[e]) for e in range(E)]
        r = [synth.mxfp4_quantize(dn[e]) for e in range(E)]
        w = synth.Weights(1, np.stack([a for a, _ in q]), np.stack([a for a, _ in r]),
                          np.stack([b for _, b in q]), np.stack([b for _, b in r]))
    return x, wr, w


def _f64(b):
    return synth.f32_from_bf16(b).astype(np.float64)


def decode_independent(w: synth.Weights, which: str, e: int) -> np.ndarray:
    """Decode one expert matrix without the oracle: bf16 by widening, MXFP4 by
    the golden E2M1 table times 2^(S-127)."""
    if w.wfmt == 0:
        return _f64(getattr(w, which)[e])
    data = getattr(w, which)[e]
    scales = getattr(w, which + "_scale")[e]
    table = golden_e2m1()
    lut = np.array([table[c] for c in range(16)])
    codes = np.empty((data.shape[0], data.shape[1] * 2), np.int64)
    codes[:, 0::2] = data & 15
    codes[:, 1::2] = data >> 4
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return lut[codes] * np.repeat(sc, 32, axis=1)


def dense_swiglu(xf, wgu, wd):
    """Textbook dense SwiGLU FFN, numpy: (silu(X Wg^T) * (X Wu^T)) Wd^T."""
    I = wd.shape[1]
    g = xf @ wgu[:I].T
    u = xf @ wgu[I:].T
    return ((g / (1.0 + np.exp(-g))) * u) @ wd.T


def _close(a, b, rtol=1e-12, atol=1e-12):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if b.size else 0.0
    assert err <= atol + rtol * scale, f"max |diff| {err:.3e} > {atol + rtol * scale:.3e}"


# --------------------------------------------------------------------------- decode pins


def pin_bf16_golden(o):
    for hexbits, val in _golden_rows("bf16_values.txt"):
        got = o.bf16_value(int(hexbits, 16))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (hexbits, got, val)


def pin_e2m1_golden(o):
    for c, v in golden_e2m1().items():
        got = o.e2m1_value(c)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), (c, got, v)


def pin_mxfp4_exhaustive(o):
    """All 16 codes x 255 finite scales, through the matrix decoder, against
    golden E2M1 x 2^(S-127); S = 255 decodes to NaN."""
    table = golden_e2m1()
    codes = np.arange(16, dtype=np.uint8)
    for s in range(256):
        row = np.zeros((1, 16), np.uint8)  # 32 elements: code c at element 2c (low nibble)
        row[0, :] = codes
        sc = np.array([[s]], np.uint8)
        got = o.decode_matrix(1, row[None], sc[None], 1, 32, 0)[0]
        for c in range(16):
            if s == 255:
                assert math.isnan(got[2 * c]), (c, s)
            else:
                assert got[2 * c] == table[c] * math.ldexp(1.0, s - 127), (c, s, got[2 * c])
            if s != 255:
                assert got[2 * c + 1] == 0.0  # high nibbles hold code 0


def pin_mxfp4_nibble_order(o):
    """Element 2b is the low nibble of byte b, 2b+1 the high nibble; one scale
    per 32 elements along the row."""
    row = np.zeros((1, 1, 32), np.uint8)
    row[0, 0, 0] = 0x72   # element 0 -> code 2 (1.0), element 1 -> code 7 (6.0)
    row[0, 0, 16] = 0x9A  # element 32 -> code 10 (-1.0), element 33 -> code 9 (-0.5)
    sc = np.array([[[127, 130]]], np.uint8)  # block 0: 2^0, block 1: 2^3
    got = o.decode_matrix(1, row, sc, 1, 64, 0)[0]
    assert got[0] == 1.0 and got[1] == 6.0, got[:2]
    assert got[32] == -8.0 and got[33] == -4.0, got[32:34]


def pin_quantize_decode_identity(o):
    """Rows whose values lie on the MXFP4 grid (E2M1 value x 2^X, amax fixing
    X) survive the generator's quantizer and the oracle's decoder unchanged."""
    rng = np.random.default_rng(7)
    table = golden_e2m1()
    mags = np.array([table[c] for c in range(8)])
    rows = []
    for X in (-9, -5, 0, 3):
        v = rng.choice(mags, size=(4, 64)) * rng.choice([-1.0, 1.0], size=(4, 64))
        v[:, 0] = 6.0  # pins amax of block 0 so its shared exponent is X
        v[:, 32] = -4.0  # block 1: amax 4 -> exponent floor(log2 4)-2 = 0
        rows.append(v * math.ldexp(1.0, X))
    w = np.concatenate(rows)
    q, s = synth.mxfp4_quantize(w)
    back = o.decode_matrix(1, q[None], s[None], w.shape[0], w.shape[1], 0)
    assert np.array_equal(back, w)


# --------------------------------------------------------------------------- quantizer pins


def _bf16_exact(vals):
    """bf16 bits of doubles that are exactly bf16 values (checked)."""
    f = np.asarray(vals, np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(vals, np.float64)), "value not exact in fp32"
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def _codes_of(q):
    """Unpack [rows][cols/2] bytes into [rows][cols] codes (low nibble first)."""
    return np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[0], -1)


def pin_quantizer_grid_identity(o):
    """Grid values E2M1(c) x 2^(S-127), in blocks whose largest magnitude is 4
    or 6 (so floor(log2 amax) - 2 = S - 127), quantise back to the same codes
    and scale bytes; -0 becomes code 0.  Scales span 0..252 (bf16 subnormals
    at the bottom, near bf16's maximum at the top); decoded with the printed
    E2M1 table."""
    rng = np.random.default_rng(11)
    table = golden_e2m1()
    S = np.concatenate([np.arange(0, 253, 4), [1, 2, 3, 127, 250, 251, 252]]).astype(np.int64)
    nb = S.size
    codes = rng.integers(0, 16, size=(nb, 32))
    codes[:, 5] = rng.choice([6, 7, 14, 15], size=nb)  # amax is 4 or 6 times the scale
    vals = np.array([[table[int(c)] for c in row] for row in codes]) * np.ldexp(1.0, S - 127)[:, None]
    w = _bf16_exact(vals.reshape(1, -1))
    q, s = o.mxfp4_quantize(w)
    assert np.array_equal(s[0], S.astype(np.uint8)), (s[0], S)
    want = np.where(codes == 8, 0, codes).reshape(1, -1)
    assert np.array_equal(_codes_of(q), want)


def pin_quantizer_closed_forms(o):
    """Hand-worked blocks: every E2M1 midpoint goes to the even code, values
    past 6 saturate, the sign is dropped on code 0, all-zero blocks store scale
    byte 0, and the shared exponent follows floor(log2 amax) - 2 with the
    clamp at S = 0 below."""
    blocks, want_codes, want_S = [], [], []

    def block(vals, codes, S):
        v = np.zeros(32)
        c = np.zeros(32, np.int64)
        v[:len(vals)] = vals
        c[:len(codes)] = codes
        blocks.append(v)
        want_codes.append(c)
        want_S.append(S)

    # amax 4 -> X = 0: midpoints 0.25 .. 5 and their neighbours
    block([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 0.3125, 0.6875, 2.625, -3.375, 5.5],
          [6, 0, 2, 2, 4, 4, 6, 6, 0, 14, 1, 1, 5, 13, 7], 127)
    # amax 7.5 -> floor(log2) = 2, X = 0: saturation at 6
    block([7.5, -7.0, 6.5, 0.5], [7, 15, 7, 1], 127)
    # amax 5.125 * 2^-8 (about 0.02): floor(log2) = -6, X = -8, S = 119; the
    # elements 5.125, 2.5625, -1.28125 (times 2^-8) sit just past midpoints
    block([5.125 * 2.0 ** -8, 2.5625 * 2.0 ** -8, -1.28125 * 2.0 ** -8], [7, 5, 11], 119)
    # all zero, and all negative zero
    block([], [], 0)
    block([-0.0] * 32, [0] * 32, 0)
    # amax 2^-126 (smallest normal): X = -128 clamps to S = 0, element 2^-126 * 2^127 = 2
    block([2.0 ** -126, 2.0 ** -127], [4, 2], 0)
    # amax 2^-130 (bf16 subnormal): S = 0, element 2^-130 * 2^127 = 1/8 -> code 0
    block([2.0 ** -130], [0], 0)
    w = _bf16_exact(np.array(blocks).reshape(1, -1))
    q, s = o.mxfp4_quantize(w)
    assert list(s[0]) == want_S, (list(s[0]), want_S)
    assert np.array_equal(_codes_of(q)[0], np.concatenate(want_codes)), _codes_of(q)[0].reshape(-1, 32)[:3, :16]


def pin_quantizer_vs_generator(o):
    """On N(0, 0.02) weights and on values spread over 40 octaves, the oracle's
    quantiser agrees byte for byte with the input generator's numpy one (an
    independent implementation of the same rule: threshold search instead of
    a nearest-value scan)."""
    rng = np.random.default_rng(12)
    a = rng.standard_normal((8, 256)) * 0.02
    b = rng.standard_normal((8, 256)) * np.ldexp(1.0, rng.integers(-20, 20, size=(8, 256)))
    for m in (a, b):
        w = synth.bf16_from_f32(m.astype(np.float32))
        q, s = o.mxfp4_quantize(w)
        q2, s2 = synth.mxfp4_quantize(synth.f32_from_bf16(w).astype(np.float64))
        assert np.array_equal(s, s2) and np.array_equal(q, q2)


def pin_fakequant(o):
    """decode(quantize(w)) in bf16: equals the printed-table decode of the
    quantised bytes, is idempotent, and stays within one grid step: the error
    is at most 2^(S-127) (half the widest gap, 4..6) below the saturation
    point and at most 2^(S-126) past it."""
    rng = np.random.default_rng(13)
    table = golden_e2m1()
    w = synth.bf16_from_f32((rng.standard_normal((6, 128)) * 0.02).astype(np.float32))
    fq = o.mxfp4_fakequant(w)
    q, s = o.mxfp4_quantize(w)
    codes = _codes_of(q)
    dec = np.vectorize(lambda c: table[int(c)])(codes) * np.ldexp(1.0, s.astype(np.int64) - 127).repeat(32, axis=1)
    assert np.array_equal(fq, _bf16_exact(dec))
    assert np.array_equal(o.mxfp4_fakequant(fq), fq)
    err = np.abs(synth.f32_from_bf16(fq).astype(np.float64) - synth.f32_from_bf16(w).astype(np.float64))
    unit = np.ldexp(1.0, s.astype(np.int64) - 127).repeat(32, axis=1)
    assert np.all(err <= 2 * unit)


def pin_quantized_forward_equals_fakequant_forward(o):
    """The layer with MXFP4 weights quantize(W) and the layer with bf16 weights
    decode(quantize(W)) compute the same reals, so the oracle's outputs agree
    exactly (the quantiser and the MXFP4 decode path agree)."""
    T, H, E, k, I = 6, 64, 4, 2, 96
    rng = np.random.default_rng(14)
    x = _bf16(rng.standard_normal((T, H)))
    wr = _bf16(rng.standard_normal((E, H)) * 0.1)
    gu = _bf16(rng.standard_normal((E * 2 * I, H)) * 0.05)
    dn = _bf16(rng.standard_normal((E * H, I)) * 0.05)
    qgu, sgu = o.mxfp4_quantize(gu)
    qdn, sdn = o.mxfp4_quantize(dn)
    wq = synth.Weights(1, qgu.reshape(E, 2 * I, H // 2), qdn.reshape(E, H, I // 2), sgu.reshape(E, 2 * I, H // 32),
                       sdn.reshape(E, H, I // 32))
    wf = synth.Weights(0, o.mxfp4_fakequant(gu).reshape(E, 2 * I, H), o.mxfp4_fakequant(dn).reshape(E, H, I))
    tok = np.arange(T, dtype=np.int32)
    yq = o.forward_tokens(x, wr, wq, k, I, tok)[0]
    yf = o.forward_tokens(x, wr, wf, k, I, tok)[0]
    assert np.array_equal(yq, yf)


# --------------------------------------------------------------------------- backward pins


def _bwd_inputs(seed, T, H, E, k, I, scale=0.3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) * scale
    wgu = rng.standard_normal((E, 2 * I, H)) * scale
    wd = rng.standard_normal((E, H, I)) * scale
    dy = rng.standard_normal((T, H))
    return x, wr, wgu, wd, dy


def pin_backward_finite_differences(o):
    """Central differences of the oracle's own loss sum(dy * y) (double
    inputs, step 1e-6) match its analytic gradients on sampled entries of x,
    W_router, W_gate_up (gate and up rows) and W_down, at points where the
    routing does not change within the step."""
    T, H, E, k, I = 5, 8, 4, 2, 6
    x, wr, wgu, wd, dy = _bwd_inputs(21, T, H, E, k, I)
    dx, dwr, dgu, ddn, _, idx = o.backward_f64(x, wr, wgu, wd, dy, k)
    grads = {"x": dx, "wr": dwr, "wgu": dgu, "wd": ddn}
    rng = np.random.default_rng(22)
    eps = 1e-6
    for name in ("x", "wr", "wgu", "wd"):
        for _ in range(10):
            arrs = {"x": x.copy(), "wr": wr.copy(), "wgu": wgu.copy(), "wd": wd.copy()}
            pos = tuple(int(rng.integers(n)) for n in arrs[name].shape)
            lv = []
            for sgn in (1.0, -1.0):
                a = {kk: v.copy() for kk, v in arrs.items()}
                a[name][pos] += sgn * eps
                r = o.backward_f64(a["x"], a["wr"], a["wgu"], a["wd"], dy, k)
                assert np.array_equal(r[5], idx), "routing changed within the step"
                lv.append(r[4])
            fd = (lv[0] - lv[1]) / (2 * eps)
            g = grads[name][pos]
            assert abs(fd - g) <= 1e-6 * max(1.0, abs(g)), (name, pos, fd, g)


def _torch_layer_grads(x, wr, wgu, wd, dy, k):
    """The layer written again with torch float64 ops (top-k by a descending
    sort of the logits; inputs have no ties) and differentiated by autograd."""
    import torch
    t = {n: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for n, v in (("x", x), ("wr", wr), ("wgu", wgu), ("wd", wd))}
    I = wd.shape[2]
    logits = t["x"] @ t["wr"].T
    sel = torch.argsort(logits.detach(), dim=1, descending=True)[:, :k]
    w = torch.softmax(torch.gather(logits, 1, sel), dim=1)
    y = torch.zeros_like(t["x"])
    for j in range(k):
        e = sel[:, j]
        gu = torch.einsum("th,trh->tr", t["x"], t["wgu"][e])
        a = torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]
        o_ = torch.einsum("ti,thi->th", a, t["wd"][e])
        y = y + w[:, j:j + 1] * o_
    (y * torch.tensor(dy)).sum().backward()
    return [t[n].grad.numpy() for n in ("x", "wr", "wgu", "wd")], sel.numpy()


def pin_backward_torch_autograd(o):
    """All four gradients equal torch's autograd of an independent float64
    implementation of the layer, on a non-square shape (H != I) where most
    experts have tokens and one may have none."""
    T, H, E, k, I = 9, 12, 5, 2, 7
    x, wr, wgu, wd, dy = _bwd_inputs(23, T, H, E, k, I)
    dx, dwr, dgu, ddn, _, idx = o.backward_f64(x, wr, wgu, wd, dy, k)
    (tx, twr, tgu, tdn), sel = _torch_layer_grads(x, wr, wgu, wd, dy, k)
    assert np.array_equal(sel, idx)
    for got, want in ((dx, tx), (dwr, twr), (dgu, tgu), (ddn, tdn)):
        assert np.allclose(got, want, rtol=1e-10, atol=1e-12), float(np.max(np.abs(got - want)))


def pin_backward_special_cases(o):
    """E = 1, k = 1: the weight is 1 whatever the logit, so the router
    gradient is exactly zero; gradients are linear in dy (doubling dy doubles
    every gradient exactly); the bf16 entry point equals the double one on the
    same values."""
    x, wr, wgu, wd, dy = _bwd_inputs(24, 4, 6, 1, 1, 5)
    r = o.backward_f64(x, wr, wgu, wd, dy, 1)
    assert np.all(r[1] == 0.0)
    x, wr, wgu, wd, dy = _bwd_inputs(25, 6, 8, 4, 2, 8)
    a = o.backward_f64(x, wr, wgu, wd, dy, 2)
    b = o.backward_f64(x, wr, wgu, wd, 2.0 * dy, 2)
    for u, v in zip(a[:4], b[:4]):
        assert np.array_equal(2.0 * u, v)
    bf = [_bf16(v) for v in (x, wr, wgu, wd, dy)]
    dec = [synth.f32_from_bf16(v).astype(np.float64) for v in bf]
    c = o.backward(*bf, 2)
    d = o.backward_f64(*dec, 2)
    for u, v in zip(c, d[:4]):
        assert np.array_equal(u, v)


# --------------------------------------------------------------------------- route pins


def _kpass_argmax(l, k):
    """Independent top-k: k passes of argmax (numpy argmax returns the first,
    i.e. lowest-index, maximum), removing the winner each time."""
    l = l.copy()
    out = []
    for _ in range(k):
        j = int(np.argmax(l))
        out.append(j)
        l[j] = -np.inf
    return out


def pin_route_bruteforce(o):
    for seed, (T, H, E, k) in enumerate([(40, 24, 8, 3), (16, 64, 32, 4), (5, 32, 128, 4), (7, 16, 6, 6)]):
        x, wr, _ = _rand_layer(seed, T, H, E, k, 32)
        logits, idx, w = o.route(x, wr, k)
        ref = _f64(x) @ _f64(wr).T
        _close(logits, ref, rtol=1e-13)
        for t in range(T):
            assert list(idx[t]) == _kpass_argmax(ref[t], k), (t, idx[t])
            sel = ref[t, idx[t]]
            ew = np.exp(sel - sel.max())
            _close(w[t], ew / ew.sum(), rtol=1e-13)


def pin_route_exact_ties(o):
    """Duplicate router rows give exactly equal logits; the lower index wins
    and comes first.  Rows 2 and 5 become copies of the token's best row."""
    x, wr, _ = _rand_layer(11, 8, 32, 8, 3, 32)
    l = _f64(x) @ _f64(wr).T
    for t in range(x.shape[0]):
        best = int(np.argmax(l[t]))
        wr2 = wr.copy()
        wr2[2] = wr[best]
        wr2[5] = wr[best]
        _, idx, w = o.route(x[t:t + 1], wr2, 3)
        if best in (2, 5):
            assert list(idx[0][:2]) == [2, 5] and w[0][0] == w[0][1], (t, idx)
        else:
            assert list(idx[0]) == sorted([2, 5, best]), (t, best, idx)
            assert w[0][0] == w[0][1] == w[0][2], w


def pin_route_zero_router(o):
    x, _, _ = _rand_layer(3, 4, 16, 8, 3, 32)
    wr = np.zeros((8, 16), np.uint16)
    _, idx, w = o.route(x, wr, 3)
    assert (idx == np.array([0, 1, 2])).all()
    assert (w == 1.0 / 3.0).all()


def pin_route_weights(o):
    x, wr, _ = _rand_layer(5, 64, 48, 16, 4, 32, w_std=0.2)
    lg, idx, w = o.route(x, wr, 4)
    assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-12)
    assert np.all(w > 0) and np.all(np.diff(w, axis=1) <= 0)  # descending-logit slots
    _, idx1, w1 = o.route(x, wr, 1)
    assert (w1 == 1.0).all() and (idx1[:, 0] == idx[:, 0]).all()
    _, idx2, w2 = o.route(x, wr, 2)
    l0 = lg[np.arange(64), idx2[:, 0]]
    l1 = lg[np.arange(64), idx2[:, 1]]
    _close(w2[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-14)


def pin_route_shift_invariance(o):
    """A constant input channel with the same router weight c for every expert
    adds c to every logit: the selection and the weights do not change."""
    x, wr, _ = _rand_layer(9, 32, 31, 8, 3, 32)
    _, idx, w = o.route(x, wr, 3)
    xs = np.concatenate([x, np.full((32, 1), 0x3F80, np.uint16)], axis=1)  # channel of 1.0
    wrs = np.concatenate([wr, np.full((8, 1), 0x4040, np.uint16)], axis=1)  # c = 3.0
    _, idx2, w2 = o.route(xs, wrs, 3)
    assert (idx == idx2).all()
    _close(w2, w, rtol=1e-12)


def pin_route_k_equals_E(o):
    x, wr, _ = _rand_layer(13, 10, 40, 6, 6, 32, w_std=0.3)
    lg, idx, w = o.route(x, wr, 6)
    for t in range(10):
        assert sorted(idx[t]) == list(range(6))
        full = np.exp(lg[t] - lg[t].max())
        full /= full.sum()
        _close(w[t], full[idx[t]], rtol=1e-13)


def pin_route_nan_logits(o):
    """Reading for non-finite inputs: a NaN logit ranks below every number
    (as -infinity), ties still to the lower index.  A NaN in a token's row
    makes all its logits NaN: experts 0..k-1 in order, NaN weights.  A NaN in
    one expert's router row makes that expert's logit NaN for every token: it
    is never selected while k < E, and it comes last when k = E.  Checked
    against an independent k-pass argmax over numpy logits with NaN replaced
    by -inf, and other tokens must be unaffected."""
    x, wr, _ = _rand_layer(17, 12, 32, 8, 3, 32)
    nan = np.uint16(0x7FC0)
    xn = x.copy()
    xn[4, 7] = nan
    _, idx, w = o.route(xn, wr, 3)
    assert list(idx[4]) == [0, 1, 2] and np.isnan(w[4]).all(), (idx[4], w[4])
    _, idx0, w0 = o.route(x, wr, 3)
    keep = np.arange(12) != 4
    assert (idx[keep] == idx0[keep]).all() and np.array_equal(w[keep], w0[keep])
    wrn = wr.copy()
    wrn[1, 5] = nan
    ref = _f64(x) @ _f64(wrn).T
    ref = np.where(np.isnan(ref), -np.inf, ref)
    def kpass(l, k):  # k passes over the remaining experts: largest value, lowest index on ties
        left = list(range(len(l)))
        out = []
        for _ in range(k):
            j = max(left, key=lambda e: (l[e], -e))
            out.append(j)
            left.remove(j)
        return out

    for k in (3, 8):
        _, idx, w = o.route(x, wrn, k)
        for t in range(12):
            assert list(idx[t]) == kpass(ref[t], k), (k, t, idx[t])
            assert np.isfinite(w[t]).all() and abs(w[t].sum() - 1.0) <= 1e-12
        if k == 8:
            assert (idx[:, -1] == 1).all() and (w[:, -1] == 0.0).all()
        else:
            assert not (idx == 1).any()


def pin_route_near_ties(o):
    """Near ties decided by 2^-20 in logits near 512 (relative 2^-29) and an
    exact tie, on inputs whose logits are exact in fp64 in any order
    (synth.near_tie_router): every token must take A2, A1, B1, B2 in that
    order (the bump puts A2 before the lower-index A1; B1 and B2 tie exactly
    and the lower index goes first; C, 2^-20 below them, is fifth), and the
    logits must equal the exact sums computed in integers."""
    for T, H, E in [(6, 64, 32), (3, 40, 128)]:
        x, wr = synth.near_tie_router(T, H, E, seed=T)
        lg, idx, w = o.route(x, wr, 4)
        nt = synth.NEAR_TIE
        want = [nt["A2"], nt["A1"], nt["B1"], nt["B2"]]
        assert (idx == np.array(want)).all(), idx
        # exact logits in units of 2^-20 (x integers, router entries multiples of 2^-20)
        xi = np.rint(_f64(x)).astype(np.int64)
        wi = np.rint(_f64(wr) * 2.0 ** 20).astype(np.int64)
        exact = (xi @ wi.T).astype(np.float64) * 2.0 ** -20
        assert np.array_equal(lg, exact)
        _, idx5, _ = o.route(x, wr, 5)
        assert (idx5[:, 4] == nt["C"]).all()
        assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-12)


# --------------------------------------------------------------------------- permute pins


def pin_permute(o):
    rng = np.random.default_rng(21)
    for T, k, E in [(37, 4, 32), (1, 4, 128), (64, 2, 8), (0, 4, 8), (100, 1, 3)]:
        idx = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], np.int32).reshape(T, k)
        off, sp, pr = o.permute(idx, E)
        flat = idx.ravel()
        assert (off == np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))])).all()
        assert (sp == np.argsort(flat, kind="stable")).all()
        if T:
            assert (pr[sp] == np.arange(T * k)).all() and (sp[pr] == np.arange(T * k)).all()
            for e in range(E):
                seg = sp[off[e]:off[e + 1]]
                assert (np.diff(seg) > 0).all() and (flat[seg] == e).all()


# --------------------------------------------------------------------------- expert pins


def pin_dense_reduction(o):
    """E=1, k=1: the layer is the textbook dense SwiGLU FFN (weight 1)."""
    for wfmt in (0, 1):
        T, H, I = 9, 64, 96
        x, wr, w = _rand_layer(31 + wfmt, T, H, 1, 1, I, wfmt=wfmt)
        y, idx, wts = o.forward_tokens(x, wr, w, 1, I, np.arange(T))
        assert (idx == 0).all() and (wts == 1.0).all()
        ref = dense_swiglu(_f64(x), decode_independent(w, "gate_up", 0), decode_independent(w, "down", 0))
        _close(y, ref, rtol=1e-12)


def pin_identical_experts(o):
    """All experts equal: y is the dense FFN for any routing (weights sum to 1)."""
    T, H, E, k, I = 12, 32, 6, 3, 64
    x, wr, w = _rand_layer(41, T, H, E, k, I)
    w = synth.Weights(0, np.repeat(w.gate_up[:1], E, 0).copy(), np.repeat(w.down[:1], E, 0).copy())
    y, _, _ = o.forward_tokens(x, wr, w, k, I, np.arange(T))
    ref = dense_swiglu(_f64(x), _f64(w.gate_up[0]), _f64(w.down[0]))
    _close(y, ref, rtol=1e-12)


def pin_mixture_k_equals_E(o):
    """k = E: y = sum over all experts of full-softmax weight x expert FFN."""
    T, H, E, I = 6, 32, 4, 48
    x, wr, w = _rand_layer(43, T, H, E, E, I, w_std=0.1)
    y, _, _ = o.forward_tokens(x, wr, w, E, I, np.arange(T))
    xf = _f64(x)
    lg = xf @ _f64(wr).T
    p = np.exp(lg - lg.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = sum(p[:, e:e + 1] * dense_swiglu(xf, _f64(w.gate_up[e]), _f64(w.down[e])) for e in range(E))
    _close(y, ref, rtol=1e-12)


def pin_token_independence_and_pairs(o):
    """A token's output is the same alone or in a batch, and equals the
    weighted sum of its per-pair expert outputs."""
    T, H, E, k, I = 20, 32, 8, 2, 64
    x, wr, w = _rand_layer(47, T, H, E, k, I)
    y_all, idx, wts = o.forward_tokens(x, wr, w, k, I, np.arange(T))
    sub = np.array([3, 17, 4])
    y_sub, _, _ = o.forward_tokens(x, wr, w, k, I, sub)
    assert np.array_equal(y_sub, y_all[sub])
    y_one, _, _ = o.forward_tokens(x[5:6], wr, w, k, I, np.array([0]))
    assert np.array_equal(y_one[0], y_all[5])
    pt = np.repeat(np.arange(T), k)
    oo = o.ffn_pairs(x, w, I, E, pt, idx.ravel())
    ref = (wts.reshape(T, k, 1) * oo.reshape(T, k, H)).sum(1)
    _close(y_all, ref, rtol=1e-13)


def pin_linearity_and_silu_zero(o):
    T, H, E, k, I = 8, 32, 4, 2, 32
    x, wr, w = _rand_layer(53, T, H, E, k, I)
    y, _, _ = o.forward_tokens(x, wr, w, k, I, np.arange(T))
    w2 = synth.Weights(0, w.gate_up, _bf16(_f64(w.down) * 2.0))
    y2, _, _ = o.forward_tokens(x, wr, w2, k, I, np.arange(T))
    assert np.array_equal(y2, 2.0 * y)
    gz = w.gate_up.copy()
    gz[:, :I, :] = 0  # gate rows zero -> silu(0) = 0 -> y = 0
    y0, _, _ = o.forward_tokens(x, wr, synth.Weights(0, gz, w.down), k, I, np.arange(T))
    assert not np.any(y0)


def pin_hand_layer(o):
    g = golden_hand_layer()
    x = _bf16([g["x"]])
    wr = _bf16(np.array(g["router"]).reshape(3, 2))
    gu = _bf16(np.stack([np.array(g[f"gate_up_e{e}"]).reshape(4, 2) for e in range(3)]))
    dn = _bf16(np.stack([np.array(g[f"down_e{e}"]).reshape(2, 2) for e in range(3)]))
    y, idx, w = o.forward_tokens(x, wr, synth.Weights(0, gu, dn), 2, 2, np.array([0]))
    assert list(idx[0]) == [int(v) for v in g["topk_idx"]]
    _close(w[0], g["topk_w"], rtol=1e-15, atol=0)
    _close(y[0], g["y"], rtol=1e-14, atol=0)


# --------------------------------------------------------------------------- packed MXFP4 order


def _packed_tensor(seed, gate_up, E, I, H):
    R, K = (2 * I, H) if gate_up else (H, I)
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 256, (E, R, K // 2), dtype=np.uint8), rng.integers(0, 256, (E, R, K // 32), dtype=np.uint8))


def pin_packed_hand_positions(o):
    """Pieces land where the hand-worked fixture puts them."""
    for kind, E, I, H, e, r, kb, off, soff in _golden_rows("mxfp4_packed_positions.txt"):
        gate_up = kind == "gu"
        E, I, H, e, r, kb, off, soff = (int(v) for v in (E, I, H, e, r, kb, off, soff))
        w, s = _packed_tensor(7, gate_up, E, I, H)
        wp, sp = o.mxfp4_pack(gate_up, E, I, H, w, s)
        assert np.array_equal(wp.reshape(-1)[off:off + 16], w[e, r, 16 * kb:16 * kb + 16]), (kind, e, r, kb)
        assert sp.reshape(-1)[soff] == s[e, r, kb], (kind, e, r, kb)


def pin_packed_round_trip(o):
    """pack and unpack are inverse permutations, over K-block counts below,
    at and across one chunk (1, 3, 16, 17, 90) and both tensor kinds."""
    for gate_up, E, I, H in [(True, 2, 16, 32), (True, 1, 32, 96), (False, 2, 64, 512), (False, 1, 544, 32),
                             (True, 1, 48, 2880), (False, 1, 2880, 64)]:
        w, s = _packed_tensor(11, gate_up, E, I, H)
        wp, sp = o.mxfp4_pack(gate_up, E, I, H, w, s)
        w2, s2 = o.mxfp4_unpack(gate_up, E, I, H, wp, sp)
        assert np.array_equal(w2, w) and np.array_equal(s2, s), (gate_up, E, I, H)
        w3, s3 = o.mxfp4_pack(gate_up, E, I, H, *o.mxfp4_unpack(gate_up, E, I, H, w, s))
        assert np.array_equal(w3, w) and np.array_equal(s3, s), (gate_up, E, I, H)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
