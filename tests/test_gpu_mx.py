"""The MX path (MOE_PATH_TILED_MX): MXFP4 expert weights on the MX matrix
cores with the activations split into two MXFP6 (E2M3) terms.

- moe_mx_split against an independent numpy implementation of the split's
  definition (include/moe.h): scale bytes equal, codes equal (a code of zero
  may carry either sign: both encode 0), on N(0, 1) rows, rows spanning many
  octaves, exact E2M3 midpoints (ties to the even code), saturation, zero
  blocks and bf16 subnormals.
- The layer on the MX path against the oracle (MXFP4 weights, W4A16 exact):
  routing and permutation bit-exact, h, y_sorted and y within 1e-2 * max|ref|,
  for the 20b MXFP4 prefill (32768 tokens, 512 checked) and decode configs in
  the row-major and the packed order, and ragged shapes (segments over several
  256-token tiles and tails, output widths off the 256-row tile, a single
  64-wide K stage, E = 1, k = E).
- moe_forward and moe_grouped_ffn (h split inside the gate/up kernel) against
  the stage entry points (bf16 h, split by moe_down): identical bits."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_ffn_05_amd as moe
import oracle
import synth
from tests.gpu_layer import GpuLayer, bf16_dev_to_f64, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-2
MX = moe.MOE_PATH_TILED_MX

# E2M3 magnitudes by code 0..31 (sign bit 5, exponent bits 4:3 with bias 1,
# mantissa bits 2:0; exponent 0 is subnormal m/8)
E2M3 = np.array([(m / 8.0) if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 1) for e in range(4) for m in range(8)])


def _e2m3_round(v):
    """Nearest E2M3 magnitude index of |v| (ties to the even code), saturating."""
    a = np.abs(v)
    i = np.clip(np.searchsorted(E2M3, a), 1, 31)
    lo, hi = E2M3[i - 1], E2M3[i]
    up = (a - lo > hi - a) | ((a - lo == hi - a) & ((i - 1) % 2 == 1))
    code = np.where(up, i, i - 1)
    return np.where(a >= E2M3[31], 31, code)


def _scale_byte(amax):
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))), -200)
    return np.clip(e - 2 + 127, 1, 254).astype(np.int64)


def split_reference(x_bf16):
    """(codes [rows][K/32][48], scales [rows][K/32][2]) of the two-term split."""
    x = synth.f32_from_bf16(x_bf16).astype(np.float64)
    rows, K = x.shape
    b = x.reshape(rows, K // 32, 32)
    out_codes, out_scales = [], []
    for term in range(2):
        S = _scale_byte(np.abs(b).max(axis=2))
        sc = np.ldexp(1.0, S - 127)[:, :, None]
        mag = _e2m3_round(b / sc)
        code = mag | np.where(b < 0, 32, 0)
        out_codes.append(code)
        out_scales.append(S)
        b = b - np.sign(b) * E2M3[mag] * sc  # the remainder, exact in double
    packed = np.zeros((rows, K // 32, 48), np.uint8)
    for term, code in enumerate(out_codes):
        bits = np.zeros((rows, K // 32, 192), np.uint8)
        for j in range(32):
            for k in range(6):
                bits[:, :, 6 * j + k] = (code[:, :, j] >> k) & 1
        packed[:, :, 24 * term:24 * term + 24] = np.packbits(bits.reshape(rows, K // 32, 24, 8), axis=3,
                                                             bitorder="little")[..., 0]
    scales = np.stack(out_scales, axis=2).astype(np.uint8)
    return packed, scales


def _unpack6(packed):
    bits = np.unpackbits(packed[..., None], axis=-1, bitorder="little").reshape(*packed.shape[:-1], -1)
    hi = bits[..., :192].reshape(*bits.shape[:-1], 32, 6)
    lo = bits[..., 192:].reshape(*bits.shape[:-1], 32, 6)
    w = 1 << np.arange(6)
    return (hi * w).sum(-1), (lo * w).sum(-1)


def _split_inputs():
    rng = np.random.default_rng(31)
    rows = []
    rows.append(rng.standard_normal((64, 256)).astype(np.float32))                     # N(0, 1)
    rows.append((rng.standard_normal((32, 256)) * np.exp2(rng.integers(-30, 30, (32, 256)))).astype(np.float32))
    grid = np.concatenate([E2M3, (E2M3[1:] + E2M3[:-1]) / 2, [7.6, 7.75, 7.9]])  # grid, midpoints, saturation
    g = rng.choice(np.concatenate([grid, -grid]), (32, 256)) * np.exp2(rng.integers(-6, 6, (32, 1)))
    g[:, ::32] = 7.99 * np.exp2(np.floor(np.log2(np.abs(g[:, ::32]).max() + 1)))     # pin each block's amax
    rows.append(g.astype(np.float32))
    z = np.zeros((8, 256), np.float32)
    z[1, :32] = 1e-40  # bf16 subnormals
    z[2, 5] = -3.0
    rows.append(z)
    return synth.bf16_from_f32(np.concatenate(rows))


def test_split_matches_definition():
    x = _split_inputs()
    rows, K = x.shape
    codes = torch.empty((rows, K // 32, 48), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, K // 32, 2), dtype=torch.uint8, device="cuda")
    moe.moe_mx_split(rows, K, to_dev(x), codes, scales)
    torch.cuda.synchronize()
    ref_codes, ref_scales = split_reference(x)
    assert np.array_equal(scales.cpu().numpy(), ref_scales)
    got_hi, got_lo = _unpack6(codes.cpu().numpy())
    ref_hi, ref_lo = _unpack6(ref_codes)
    for got, ref in ((got_hi, ref_hi), (got_lo, ref_lo)):
        zero = (got & 31) == 0
        assert np.array_equal(np.where(zero, 0, got), np.where((ref & 31) == 0, 0, ref))
    # hi + lo reconstructs x to within the lo term's half step
    xs = synth.f32_from_bf16(x).astype(np.float64).reshape(rows, K // 32, 32)
    val = lambda c, s: np.where(c & 32, -1, 1) * E2M3[c & 31] * np.ldexp(1.0, s.astype(np.int64) - 127)[..., None]
    rec = val(got_hi, scales.cpu().numpy()[..., 0]) + val(got_lo, scales.cpu().numpy()[..., 1])
    step = np.ldexp(1.0, scales.cpu().numpy()[..., 1].astype(np.int64) - 127 - 1)[..., None]  # half of 2^(S2-127) * 1
    assert np.all(np.abs(rec - xs) <= step * 1.0 + 1e-300)


def _layer(T, H, E, k, I, seed=5, zipf=0.0):
    cfg = synth.LayerConfig(f"mx_T{T}_H{H}_E{E}_k{k}_I{I}", T=T, H=H, E=E, k=k, I=I, wfmt=1, seed=seed, zipf_s=zipf)
    return synth.make_layer(cfg)


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("shape", [(37, 128, 5, 2, 192), (300, 192, 7, 3, 128), (700, 256, 4, 2, 320),
                                   (50, 64, 3, 2, 64), (260, 128, 1, 1, 64), (90, 64, 6, 6, 128),
                                   (1100, 320, 16, 4, 192)],
                         ids=lambda s: "T{}_H{}_E{}_k{}_I{}".format(*s))
def test_mx_ragged(shape, packed):
    layer = _layer(*shape, zipf=1.1 if shape[0] >= 700 else 0.0)
    c = layer.cfg
    print(f"[mx] {c.name} packed={packed}", flush=True)
    y_ref, idx_ref, w_ref, o_ref, h_ref = oracle.get().forward_tokens(layer.x, layer.w_router, layer.weights, c.k,
                                                                      c.I, np.arange(c.T), want_pairs=True)
    g = GpuLayer(layer, MX, packed=packed)
    g.forward()
    torch.cuda.synchronize()
    assert np.array_equal(g.topk_idx.cpu().numpy(), idx_ref)
    e = rel_err(bf16_dev_to_f64(g.y), y_ref)
    assert e <= TOL, e
    y_fused = g.y.clone()
    # stage by stage on the same path: h and y_sorted per pair
    g.stages()
    torch.cuda.synchronize()
    pr = g.pair_rank.cpu().numpy()
    e_h = rel_err(bf16_dev_to_f64(g.h)[pr], h_ref.reshape(-1, c.I))
    e_o = rel_err(bf16_dev_to_f64(g.y_sorted)[pr], o_ref.reshape(-1, c.H))
    print(f"[mx] {c.name} rel err y {e:.2e} h {e_h:.2e} y_sorted {e_o:.2e}")
    assert e_h <= TOL and e_o <= TOL, (e_h, e_o)
    # moe_forward and moe_grouped_ffn split h inside the gate/up kernel; the
    # stage entry points write bf16 h and split it in the down stage: same bits
    assert torch.equal(y_fused, g.y)
    ys_stages = g.y_sorted.clone()
    g.y_sorted.fill_(0)
    g.grouped_ffn()
    torch.cuda.synchronize()
    assert torch.equal(ys_stages, g.y_sorted)


@pytest.mark.parametrize("name", ["20b_mxfp4_prefill", "20b_mxfp4_prefill+packed", "20b_mxfp4_decode+packed"])
def test_mx_configs(name):
    print(f"[mx] {name}", flush=True)
    layer = synth.make_layer(name.split("+")[0])
    c = layer.cfg
    tokens = synth.sample_tokens(c.T, 512, c.seed + 1)
    orc = oracle.get()
    _, idx_all, _ = orc.route(layer.x, layer.w_router, c.k)
    y_ref, _, _ = orc.forward_tokens(layer.x, layer.w_router, layer.weights, c.k, c.I, tokens)
    g = GpuLayer(layer, MX, packed=name.endswith("+packed"))
    g.forward()
    torch.cuda.synchronize()
    assert np.array_equal(g.topk_idx.cpu().numpy(), idx_all)
    y = bf16_dev_to_f64(g.y.index_select(0, torch.from_numpy(tokens.astype(np.int64)).to(g.device)))
    e = rel_err(y, y_ref)
    print(f"[mx] {name} rel err y {e:.2e}")
    assert e <= TOL, e
    y1 = g.y.clone()
    g.forward()
    torch.cuda.synchronize()
    assert torch.equal(y1, g.y)  # deterministic
    g.stages()  # h written as bf16 and split by the down stage: the same bits as the fused split
    torch.cuda.synchronize()
    assert torch.equal(y1, g.y)


def test_mx_refuses_what_it_cannot_run():
    for d in (moe.dims(16, 96, 4, 2, 64, moe.MOE_WFMT_MXFP4, MX), moe.dims(16, 64, 4, 2, 64, moe.MOE_WFMT_BF16, MX)):
        with pytest.raises(moe.MoeError) as ex:
            moe.moe_workspace_size(d)
        assert ex.value.code == moe.MOE_ERR_UNSUPPORTED
