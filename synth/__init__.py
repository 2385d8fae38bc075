"""Seeded synthetic inputs for the MoE FFN layer.

This module only *defines data*: it draws seeded normals, rounds them to bf16,
quantizes expert weights to MXFP4, and biases the router for the skewed
(Zipf) prefill workload.  It holds none of the layer's arithmetic (no routing,
no permutation, no expert math) and is shared by the oracle tests, the GPU
parity tests and the benchmark alike.

Workload shapes follow the gpt-oss layer the pages describe: hidden 2880,
top-4 of 32 experts ("Persona Kappa: training a 20B LLM on desktop GPUs",
table "Architecture Summary"), 128 experts for the 120b model
("hearth-lean-loomed-v1", section "Why 12-16 streams can be slow on Vulkan"),
and natively MXFP4 expert weights with bf16 activations (Persona Kappa,
section "Quantization-Aware Training (QAT)").  No model weights exist here;
every tensor is drawn from the distributions stated per preset.

Conventions: bf16 tensors are numpy.uint16 bit patterns; MXFP4 tensors are
numpy.uint8 packed nibbles (element 2b in the low nibble of byte b) plus one
numpy.uint8 E8M0 scale per 32 elements along K; weights are [out][in].
"""
from __future__ import annotations

import dataclasses
import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# --------------------------------------------------------------------------- presets


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int                 # tokens
    H: int                 # hidden size
    E: int                 # experts
    k: int                 # experts per token
    I: int                 # expert FFN width (gate/up each I rows, down I columns)
    wfmt: int = 0          # 0 = bf16 expert weights, 1 = MXFP4
    zipf_s: float = 0.0    # > 0: router biased so expert popularity follows Zipf(s)
    seed: int = 0
    w_std: float = 0.02    # std of router and expert weights
    x_std: float = 1.0     # std of the activations
    mx_gen: str = "quantize"  # MXFP4 weights: "quantize" N(0, w_std) draws, or "sampled" (see make_weights)

    @property
    def P(self) -> int:
        return self.T * self.k

    def with_T(self, T: int) -> "LayerConfig":
        return dataclasses.replace(self, T=T)


CONFIGS = {
    # small case the oracle finishes in well under a second
    "tiny": LayerConfig("tiny", T=64, H=256, E=8, k=2, I=512),
    # 20b-shaped layer, decode: 16 tokens, ~2 tokens per expert
    "20b_decode": LayerConfig("20b_decode", T=16, H=2880, E=32, k=4, I=2880),
    # 20b-shaped layer, prefill: 8192 packed tokens, Zipf(1.1) expert popularity
    "20b_prefill_zipf": LayerConfig("20b_prefill_zipf", T=8192, H=2880, E=32, k=4, I=2880, zipf_s=1.1),
    # 120b-shaped layer (128 experts); swept over SWEEP_120B token counts
    "120b_sweep": LayerConfig("120b_sweep", T=32, H=2880, E=128, k=4, I=2880),
    # 20b-shaped layer with MXFP4 expert weights: decode and prefill
    "20b_mxfp4_decode": LayerConfig("20b_mxfp4_decode", T=16, H=2880, E=32, k=4, I=2880, wfmt=1),
    "20b_mxfp4_prefill": LayerConfig("20b_mxfp4_prefill", T=32768, H=2880, E=32, k=4, I=2880, wfmt=1),
    # 120b-shaped layer with MXFP4 expert weights (the 120b model's experts are
    # MXFP4 too), swept over SWEEP_120B; codes and scales sampled with the
    # frequencies of quantised N(0, 0.02) draws (4x the 20b tensors: drawing and
    # quantising that many normals on the host would take minutes)
    "120b_mxfp4_sweep": LayerConfig("120b_mxfp4_sweep", T=32, H=2880, E=128, k=4, I=2880, wfmt=1,
                                    mx_gen="sampled"),
}
SWEEP_120B = (1, 4, 8, 12, 16, 32)

# Gain of the constant router channel that carries the Zipf bias (see
# zipf_router_bias).  With x[:, H-1] = 1 the router adds ZIPF_GAIN*ln(p_e) to
# expert e's logit; the logits' own spread is ~N(0, 0.02^2 * (H-1)) ~ 1.07^2,
# and this gain makes the first-choice share of each expert track p_e.
ZIPF_GAIN = 0.62

# Tensor ids of the per-tensor random streams.
_X, _WR, _WGU, _WD = 0, 1, 2, 3


# --------------------------------------------------------------------------- number formats


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns, round-to-nearest-even.
    (Inputs are finite; NaN/Inf never occur in the generated data.)"""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def f32_from_bf16(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# E2M1 grid magnitudes by code 0..7 (OCP Microscaling v1.0, FP4 E2M1) and the
# midpoints between neighbours.
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MID = (_E2M1_MAG[1:] + _E2M1_MAG[:-1]) / 2


def mxfp4_quantize(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantize rows of w [rows][cols] (cols % 32 == 0) to MXFP4.

    Per block of 32 consecutive elements along a row: shared exponent
    X = floor(log2(amax)) - 2 (2 = the largest E2M1 exponent), stored as the
    E8M0 byte X + 127 clamped to [0, 254]; an all-zero block stores 0.  Each
    element v/2^X is rounded to the nearest E2M1 value, ties to the even code,
    saturating at +-6.  Returns (packed bytes [rows][cols/2], scales
    [rows][cols/32])."""
    w = np.asarray(w, np.float64)
    rows, cols = w.shape
    assert cols % 32 == 0
    blk = w.reshape(rows, cols // 32, 32)
    amax = np.abs(blk).max(axis=2)
    with np.errstate(divide="ignore"):
        xexp = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    sbyte = np.clip(xexp + 127, 0, 254).astype(np.uint8)
    scaled = blk / np.ldexp(1.0, sbyte.astype(np.int32) - 127)[:, :, None]
    mag = np.abs(scaled)
    code = np.searchsorted(_E2M1_MID, mag, side="left")
    tie = (code < 7) & (mag == _E2M1_MID[np.minimum(code, 6)]) & (code % 2 == 1)
    code = np.minimum(code + tie, 7).astype(np.uint8)
    code = code | np.where((scaled < 0) & (code > 0), np.uint8(8), np.uint8(0)).astype(np.uint8)
    code = code.reshape(rows, cols)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(sbyte.reshape(rows, cols // 32))


# --------------------------------------------------------------------------- tensors


@dataclasses.dataclass
class Weights:
    """Batched expert weights of one layer (host arrays)."""
    wfmt: int
    gate_up: np.ndarray                      # bf16 [E][2I][H] or u8 [E][2I][H/2]
    down: np.ndarray                         # bf16 [E][H][I] or u8 [E][H][I/2]
    gate_up_scale: np.ndarray | None = None  # u8 [E][2I][H/32] (MXFP4 only)
    down_scale: np.ndarray | None = None     # u8 [E][H][I/32] (MXFP4 only)

    def nbytes_per_expert(self) -> int:
        n = self.gate_up[0].nbytes + self.down[0].nbytes
        if self.wfmt == 1:
            n += self.gate_up_scale[0].nbytes + self.down_scale[0].nbytes
        return n


@dataclasses.dataclass
class Layer:
    cfg: LayerConfig
    x: np.ndarray            # bf16 [T][H]
    w_router: np.ndarray     # bf16 [E][H]
    weights: Weights


def _rng(seed: int, tensor: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, sub])))


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return bf16_from_f32(a)


def zipf_probs(E: int, s: float) -> np.ndarray:
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


def make_x(cfg: LayerConfig, T: int | None = None) -> np.ndarray:
    """Activations x ~ N(0, x_std^2) in bf16; with a Zipf bias the last channel
    is the constant 1.0 that carries it."""
    T = cfg.T if T is None else T
    x = _normal_bf16(_rng(cfg.seed, _X), (T, cfg.H), cfg.x_std)
    if cfg.zipf_s > 0:
        x[:, cfg.H - 1] = 0x3F80  # 1.0
    return x


# Experts of the near-tie router (near_tie_router): slot order by design.
NEAR_TIE = {"A2": 17, "A1": 3, "B1": 5, "B2": 9, "C": 2}


def near_tie_router(T: int, H: int, E: int, seed: int = 0):
    """x [T][H] and a router [E][H] (bf16) whose logits are exact in fp64
    whatever the summation order, with near ties at the top.  Every value is
    a small integer times a power of two: x[:, 2:] integers in [-8, 8],
    router entries integers in [-16, 16] / 256, so a logit is a multiple of
    2^-20 below 2^11 in magnitude (31 bits).  Channel 0 of x is 1 and carries
    a bias, channel 1 is 1 and carries a bump of +-2^-20.  Experts NEAR_TIE
    share one random row: A1 and A2 have bias 512 and A2 the bump +2^-20, B1
    and B2 are identical with bias 256, C has bias 256 and the bump -2^-20;
    every other expert has its own random row and no bias (|logit| <= 127)."""
    assert H >= 8 and E >= 18
    rng = _rng(seed, 7)
    x = rng.integers(-8, 9, size=(T, H)).astype(np.float32)
    x[:, 0] = 1.0
    x[:, 1] = 1.0
    w = rng.integers(-16, 17, size=(E, H)).astype(np.float32) / 256.0
    w[:, :2] = 0.0
    common = rng.integers(-16, 17, size=H).astype(np.float32) / 256.0
    for name, e in NEAR_TIE.items():
        w[e, 2:] = common[2:]
        w[e, 0] = 512.0 if name.startswith("A") else 256.0
    w[NEAR_TIE["A2"], 1] = 2.0 ** -20
    w[NEAR_TIE["C"], 1] = -(2.0 ** -20)
    return bf16_from_f32(x), bf16_from_f32(w)


def zipf_router_bias(cfg: LayerConfig) -> np.ndarray:
    """bf16 bias column ZIPF_GAIN * ln(p_e) for the router's last channel."""
    p = zipf_probs(cfg.E, cfg.zipf_s)
    return bf16_from_f32((ZIPF_GAIN * np.log(p)).astype(np.float32))


def make_router(cfg: LayerConfig) -> np.ndarray:
    wr = _normal_bf16(_rng(cfg.seed, _WR), (cfg.E, cfg.H), cfg.w_std)
    if cfg.zipf_s > 0:
        wr[:, cfg.H - 1] = zipf_router_bias(cfg)
    return wr


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@functools.lru_cache(maxsize=4)
def _mx_sample_tables(std: float):
    """256-entry lookup tables that turn a uniform random byte into an E2M1
    code, or into an E8M0 scale byte, with the frequencies that
    mxfp4_quantize gives N(0, std^2) data (measured once on a seeded sample of
    512 x 2880 draws)."""
    a = _rng(0x4D58, 0).standard_normal((512, 2880), dtype=np.float32) * np.float32(std)
    packed, scales = mxfp4_quantize(a)
    codes = np.concatenate([packed & 15, packed >> 4]).ravel()

    def table(values):
        vals, counts = np.unique(values, return_counts=True)
        cdf = np.cumsum(counts) / counts.sum()
        return vals[np.minimum(np.searchsorted(cdf, (np.arange(256) + 0.5) / 256), len(vals) - 1)].astype(np.uint8)

    return table(codes), table(scales.ravel())


def _mx_sampled(rng: np.random.Generator, rows: int, cols: int, std: float):
    """MXFP4 bytes [rows][cols/2] and scales [rows][cols/32] whose codes and
    scale bytes are drawn independently with the frequencies of quantised
    N(0, std^2) data."""
    ctab, stab = _mx_sample_tables(std)
    c = ctab[rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)]
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    scales = stab[rng.integers(0, 256, size=(rows, cols // 32), dtype=np.uint8)]
    return np.ascontiguousarray(packed), np.ascontiguousarray(scales)


def make_weights(cfg: LayerConfig) -> Weights:
    """Expert weights ~N(0, w_std^2): bf16, or MXFP4 quantized from the same
    float draws.  One random stream per (tensor, expert).  With mx_gen =
    "sampled" the MXFP4 codes and scales are drawn directly from the
    frequencies quantised N(0, w_std^2) data has (_mx_sampled)."""
    E, H, I = cfg.E, cfg.H, cfg.I
    if cfg.wfmt == 0:
        gu = np.empty((E, 2 * I, H), np.uint16)
        dn = np.empty((E, H, I), np.uint16)

        def one(e):
            gu[e] = _normal_bf16(_rng(cfg.seed, _WGU, e), (2 * I, H), cfg.w_std)
            dn[e] = _normal_bf16(_rng(cfg.seed, _WD, e), (H, I), cfg.w_std)

        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, range(E)))
        return Weights(0, gu, dn)
    assert H % 32 == 0 and I % 32 == 0, "MXFP4 needs K dims that are multiples of 32"
    gu = np.empty((E, 2 * I, H // 2), np.uint8)
    gus = np.empty((E, 2 * I, H // 32), np.uint8)
    dn = np.empty((E, H, I // 2), np.uint8)
    dns = np.empty((E, H, I // 32), np.uint8)

    def oneq(e):
        if cfg.mx_gen == "sampled":
            gu[e], gus[e] = _mx_sampled(_rng(cfg.seed, _WGU, e), 2 * I, H, cfg.w_std)
            dn[e], dns[e] = _mx_sampled(_rng(cfg.seed, _WD, e), H, I, cfg.w_std)
            return
        a = _rng(cfg.seed, _WGU, e).standard_normal((2 * I, H), dtype=np.float32) * np.float32(cfg.w_std)
        gu[e], gus[e] = mxfp4_quantize(a)
        b = _rng(cfg.seed, _WD, e).standard_normal((H, I), dtype=np.float32) * np.float32(cfg.w_std)
        dn[e], dns[e] = mxfp4_quantize(b)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(oneq, range(E)))
    return Weights(1, gu, dn, gus, dns)


def make_layer(cfg: LayerConfig | str, T: int | None = None) -> Layer:
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if T is not None:
        cfg = cfg.with_T(T)
    return Layer(cfg, make_x(cfg), make_router(cfg), make_weights(cfg))


def sample_tokens(T: int, n: int, seed: int) -> np.ndarray:
    """n distinct token indices (sorted), uniform without replacement, drawn
    from a stream seeded with `seed`; all tokens when n >= T."""
    if n >= T:
        return np.arange(T, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x5EED])))
    return np.sort(rng.choice(T, size=n, replace=False)).astype(np.int32)


def expected_touched(E: int, k: int, T: int) -> float:
    """Expected number of distinct experts hit by T uniformly routed tokens."""
    return E * (1.0 - (1.0 - k / E) ** T)


__all__ = ["LayerConfig", "CONFIGS", "SWEEP_120B", "ZIPF_GAIN", "Weights", "Layer", "bf16_from_f32", "f32_from_bf16",
           "mxfp4_quantize", "make_layer", "make_x", "make_router", "make_weights", "sample_tokens", "zipf_probs",
           "zipf_router_bias", "expected_touched"]
