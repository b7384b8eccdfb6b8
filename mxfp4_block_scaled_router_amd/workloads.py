"""Seeded synthetic workloads for the MXFP4 routed-expert MoE layer.

This module only draws random inputs; it holds none of the layer's arithmetic
(no E2M1 decoding, no quantiser, no routing).  Both the GPU path and the CPU
oracle consume what it returns, in the canonical layout:

  x       uint16 bf16 bits [T, H]
  logits  float32 [T, E_global]
  w13     uint8 [E_local, 2I, H/2]  two E2M1 codes per byte, low nibble first
  w13s    uint8 [E_local, 2I, H/32] UE8M0 scale bytes
  w2      uint8 [E_local, H, I/2],  w2s uint8 [E_local, H, I/32]

Workloads (shapes and value distributions of the layer's five configurations):

  tiny     T=16   H=512  I=256  E=8/8     k=2  x~N(0,1), logits~N(0,1),
           uniform code bytes, scale bytes uniform in [120, 124]
  decode   T=16   H=2048 I=1536 E=64/64   k=8  as tiny, scale bytes in [118, 124]
  ep_share T=256  H=5120 I=1536 E=64/256  k=8  first_local=0; logits N(0,1) plus a
           per-expert bias -1.1*ln(rank), rank a seeded permutation of 1..256, so the
           noise-free router probabilities follow Zipf's law with s=1.1
  prefill  T=8192 H=4096 I=1536 E=128/128 k=8  x: N(0,1) with round(0.005*H)
           channels (drawn without replacement) scaled x20 before the bf16 rounding
  a4       T=4096 H=4096 I=1536 E=128/128 k=8  x~N(0,1); weights are Student-t(3)
           values times (3K)^-1/2 in fp32 (K = H for w13, K = I for w2), handed over
           unquantised: each side applies its own MXFP4 quantiser
  a8       as a4 with the activations quantised to MXFP8 (E4M3) instead of MXFP4
  verify_bB  T=6B (B = 1, 8, 16, 32, 48) with decode's dims and distributions:
           speculative verification of 5 draft tokens + 1 per sequence

Experts kept in bf16 (per-expert exclusions inside a fused buffer): uniform-code
workloads draw their bf16 weights from N(0, 0.16^2) (about the rms of their MXFP4
experts' values), one generator per (expert, matrix); Student-t workloads round
the expert's own Student-t draw to bf16.  `fuse` lays experts of both kinds back
to back in one byte buffer, the format a loader has to split per expert.

Every array comes from its own child stream of numpy's SeedSequence(seed), so an
array does not depend on which other arrays were drawn.  The Student-t weights are
drawn with torch generators, one per expert, so that any subset of experts can be
regenerated on the device that needs it.  bf16 rounding of x uses torch's
float32 -> bfloat16 conversion (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E_global: int
    E_local: int
    first_local: int
    top_k: int
    clamp_limit: float = 7.0
    scale_lo: int = 120
    scale_hi: int = 124
    x_kind: str = "normal"          # "normal" | "outliers"
    logits_kind: str = "normal"     # "normal" | "zipf_bias"
    weight_kind: str = "uniform"    # "uniform" | "student_t"
    a4: bool = False
    a8: bool = False
    seed: int = 1000

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    # sizes -------------------------------------------------------------
    @property
    def expert_bytes(self) -> int:
        """Packed codes + scale bytes of one expert (w13 and w2)."""
        return 3 * self.I * self.H // 2 + 3 * self.I * self.H // 32


WORKLOADS = {
    "tiny": Workload("tiny", 16, 512, 256, 8, 8, 0, 2, scale_lo=120, scale_hi=124, seed=1000),
    "decode": Workload("decode", 16, 2048, 1536, 64, 64, 0, 8, scale_lo=118, scale_hi=124,
                       seed=1001),
    "ep_share": Workload("ep_share", 256, 5120, 1536, 256, 64, 0, 8, scale_lo=118, scale_hi=124,
                         logits_kind="zipf_bias", seed=1002),
    "prefill": Workload("prefill", 8192, 4096, 1536, 128, 128, 0, 8, scale_lo=118, scale_hi=124,
                        x_kind="outliers", seed=1003),
    "a4": Workload("a4", 4096, 4096, 1536, 128, 128, 0, 8, weight_kind="student_t", a4=True,
                   seed=1004),
}
# MXFP8 activations (A8) on the a4 workload's shapes and weights
WORKLOADS["a8"] = WORKLOADS["a4"].replace(name="a8", a4=False, a8=True, seed=1010)
# Speculative-verify shapes: the decode layer's dims with T = 6 tokens per
# sequence (5 draft tokens + 1) for batches 1..48.
for _b, _seed in ((1, 1005), (8, 1006), (16, 1007), (32, 1008), (48, 1009)):
    WORKLOADS["verify_b%d" % _b] = Workload("verify_b%d" % _b, 6 * _b, 2048, 1536, 64, 64, 0, 8,
                                            scale_lo=118, scale_hi=124, seed=_seed)

_STREAMS = ("x", "logits", "bias", "w13", "w13s", "w2", "w2s", "outlier_channels", "student_t")


def _rng(wl: Workload, stream: str) -> np.random.Generator:
    child = np.random.SeedSequence(wl.seed).spawn(len(_STREAMS))[_STREAMS.index(stream)]
    return np.random.Generator(np.random.PCG64(child))


def bf16_bits_of(f32: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns via torch's RNE conversion."""
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def make_x(wl: Workload) -> np.ndarray:
    x = _rng(wl, "x").standard_normal((wl.T, wl.H), dtype=np.float32)
    if wl.x_kind == "outliers":
        n_out = int(round(0.005 * wl.H))
        ch = _rng(wl, "outlier_channels").choice(wl.H, size=n_out, replace=False)
        x[:, ch] *= np.float32(20.0)
    return bf16_bits_of(x)


def make_logits(wl: Workload, variant: int = 0) -> np.ndarray:
    """Router logits [T, E_global].  variant > 0 draws another batch of tokens'
    logits from its own stream; the per-expert bias (a property of the
    experts, not of the tokens) is the same for every variant."""
    rng = _rng(wl, "logits") if variant == 0 else \
        np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 0x106175, variant])))
    lg = rng.standard_normal((wl.T, wl.E_global), dtype=np.float32)
    if wl.logits_kind == "zipf_bias":
        rank = _rng(wl, "bias").permutation(wl.E_global) + 1
        bias = (-1.1 * np.log(rank.astype(np.float64))).astype(np.float32)
        lg = lg + bias[None, :]
    return np.ascontiguousarray(lg, dtype=np.float32)


def make_uniform_weights(wl: Workload):
    """Uniform code bytes and scale bytes uniform in [scale_lo, scale_hi]."""
    E, H, I = wl.E_local, wl.H, wl.I
    w13 = _rng(wl, "w13").integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w13s = _rng(wl, "w13s").integers(wl.scale_lo, wl.scale_hi + 1, (E, 2 * I, H // 32),
                                     dtype=np.uint8)
    w2 = _rng(wl, "w2").integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w2s = _rng(wl, "w2s").integers(wl.scale_lo, wl.scale_hi + 1, (E, H, I // 32),
                                   dtype=np.uint8)
    return w13, w13s, w2, w2s


def student_t_expert(wl: Workload, expert: int, which: str, device="cpu") -> torch.Tensor:
    """fp32 Student-t(3) weights of one expert, times (3K)^-1/2.

    which = "w13" -> [2I, H] (K = H); which = "w2" -> [H, I] (K = I).
    t3 = z0 / sqrt((z1^2 + z2^2 + z3^2) / 3) from four standard normals.
    """
    if which == "w13":
        shape, K, tag = (2 * wl.I, wl.H), wl.H, 0
    elif which == "w2":
        shape, K, tag = (wl.H, wl.I), wl.I, 1
    else:
        raise ValueError(which)
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 100003 + expert * 2 + tag)
    z = torch.randn((4,) + shape, generator=g, device=device, dtype=torch.float32)
    chi2 = z[1] * z[1] + z[2] * z[2] + z[3] * z[3]
    t = z[0] / torch.sqrt(chi2 / 3.0)
    return (t * (1.0 / math.sqrt(3.0 * K))).contiguous()


def make_inputs(wl: Workload, weights: bool = True) -> dict:
    """x, logits and (for uniform-code workloads) canonical weights as numpy arrays."""
    out = {"x": make_x(wl), "logits": make_logits(wl)}
    if weights and wl.weight_kind == "uniform":
        out["w13"], out["w13s"], out["w2"], out["w2s"] = make_uniform_weights(wl)
    return out


def scaled_down(wl: Workload, **kw) -> Workload:
    """The same distributions at other sizes (for tests that must run in seconds)."""
    return wl.replace(**kw)


# ---------------------------------------------------------------- bf16 experts

BF16_EXPERT_STD = 0.16


def bf16_expert(wl: Workload, expert: int, which: str, device="cpu") -> np.ndarray:
    """bf16 bits of one expert kept in bf16: [2I, H] for "w13", [H, I] for "w2"."""
    shape = (2 * wl.I, wl.H) if which == "w13" else (wl.H, wl.I)
    if wl.weight_kind == "student_t":
        t = student_t_expert(wl, int(expert), which, device=device)
        return t.to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16).copy()
    tag = 0 if which == "w13" else 1
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 0xB16, int(expert), tag])))
    return bf16_bits_of(g.standard_normal(shape, dtype=np.float32) * np.float32(BF16_EXPERT_STD))


def fuse(codes: np.ndarray, scales: np.ndarray, bf16: np.ndarray, excluded) -> tuple:
    """One fused expert buffer with per-expert dtypes: experts back to back in
    expert order, packed codes [R, K/2] for a packed expert or bf16 [R, K] (2
    bytes each) for an excluded one; the scale tensor holds the packed experts'
    [R, K/32] scale bytes back to back.  codes/scales: [E, R, K/2], [E, R, K/32]
    (slots of excluded experts unused); bf16: [n, R, K] uint16, the j-th
    excluded expert in slot j.  Returns (fused uint8 [bytes], scales uint8 [bytes])."""
    ex = np.asarray(excluded, dtype=bool)
    parts, sparts, j = [], [], 0
    for e in range(ex.size):
        if ex[e]:
            parts.append(np.ascontiguousarray(bf16[j], dtype=np.uint16).reshape(-1).view(np.uint8))
            j += 1
        else:
            parts.append(np.ascontiguousarray(codes[e], dtype=np.uint8).reshape(-1))
            sparts.append(np.ascontiguousarray(scales[e], dtype=np.uint8).reshape(-1))
    assert j == len(bf16)
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.uint8)
    return cat(parts), cat(sparts)
