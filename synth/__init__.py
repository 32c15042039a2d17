"""Seeded synthetic inputs for the block-scaled FP4 MoE path.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds none of the method's arithmetic: it only draws random numbers and casts
them with library routines (torch's bfloat16 / float8_e4m3fn casts).  It
imports neither the oracle nor the HIP library.

Every array is drawn from numpy ``PCG64`` streams keyed by
(seed, stream id[, expert]), so one expert's weights can be regenerated
without drawing the whole layer.  Shapes and distributions follow the
workloads of the pages (GLM-5.2 MoE layers quantised to NVFP4 group16 or to
FP4 + UE8M0 group32); there is no dataset or checkpoint behind them.

Layouts (all row-major, K contiguous):
  x       A16: [T, H] bfloat16 bit patterns (uint16)
          A8 : [T, H] E4M3 bytes + x_sf [T, H/32] UE8M0 bytes
  topk    ids [T, k] int32, weights [T, k] float32
  w13     [E, 2I, H/2] uint8 (two E2M1 codes per byte, even K in low nibble)
  w13_sf  [E, 2I, H/gran] uint8 (E4M3 for gran 16, UE8M0 for gran 32)
  w13_gs  [E] float32 or None
  w2      [E, H, I/2], w2_sf [E, H, I/gran], w2_gs [E] or None
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch

# stream ids
_S_ROUTER, _S_X = 1, 2
_S_W13, _S_W2, _S_GS = 10, 12, 14


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    E: int
    k: int
    H: int
    I: int
    gran: int                 # 16: E4M3 block scales, 32: UE8M0 block scales
    act: str                  # "bf16" or "fp8"
    routing: str              # "softmax_topk" or "zipf"
    scale_log2: tuple = (-10.0, -3.0)   # gran 16: log-uniform E4M3 scale range
    ue8m0_exp: tuple = (-10, -2)        # gran 32: uniform integer exponents
    global_scale: str = "uniform"       # "uniform" U[0.5, 2], "one", "none"
    zipf_s: float = 1.1
    seed: int = 0
    weight_seed: int | None = None      # weights drawn from this seed (default: seed)

    @property
    def wseed(self) -> int:
        return self.seed if self.weight_seed is None else self.weight_seed


@dataclass(frozen=True)
class RequantConfig:
    name: str
    E: int
    shapes: tuple             # ((N, K), ...) one per tensor, e.g. w13 and w2
    scale_log2: tuple = (-10.0, -3.0)
    seed: int = 4


CONFIGS = {
    "tiny": MoEConfig("tiny", T=32, E=8, k=2, H=512, I=256, gran=16, act="bf16",
                      routing="softmax_topk", scale_log2=(-8.0, -2.0),
                      global_scale="one", seed=0),
    "decode16": MoEConfig("decode16", T=64, E=256, k=8, H=6144, I=2048, gran=16,
                          act="bf16", routing="softmax_topk", seed=1),
    "decode32": MoEConfig("decode32", T=256, E=256, k=8, H=6144, I=2048, gran=32,
                          act="fp8", routing="softmax_topk", global_scale="none",
                          seed=2),
    # the prefill layer reuses the decode32 layer's weights (same weight seed)
    "prefill32": MoEConfig("prefill32", T=8192, E=256, k=8, H=6144, I=2048, gran=32,
                           act="fp8", routing="zipf", global_scale="none", seed=3,
                           weight_seed=2),
}

REQUANT_CONFIGS = {
    # the full decode16 layer (same seed and streams): w13 and w2 of 256 experts
    "requant": RequantConfig("requant", E=256, shapes=((4096, 6144), (6144, 2048)), seed=1),
}


def variant(cfg: MoEConfig, **kw) -> MoEConfig:
    """A copy of ``cfg`` with some fields changed (reduced sizes for tests)."""
    return replace(cfg, **kw)


# ----------------------------------------------------------------------------
# routing


def make_routing(cfg: MoEConfig):
    """Router outputs (outside the library, which takes ids/weights as input).

    softmax_topk: logits N(0,1) [T, E], probabilities = softmax over all E,
      ids = the k largest (ties to the lower index), weights = their
      probabilities, not renormalised.
    zipf: expert popularity p_r ~ r**-s over a seeded permutation of the
      experts; ids = the k largest of log p + Gumbel noise per token (sampling
      without replacement); weights = softmax over k fresh N(0,1) logits.
    """
    rng = _rng(cfg.seed, _S_ROUTER)
    T, E, k = cfg.T, cfg.E, cfg.k
    if cfg.routing == "softmax_topk":
        logits = rng.standard_normal((T, E))
        z = np.exp(logits - logits.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        ids = np.argsort(-p, axis=1, kind="stable")[:, :k]
        w = np.take_along_axis(p, ids, axis=1)
    elif cfg.routing == "zipf":
        perm = rng.permutation(E)
        pop = np.empty(E)
        pop[perm] = np.arange(1, E + 1, dtype=np.float64) ** (-cfg.zipf_s)
        pop /= pop.sum()
        g = rng.gumbel(size=(T, E))
        ids = np.argsort(-(np.log(pop)[None, :] + g), axis=1, kind="stable")[:, :k]
        lw = rng.standard_normal((T, k))
        z = np.exp(lw - lw.max(axis=1, keepdims=True))
        w = z / z.sum(axis=1, keepdims=True)
    else:
        raise ValueError(cfg.routing)
    return ids.astype(np.int32), w.astype(np.float32)


# ----------------------------------------------------------------------------
# activations


def make_activations(cfg: MoEConfig):
    """A16: x ~ N(0,1) cast to bfloat16 (torch RNE cast) -> (bits, None); the
         same for "bf16q" / "bf16q4" (bfloat16 x that the library quantises
         to FP8 / MXFP4).
    A8 : per 32-block UE8M0 byte uniform in {119, 120, 121} and E4M3 payload
         = torch cast of clip(64 * N(0,1), +-448) -> (fp8 bytes, sf bytes)."""
    rng = _rng(cfg.seed, _S_X)
    T, H = cfg.T, cfg.H
    if cfg.act in ("bf16", "bf16q", "bf16q4"):
        xf = rng.standard_normal((T, H), dtype=np.float32)
        bits = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return bits.copy(), None
    if cfg.act == "fp8":
        sf = rng.integers(119, 122, size=(T, H // 32), dtype=np.uint8)
        xf = np.clip(64.0 * rng.standard_normal((T, H), dtype=np.float32), -448.0, 448.0)
        q = torch.from_numpy(xf).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        return q.copy(), sf
    raise ValueError(cfg.act)


# ----------------------------------------------------------------------------
# weights


def _e4m3_log_uniform(rng, shape, lo, hi):
    u = rng.uniform(lo, hi, size=shape)
    v = torch.from_numpy(np.exp2(u).astype(np.float32))
    return v.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def make_fp4_tensor(seed, stream, e, N, K, gran, scale_log2=(-10.0, -3.0),
                    ue8m0_exp=(-10, -2)):
    """One expert's [N, K/2] packed codes (uniform random bytes, i.e. uniform
    E2M1 codes) and its [N, K/gran] block scales."""
    codes = np.frombuffer(_rng(seed, stream, e).bytes(N * K // 2), dtype=np.uint8)
    codes = codes.reshape(N, K // 2)
    srng = _rng(seed, stream + 100, e)
    if gran == 16:
        sf = _e4m3_log_uniform(srng, (N, K // 16), *scale_log2)
    elif gran == 32:
        sf = srng.integers(127 + ue8m0_exp[0], 127 + ue8m0_exp[1] + 1,
                           size=(N, K // 32), dtype=np.uint8)
    else:
        raise ValueError(gran)
    return codes, sf


def make_global_scales(seed, stream, E, mode):
    if mode == "none":
        return None
    if mode == "one":
        return np.ones(E, dtype=np.float32)
    if mode == "uniform":
        return _rng(seed, _S_GS, stream).uniform(0.5, 2.0, size=E).astype(np.float32)
    raise ValueError(mode)


@dataclass
class MoEInputs:
    cfg: MoEConfig
    x: np.ndarray
    x_sf: np.ndarray | None
    topk_ids: np.ndarray
    topk_w: np.ndarray
    w13: np.ndarray
    w13_sf: np.ndarray
    w13_gs: np.ndarray | None
    w2: np.ndarray
    w2_sf: np.ndarray
    w2_gs: np.ndarray | None
    extra: dict = field(default_factory=dict)


def make_moe_inputs(cfg: MoEConfig) -> MoEInputs:
    ids, w = make_routing(cfg)
    x, x_sf = make_activations(cfg)
    E, H, I, g = cfg.E, cfg.H, cfg.I, cfg.gran
    w13 = np.empty((E, 2 * I, H // 2), np.uint8)
    w13_sf = np.empty((E, 2 * I, H // g), np.uint8)
    w2 = np.empty((E, H, I // 2), np.uint8)
    w2_sf = np.empty((E, H, I // g), np.uint8)
    ws = cfg.wseed
    for e in range(E):
        w13[e], w13_sf[e] = make_fp4_tensor(ws, _S_W13, e, 2 * I, H, g,
                                            cfg.scale_log2, cfg.ue8m0_exp)
        w2[e], w2_sf[e] = make_fp4_tensor(ws, _S_W2, e, H, I, g,
                                          cfg.scale_log2, cfg.ue8m0_exp)
    gs1 = make_global_scales(ws, _S_W13, E, cfg.global_scale)
    gs2 = make_global_scales(ws, _S_W2, E, cfg.global_scale)
    return MoEInputs(cfg, x, x_sf, ids, w, w13, w13_sf, gs1, w2, w2_sf, gs2)


@dataclass
class RequantInputs:
    cfg: RequantConfig
    tensors: list   # [(src [E, N, K/2], src_sf [E, N, K/16], gs [E]), ...]


def make_requant_tensor(cfg: RequantConfig, which: int, experts=None):
    """Tensor ``which`` of the layer (0: w13, 1: w2) for the listed experts."""
    N, K = cfg.shapes[which]
    ex = range(cfg.E) if experts is None else list(experts)
    src = np.empty((len(ex), N, K // 2), np.uint8)
    sf = np.empty((len(ex), N, K // 16), np.uint8)
    for i, e in enumerate(ex):
        src[i], sf[i] = make_fp4_tensor(cfg.seed, _S_W13 + 2 * which, e, N, K, 16,
                                        cfg.scale_log2)
    gs = make_global_scales(cfg.seed, _S_W13 + 2 * which, cfg.E, "uniform")
    if experts is not None:
        gs = gs[list(experts)]
    return src, sf, gs


def make_requant_inputs(cfg: RequantConfig) -> RequantInputs:
    return RequantInputs(cfg, [make_requant_tensor(cfg, i) for i in range(len(cfg.shapes))])
