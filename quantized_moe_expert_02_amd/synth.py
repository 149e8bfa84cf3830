"""Seeded synthetic inputs for the quantised MoE FFN layer.

This module only draws random numbers and encodes them into the canonical
storage format; it holds none of the layer's arithmetic (no routing, no
decode of codes back to weights, no products).  Both the GPU path and the
CPU oracle consume the bytes it produces.

Canonical storage format (all row-major, little-endian):

* ``q[rows][cols*bits/8]`` uint8 per matrix (gate ``[I][H]``, up ``[I][H]``,
  down ``[H][I]``).  4-bit codes: element ``2j`` sits in the low nibble of
  byte ``j``, element ``2j+1`` in the high nibble.  INT8_ROW: one
  two's-complement byte per element.  INT2_ROW: element ``4j+i`` in bits
  ``2i..2i+1`` of byte ``j``, two's complement in [-2, 1].
* INT4_ROW: a nibble is a two's-complement integer in [-8, 7]; one binary16
  scale per output row (``s[rows]``).  This is the
  "int4 with a per-row scale" format of the Colibrì engine (hakusoku.com
  story 8412, section 実装済み機能).  INT8_ROW and INT2_ROW are that engine's
  int8 and int2 kernels' formats, with the same per-row binary16 scale.
* E2M1_B16: a nibble is an OCP FP4 E2M1 code; one OCP FP8 E4M3 scale byte per
  16 consecutive weights along the row (``s[rows][cols/16]``) and one fp32
  tensor scale per matrix (``g``).  This is the NVFP4-style format that the
  Ornith engine decodes inside its matmul kernel (648news.com, Ornith
  inference engine article, section on splitting weights between VRAM and
  system memory).

Value distributions follow the layer workloads: activations ~ N(0, 1) rounded
to binary16, router weights ~ N(0, 0.02) fp32, expert weights ~ N(0, 0.02)
quantised symmetrically (int4: scale = amax_row / 7; int8: amax_row / 127;
int2: amax_row / 2, codes clamped to [-2, 1]; e2m1: tensor scale
g = amax / (6 * 448), block scale = e4m3(amax_block / (6 g))).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional

import numpy as np
import torch

INT4_ROW = 0
E2M1_B16 = 1
INT8_ROW = 2
INT2_ROW = 3
ROW_SCALED = (INT4_ROW, INT8_ROW, INT2_ROW)


def code_bits(wfmt: int) -> int:
    """Bits per stored weight code."""
    return {INT4_ROW: 4, E2M1_B16: 4, INT8_ROW: 8, INT2_ROW: 2}[wfmt]

# Binary16/E4M3 encoders are torch's own conversions; the e2m1 encoder below
# picks the nearest representable magnitude by bucketing at the midpoints of
# the E2M1 value grid.  These choose *inputs*; any deterministic choice would
# serve, since both implementations consume the resulting codes as given.
_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


@dataclasses.dataclass(frozen=True)
class Dims:
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    has_shared: int = 1
    wfmt: int = INT4_ROW
    top_p: float = 0.0  # adaptive top-p threshold; 0 keeps all top_k slots

    def as_tuple(self):
        """The six integer fields (top_p travels separately)."""
        return (self.hidden, self.inter, self.n_experts, self.top_k, self.has_shared, self.wfmt)


# Named workloads.  Sizes follow the pages: ~19 MB per int4 expert and 256
# experts per MoE layer (hakusoku.com story 8412, section Colibrì), 8 experts
# per token (same page, section 性能・要件).
WORKLOADS = {
    "tiny": dict(dims=Dims(256, 128, 8, 2, 1, INT4_ROW), tokens=4),
    "decode_b1": dict(dims=Dims(6144, 2048, 256, 8, 1, INT4_ROW), tokens=1),
    "decode_b8": dict(dims=Dims(6144, 2048, 256, 8, 1, INT4_ROW), tokens=8),
    # adaptive expert top-p 0.7 (hakusoku.com story 8412, section 実行・チューニングパラメータ)
    "decode_b1_topp": dict(dims=Dims(6144, 2048, 256, 8, 1, INT4_ROW, top_p=0.7), tokens=1),
    "e2m1_b1": dict(dims=Dims(2048, 512, 256, 8, 1, E2M1_B16), tokens=1),
    "e2m1_b4": dict(dims=Dims(2048, 512, 256, 8, 1, E2M1_B16), tokens=4),
    "prefill_2048": dict(dims=Dims(6144, 2048, 256, 8, 1, INT4_ROW), tokens=2048, zipf=1.1),
    # the same prefill without the Zipf bias: routing spread over all experts
    "prefill_2048_uniform": dict(dims=Dims(6144, 2048, 256, 8, 1, INT4_ROW), tokens=2048, zipf=0.0),
    # the same layer with int8 / int2 per-row-scale weights (hakusoku.com
    # story 8412, section 実装済み機能: int8/int4/int2 kernels, row scales)
    "int8_b1": dict(dims=Dims(6144, 2048, 256, 8, 1, INT8_ROW), tokens=1),
    "int2_b1": dict(dims=Dims(6144, 2048, 256, 8, 1, INT2_ROW), tokens=1),
    "int2_b8": dict(dims=Dims(6144, 2048, 256, 8, 1, INT2_ROW), tokens=8),
}


def _seed(*parts) -> int:
    h = hashlib.sha256(("moe:" + ":".join(str(p) for p in parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def pack_nibbles(codes: torch.Tensor) -> torch.Tensor:
    """codes int [.., cols] with values 0..15 -> uint8 [.., cols/2], even element in the low nibble."""
    c = codes.to(torch.uint8) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).contiguous()


def quantize_int4_rows(w: torch.Tensor):
    """fp32 [.., rows, cols] -> (q uint8 [.., rows, cols/2], s binary16 [.., rows])."""
    amax = w.abs().amax(dim=-1)
    s16 = (amax / 7.0).to(torch.float16)
    s16 = torch.where(s16 == 0, torch.ones_like(s16), s16)
    q = torch.clamp(torch.round(w / s16.float().unsqueeze(-1)), -8, 7).to(torch.int16)
    return pack_nibbles(q & 0xF), s16


def quantize_int_rows(w: torch.Tensor, wfmt: int):
    """fp32 [.., rows, cols] -> (q uint8 [.., rows, cols*bits/8], s binary16 [.., rows]) for
    INT4_ROW, INT8_ROW or INT2_ROW."""
    if wfmt == INT4_ROW:
        return quantize_int4_rows(w)
    qmin, qmax, div = (-128, 127, 127.0) if wfmt == INT8_ROW else (-2, 1, 2.0)
    amax = w.abs().amax(dim=-1)
    s16 = (amax / div).to(torch.float16)
    s16 = torch.where(s16 == 0, torch.ones_like(s16), s16)
    q = torch.clamp(torch.round(w / s16.float().unsqueeze(-1)), qmin, qmax).to(torch.int16)
    if wfmt == INT8_ROW:
        return (q & 0xFF).to(torch.uint8).contiguous(), s16
    c = (q & 0x3).to(torch.uint8)
    packed = c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)
    return packed.contiguous(), s16


def quantize_e2m1_blocks(w: torch.Tensor):
    """fp32 [.., rows, cols] -> (q uint8 [.., rows, cols/2], s uint8 e4m3 [.., rows, cols/16], g fp32 [..])."""
    lead = w.shape[:-2]
    rows, cols = w.shape[-2], w.shape[-1]
    amax_t = w.abs().flatten(-2).amax(dim=-1)
    g = (amax_t / (6.0 * 448.0)).clamp_min(1e-30)
    blk = w.reshape(*lead, rows, cols // 16, 16)
    amax_b = blk.abs().amax(dim=-1)
    sc = (amax_b / (6.0 * g[..., None, None])).clamp(max=448.0).to(torch.float8_e4m3fn)
    sc_val = sc.float()
    denom = (g[..., None, None] * sc_val).unsqueeze(-1)
    v = torch.where(denom > 0, blk / torch.where(denom > 0, denom, torch.ones_like(denom)), torch.zeros_like(blk))
    mids = torch.tensor(_E2M1_MIDPOINTS, dtype=v.dtype, device=v.device)
    mag = torch.bucketize(v.abs().contiguous(), mids, right=False)  # 0..7
    sign = (v < 0).to(torch.int64) << 3
    codes = (mag | sign).reshape(*lead, rows, cols)
    return pack_nibbles(codes), sc.view(torch.uint8), g.to(torch.float32)


@dataclasses.dataclass
class Layer:
    """One MoE layer in canonical format.  Expert tensors are stacked with
    index ``n_experts`` holding the shared expert (when ``has_shared``)."""
    dims: Dims
    q_gate: torch.Tensor  # uint8 [E+S][I][H*bits/8]
    s_gate: torch.Tensor  # integer formats: binary16 [E+S][I]; e2m1: uint8 e4m3 [E+S][I][H/16]
    q_up: torch.Tensor
    s_up: torch.Tensor
    q_down: torch.Tensor  # uint8 [E+S][H][I*bits/8]
    s_down: torch.Tensor
    g3: torch.Tensor      # fp32 [E+S][3] (1.0 for INT4_ROW)
    router_w: torch.Tensor  # fp32 [E][H]
    router_b: Optional[torch.Tensor]  # fp32 [E] or None

    @property
    def n_stored(self):
        return self.q_gate.shape[0]

    def to(self, device):
        f = lambda t: None if t is None else t.to(device)
        return Layer(self.dims, *(f(getattr(self, n)) for n in
                     ("q_gate", "s_gate", "q_up", "s_up", "q_down", "s_down", "g3", "router_w", "router_b")))


def make_experts(dims: Dims, n: int, seed_tag, device="cpu", std=0.02, batch=8):
    """Quantised expert weights for ``n`` experts (the last one is the shared
    expert when the caller counts it in ``n``)."""
    H, I = dims.hidden, dims.inter
    b = code_bits(dims.wfmt)
    qg = torch.empty((n, I, H * b // 8), dtype=torch.uint8, device=device)
    qu = torch.empty_like(qg)
    qd = torch.empty((n, H, I * b // 8), dtype=torch.uint8, device=device)
    if dims.wfmt in ROW_SCALED:
        sg = torch.empty((n, I), dtype=torch.float16, device=device)
        su = torch.empty_like(sg)
        sd = torch.empty((n, H), dtype=torch.float16, device=device)
    else:
        sg = torch.empty((n, I, H // 16), dtype=torch.uint8, device=device)
        su = torch.empty_like(sg)
        sd = torch.empty((n, H, I // 16), dtype=torch.uint8, device=device)
    g3 = torch.ones((n, 3), dtype=torch.float32, device=device)
    for e0 in range(0, n, batch):
        e1 = min(n, e0 + batch)
        mats = []
        for m, shape in enumerate(((I, H), (I, H), (H, I))):
            w = torch.stack([
                torch.randn(shape, generator=_gen(device, seed_tag, e, m), device=device, dtype=torch.float32)
                for e in range(e0, e1)]) * std
            mats.append(w)
        for m, (qdst, sdst) in enumerate(((qg, sg), (qu, su), (qd, sd))):
            if dims.wfmt in ROW_SCALED:
                q, s = quantize_int_rows(mats[m], dims.wfmt)
                qdst[e0:e1] = q
                sdst[e0:e1] = s
            else:
                q, s, g = quantize_e2m1_blocks(mats[m])
                qdst[e0:e1] = q
                sdst[e0:e1] = s
                g3[e0:e1, m] = g
        del mats
    return qg, sg, qu, su, qd, sd, g3


def make_router(dims: Dims, seed_tag, device="cpu", zipf: float = 0.0):
    E, H = dims.n_experts, dims.hidden
    rw = torch.randn((E, H), generator=_gen(device, seed_tag, "router"), device=device, dtype=torch.float32) * 0.02
    rb = None
    if zipf > 0:
        # Skewed per-expert logit bias: b_e = ln p_{pi(e)} - mean, p_r ~ r^-zipf,
        # pi a seeded permutation, so token counts per expert are uneven.
        rng = np.random.Generator(np.random.PCG64(_seed(seed_tag, "zipf")))
        perm = rng.permutation(E)
        r = np.arange(1, E + 1, dtype=np.float64)
        logp = -zipf * np.log(r)
        logp = logp - np.log(np.exp(logp).sum())
        b = logp[perm]
        b = b - b.mean()
        rb = torch.tensor(b, dtype=torch.float32, device=device)
    return rw, rb


def make_layer(dims: Dims, seed_tag, device="cpu", zipf: float = 0.0) -> Layer:
    n = dims.n_experts + (1 if dims.has_shared else 0)
    qg, sg, qu, su, qd, sd, g3 = make_experts(dims, n, (seed_tag, "experts"), device=device)
    rw, rb = make_router(dims, seed_tag, device=device, zipf=zipf)
    return Layer(dims, qg, sg, qu, su, qd, sd, g3, rw, rb)


# ---- crafted codes: every stored code value --------------------------------
# The random encoders above never emit some codes (int4 -8, int8 -128: they
# scale by amax/7 and amax/127) and pin the e2m1 block scales near the top of
# the e4m3 range.  The layers below write codes directly, so that every code
# of a format appears: integer codes cycle through all 2^bits two's-complement
# values along each row (from a seeded random offset per row); e2m1 codes
# cycle through all 16 codes inside every 16-column block; e2m1 block scales cycle
# through one e4m3 binade ("band": exponent field b, both signs, every
# mantissa) per matrix, so that all 254 finite e4m3 codes -- zero and the
# subnormals (b = 0) included -- appear across a layer's matrices, each in a
# matrix where its blocks carry the weight.  Row scales (integer formats)
# cycle through factors 1/16 .. 2 of a base chosen so that the weights have a
# spread near 0.02 (int8 rows at 1/16 get binary16-subnormal scales); the
# e2m1 tensor scale g of a matrix brings its band to the same spread.
_ROW_FACTORS = (1.0 / 16, 0.25, 0.5, 1.0, 1.5, 2.0)
_CODE_SPREAD = {INT4_ROW: 4.6, INT8_ROW: 74.0, INT2_ROW: 1.1}


def e4m3_band_codes(b: int):
    """The finite e4m3 codes with exponent field b (0..15), both signs."""
    pos = [(b << 3) | m for m in range(8) if not (b == 15 and m == 7)]
    return pos + [0x80 | c for c in pos]


def _sweep_fields(rows: int, cols: int, n: int, seed_tag) -> torch.Tensor:
    """Row r holds (c + o_r) mod n along its columns, o_r a seeded random
    offset: every row walks the whole code cycle, and rows are not periodic
    (a periodic pattern lets the down projection cancel exactly)."""
    off = torch.randint(0, n, (rows, 1), generator=_gen("cpu", seed_tag, "sweep"))
    c = torch.arange(cols).unsqueeze(0)
    return ((c + off) % n).to(torch.int64)


def _pack_fields(u: torch.Tensor, wfmt: int) -> torch.Tensor:
    """Unsigned fields (two's-complement bit patterns) -> canonical bytes."""
    if wfmt == INT8_ROW:
        return u.to(torch.uint8).contiguous()
    if wfmt == INT2_ROW:
        c = u.to(torch.uint8)
        return (c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)).contiguous()
    return pack_nibbles(u)


def make_code_sweep_layer(dims: Dims, seed_tag, band_of=None) -> Layer:
    """A layer whose stored codes cover every value of its format (see above).
    band_of(e, m) picks the e4m3 band of matrix m (0 gate, 1 up, 2 down) of
    expert e (default (3e + m) mod 16).  The router is the usual random one."""
    H, I = dims.hidden, dims.inter
    n = dims.n_experts + (1 if dims.has_shared else 0)
    if band_of is None:
        band_of = lambda e, m: (3 * e + m) % 16  # noqa: E731
    qs, ss = [[], [], []], [[], [], []]
    g3 = torch.ones((n, 3), dtype=torch.float32)
    for e in range(n):
        for m, (rows, cols) in enumerate(((I, H), (I, H), (H, I))):
            if dims.wfmt in ROW_SCALED:
                nb = 1 << code_bits(dims.wfmt)
                qs[m].append(_pack_fields(_sweep_fields(rows, cols, nb, (seed_tag, e, m, "q")), dims.wfmt))
                base = 0.02 / _CODE_SPREAD[dims.wfmt]
                f = torch.tensor([_ROW_FACTORS[(r + e + m) % len(_ROW_FACTORS)] for r in range(rows)])
                ss[m].append((base * f).to(torch.float16))
            else:
                qs[m].append(_pack_fields(_sweep_fields(rows, cols, 16, (seed_tag, e, m, "q")), dims.wfmt))
                band = e4m3_band_codes(band_of(e, m))
                idx = _sweep_fields(rows, cols // 16, len(band), (seed_tag, e, m, "s"))
                sc = torch.tensor(band, dtype=torch.uint8)[idx]
                mags = torch.tensor(band, dtype=torch.uint8).view(torch.float8_e4m3fn).float().abs()
                typ = float(mags[mags > 0].mean())
                g3[e, m] = 0.02 / (2.25 * typ)  # 2.25: mean |e2m1| over the 16 codes
                ss[m].append(sc.contiguous())
    rw, rb = make_router(dims, (seed_tag, "router"))
    st = [torch.stack(v) for v in ss]
    return Layer(dims, torch.stack(qs[0]), st[0], torch.stack(qs[1]), st[1], torch.stack(qs[2]), st[2], g3, rw, rb)


def make_tokens(dims: Dims, T: int, seed_tag, device="cpu") -> torch.Tensor:
    """x ~ N(0,1) rounded to binary16, shape [T][H]."""
    if T == 0:
        return torch.empty((0, dims.hidden), dtype=torch.float16, device=device)
    return torch.randn((T, dims.hidden), generator=_gen(device, seed_tag, "x"), device=device,
                       dtype=torch.float32).to(torch.float16)


def workload(name: str, seed=0, device="cpu", layer_idx=0):
    w = WORKLOADS[name]
    dims = w["dims"]
    layer = make_layer(dims, (name, seed, layer_idx), device=device, zipf=w.get("zipf", 0.0))
    x = make_tokens(dims, w["tokens"], (name, seed, layer_idx), device=device)
    return layer, x
