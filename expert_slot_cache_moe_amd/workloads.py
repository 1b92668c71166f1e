"""Seeded synthetic inputs shaped like the decode workloads on the pages.

This module only draws numbers and lays them out in the storage formats
the library and the oracle read (bf16 bit patterns, 4-bit codes with e4m3
or e8m0 scales); it holds none of the decode step's arithmetic and imports neither
the oracle nor the HIP binding, so both can be fed from it.

Recipes (numpy PCG64; each purpose gets its own stream spawned from the
seed):
  - expert weights: N(0, 0.02), stored as bf16 (round to nearest even via
    torch), or quantized per 16 consecutive elements of a row: scale =
    e4m3(amax / 6) (torch's float8_e4m3fn conversion), code = the nearest
    E2M1 value of w / scale, global scale 1.0; or MXFP4 (per 32 elements,
    a power-of-two e8m0 scale, the OCP MX recipe);
  - hidden states: N(0, 1) as bf16;
  - router logits: N(0, 1) plus a Zipf rank bias -s * ln(rank + 1) over a
    seeded expert permutation, so the softmax favours experts with
    probability ~ 1 / (rank + 1)^s.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass

import numpy as np
import torch

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def rng(seed: int, *purpose) -> np.random.Generator:
    """An independent generator per (seed, purpose...)."""
    key = tuple(zlib.crc32(str(p).encode()) for p in purpose)
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def bf16_bits(a) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_bf16(g: np.random.Generator, shape, std=1.0) -> np.ndarray:
    return bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(std))


# ---------------------------------------------------------------- weights

def bf16_expert_rows(g: np.random.Generator, rows: int, H: int, F: int, std=0.02):
    """Two banks [rows, bytes]: w13 [2F][H] and w2 [H][F], bf16."""
    w13 = normal_bf16(g, (rows, 2 * F * H), std).view(np.uint8).reshape(rows, -1)
    w2 = normal_bf16(g, (rows, H * F), std).view(np.uint8).reshape(rows, -1)
    return [w13, w2]


def _quantize_e2m1(w: np.ndarray):
    """w [n, cols] float32 -> (codes [n, cols/2] u8, scales [n, cols/16] u8)."""
    n, cols = w.shape
    blk = w.reshape(n, cols // 16, 16)
    amax = np.abs(blk).max(axis=2)
    sc8 = torch.from_numpy((amax / 6.0).astype(np.float32)).to(torch.float8_e4m3fn)
    scale = sc8.float().numpy()
    safe = np.where(scale > 0, scale, 1.0)
    mag = np.abs(blk) / safe[:, :, None]
    mids = (E2M1_VALUES[1:] + E2M1_VALUES[:-1]) / 2
    code = np.searchsorted(mids, mag).astype(np.uint8)          # 0..7, saturating at 6
    code |= (blk < 0).astype(np.uint8) << 3
    code = code.reshape(n, cols)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sc8.view(torch.uint8).numpy()


def e2m1_expert_rows(g: np.random.Generator, rows: int, H: int, F: int, std=0.02):
    """Six banks [rows, bytes]: w13 codes/scales/global, w2 codes/scales/global."""
    banks = [[], [], [], [], [], []]
    for _ in range(rows):
        for m, (nr, nc) in enumerate(((2 * F, H), (H, F))):
            w = g.standard_normal((nr, nc), dtype=np.float32) * np.float32(std)
            codes, scales = _quantize_e2m1(w)
            banks[3 * m].append(codes.reshape(-1))
            banks[3 * m + 1].append(scales.reshape(-1))
            banks[3 * m + 2].append(np.array([1.0], np.float32).view(np.uint8))
    return [np.stack(b) for b in banks]


def _quantize_mxfp4(w: np.ndarray):
    """w [n, cols] float32 -> (codes [n, cols/2] u8, e8m0 scales [n, cols/32] u8):
    the OCP MX recipe, shared scale 2^(floor(log2(amax)) - 2) per 32
    consecutive elements (2 = the largest E2M1 exponent), codes the nearest
    E2M1 value of w / scale, saturating at 6."""
    n, cols = w.shape
    blk = w.reshape(n, cols // 32, 32).astype(np.float64)
    amax = np.abs(blk).max(axis=2)
    e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    code8 = np.clip(e + 127, 0, 254).astype(np.uint8)
    scale = np.ldexp(1.0, code8.astype(np.int64) - 127)
    mag = np.abs(blk) / scale[:, :, None]
    mids = (E2M1_VALUES[1:] + E2M1_VALUES[:-1]) / 2
    code = np.searchsorted(mids, mag).astype(np.uint8)
    code |= (blk < 0).astype(np.uint8) << 3
    code = code.reshape(n, cols)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, code8


def mxfp4_expert_rows(g: np.random.Generator, rows: int, H: int, F: int, std=0.02):
    """Four banks [rows, bytes]: w13 codes/e8m0 scales, w2 codes/e8m0 scales."""
    banks = [[], [], [], []]
    for _ in range(rows):
        for m, (nr, nc) in enumerate(((2 * F, H), (H, F))):
            w = g.standard_normal((nr, nc), dtype=np.float32) * np.float32(std)
            codes, scales = _quantize_mxfp4(w)
            banks[2 * m].append(codes.reshape(-1))
            banks[2 * m + 1].append(scales.reshape(-1))
    return [np.stack(b) for b in banks]


def expert_rows(fmt: int, g, rows, H, F, std=0.02):
    if fmt == 0:
        return bf16_expert_rows(g, rows, H, F, std)
    if fmt == 1:
        return e2m1_expert_rows(g, rows, H, F, std)
    return mxfp4_expert_rows(g, rows, H, F, std)


# ---------------------------------------------------------------- weights drawn on the device

def _torch_generator(device, seed, *purpose) -> torch.Generator:
    key = zlib.crc32(repr((seed,) + purpose).encode())
    gen = torch.Generator(device=device)
    gen.manual_seed(key)
    return gen


def _quantize_e2m1_torch(w: torch.Tensor):
    """The numpy E2M1 recipe (_quantize_e2m1) in torch, on w's device."""
    n, cols = w.shape
    blk = w.reshape(n, cols // 16, 16)
    amax = blk.abs().amax(dim=2)
    sc8 = (amax / 6.0).to(torch.float8_e4m3fn)
    scale = sc8.float()
    safe = torch.where(scale > 0, scale, torch.ones_like(scale))
    mag = blk.abs() / safe[:, :, None]
    vals = torch.tensor(E2M1_VALUES, dtype=torch.float32, device=w.device)
    mids = (vals[1:] + vals[:-1]) / 2
    code = torch.bucketize(mag, mids).to(torch.uint8)           # same ties as searchsorted 'left'
    code |= (blk < 0).to(torch.uint8) << 3
    code = code.reshape(n, cols)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), sc8.view(torch.uint8).contiguous()


def _quantize_mxfp4_torch(w: torch.Tensor):
    """The numpy MXFP4 recipe (_quantize_mxfp4) in torch, on w's device."""
    n, cols = w.shape
    blk = w.reshape(n, cols // 32, 32).double()
    amax = blk.abs().amax(dim=2)
    pos = amax > 0
    e = torch.where(pos, torch.floor(torch.log2(torch.where(pos, amax, torch.ones_like(amax)))) - 2,
                    torch.full_like(amax, -127.0))
    code8 = torch.clamp(e + 127, 0, 254).to(torch.uint8)
    scale = torch.ldexp(torch.ones_like(amax), code8.to(torch.int64) - 127)
    mag = blk.abs() / scale[:, :, None]
    vals = torch.tensor(E2M1_VALUES, dtype=torch.float64, device=w.device)
    mids = (vals[1:] + vals[:-1]) / 2
    code = torch.bucketize(mag, mids).to(torch.uint8)
    code |= (blk < 0).to(torch.uint8) << 3
    code = code.reshape(n, cols)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), code8.contiguous()


def e2m1_global_scales(rows: int, matrix: int) -> np.ndarray:
    """Per-expert fp32 global scales of the E2M1 pools drawn on the device,
    distinct for up to 509 experts: 1 + (e mod 509) / 512 for w13 and
    1 - (e mod 509) / 1024 for w2 (exact in fp32)."""
    e = np.arange(rows) % 509
    g = 1.0 + e / 512.0 if matrix == 0 else 1.0 - e / 1024.0
    return g.astype(np.float32)


def device_expert_rows(fmt: int, seed, rows: int, H: int, F: int, device="cuda", std=0.02,
                       chunk_rows: int = 16):
    """Banks [rows, bytes] (uint8 tensors on `device`) in which every
    expert's weights are drawn afresh: N(0, std) from torch's seeded
    generator, stored as bf16 or quantized with the same E2M1 / MXFP4
    recipes as the numpy generators.  E2M1 pools get distinct per-expert
    global scales (e2m1_global_scales), so no two experts share bytes.
    Full-size pools (gigabytes) are drawn this way in seconds."""
    gen = _torch_generator(device, seed, "device-experts", fmt, rows, H, F)
    shapes = ((2 * F, H), (H, F))
    if fmt == 0:
        banks = [torch.empty((rows, 2 * nr * nc), dtype=torch.uint8, device=device) for nr, nc in shapes]
    elif fmt == 1:
        banks = []
        for nr, nc in shapes:
            banks += [torch.empty((rows, nr * nc // 2), dtype=torch.uint8, device=device),
                      torch.empty((rows, nr * nc // 16), dtype=torch.uint8, device=device),
                      torch.empty((rows, 4), dtype=torch.uint8, device=device)]
    else:
        banks = []
        for nr, nc in shapes:
            banks += [torch.empty((rows, nr * nc // 2), dtype=torch.uint8, device=device),
                      torch.empty((rows, nr * nc // 32), dtype=torch.uint8, device=device)]
    for r0 in range(0, rows, chunk_rows):
        n = min(chunk_rows, rows - r0)
        for m, (nr, nc) in enumerate(shapes):
            w = torch.randn((n * nr, nc), generator=gen, device=device, dtype=torch.float32).mul_(std)
            if fmt == 0:
                banks[m][r0:r0 + n] = w.to(torch.bfloat16).view(torch.uint8).reshape(n, -1)
            elif fmt == 1:
                codes, scales = _quantize_e2m1_torch(w)
                banks[3 * m][r0:r0 + n] = codes.reshape(n, -1)
                banks[3 * m + 1][r0:r0 + n] = scales.reshape(n, -1)
            else:
                codes, scales = _quantize_mxfp4_torch(w)
                banks[2 * m][r0:r0 + n] = codes.reshape(n, -1)
                banks[2 * m + 1][r0:r0 + n] = scales.reshape(n, -1)
    if fmt == 1:
        for m in range(2):
            g = torch.from_numpy(e2m1_global_scales(rows, m).view(np.uint8).reshape(rows, 4))
            banks[3 * m + 2].copy_(g)
    return banks


def pinned_copy(t: torch.Tensor) -> torch.Tensor:
    """A pinned host copy of a device tensor."""
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


# ---------------------------------------------------------------- routing

def zipf_bias(g: np.random.Generator, E: int, s: float) -> np.ndarray:
    """Per-expert logit bias -s * ln(rank + 1) over a random rank order."""
    rank = g.permutation(E)
    return (-s * np.log(rank + 1.0)).astype(np.float32)


def zipf_logits(g: np.random.Generator, T: int, E: int, s: float, bias=None) -> np.ndarray:
    if bias is None:
        bias = zipf_bias(g, E, s)
    return (g.standard_normal((T, E), dtype=np.float32) + bias[None, :]).astype(np.float32)


def forced_logits(g: np.random.Generator, chosen: np.ndarray, E: int, bonus=10.0) -> np.ndarray:
    """N(0,1) logits with +bonus on chosen[t, :] so those experts are each
    row's top-k (the router stays in the path; the recipe picks experts)."""
    T = chosen.shape[0]
    lg = g.standard_normal((T, E), dtype=np.float32)
    np.put_along_axis(lg, chosen, np.take_along_axis(lg, chosen, 1) + np.float32(bonus), 1)
    return lg


# ---------------------------------------------------------------- configurations

@dataclass(frozen=True)
class Shape:
    name: str
    layers: int
    experts: int
    top_k: int
    hidden: int
    ffn: int
    slots: int
    tokens: int
    fmt: int = 0
    shared: bool = False


TINY = Shape("tiny", 1, 8, 2, 64, 128, 4, 1)
ADMISSION_ONLY = Shape("admission-only", 48, 512, 10, 0, 0, 2100, 1)
SHARED_DECODE = Shape("shared-expert-decode", 40, 256, 8, 2048, 512, 3164, 1, shared=True)
WIDE_BF16 = Shape("wide-decode-bf16", 1, 160, 2, 1024, 256, 160, 150)
WIDE_E2M1 = Shape("wide-decode-e2m1", 1, 160, 2, 1024, 256, 1100, 600, fmt=1)
PREFILL_256 = Shape("prefill-chunk-256", 1, 256, 6, 4096, 1024, 256, 42)
PREFILL_640 = Shape("prefill-chunk-640", 1, 640, 6, 4096, 1024, 640, 50)

ADMISSION_BATCHES = (1, 4, 8, 12, 13, 16, 24, 32, 48, 128)


def tiny_logits(seed: int = 0, steps: int = 32) -> np.ndarray:
    """[steps, 1, 8] router logits, N(0,1) + Zipf(1.1) bias."""
    g = rng(seed, "tiny", "logits")
    bias = zipf_bias(g, TINY.experts, 1.1)
    return zipf_logits(g, steps, TINY.experts, 1.1, bias)[:, None, :]


def admission_ids(seed: int, requests: int, experts=512, per_request=10) -> np.ndarray:
    """One step's routes: each request picks per_request distinct uniform ids."""
    g = rng(seed, "admission", requests)
    return np.concatenate([g.choice(experts, per_request, replace=False)
                           for _ in range(requests)]).astype(np.int32)


def wide_bf16_routes(seed: int = 0) -> np.ndarray:
    """150 rows x top-2 over 160 experts: rows 0..79 take experts (2i, 2i+1)
    of a seeded permutation, the rest 2 distinct uniform experts."""
    g = rng(seed, "wide-bf16", "routes")
    perm = g.permutation(160)
    chosen = np.empty((150, 2), np.int64)
    for r in range(150):
        chosen[r] = perm[2 * r:2 * r + 2] if r < 80 else g.choice(160, 2, replace=False)
    return chosen


# ---------------------------------------------------------------- the decode trace

class DecodeTrace:
    """Batch-1 decode routing for L layers x E experts, top-K, with
    per-layer Zipf(s) popularity and temporal locality: each layer keeps a
    working set of K experts; at every token each member is kept with
    probability `stay`, else replaced by a fresh Zipf draw.  The logits put
    the working set on top (+bonus), so the router selects it."""

    # stay = 0.73 gives ~28 misses per token on 40 x 256 experts, top-8,
    # 3164 slots after a 64-token warm-up (checked against the oracle's
    # admission in the tests).
    def __init__(self, seed: int, layers: int, experts: int, top_k: int, s: float = 1.05,
                 stay: float = 0.73):
        self.L, self.E, self.K, self.stay = layers, experts, top_k, stay
        g = rng(seed, "trace", "popularity")
        self.p = np.empty((layers, experts))
        for l in range(layers):
            rank = g.permutation(experts)
            w = 1.0 / (rank + 1.0) ** s
            self.p[l] = w / w.sum()
        self.g = rng(seed, "trace", "steps")
        self.sets = [list(self.g.choice(experts, top_k, replace=False, p=self.p[l]))
                     for l in range(layers)]

    def _advance(self):
        for l in range(self.L):
            cur = self.sets[l]
            for i in range(self.K):
                if self.g.random() >= self.stay:
                    while True:
                        e = int(self.g.choice(self.E, p=self.p[l]))
                        if e not in cur:
                            break
                    cur[i] = e

    def step_sets(self) -> np.ndarray:
        """Advances one token; returns the [L, K] expert working sets."""
        self._advance()
        return np.array(self.sets, np.int64)

    def logits(self, sets: np.ndarray) -> np.ndarray:
        return forced_logits(self.g, sets, self.E)
