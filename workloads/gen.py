"""Workload definitions and seeded generators (inputs only, no attention math).

Shapes follow the video-DiT attention layers that the FG-Attn page measures on
(Wan 2.1 14B 480p/720p 81 frames, HunyuanVideo 720p 129 frames; "Recorded
benchmark results" on the FG-Attn page).  Model weights are not available, so
Q/K/V are i.i.d. normal and keep-masks follow the recipes below.

Mask bitmap format (shared by every consumer): uint32 words, row-major
[B][H][T_q][words], bit (j % 32) of word (j // 32) is key tile j, LSB first,
1 = tile kept.  Padding bits past T_k are zero here; consumers ignore them.

Random streams:
  * Q, K, V, offsets: torch CPU generator seeded with seed*8 + {0,1,2,4},
    fp32 normal draws, rounded to bf16 (round-to-nearest-even) for bf16 runs.
  * i.i.d. / frame-structured masks: a counter-based generator, SplitMix64
    (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
    OOPSLA 2014): output number ctr+1 of a SplitMix64 stream whose state starts
    at seed*8 + 3, where ctr = ((b*H + h)*T_q + i)*T_k + j.  A tile is kept iff
    (z >> 40) < thr with thr = round(p * 2**24), integer-only, so the GPU
    generator reproduces it bit for bit.
  * exact-count masks: numpy Generator(PCG64(seed*8 + 3)).choice per head.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)


# --------------------------------------------------------------------------
# SplitMix64 (published definition), vectorised over counters
# --------------------------------------------------------------------------
def splitmix64(state0: int, ctr) -> np.ndarray:
    """Output number ctr+1 of a SplitMix64 stream whose state starts at state0.

    SplitMix64 advances its state by the golden gamma 0x9E3779B97F4A7C15 and
    returns a mixed copy of it, so output n depends only on state0 + n*gamma:
    a counter-based generator.
    """
    c = np.asarray(ctr, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(state0 & 0xFFFFFFFFFFFFFFFF) + (c + np.uint64(1)) * GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        z = z ^ (z >> np.uint64(31))
    return z


def prob_threshold(p: float) -> int:
    """24-bit integer threshold for keep probability p."""
    return int(round(p * (1 << 24)))


# --------------------------------------------------------------------------
# Workload description
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class MaskRecipe:
    kind: str                     # "hash" | "exact_drop" | "predicted" | "ones" | "diag_only" | "structured"
    p_near: float = 0.0           # hash: keep probability near the query frame (or everywhere)
    p_far: float = 0.0            # hash: keep probability outside the frame window
    frame_tokens: int = 0         # hash: tokens per latent frame (0: no frame structure)
    frame_radius: int = 2         # hash: |q_frame - k_frame| <= radius is "near"
    drop_fraction: float = 0.0    # exact_drop
    sparsity_percent: int = 0     # predicted
    force_diag: bool = True
    # structured: one pattern per head (PATTERN_* codes of tsa_workload.h);
    # frame_tokens is the multi-diagonal spacing
    patterns: tuple = ()
    diag_width: int = 0
    band_width: int = 0
    reach: int = 0
    stripe_period: int = 0
    stripe_width: int = 0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    M: int
    N: int
    dtype: str                    # "f32" | "bf16"
    mask: MaskRecipe
    seed: int
    offset_frame_tokens: int = 0  # >0: per-frame shared offset added to Q and K
    offset_sigma: float = 0.0
    description: str = ""

    @property
    def T_q(self) -> int:
        return -(-self.L // self.M)

    @property
    def T_k(self) -> int:
        return -(-self.L // self.N)

    @property
    def words(self) -> int:
        return row_words(self.L, self.N)

    @property
    def scale(self) -> float:
        """1/sqrt(d), rounded to fp32 (the value that crosses the C ABI)."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def row_words(L: int, N: int) -> int:
    return -(-(-(-L // N)) // 32)


def frame_thresholds(w: Workload, p_near_nominal: float, p_far_nominal: float,
                     target: float) -> tuple[float, float]:
    """Scale nominal near/far keep probabilities so the expected kept fraction is `target`.

    A tile's frame is the frame of its first token; the near fraction f is
    counted over the real tile grid.
    """
    ft = w.mask.frame_tokens
    fq = (np.arange(w.T_q, dtype=np.int64) * w.M) // ft
    fk = (np.arange(w.T_k, dtype=np.int64) * w.N) // ft
    nf = int(max(fq.max(), fk.max())) + 1
    cq = np.bincount(fq, minlength=nf).astype(np.float64)
    ck = np.bincount(fk, minlength=nf).astype(np.float64)
    r = w.mask.frame_radius
    near = 0.0
    for a in range(nf):
        lo, hi = max(0, a - r), min(nf, a + r + 1)
        near += cq[a] * ck[lo:hi].sum()
    f = near / (w.T_q * w.T_k)
    c = target / (p_near_nominal * f + p_far_nominal * (1.0 - f))
    return p_near_nominal * c, p_far_nominal * c


def _frames_recipe(L, M, N, frame_tokens, radius=2):
    # near/far probabilities are filled in by _finalise (they depend on the grid)
    return MaskRecipe(kind="hash", frame_tokens=frame_tokens, frame_radius=radius,
                      force_diag=True)


def _finalise(w: Workload) -> Workload:
    if w.mask.kind == "hash" and w.mask.frame_tokens > 0 and w.mask.p_near == 0.0:
        pn, pf = frame_thresholds(w, 0.6, 0.15, 0.30)
        w = w.replace(mask=dataclasses.replace(w.mask, p_near=pn, p_far=pf))
    return w


BASE_SEED = 20250920

CONFIGS: dict[str, Workload] = {}


def _add(w: Workload):
    CONFIGS[w.name] = _finalise(w)


_add(Workload("tiny", 1, 2, 512, 64, 16, 16, "f32",
              MaskRecipe("hash", p_near=0.5, p_far=0.5), BASE_SEED + 1,
              description="1x2x512x64 fp32, 16x16 tiles, i.i.d. keep p=0.5, diagonal kept"))
_add(Workload("wan480_coarse", 1, 40, 32760, 128, 64, 64, "bf16",
              MaskRecipe("exact_drop", drop_fraction=0.70), BASE_SEED + 2,
              description="Wan 2.1 14B 480p 81f shape (21 x 30x52 tokens), 64x64 block-sparse, "
                          "70% of tiles dropped uniformly per head, diagonal kept"))
_add(Workload("wan480_fine", 1, 40, 32760, 128, 16, 8, "bf16",
              _frames_recipe(32760, 16, 8, 1560), BASE_SEED + 3,
              description="Wan 2.1 14B 480p 81f shape, 16x8 tiles, frame-structured 70% sparsity "
                          "(+-2 latent frames kept w.p. 0.6, others 0.15, renormalised to 30%), "
                          "diagonal kept"))
_add(Workload("wan720_n1", 1, 40, 75600, 128, 16, 1, "bf16",
              MaskRecipe("hash", p_near=0.2, p_far=0.2), BASE_SEED + 4,
              description="Wan 2.1 720p 81f shape (21 x 45x80 tokens), 16x1 tiles (per-key column "
                          "skip), 80% i.i.d. sparsity, diagonal 16x16 region kept"))
_add(Workload("hunyuan720", 1, 24, 118800, 128, 16, 16, "bf16",
              MaskRecipe("predicted", sparsity_percent=85, force_diag=False), BASE_SEED + 5,
              offset_frame_tokens=3600, offset_sigma=0.5,
              description="HunyuanVideo 720p 129f shape (33 x 45x80 tokens), 16x16 tiles, mask "
                          "predicted from pooled Q . pooled K at the per-row 85th percentile"))

# Wan 2.1 480p shape with per-head structured patterns: 2 of 40 heads skipped
# (the abstract's 3-6% range), the rest diagonal (width 0.15 L), multi-diagonal
# (width 128 tokens, repeated every 1560-token latent frame over +-20 frames)
# and vertical stripes (390 of every 1560 keys).
_STRUCT_PATTERNS = tuple([0, 0] + [1] * 12 + [2] * 13 + [3] * 13)
_add(Workload("wan480_struct", 1, 40, 32760, 128, 16, 8, "bf16",
              MaskRecipe("structured", frame_tokens=1560, patterns=_STRUCT_PATTERNS, diag_width=4914,
                         band_width=128, reach=20, stripe_period=1560, stripe_width=390,
                         force_diag=False),
              BASE_SEED + 6,
              description="Wan 2.1 480p shape, 16x8 tiles, per-head structured masks: 2 heads "
                          "skipped, 12 diagonal (|q-k| <= 4914), 13 multi-diagonal (|q-k-1560t| <= "
                          "128, |t| <= 20), 13 vertical-stripe (k mod 1560 < 390)"))

# Small bf16 problems for the benchmark's output-contract tests (every line of
# bench.py in seconds); not workloads of the pages.
_add(Workload("small_fine", 1, 2, 2048, 128, 16, 8, "bf16",
              MaskRecipe("hash", p_near=0.3, p_far=0.3), BASE_SEED + 7,
              description="1x2x2048x128 bf16, 16x8 tiles, i.i.d. keep p=0.3, diagonal kept"))
_add(Workload("small_pred", 1, 2, 2048, 128, 16, 16, "bf16",
              MaskRecipe("predicted", sparsity_percent=85, force_diag=False), BASE_SEED + 8,
              description="1x2x2048x128 bf16, 16x16 tiles, mask predicted at the per-row 85th "
                          "percentile of pooled scores"))

HEADLINE = "wan480_fine"


def get(name: str) -> Workload:
    return CONFIGS[name]


# --------------------------------------------------------------------------
# Masks
# --------------------------------------------------------------------------
def diag_tiles(w: Workload, i: int) -> np.ndarray:
    """Key tiles j whose key range overlaps query tile i's row range."""
    r0, r1 = i * w.M, min(i * w.M + w.M, w.L)
    j0 = r0 // w.N
    j1 = -(-r1 // w.N)
    return np.arange(j0, min(j1, w.T_k), dtype=np.int64)


def pack_bits(keep: np.ndarray) -> np.ndarray:
    """bool [..., T_k] -> uint32 [..., ceil(T_k/32)], bit j%32 of word j//32, LSB first."""
    keep = np.asarray(keep, dtype=bool)
    T_k = keep.shape[-1]
    nw = -(-T_k // 32)
    pad = nw * 32 - T_k
    if pad:
        keep = np.concatenate([keep, np.zeros(keep.shape[:-1] + (pad,), dtype=bool)], axis=-1)
    by = np.packbits(keep, axis=-1, bitorder="little")
    return np.ascontiguousarray(by).view("<u4").astype(np.uint32, copy=False)


def _hash_rows(w: Workload, rows: np.ndarray) -> np.ndarray:
    """Hash-recipe keep bits for rows given as (b, h, i) triples -> bool [n, T_k]."""
    m = w.mask
    j = np.arange(w.T_k, dtype=np.uint64)
    out = np.empty((len(rows), w.T_k), dtype=bool)
    thr_n = np.uint64(prob_threshold(m.p_near))
    thr_f = np.uint64(prob_threshold(m.p_far))
    if m.frame_tokens > 0:
        fk = (np.arange(w.T_k, dtype=np.int64) * w.N) // m.frame_tokens
    state0 = w.seed * 8 + 3
    for r, (b, h, i) in enumerate(rows):
        base = np.uint64(((int(b) * w.H + int(h)) * w.T_q + int(i)) * w.T_k)
        u = splitmix64(state0, base + j) >> np.uint64(40)
        if m.frame_tokens > 0:
            fq = (int(i) * w.M) // m.frame_tokens
            thr = np.where(np.abs(fk - fq) <= m.frame_radius, thr_n, thr_f)
        else:
            thr = thr_n
        keep = u < thr
        if m.force_diag:
            keep[diag_tiles(w, int(i))] = True
        out[r] = keep
    return out


# Structured patterns (tsa_workload.h), per head: the diagonal, multi-diagonal
# and vertical-stripe structures and skipped heads that the Sparse-vDiT
# abstract names.  A tile is kept iff its rule holds for some (query, key)
# token pair inside it.
PATTERN_EMPTY, PATTERN_DIAGONAL, PATTERN_MULTI_DIAGONAL, PATTERN_VERTICAL_STRIPE, PATTERN_DENSE = range(5)


def _structured_rows(w: Workload, rows: np.ndarray) -> np.ndarray:
    m = w.mask
    j = np.arange(w.T_k, dtype=np.int64)
    k0 = j * w.N
    k1 = np.minimum(k0 + w.N, w.L) - 1
    out = np.zeros((len(rows), w.T_k), dtype=bool)
    for r, (_, h, i) in enumerate(rows):
        pat = m.patterns[int(h)]
        q0 = int(i) * w.M
        q1 = min(q0 + w.M, w.L) - 1
        if pat == PATTERN_DENSE:
            out[r] = True
        elif pat == PATTERN_DIAGONAL:
            out[r] = (k0 <= q1 + m.diag_width) & (k1 >= q0 - m.diag_width)
        elif pat == PATTERN_MULTI_DIAGONAL:
            for t in range(-m.reach, m.reach + 1):
                sft = t * m.frame_tokens
                out[r] |= (k0 <= q1 + sft + m.band_width) & (k1 >= q0 + sft - m.band_width)
        elif pat == PATTERN_VERTICAL_STRIPE and m.stripe_width > 0:
            rem = k0 % m.stripe_period
            first = np.where(rem < m.stripe_width, k0, k0 + (m.stripe_period - rem))
            out[r] = first <= k1
    return out


def structured_params(w: Workload) -> dict:
    """Arguments of the GPU structured-mask generator for this workload."""
    m = w.mask
    if m.kind != "structured":
        raise ValueError(f"mask recipe {m.kind!r} is not structured")
    return dict(head_patterns=list(m.patterns), diag_width=m.diag_width, band_width=m.band_width,
                frame_tokens=m.frame_tokens, reach=m.reach, stripe_period=m.stripe_period,
                stripe_width=m.stripe_width)


def hash_params(w: Workload) -> dict:
    """Parameters of the counter-based mask recipe, as the GPU generator takes them."""
    m = w.mask
    if m.kind != "hash":
        raise ValueError(f"mask recipe {m.kind!r} is not counter-based")
    return dict(state0=w.seed * 8 + 3, thr_near=prob_threshold(m.p_near),
                thr_far=prob_threshold(m.p_far), frame_tokens=m.frame_tokens,
                frame_radius=m.frame_radius if m.frame_tokens > 0 else 0,
                force_diag=m.force_diag)


def mask_rows_bool(w: Workload, rows) -> np.ndarray:
    """Keep bits (bool [n, T_k]) of the given (b, h, i) rows, for recipes that
    can be evaluated row by row (hash, structured, ones, diag_only)."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    k = w.mask.kind
    if k == "hash":
        return _hash_rows(w, rows)
    if k == "structured":
        return _structured_rows(w, rows)
    if k == "ones":
        return np.ones((len(rows), w.T_k), dtype=bool)
    if k == "diag_only":
        out = np.zeros((len(rows), w.T_k), dtype=bool)
        for r, (_, _, i) in enumerate(rows):
            out[r, diag_tiles(w, int(i))] = True
        return out
    raise ValueError(f"mask recipe {k!r} is not row-separable")


def mask_bits(w: Workload) -> np.ndarray:
    """Whole bitmap uint32 [B, H, T_q, words] (CPU)."""
    k = w.mask.kind
    if k == "exact_drop":
        rng = np.random.Generator(np.random.PCG64(w.seed * 8 + 3))
        out = np.empty((w.B, w.H, w.T_q, w.words), dtype=np.uint32)
        ii = np.arange(w.T_q)
        diag = np.zeros((w.T_q, w.T_k), dtype=bool)
        for i in ii:
            diag[i, diag_tiles(w, int(i))] = True
        nondiag = np.flatnonzero(~diag.ravel())
        n_drop = int(round(w.mask.drop_fraction * w.T_q * w.T_k))
        for b in range(w.B):
            for h in range(w.H):
                drop = rng.choice(nondiag.size, size=n_drop, replace=False)
                keep = np.ones(w.T_q * w.T_k, dtype=bool)
                keep[nondiag[drop]] = False
                out[b, h] = pack_bits(keep.reshape(w.T_q, w.T_k))
        return out
    if k == "predicted":
        raise ValueError("predicted masks come from the predictor, not from a generator")
    out = np.empty((w.B, w.H, w.T_q, w.words), dtype=np.uint32)
    for b in range(w.B):
        for h in range(w.H):
            rows = np.stack([np.full(w.T_q, b), np.full(w.T_q, h), np.arange(w.T_q)], axis=1)
            out[b, h] = pack_bits(mask_rows_bool(w, rows))
    return out


# --------------------------------------------------------------------------
# Q / K / V
# --------------------------------------------------------------------------
def make_qkv(w: Workload, heads=None):
    """Seeded Q, K, V as torch CPU tensors [B, H, L, d] in the workload dtype.

    `heads` restricts generation to a prefix of heads (the full draw is made and
    sliced, so the values equal those of the full tensors).
    """
    import torch

    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    out = []
    offs = None
    if w.offset_frame_tokens > 0:
        g = torch.Generator().manual_seed(w.seed * 8 + 4)
        nf = -(-w.L // w.offset_frame_tokens)
        offs = torch.randn(w.B, w.H, nf, w.d, generator=g, dtype=torch.float32) * w.offset_sigma
        frame = torch.arange(w.L) // w.offset_frame_tokens
    for s, add_off in ((0, True), (1, True), (2, False)):
        g = torch.Generator().manual_seed(w.seed * 8 + s)
        x = torch.randn(w.B, w.H, w.L, w.d, generator=g, dtype=torch.float32)
        if offs is not None and add_off:
            for b in range(w.B):
                for h in range(w.H):
                    x[b, h] += offs[b, h].index_select(0, frame)
        x = x.to(tdt)
        if heads is not None:
            x = x[:, :heads].contiguous()
        out.append(x)
    return tuple(out)


def make_do(w: Workload, heads=None):
    """Seeded upstream gradient dO for the backward: torch CPU [B, H, L, d] in the
    workload dtype, standard normal from its own stream (seed * 8 + 5)."""
    import torch

    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    g = torch.Generator().manual_seed(w.seed * 8 + 5)
    x = torch.randn(w.B, w.H, w.L, w.d, generator=g, dtype=torch.float32).to(tdt)
    return x[:, :heads].contiguous() if heads is not None else x


# --------------------------------------------------------------------------
# Parity sampling
# --------------------------------------------------------------------------
def sample_tiles(w: Workload, per_head: int = 256) -> np.ndarray:
    """Query tiles compared per (b, h): [B, H, n] int64.

    Tile 0 and the last (possibly partial) tile always; the rest drawn without
    replacement from a PCG64 stream seeded with seed + 100.  All tiles when
    T_q <= per_head.
    """
    T = w.T_q
    if T <= per_head:
        return np.broadcast_to(np.arange(T), (w.B, w.H, T)).copy()
    rng = np.random.Generator(np.random.PCG64(w.seed + 100))
    out = np.empty((w.B, w.H, per_head), dtype=np.int64)
    for b in range(w.B):
        for h in range(w.H):
            mid = 1 + rng.choice(T - 2, size=per_head - 2, replace=False)
            out[b, h] = np.sort(np.concatenate([[0, T - 1], mid]))
    return out
