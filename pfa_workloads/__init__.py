"""Seeded synthetic inputs for packed varlen attention (shared by tests, smoke and bench).

This module holds no attention arithmetic.  It draws the inputs, rounds them to bf16
and builds segment tables; the oracle and the HIP path both consume what it returns.

Recipe (every workload): ``numpy.random.default_rng(seed)`` draws Q, then K, then V,
each ``standard_normal((T, H, d), float32)``; any per-head scaling is applied next;
values are then rounded to bf16 (round-to-nearest-even) and returned as uint16 bit
patterns.  Segment lengths follow the patch counts of the Mage-Flow page (section on
native-resolution sequence packing: 512x512 -> 1024 tokens, 1024x1024 -> 4096,
768x432 -> 1296 at patch 16) and the [batch 8, heads 8, 4096, 64] shape of the
GigaPath-Flash page, section 4.1.  No dataset or trained weights are involved.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# ----------------------------------------------------------------------------- bf16

def bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even.

    Finite inputs only (the largest finite pattern plus the rounding increment still fits
    in 32 bits); NaN and infinity patterns are passed through by truncation."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    finite = np.isfinite(f)
    r = (u >> 16) & 1
    r += u
    r += np.uint32(0x7FFF)
    r >>= 16
    if not finite.all():
        r[~finite] = u[~finite] >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(bits) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


# ----------------------------------------------------------------------- workloads

def _c3_lengths():
    base = [4096] * 7 + [1296] * 5 + [1024] * 4
    perm = np.random.default_rng(0).permutation(len(base))
    return [base[i] for i in perm]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    lengths: tuple
    heads: int
    head_dim: int
    description: str
    per_head_qk_scale: bool = False


CONFIGS = {
    "C1": Config("C1", (256, 64), 4, 64,
                 "2 images (256^2 and 128^2 at patch 16), seg [256,64], 4 heads, d 64"),
    "C2": Config("C2", (4096,) * 8, 8, 64,
                 "8 sequences of 4096 packed, 8 heads, d 64 (GigaPath-Flash 4.1 shape)"),
    "C3": Config("C3", tuple(_c3_lengths()), 24, 128,
                 "Mage-Flow mixed pack: 7x4096 + 5x1296 + 4x1024 (seed-0 permutation), "
                 "39,248 tokens, 24 heads, d 128"),
    "C4": Config("C4", (4096,) * 8, 24, 128,
                 "8x4096 packed, 24 heads, d 128, Q and K of head h scaled by 0.5+1.5h/23",
                 per_head_qk_scale=True),
    "C5a": Config("C5a", (65536,), 16, 128, "one segment of 65536 tokens, 16 heads, d 128"),
    "C5b": Config("C5b", (65536, 16384, 4096, 1296, 1), 16, 128,
                  "5-segment pack [65536,16384,4096,1296,1], 16 heads, d 128"),
}


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def flops(lengths, heads: int, head_dim: int) -> float:
    """Counted work 4 * sum(L^2) * H * d (QK^T and PV, 2 flops per multiply-add)."""
    return 4.0 * float(sum(int(L) * int(L) for L in lengths)) * heads * head_dim


@dataclasses.dataclass
class Workload:
    name: str
    q: np.ndarray          # uint16 bf16 bits [T, H, d]
    k: np.ndarray
    v: np.ndarray
    cu_seqlens: np.ndarray  # int32 [num_seqs + 1]
    lengths: tuple
    heads: int
    head_dim: int
    scale: float
    max_seqlen: int
    seed: int

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def num_seqs(self) -> int:
        return len(self.lengths)

    @property
    def flops(self) -> float:
        return flops(self.lengths, self.heads, self.head_dim)


def make(lengths, heads: int, head_dim: int, seed: int = 0, name: str = "custom",
         per_head_qk_scale: bool = False, scale: float | None = None) -> Workload:
    lengths = tuple(int(L) for L in lengths)
    T = int(sum(lengths))
    rng = np.random.default_rng(seed)
    shape = (T, heads, head_dim)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if per_head_qk_scale:
        s = (0.5 + 1.5 * np.arange(heads, dtype=np.float64) / max(heads - 1, 1)).astype(np.float32)
        q *= s[None, :, None]
        k *= s[None, :, None]
    return Workload(name=name, q=bf16_bits(q), k=bf16_bits(k), v=bf16_bits(v),
                    cu_seqlens=cu_from_lengths(lengths), lengths=lengths, heads=heads,
                    head_dim=head_dim,
                    scale=float(scale) if scale is not None else 1.0 / math.sqrt(head_dim),
                    max_seqlen=max(lengths) if lengths else 0, seed=seed)


def generate(name: str, seed: int = 0) -> Workload:
    c = CONFIGS[name]
    return make(c.lengths, c.heads, c.head_dim, seed=seed, name=name,
                per_head_qk_scale=c.per_head_qk_scale)


@dataclasses.dataclass
class CrossWorkload:
    """Separate query and key segment tables: queries of segment s attend keys of s."""
    name: str
    q: np.ndarray          # uint16 bf16 bits [Tq, H, d]
    k: np.ndarray          # [Tk, H, d]
    v: np.ndarray          # [Tk, H, d]
    cu_q: np.ndarray       # int32 [num_seqs + 1]
    cu_k: np.ndarray
    lengths_q: tuple
    lengths_k: tuple
    heads: int
    head_dim: int
    scale: float
    seed: int

    @property
    def total_q(self) -> int:
        return int(self.cu_q[-1])

    @property
    def total_k(self) -> int:
        return int(self.cu_k[-1])

    @property
    def num_seqs(self) -> int:
        return len(self.lengths_q)

    @property
    def max_q(self) -> int:
        return max(max(self.lengths_q), 1)

    @property
    def max_k(self) -> int:
        return max(max(self.lengths_k), 1)

    @property
    def flops(self) -> float:
        return 4.0 * float(sum(int(a) * int(b) for a, b in zip(self.lengths_q, self.lengths_k))) \
            * self.heads * self.head_dim


def make_cross(lengths_q, lengths_k, heads: int, head_dim: int, seed: int = 0,
               name: str = "cross", scale: float | None = None) -> CrossWorkload:
    """Draw Q [Tq, H, d], then K and V [Tk, H, d], N(0,1) float32, rounded to bf16."""
    lengths_q = tuple(int(L) for L in lengths_q)
    lengths_k = tuple(int(L) for L in lengths_k)
    if len(lengths_q) != len(lengths_k):
        raise ValueError("one key length per query segment")
    rng = np.random.default_rng(seed)
    tq, tk = int(sum(lengths_q)), int(sum(lengths_k))
    q = rng.standard_normal((tq, heads, head_dim), dtype=np.float32)
    k = rng.standard_normal((tk, heads, head_dim), dtype=np.float32)
    v = rng.standard_normal((tk, heads, head_dim), dtype=np.float32)
    return CrossWorkload(name=name, q=bf16_bits(q), k=bf16_bits(k), v=bf16_bits(v),
                         cu_q=cu_from_lengths(lengths_q), cu_k=cu_from_lengths(lengths_k),
                         lengths_q=lengths_q, lengths_k=lengths_k, heads=heads,
                         head_dim=head_dim,
                         scale=float(scale) if scale is not None else 1.0 / math.sqrt(head_dim),
                         seed=seed)


# Cross-attention workload: the Mage-Flow mixed pack's image tokens (C3's segments, same
# order) as queries, each image attending its own 256-token condition sequence ("long Q,
# short KV").  The pages give no condition length; 256 is the reading used here.
CROSS_CONFIGS = {
    "X1": dict(lengths_q=tuple(_c3_lengths()), lengths_k=(256,) * 16, heads=24, head_dim=128,
               description="cross-attention: 16 images (7x4096+5x1296+4x1024 query tokens) "
                           "each attending 256 condition tokens, 24 heads, head_dim 128"),
}


def generate_cross(name: str, seed: int = 0) -> CrossWorkload:
    c = CROSS_CONFIGS[name]
    return make_cross(c["lengths_q"], c["lengths_k"], c["heads"], c["head_dim"], seed=seed,
                      name=name)


# ------------------------------------------------- fused QKV input and angle tables

def grid_positions(lengths) -> tuple:
    """(row, col) patch coordinates of every packed token: a segment of L tokens is an
    image laid out row-major on a grid ceil(sqrt(L)) patches wide (4096 -> 64 x 64,
    1296 -> 36 x 36), restarting at (0, 0) for every segment."""
    rows, cols = [], []
    for L in lengths:
        L = int(L)
        w = max(1, math.isqrt(L - 1) + 1) if L > 0 else 1
        i = np.arange(L, dtype=np.int64)
        rows.append(i // w)
        cols.append(i % w)
    if not rows:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return np.concatenate(rows), np.concatenate(cols)


def rope_tables_2d(lengths, head_dim: int, base: float = 10000.0) -> tuple:
    """Axial 2-D rotary angle tables (cos, sin), float32 [T, head_dim / 2]: the first half
    of the head_dim / 2 frequency pairs turns with the patch row, the second half with
    the patch column, at frequencies base^(-j / (head_dim / 4)), j = 0 .. head_dim/4 - 1.
    Angles are formed in fp64 and their cosine and sine rounded once to float32."""
    if head_dim % 4:
        raise ValueError("head_dim must be a multiple of 4")
    r, c = grid_positions(lengths)
    nf = head_dim // 4
    freq = base ** (-np.arange(nf, dtype=np.float64) / nf)
    ang = np.concatenate([r[:, None] * freq[None, :], c[:, None] * freq[None, :]], axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def fuse_qkv(q, k, v) -> np.ndarray:
    """[T, 3, H, d] bf16 bits: the layout of one projection whose output features are q,
    then k, then v (row t holds 3 * H * d consecutive values)."""
    return np.ascontiguousarray(np.stack([q, k, v], axis=1))


# ---------------------------------------------------------- block-sparse tile layouts

SPARSE_BLOCK_Q = 256    # query rows per listed block (one query tile of the kernel)
SPARSE_BLOCK_K = 64     # keys per key block


def band_layout(lengths, radius: int, block_q: int = SPARSE_BLOCK_Q,
                block_k: int = SPARSE_BLOCK_K) -> list:
    """A sliding-tile band: query block I of a segment lists every key block that overlaps
    [I*block_q - radius, (I+1)*block_q + radius) inside the segment.  For an image in raster
    order at 64 patches per row, radius 1024 is a band of +-16 patch rows around the
    query tile's 4 rows.  Returns layout[0][s][I] (one layout shared by every head)."""
    segs = []
    for L in lengths:
        L = int(L)
        nkb = -(-L // block_k)
        rows = []
        for I in range(-(-L // block_q)):
            lo = max(0, I * block_q - radius)
            hi = min(L, (I + 1) * block_q + radius)
            rows.append(list(range(lo // block_k, min(nkb, -(-hi // block_k)))))
        segs.append(rows)
    return [segs]


def random_layout(rng: np.random.Generator, lengths, heads_layout: int, density: float,
                  block_q: int = SPARSE_BLOCK_Q, block_k: int = SPARSE_BLOCK_K) -> list:
    """Each key block of a segment is listed for a query block with probability
    ``density``, in a random order; layout[hl][s][I] for hl < heads_layout."""
    lay = []
    for _ in range(heads_layout):
        segs = []
        for L in lengths:
            nkb = -(-int(L) // block_k)
            segs.append([[int(J) for J in rng.permutation(nkb) if rng.random() < density]
                         for _ in range(-(-int(L) // block_q))])
        lay.append(segs)
    return lay


def layout_pairs(layout, lengths, heads: int, block_q: int = SPARSE_BLOCK_Q,
                 block_k: int = SPARSE_BLOCK_K) -> int:
    """Allowed (query, key) pairs summed over heads: the work a block-sparse pass must do
    (rows of each query block times keys of each listed block, clipped to the segment)."""
    total = 0
    for h in range(heads):
        hl = layout[h if len(layout) == heads else 0]
        for s, L in enumerate(lengths):
            L = int(L)
            for I, row in enumerate(hl[s]):
                nq = min(block_q, L - I * block_q)
                nk = sum(min(block_k, L - J * block_k) for J in set(row) if 0 <= J * block_k < L)
                total += nq * nk
    return total


def sample_rows(cu_seqlens, stride: int = 61, edge: int = 128, full_upto: int = 4096) -> np.ndarray:
    """Deterministic row sample for configurations too large for the oracle in full.

    Keeps rows r of segment [a, b) with (r - a) % stride == 0, rows within ``edge`` of
    either segment end, and every row of segments no longer than ``full_upto``.  A prime
    stride walks every residue of a power-of-two tile size.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    keep = []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        r = np.arange(a, b)
        if b - a <= full_upto:
            keep.append(r)
            continue
        m = ((r - a) % stride == 0) | (r - a < edge) | (b - 1 - r < edge)
        keep.append(r[m])
    return np.concatenate(keep) if keep else np.zeros(0, dtype=np.int64)


def random_lengths(rng: np.random.Generator, n: int, max_len: int, p_zero: float = 0.1,
                   p_one: float = 0.1) -> list:
    """Random segment lengths including the degenerate 0 and 1 cases."""
    out = []
    for _ in range(n):
        u = rng.random()
        if u < p_zero:
            out.append(0)
        elif u < p_zero + p_one:
            out.append(1)
        else:
            out.append(int(rng.integers(2, max_len + 1)))
    return out


# ------------------------------------------------- SparseAttn worked-example inputs

@dataclasses.dataclass
class WorkedExample:
    q: np.ndarray       # float64 [2 heads, n, d]; k is the same array
    v: np.ndarray       # float64 [n, 3], shared by both heads
    frame: np.ndarray   # frame index of each token (frame-major order)
    pixel: np.ndarray   # position index within the frame
    frames: int
    positions: int


def worked_example() -> WorkedExample:
    """Inputs of the worked experiment in section 4 of the jefxiong.cn SparseAttn article.

    The article describes a video of 4 frames on a 4 x 4 grid of positions, 64 tokens in
    frame-major order, and two synthetic heads: in the first ("spatial") every token
    carries a signal of strength 6 on a feature naming its frame, in the second
    ("temporal") on a feature naming its position within the frame.  Features are one-hot:
    the 4 frame features come first, then the 16 position features (d = 20).  Gaussian
    noise of standard deviation 0.15 is added to both heads, keys equal queries, and the
    values are standard normal of width 3, shared by both heads; the generator is
    numpy's default_rng seeded with 7, the noise drawn before the values (the order that
    reproduces the printed numbers).
    """
    frames, positions = 4, 16
    order = [(f, p) for f in range(frames) for p in range(positions)]   # frame-major
    frame = np.array([f for f, _ in order])
    pixel = np.array([p for _, p in order])
    features = np.eye(frames + positions)
    # head 0 names the frame feature, head 1 the position feature after the frame block
    signal = np.stack([6.0 * features[frame], 6.0 * features[frames + pixel]])
    gen = np.random.default_rng(7)
    noise = gen.normal(0.0, 0.15, size=signal.shape)
    values = gen.standard_normal((len(order), 3))
    return WorkedExample(q=signal + noise, v=values, frame=frame, pixel=pixel, frames=frames,
                         positions=positions)
