"""Oracle: a plain CPU restatement of the Summaryformer per-block memory.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports, calls or links it,
and this module imports nothing from the product.  The two share only the
seeded input generators of ``sf_inputs``.

Everything is numpy on the host.  Floating-point arithmetic is fp64.  Stored
buffer contents keep the bytes the caller handed in (float32 values, or the
uint16 bit patterns of bfloat16), so byte-exact comparison is direct.

Source.  The method is described on one web page, the model card titled
"GTA world model: weights and inference code" (Summaryformer).  Citations in
this file name its parts:

  [caption]  the caption at the top of the page: the start image and the
             newest three frames kept whole, 22 older frames kept as 96
             summary tokens each; 6,528 keys instead of 26,208.
  [record]   section "A frame is a record": record(t) is the H*W raw tokens
             followed by the X summary tokens.
  [attends]  section "What a frame attends to": the four-item list.
  [buffer]   section "One buffer, no mask": the Z0 | RAW | SUM layout, the
             eviction paragraph, the figure "The buffer one frame apart",
             the parameter table and the dense, unmasked read.
  [sampling] section "The rest of the model", the "Sampling" item: a clean
             pass rewrites the frame's entry in memory.
  [sink]     section "Running for a long time: the start image follows the
             window": rotary keys compose, rotation(id + T) = rotation(id) *
             rotation(T); when the gap between the start image and the oldest
             frame in memory reaches 5, the start image's keys are rotated
             forward to bring it back to 1, values untouched.
  [level]    section "Telling a summary from a pixel: level planes": 12
             temporal planes per head; the two slowest turn by less than half
             a radian over 1024 frames; summary tokens take an exact quarter
             turn on those two; the model refuses to build unless they are idle.
  [positions] section "The rest of the model", the "Positions" item: one
             rotary table with temporal, height and width bands, indexed in
             time by frame id, adapted from Wan2.1.
  [files]    section "Files": the model's files include an optional recency
             bias on summary keys.
  [credits]  section "Credits": that bias follows the Recency Forcing paper,
             which the page does not reproduce.

Readings where the page leaves a step open:
  * Frame 0 is the start image and lives in Z0; generated frames are t >= 1.
  * RAW slot of frame t is t mod (Y+1); SUM slot of frame f is f mod (W-Y).
  * In one step, the eviction runs before the new record is written.
  * Softmax scale defaults to 1/sqrt(head_dim).
  * Empty slots hold zeros and are never read.
  * [sink] The temporal band is laid out as in Wan2.1's table (which
    [positions] credits): the first hd/2 - 2*floor(hd/6) complex planes of a
    head, plane i being dims (2i, 2i+1) as (real, imaginary), turning at
    theta^(-2i / (hd - 4*floor(hd/6))) radians per frame, theta = 10000.
    This gives the 12 temporal planes of [level] at head_dim 64, and exactly
    its two slowest stay under half a radian over 1024 frames.
  * [sink] "The oldest frame in memory" is the oldest generated frame held in
    a RAW or SUM slot; the check runs after each frame's eviction step (the
    only time that frame can change), and the rotation turns every Z0 key row
    (raw and summary rows of the start image) on all temporal planes by
    rotation(T), T = oldest - 1 - (Z0's frame id).
  * [level] Whether a summary row's quarter turn takes the place of the time
    angle on the two slowest planes or is added to it, the page does not say;
    both are built (ROPE_LEVEL_REPLACE, the plainer reading, and
    ROPE_LEVEL_ADD).  Under REPLACE those planes of Z0's summary rows hold no
    time, so the sink leaves them; under ADD the sink's plain multiply is the
    exact composition.  Queries take the same rotation as keys, row by row.
    "Idle" is checked as the page states it: both planes below half a radian
    over 1024 frames.  Only the temporal band is applied; the height and
    width bands do not depend on the frame and stay the caller's.
  * [files], [credits] The recency bias is read as an additive term on the
    scaled scores (natural-log units) of summary keys that depends only on
    the head and on the age t - f of the key's frame f: a table of W+1
    values per head (ages 0 .. W, all a summary row can have), given by the
    caller, since its form comes from a paper the page does not reproduce.
    It reaches every summary row of a generated frame (in the record, in a
    RAW slot, in a SUM slot); raw rows and the start image's rows get none.

Pin status.  Every function below is pinned by tests/test_oracle_pins.py
against facts the page fixes (the figure's worked example, the caption's key
counts, brute-force equality with the attention-set rule, closed forms of
softmax attention, torch's float64 SDPA over gathered rows, the 12 temporal
planes and the half-radian bound of [level], the composition law of [sink],
numpy's float32 conversion for the rounding), and by
tests/test_oracle_bias_pins.py for the recency bias (a bias of ln n equals n
copies of those keys; a bias of -inf equals leaving them out, checked against
the frame-level attention rule and the figure's example).  No function here is
"parity unpinned"; the values of the recency bias table are the caller's.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


# --------------------------------------------------------------------------
# Geometry of one buffer
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Geometry:
    """Shape of the memory of one session ([record], [buffer] parameter table).

    hw: raw tokens per frame (one per latent grid cell); x: summary tokens per
    frame; y: frames kept whole before the current one; w: memory window in
    frames; plus heads, head_dim, blocks and the storage type of Q/K/V.
    """

    hw: int
    x: int
    y: int
    w: int
    n_heads: int
    head_dim: int
    n_blocks: int = 1
    dtype: str = "bf16"

    @property
    def r(self) -> int:
        """Rows of one record: H*W raw rows then X summary rows ([record])."""
        return self.hw + self.x

    @property
    def n_raw(self) -> int:
        """RAW slots: the current frame and the Y before it ([buffer])."""
        return self.y + 1

    @property
    def n_sum(self) -> int:
        """SUM slots: one per older frame inside the window ([buffer])."""
        return self.w - self.y

    @property
    def capacity(self) -> int:
        """Rows of the whole buffer: Z0, then Y+1 records, then W-Y summaries."""
        return self.r * (self.y + 2) + self.n_sum * self.x

    def z0_rows(self):
        return 0, self.r

    def raw_rows(self, s: int):
        return self.r * (1 + s), self.r * (2 + s)

    def sum_rows(self, u: int):
        base = self.r * (self.y + 2)
        return base + u * self.x, base + (u + 1) * self.x

    @classmethod
    def from_workload(cls, wl: dict) -> "Geometry":
        return cls(wl["hw"], wl["x"], wl["y"], wl["w"], wl["n_heads"],
                   wl["head_dim"], wl["n_blocks"], wl["dtype"])


# --------------------------------------------------------------------------
# Numbers
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns: they are the top half of a float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def stored_to_f64(a: np.ndarray) -> np.ndarray:
    """fp64 value of stored Q/K/V bytes (uint16 = bfloat16 bits, else a float type)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of fp64 values, rounded once to nearest (ties to even).

    Finite values only.  The significand is scaled to 8 bits, rounded with
    numpy's rint (ties to even) and the exact result converted to float32,
    whose upper 16 bits are the bfloat16 pattern; below 2**-126 the quantum
    is the subnormal step 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # subnormal range: fixed quantum 2**-133
    r = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    bits = r.astype(np.float32).view(np.uint32)
    return (bits >> np.uint32(16)).astype(np.uint16)


def f64_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored form of fp64 values: bfloat16 bits (single rounding) or float32."""
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def default_scale(head_dim: int) -> float:
    """Softmax scale when the caller gives none: 1/sqrt(head_dim)."""
    return 1.0 / np.sqrt(float(head_dim))


def attention_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, bias=None) -> np.ndarray:
    """Exact softmax attention, every query row against every key row, per head.

    q: [n][H][d], k and v: [m][H][d], all fp64.  Returns [n][H][d] fp64:
    O[i,h] = sum_j softmax_j(scale * <q[i,h], k[j,h]> + bias[j,h]) v[j,h].  No
    mask and no causal order ([buffer]: the read is one dense, unmasked
    attention).  ``bias`` ([m][H], natural-log units; None = 0) is the
    recency bias of summary keys.  Subtracting the row maximum before exp
    leaves the exact value unchanged.
    """
    n, n_heads, _ = q.shape
    out = np.empty((n, n_heads, v.shape[2]), dtype=np.float64)
    for h in range(n_heads):
        s = (q[:, h, :] @ k[:, h, :].T) * scale
        if bias is not None:
            s = s + bias[None, :, h]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        out[:, h, :] = (p @ v[:, h, :]) / p.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------
# The attention-set rule, stated on frame ids (no buffer)
# --------------------------------------------------------------------------
def frame_visibility(g: Geometry, t: int, f: int) -> str:
    """What frame t's tokens see of frame f ([attends]): 'whole', 'summary' or 'none'.

    Frame 0 (the start image) is always seen whole.  Frame t itself and the Y
    frames before it are seen whole.  Older frames inside the window of W
    frames before t are seen through their X summary rows only.  Generated
    frames are numbered from 1.
    """
    if f == 0:
        return "whole"
    if f < 1 or f > t:
        return "none"
    if f >= t - g.y:
        return "whole"
    if f >= t - g.w:
        return "summary"
    return "none"


def history_mask(g: Geometry, t: int) -> np.ndarray:
    """Boolean mask over the concatenated records 0..t: may frame t see this row?"""
    rows = np.arange(g.r)
    parts = []
    for f in range(t + 1):
        vis = frame_visibility(g, t, f)
        if vis == "whole":
            parts.append(np.ones(g.r, dtype=bool))
        elif vis == "summary":
            parts.append(rows >= g.hw)
        else:
            parts.append(np.zeros(g.r, dtype=bool))
    return np.concatenate(parts)


def history_attention(g: Geometry, t: int, q: np.ndarray, hist_k, hist_v, scale: float) -> np.ndarray:
    """Brute-force twin: masked attention over the full history of records.

    hist_k / hist_v: sequences of fp64 [R][H][d] records for frames 0..t (the
    last write of each).  The mask is ``history_mask``; masked scores are
    dropped from the softmax.  Equal to the buffer read when the buffer keeps
    exactly what [attends] lists.
    """
    keys = np.concatenate([np.asarray(hist_k[f]) for f in range(t + 1)], axis=0)
    vals = np.concatenate([np.asarray(hist_v[f]) for f in range(t + 1)], axis=0)
    m = history_mask(g, t)
    return attention_f64(q, keys[m], vals[m], scale)


def key_count(g: Geometry, t: int) -> int:
    """Readable rows at frame t, counted from the attention-set rule ([attends]).

    Z0's record, the whole records of frames max(1, t-Y)..t, and X summary
    rows for each frame max(1, t-W)..t-Y-1.
    """
    if t == 0:
        return g.r
    whole = t - max(1, t - g.y) + 1
    summarised = max(0, (t - g.y - 1) - max(1, t - g.w) + 1)
    return g.r + whole * g.r + summarised * g.x


# --------------------------------------------------------------------------
# Rotary temporal band and the streaming sink ([sink], [level], [positions])
# --------------------------------------------------------------------------
def temporal_planes(head_dim: int) -> int:
    """Temporal planes per head: the band Wan2.1's table gives time,
    hd - 4*floor(hd/6) dims, counted in planes of two dims."""
    return (head_dim - 4 * (head_dim // 6)) // 2


def temporal_frequencies(head_dim: int, theta: float = 10000.0) -> np.ndarray:
    """Radians per frame of temporal plane i: theta^(-2i / band dims)."""
    n = temporal_planes(head_dim)
    return theta ** (-(2.0 * np.arange(n)) / (2 * n))


def rotate_temporal(k: np.ndarray, head_dim: int, frames: float, theta: float = 10000.0) -> np.ndarray:
    """Keys moved ``frames`` forward in time: every temporal plane (x, y) of every
    head turned by its frequency times ``frames``, as the complex product
    (x + iy) * exp(i a).  k: [..., head_dim] fp64; returns a new fp64 array."""
    out = np.array(k, dtype=np.float64, copy=True)
    n = temporal_planes(head_dim)
    a = temporal_frequencies(head_dim, theta) * frames
    x = out[..., 0:2 * n:2].copy()
    y = out[..., 1:2 * n:2].copy()
    c, s = np.cos(a), np.sin(a)
    out[..., 0:2 * n:2] = x * c - y * s
    out[..., 1:2 * n:2] = x * s + y * c
    return out


# How the temporal band reaches the stored keys.  CALLER: the keys arrive rotated
# and the memory never rotates at a write.  LEVEL_REPLACE / LEVEL_ADD: the memory
# rotates each record by its frame id at the write (and a query by the current
# frame); summary rows' two slowest planes hold the level axis of [level], the
# quarter turn taking the place of the time angle (REPLACE) or added to it (ADD).
ROPE_CALLER, ROPE_LEVEL_REPLACE, ROPE_LEVEL_ADD = 0, 1, 2
IDLE_SPAN_FRAMES = 1024      # [level]: the span over which the level planes must stay idle
IDLE_BOUND_RAD = 0.5         # [level]: "idle" = less than half a radian over that span


def level_planes_idle(head_dim: int, theta: float = 10000.0) -> bool:
    """[level] The construction check: the two slowest temporal planes turn by less
    than half a radian over 1024 frames (so they carry no usable position)."""
    w = temporal_frequencies(head_dim, theta)
    return bool(np.all(w[-2:] * IDLE_SPAN_FRAMES < IDLE_BOUND_RAD))


def quarter_turn(x: np.ndarray, y: np.ndarray):
    """(x + iy) * i: the exact quarter turn of a plane."""
    return -y, x


def rope_record_f64(a: np.ndarray, hw: int, t: int, head_dim: int, theta: float = 10000.0,
                    mode: int = ROPE_LEVEL_REPLACE) -> np.ndarray:
    """[level], [positions] Record(t)'s Q or K rows ([R][H][d], fp64) with the temporal
    band applied at frame id t.  Raw rows (r < hw): every temporal plane turned by its
    frequency times t.  Summary rows (r >= hw): the same on all but the two slowest
    planes; on those, REPLACE puts the exact quarter turn of the input, ADD turns by
    the time angle and then by the quarter turn."""
    if mode not in (ROPE_LEVEL_REPLACE, ROPE_LEVEL_ADD):
        raise ValueError("rope_record_f64: mode must be LEVEL_REPLACE or LEVEL_ADD")
    a = np.asarray(a, dtype=np.float64)
    out = rotate_temporal(a, head_dim, t, theta)
    n = temporal_planes(head_dim)
    lv = slice(2 * (n - 2), 2 * n)
    src = a[hw:, ..., lv] if mode == ROPE_LEVEL_REPLACE else out[hw:, ..., lv]
    x, y = quarter_turn(src[..., 0::2].copy(), src[..., 1::2].copy())
    out[hw:, ..., lv][..., 0::2] = x
    out[hw:, ..., lv][..., 1::2] = y
    return out


def rope_record(stored: np.ndarray, hw: int, t: int, head_dim: int, dtype: str, theta: float = 10000.0,
                mode: int = ROPE_LEVEL_REPLACE) -> np.ndarray:
    """rope_record_f64 on storage bytes, rounded once back to the storage type."""
    return f64_to_storage(rope_record_f64(stored_to_f64(stored), hw, t, head_dim, theta, mode), dtype)


def sink_shift(oldest: int, z0_frame: int, gap: int) -> int:
    """[sink] Frames Z0 moves forward after an eviction step: back to a gap of 1
    once the gap to the oldest generated frame in memory reaches ``gap``."""
    if gap <= 0 or oldest < 1 or oldest - z0_frame < gap:
        return 0
    return oldest - 1 - z0_frame


# --------------------------------------------------------------------------
# The buffer replay
# --------------------------------------------------------------------------
class MemoryReplay:
    """One session's per-block K/V buffers, replayed step by step on the host.

    The layout follows [buffer]: rows [0, R) hold Z0 (record 0, never evicted);
    RAW slot s holds rows [R(1+s), R(2+s)); SUM slot u holds rows
    [R(Y+2) + uX, R(Y+2) + (u+1)X).  K and V of a block are each
    [capacity][H][d] in storage bytes.  ``blocks`` limits the replay to a
    subset of blocks (blocks are independent); by default all are kept.
    """

    def __init__(self, g: Geometry, blocks=None, sink_gap: int = 0, rope_theta: float = 10000.0,
                 rope_mode: int = ROPE_CALLER, recency_bias=None):
        self.g = g
        self.recency_bias = None
        if recency_bias is not None:
            self.set_recency_bias(recency_bias)
        self.sink_gap = sink_gap
        self.rope_theta = rope_theta
        self.rope_mode = rope_mode
        self.z0_frame = 0
        self.blocks = list(range(g.n_blocks)) if blocks is None else list(blocks)
        self.index = {b: i for i, b in enumerate(self.blocks)}
        store = np.uint16 if g.dtype == "bf16" else np.float32
        shape = (len(self.blocks), g.capacity, g.n_heads, g.head_dim)
        self.k = np.zeros(shape, dtype=store)
        self.v = np.zeros(shape, dtype=store)
        self.raw_frame = [-1] * g.n_raw    # frame id held by each RAW slot
        self.sum_frame = [-1] * g.n_sum    # frame id whose summary each SUM slot holds
        self.t = -1

    # -- slot map ([buffer] figure "The buffer one frame apart") -----------
    def raw_slot(self, t: int) -> int:
        return t % self.g.n_raw

    def sum_slot(self, f: int) -> int:
        return f % self.g.n_sum

    # -- eviction ([buffer], eviction paragraph) ---------------------------
    def evict(self, t: int):
        """Before frame t is written: move the summary of the frame leaving RAW into SUM.

        The frame leaving is the one in RAW slot t mod (Y+1).  Only its X
        summary rows (record rows [HW, R)) are copied, K and V, in every block;
        its raw rows stay where they are, to be overwritten by frame t.  Frame
        0 is never in RAW, so nothing moves while that slot is still empty.
        Returns (raw slot, sum slot, frame) or None.
        """
        g = self.g
        moved = None
        if t > g.y:
            s = self.raw_slot(t)
            f = self.raw_frame[s]
            if f >= 1:
                u = self.sum_slot(f)
                src0 = g.raw_rows(s)[0] + g.hw
                src1 = g.raw_rows(s)[1]
                dst0, dst1 = g.sum_rows(u)
                self.k[:, dst0:dst1] = self.k[:, src0:src1]
                self.v[:, dst0:dst1] = self.v[:, src0:src1]
                self.sum_frame[u] = f
                moved = (s, u, f)
        self.sink_step()
        return moved

    def oldest_frame(self) -> int:
        """Oldest generated frame held in a RAW or SUM slot (-1: none)."""
        held = [f for f in self.raw_frame + self.sum_frame if f >= 1]
        return min(held) if held else -1

    def sink_step(self) -> int:
        """[sink] After an eviction step: rotate every block's Z0 keys forward when
        the gap has reached sink_gap; returns the shift (0: none).  The rotation is
        computed in fp64 from the stored keys and rounded once to the storage type."""
        T = sink_shift(self.oldest_frame(), self.z0_frame, self.sink_gap)
        if T > 0:
            g = self.g
            lo, hi = g.z0_rows()
            k = stored_to_f64(self.k[:, lo:hi])
            turned = f64_to_storage(rotate_temporal(k, g.head_dim, T, self.rope_theta), g.dtype)
            if self.rope_mode == ROPE_LEVEL_REPLACE:
                # a summary row's level planes hold a fixed quarter turn, not a time: kept
                n = temporal_planes(g.head_dim)
                turned[:, g.hw:, :, 2 * (n - 2):2 * n] = self.k[:, lo + g.hw:hi, :, 2 * (n - 2):2 * n]
            self.k[:, lo:hi] = turned
            self.z0_frame += T
        return T

    # -- record write ([buffer]; rewrite: [sampling]) ----------------------
    def write(self, block: int, t: int, k: np.ndarray, v: np.ndarray):
        """Store record(t)'s K and V ([R][H][d] storage bytes) in its rows of one block.

        Frame 0 goes to Z0; frame t >= 1 to RAW slot t mod (Y+1).  Writing the
        same t again overwrites (the clean pass rewrites the frame's entry).
        """
        g = self.g
        if t == 0:
            lo, hi = g.z0_rows()
        else:
            s = self.raw_slot(t)
            lo, hi = g.raw_rows(s)
            self.raw_frame[s] = t
        i = self.index[block]
        k = np.asarray(k).reshape(g.r, g.n_heads, g.head_dim)
        if self.rope_mode != ROPE_CALLER:
            k = rope_record(k, g.hw, t, g.head_dim, g.dtype, self.rope_theta, self.rope_mode)
        self.k[i, lo:hi] = k
        self.v[i, lo:hi] = np.asarray(v).reshape(g.r, g.n_heads, g.head_dim)
        self.t = t

    def step(self, t: int, records: dict):
        """Frame t: eviction (if due) then the write of every block in ``records``."""
        ev = self.evict(t) if t >= 1 else None
        for b, (k, v) in records.items():
            self.write(b, t, k, v)
        return ev

    # -- the dense read ([buffer]: what is in the buffer is what is seen) --
    def readable_segments(self):
        """Filled rows, ascending, as (begin, length) segments of contiguous rows."""
        g = self.g
        if self.t < 0:
            return []
        ranges = [g.z0_rows()]
        ranges += [g.raw_rows(s) for s in range(g.n_raw) if self.raw_frame[s] >= 1]
        ranges += [g.sum_rows(u) for u in range(g.n_sum) if self.sum_frame[u] >= 1]
        ranges.sort()
        segs = []
        for lo, hi in ranges:
            if segs and segs[-1][0] + segs[-1][1] == lo:
                segs[-1] = (segs[-1][0], segs[-1][1] + hi - lo)
            else:
                segs.append((lo, hi - lo))
        return segs

    def readable_rows(self) -> np.ndarray:
        segs = self.readable_segments()
        if not segs:
            return np.zeros(0, dtype=np.int64)
        return np.concatenate([np.arange(b, b + n) for b, n in segs])

    def n_keys(self) -> int:
        return sum(n for _, n in self.readable_segments())

    # -- recency bias on summary keys (file list of the page: recency_bias.py) --
    def set_recency_bias(self, table):
        """Bias table [H][W+1], natural-log units: entry [h][a] is added to head h's
        scaled scores against the summary keys of the frame a frames older than the
        current one (a = 0: the current frame's own record)."""
        g = self.g
        tab = np.asarray(table, dtype=np.float64)
        if tab.shape != (g.n_heads, g.w + 1):
            raise ValueError("recency bias table must be [n_heads][w + 1]")
        self.recency_bias = tab.copy()

    def row_frames(self, rows: np.ndarray):
        """For buffer rows: the generated frame each belongs to (-1: Z0, the start
        image) and whether it is a summary row.  Looked up in the slot tables."""
        g = self.g
        frame = np.full(len(rows), -1, dtype=np.int64)
        summary = np.zeros(len(rows), dtype=bool)
        sum0 = g.r * (g.y + 2)
        for j, row in enumerate(np.asarray(rows).tolist()):
            if row < g.r:
                continue                                   # Z0: no recency
            if row < sum0:
                s, within = divmod(row - g.r, g.r)
                frame[j] = self.raw_frame[s]
                summary[j] = within >= g.hw
            else:
                frame[j] = self.sum_frame[(row - sum0) // g.x]
                summary[j] = True
        return frame, summary

    def key_bias(self, rows: np.ndarray):
        """[len(rows)][H] recency bias of these key rows (None when off): the
        table's entry for the age t - f of a summary row's frame f, 0 for raw rows
        and for Z0."""
        if self.recency_bias is None:
            return None
        frame, summary = self.row_frames(rows)
        bias = np.zeros((len(rows), self.g.n_heads), dtype=np.float64)
        for j in np.nonzero(summary & (frame >= 1))[0]:
            bias[j] = self.recency_bias[:, self.t - frame[j]]
        return bias

    def gathered(self, block: int):
        """fp64 K and V of the readable rows of one block, ascending row order."""
        rows = self.readable_rows()
        i = self.index[block]
        return stored_to_f64(self.k[i, rows]), stored_to_f64(self.v[i, rows])

    def attend(self, block: int, q: np.ndarray, scale=None, rows=None) -> np.ndarray:
        """Frame t's record attends to every readable row of one block, fp64.

        q: [R][H][d] storage bytes (or fp64).  ``rows`` optionally restricts the
        query rows computed (for sampled checks at large sizes).  With the memory
        applying the temporal band, q arrives unrotated and is turned as record(t)'s
        rows are, t being the current frame, and rounded to the storage type.
        """
        g = self.g
        if scale is None or scale <= 0:
            scale = default_scale(g.head_dim)
        q = np.asarray(q).reshape(-1, g.n_heads, g.head_dim)
        if self.rope_mode != ROPE_CALLER:
            q = rope_record(q, g.hw, self.t, g.head_dim, g.dtype, self.rope_theta, self.rope_mode)
        qf = stored_to_f64(q)
        if rows is not None:
            qf = qf[np.asarray(rows)]
        kf, vf = self.gathered(block)
        return attention_f64(qf, kf, vf, scale, self.key_bias(self.readable_rows()))

    # -- bytes --------------------------------------------------------------
    def block_bytes(self, block: int) -> bytes:
        """Canonical bytes of one block: K [capacity][H][d] then V."""
        i = self.index[block]
        return self.k[i].tobytes() + self.v[i].tobytes()
