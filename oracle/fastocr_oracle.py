"""Plain float64 CPU oracle of FastOCR's decode-step attention.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  It shares no code,
constants or helpers with the GPU library, and the GPU library never calls it.

What it follows.  The FastOCR pages are a technical summary of the paper
("FastOCR: Dynamic Visual Fixation via KV Cache Pruning for Efficient Document
Parsing", published in Korean and French editions with the same content) and
the paper's abstract.  Citations below name the summary's sections:

* "Method": the full KV cache is kept and only the set of attended tokens
  changes per step; nothing is evicted.
* "Method / 1. Focal-Guided Pruning / Focal Layer Selection": a w-step
  warm-up profiles each layer's image-attention ratio and fixes a small set C
  of focal layers with high image concentration.
* "Method / 1. Focal-Guided Pruning / Cross-Layer Propagation": after the
  warm-up, only focal layers look at the full cache and pick the
  top-attended image tokens by kept ratio tau; the pick is passed on to every
  non-focal layer, which attends only to the pruned set.
* "Method / 2. Cross-Step Fixation Reuse / Implementation": at the start of a
  step, a non-focal first layer inherits the deepest focal layer's set of the
  previous step (F_last) as a warm start; the first focal layer refines it.
* Abstract: focal layers select the most task-relevant visual tokens each
  step; fixation is warm-started from the previous step; no token is evicted.

Readings where the pages leave a step open (each is the plainest one the rest
supports):

* token score = attention probability summed over all query heads, current
  step only; the tau-set is the k highest-scoring image tokens, ties to the
  lower token index, stored in ascending order;
* k = clamp(ceil(tau * n - 1e-9), 1, n) for n > 0 image tokens, 0 for n = 0;
* pruning touches image tokens only: prompt and generated tokens (including
  the current one) are always attended;
* one set per sequence, shared by all heads; every focal layer replaces the
  current set with its own pick; F_last is the set after the deepest focal
  layer of the previous step;
* focal layers attend to the full cache (they are the ones that "consult" it);
* image-attention ratio of a layer = image probability mass averaged over
  heads, sequences and the w warm-up steps; C = the |C| largest, ties to the
  lower layer index, in ascending order;
* the first pruned step inherits the set picked from the last warm-up step's
  scores at the deepest focal layer;
* grouped-query attention maps query head h to KV head h // (Hq / Hkv); the
  logit scale is 1 / sqrt(d);
* an empty attention set yields a zero output;
* optional periodic re-selection (the conclusion names adaptive layer
  selection as future work): after every R pruned steps a new w-step
  warm-up window picks C and F_last again from that window alone;
* image tokens may sit in several spans of the cache (pages with text
  between them): image token j is the j-th image row in ascending order,
  and every other row is text.

Parity pins: every function here is checked in tests/test_oracle_pins.py
against closed forms, hand-worked fixtures, an independent library routine
(torch's scaled_dot_product_attention on the CPU) or brute-force enumeration.
The pages print no worked example of a decode trajectory; DecodeOracle is
pinned by a hand-worked three-step, four-layer trajectory with exact
rational outputs (warm-up pick, warm start, replacement by each focal layer,
carry from the deepest one, ties) and by invariants (fixed point under
stationary inputs, layer-0 focal, no eviction, drift recovery).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Leaf operations
# ---------------------------------------------------------------------------


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h under grouped-query attention."""
    return h // (num_q_heads // num_kv_heads)


# Every function computes in float64 unless a caller asks for another
# working precision (``dtype``): the benchmark's CPU baseline also times a
# float32 run of the same definitions; parity always uses float64.


def attention_probs(q: np.ndarray, K: np.ndarray, rows, scale: float, dtype=np.float64) -> np.ndarray:
    """Softmax attention probabilities of one sequence over the given rows.

    q: [Hq, d]; K: [Hkv, S, d]; rows: a 1-D index array or a slice of cache
    rows.  Returns p: [Hq, n_rows] with
    p[h, i] = softmax_i(scale * <q_h, K[kv(h), rows[i]]>).
    (Method: the method only changes which rows are attended, never the
    softmax itself.)
    """
    Hq, Hkv = q.shape[0], K.shape[0]
    n_rows = len(range(K.shape[1])[rows]) if isinstance(rows, slice) else len(rows)
    p = np.zeros((Hq, n_rows), dtype=dtype)
    if n_rows == 0:
        return p
    for kvh in range(Hkv):
        heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == kvh]
        keys = np.asarray(K[kvh][rows], dtype=dtype)  # [n_rows, d]
        x = dtype(scale) * (np.asarray(q[heads], dtype=dtype) @ keys.T)  # [g, n_rows]
        e = np.exp(x - x.max(axis=1, keepdims=True))
        p[heads] = e / e.sum(axis=1, keepdims=True)
    return p


def _weighted_values(p: np.ndarray, V: np.ndarray, rows) -> np.ndarray:
    """out[h] = sum_i p[h, i] * V[kv(h), rows[i]] (in p's precision)."""
    Hq = p.shape[0]
    Hkv, _, d = V.shape
    out = np.zeros((Hq, d), dtype=p.dtype)
    if p.shape[1] == 0:
        return out
    for kvh in range(Hkv):
        heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == kvh]
        out[heads] = p[heads] @ np.asarray(V[kvh][rows], dtype=p.dtype)
    return out


def full_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, length: int,
                   scale: float, dtype=np.float64) -> Tuple[np.ndarray, np.ndarray]:
    """Full decode attention over cache rows [0, length) of one sequence.

    Used on every layer during the warm-up and on focal layers afterwards,
    which are the layers that consult the full KV cache (Method / 1.
    Focal-Guided Pruning / Cross-Layer Propagation).
    Returns (out [Hq, d], p [Hq, length]).
    """
    rows = slice(0, int(length))
    p = attention_probs(q, K, rows, scale, dtype)
    return _weighted_values(p, V, rows), p


def image_rows_of(spans: Sequence[Tuple[int, int]]) -> np.ndarray:
    """Cache rows of the image tokens of a sequence whose image occupies the
    given (start, count) spans (several pages or images), in ascending row
    order: image token j of the method is row image_rows_of(spans)[j].

    The method prunes visual tokens and keeps every text token (Method / 1.
    Focal-Guided Pruning); where in the cache the visual tokens sit is not
    fixed by the summary, so they are whichever rows the spans name.
    """
    rows = [np.arange(a, a + c, dtype=np.int64) for a, c in spans]
    return np.sort(np.concatenate(rows)) if rows else np.zeros(0, dtype=np.int64)


def sparse_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                     selected: Sequence[int], n_img: int, length: int,
                     scale: float, image_rows: Optional[np.ndarray] = None, dtype=np.float64) -> np.ndarray:
    """Non-focal decode attention: the selected image tokens plus all text rows.

    Non-focal layers attend only to the pruned token set (Method / 1.
    Focal-Guided Pruning / Cross-Layer Propagation); pruning applies to image
    tokens [0, n_img), and every prompt/generated row [n_img, length) is kept.
    With ``image_rows`` the image tokens are those cache rows instead (image
    token j at row image_rows[j]) and every other row below ``length`` is text.
    Returns out [Hq, d].
    """
    sel = np.sort(np.asarray(selected, dtype=np.int64))
    if image_rows is None:
        rows = np.concatenate([sel, np.arange(n_img, length, dtype=np.int64)])
    else:
        text = np.setdiff1d(np.arange(length, dtype=np.int64), image_rows)
        rows = np.concatenate([np.asarray(image_rows, dtype=np.int64)[sel], text])
    p = attention_probs(q, K, rows, scale, dtype)
    return _weighted_values(p, V, rows)


def image_scores(p: np.ndarray, n_img: int, image_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-image-token attention score: probability summed over query heads.

    Focal layers pick the "top-attended" image tokens (Method / 1.
    Focal-Guided Pruning / Cross-Layer Propagation); the head sum is the
    statistic.  p is [Hq, length] from a full-cache attention; the image
    tokens are rows [0, n_img), or the rows ``image_rows`` when given.
    """
    return (p[:, :n_img] if image_rows is None else p[:, image_rows]).sum(axis=0)


def image_mass(p: np.ndarray, n_img: int, image_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-head attention mass on image tokens, [Hq] (Focal Layer Selection)."""
    return (p[:, :n_img] if image_rows is None else p[:, image_rows]).sum(axis=1)


def kept_count(tau: float, n_img: int) -> int:
    """Number of image tokens kept at kept ratio tau (Cross-Layer Propagation)."""
    if n_img <= 0:
        return 0
    k = math.ceil(float(tau) * float(n_img) - 1e-9)
    return int(min(max(k, 1), n_img))


def select_top(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k highest scores, ties to the lower index, ascending.

    np.lexsort sorts by its last key first: primary key -score (highest score
    first), secondary key the index (lower index first on equal scores).
    """
    idx = np.arange(len(scores))
    order = np.lexsort((idx, -np.asarray(scores, dtype=np.float64)))
    return np.sort(order[:k]).astype(np.int64)


def choose_focal_layers(ratios: Sequence[float], num_focal: int) -> np.ndarray:
    """Focal layer set C: the num_focal layers with the highest image-attention
    ratio, ties to the lower layer index, ascending (Focal Layer Selection)."""
    r = np.asarray(ratios, dtype=np.float64)
    order = np.lexsort((np.arange(len(r)), -r))
    return np.sort(order[:num_focal]).astype(np.int64)


# ---------------------------------------------------------------------------
# The decode-step procedure
# ---------------------------------------------------------------------------


@dataclass
class StepRecord:
    t: int
    phase: str  # "warmup" | "pruned" | "full"
    outs: List[np.ndarray] = field(default_factory=list)  # per layer [B, Hq, d]
    sets: Dict[int, List[np.ndarray]] = field(default_factory=dict)  # focal layer -> per-seq set
    scores: Dict[int, List[np.ndarray]] = field(default_factory=dict)  # focal layer -> per-seq scores
    used_sets: Dict[int, List[np.ndarray]] = field(default_factory=dict)  # non-focal layer -> set used
    warm_start: Optional[List[np.ndarray]] = None  # F_last inherited at step start


class DecodeOracle:
    """Runs FastOCR's per-step attention on caller-supplied inputs.

    ``step(t, q_of, kv_of, lens)``:
      q_of(l)  -> queries of layer l at this step, [B, Hq, d]
      kv_of(l) -> (K, V) of layer l, each [B, Hkv, S, d]
      lens     -> [B, 2] (image tokens, valid rows)

    The first w steps are the warm-up: every layer runs full attention and
    its image mass is recorded (Focal Layer Selection).  After the last of
    them the focal set C is chosen and F_last is initialised from that step's
    scores at the deepest focal layer.  Later steps start from S = F_last
    (Cross-Step Fixation Reuse / Implementation); a focal layer runs full
    attention and replaces S with its top-k pick; a non-focal layer attends to
    S plus all text rows; at the end of the step F_last = S.

    Periodic re-selection (``reprofile_every`` = R > 0; the summary names
    adaptive layer selection as a direction its conclusion leaves open, and
    the reading here is the plainest one built from the warm-up itself):
    after every R pruned steps the next w steps are a new warm-up window, and
    C and F_last are chosen again from that window alone, exactly as after
    the first one.  Phases follow the number of steps run, not ``t``.
    """

    def __init__(self, *, num_layers: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, tau: float, num_focal: int, warmup_steps: int,
                 scale: Optional[float] = None, full_mode: bool = False,
                 reprofile_every: int = 0,
                 spans: Optional[Sequence[Sequence[Tuple[int, int]]]] = None):
        self.L = num_layers
        self.Hq = num_q_heads
        self.Hkv = num_kv_heads
        self.d = head_dim
        self.tau = tau
        self.num_focal = num_focal
        self.w = warmup_steps
        self.scale = (1.0 / math.sqrt(head_dim)) if not scale else float(scale)
        self.full_mode = full_mode
        self.reprofile_every = reprofile_every
        # image tokens of sequence b at the rows of its spans (None: rows
        # [0, n_img)), fixed for the run like the image-token counts
        self.image_rows = None if spans is None else [image_rows_of(sp) for sp in spans]
        self.mass: Dict[int, List[np.ndarray]] = {l: [] for l in range(num_layers)}
        self.warm_scores: Dict[int, List[np.ndarray]] = {}
        self.ratios: Optional[np.ndarray] = None
        self.focal: Optional[np.ndarray] = None
        self.f_last: Optional[List[np.ndarray]] = None
        self.window_pos: Optional[int] = 0  # step index inside a warm-up window, None when pruning
        self.pruned_since = 0  # pruned steps since the last profile
        self.profiles: List[Tuple[int, np.ndarray]] = []  # (t of the first pruned step, C)

    # -- warm-up profiler (Focal Layer Selection) --------------------------
    def layer_ratios(self) -> np.ndarray:
        """Mean image mass per layer over warm-up steps, sequences and heads."""
        return np.array([np.mean(np.stack(self.mass[l])) for l in range(self.L)])

    def _finish_warmup(self, lens: np.ndarray) -> None:
        self.ratios = self.layer_ratios()
        self.focal = choose_focal_layers(self.ratios, self.num_focal)
        deepest = int(self.focal.max())
        self.f_last = [select_top(self.warm_scores[deepest][b], kept_count(self.tau, int(lens[b, 0])))
                       for b in range(len(lens))]

    # -- one decode step ----------------------------------------------------
    def step(self, t: int, q_of: Callable[[int], np.ndarray],
             kv_of: Callable[[int], Tuple[np.ndarray, np.ndarray]],
             lens: np.ndarray) -> StepRecord:
        lens = np.asarray(lens)
        B = lens.shape[0]
        if self.full_mode:
            return self._full_step(t, q_of, kv_of, lens, "full")
        if self.window_pos is not None:
            last = self.window_pos == self.w - 1
            rec = self._full_step(t, q_of, kv_of, lens, "warmup", keep_scores=last)
            self.window_pos += 1
            if last:
                self._finish_warmup(lens)
                self.window_pos = None
                self.pruned_since = 0
                self.profiles.append((t + 1, self.focal.copy()))
            return rec

        rec = StepRecord(t=t, phase="pruned")
        current = [s.copy() for s in self.f_last]
        rec.warm_start = [s.copy() for s in current]
        focal = set(int(c) for c in self.focal)
        for l in range(self.L):
            q = q_of(l)
            K, V = kv_of(l)
            out = np.zeros((B, self.Hq, self.d))
            if l in focal:
                rec.sets[l], rec.scores[l] = [], []
                for b in range(B):
                    n, length = int(lens[b, 0]), int(lens[b, 1])
                    out[b], p = full_attention(q[b], K[b], V[b], length, self.scale)
                    s = image_scores(p, n, self._rows(b, n))
                    current[b] = select_top(s, kept_count(self.tau, n))
                    rec.scores[l].append(s)
                    rec.sets[l].append(current[b].copy())
            else:
                rec.used_sets[l] = [c.copy() for c in current]
                for b in range(B):
                    n, length = int(lens[b, 0]), int(lens[b, 1])
                    out[b] = sparse_attention(q[b], K[b], V[b], current[b], n, length, self.scale,
                                              self._rows(b, n))
            rec.outs.append(out)
        self.f_last = current
        self.pruned_since += 1
        if self.reprofile_every > 0 and self.pruned_since == self.reprofile_every:
            # a new warm-up window: statistics of that window alone
            self.window_pos = 0
            self.mass = {l: [] for l in range(self.L)}
            self.warm_scores = {}
        return rec

    def _rows(self, b: int, n: int) -> Optional[np.ndarray]:
        if self.image_rows is None:
            return None
        assert len(self.image_rows[b]) == n, "lens must count the spans' image tokens"
        return self.image_rows[b]

    def _full_step(self, t, q_of, kv_of, lens, phase, keep_scores=False) -> StepRecord:
        B = lens.shape[0]
        rec = StepRecord(t=t, phase=phase)
        for l in range(self.L):
            q = q_of(l)
            K, V = kv_of(l)
            out = np.zeros((B, self.Hq, self.d))
            masses, scores = [], []
            for b in range(B):
                n, length = int(lens[b, 0]), int(lens[b, 1])
                out[b], p = full_attention(q[b], K[b], V[b], length, self.scale)
                masses.append(image_mass(p, n, self._rows(b, n)))
                scores.append(image_scores(p, n, self._rows(b, n)))
            if phase == "warmup":
                self.mass[l].append(np.stack(masses))
                if keep_scores:
                    self.warm_scores[l] = scores
            rec.scores[l] = scores
            rec.outs.append(out)
        return rec
