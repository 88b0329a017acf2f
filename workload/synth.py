"""Synthetic document-page decode workloads.

The FastOCR pages (technical summary, "Method"; abstract) describe the
phenomenon the method exploits: at each decode step the model's attention
concentrates on a small region of the page image that shifts gradually from
one step to the next ("Dynamic Visual Fixation").  No dataset or trained model
is available here, so this module builds inputs of the right shapes whose
attention behaves that way:

* keys and values of every layer are i.i.d. N(0, 1) for every cache row
  (image, prompt and generated rows are all drawn up front; decoding only
  grows the valid length);
* image token j sits at grid cell (j // W, j % W) in raster order;
* the query of layer l, sequence b, head h at step t is
  alpha_l * mean(K_l[b, kv(h), window_b(t)]) + sigma * eps, where the window
  is a rows x cols box centred on a cell that advances one cell per step in
  raster order (clipped at the grid border, wrapping at the end of the grid);
* alpha_l is large on a band of layers, which makes those layers attend
  strongly to the image, and small elsewhere.

Everything is drawn from numpy PCG64 streams spawned from one SeedSequence per
workload, so any layer can be regenerated on its own.  Values are produced in
float32 and, for bfloat16 workloads, rounded to bfloat16 (round to nearest
even) before anyone consumes them, so the oracle and the GPU see identical
numbers.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# bfloat16 helpers (input preparation only)
# --------------------------------------------------------------------------


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float32."""
    return bits_to_f32(bf16_bits(x))


# --------------------------------------------------------------------------
# Workload description
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    """Shapes and generator knobs of one synthetic decode workload."""

    name: str
    description: str
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    batch: int
    dtype: str  # "f32" or "bf16"
    tau: float
    num_focal: int
    warmup_steps: int
    steps: int  # T, total decode steps including warm-up
    n_prompt: Tuple[int, int]  # inclusive range; equal ends = fixed count
    grid: Optional[Tuple[int, int]]  # (rows, cols) when fixed, else None
    n_img_range: Optional[Tuple[int, int]]  # ragged image-token counts
    window: Tuple[int, int]  # (rows, cols) of the fixation box
    jump_every: int  # 0 = no line jumps
    focal_band: Optional[Tuple[int, int]]  # inclusive layer band with alpha_hi
    planted_layers: Optional[Tuple[int, ...]]  # explicit strong layers
    alpha_hi: float
    alpha_lo: Optional[float]  # fixed low alpha, else U[0.3, 1] per layer
    sigma: float
    seed: int
    # (t, layers): from decode step t on, the strong alpha sits on these layers
    # and the layers that had it before take the low alpha (a focal set that
    # drifts during decoding); None = no drift
    drift: Optional[Tuple[int, Tuple[int, ...]]] = None
    # multi-page layout: the image (grid rows split evenly into `pages`
    # pages) sits in the cache behind page_text[0] text tokens, with
    # page_text[1] text tokens between pages; n_prompt counts every text
    # token before decoding (these included).  pages = 1 and (0, 0): the
    # image first, then the prompt.
    pages: int = 1
    page_text: Tuple[int, int] = (0, 0)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def with_overrides(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def _band(num_layers: int) -> Tuple[int, int]:
    # Layers 14..22 of a 28-layer stack, scaled by depth for deeper stacks.
    return (num_layers // 2, (22 * num_layers) // 28)


WORKLOADS: Dict[str, Workload] = {
    # 4-layer fp32 stack, 16x16 page, strong layers planted at 1 and 3.
    "tiny-fp32": Workload(
        name="tiny-fp32",
        description="tiny fp32 decode attention: B=1, 4 layers, 4 q / 2 kv heads, d=64, "
        "256 image (16x16) + 32 prompt + 16 decode tokens, tau=0.1",
        num_layers=4, num_q_heads=4, num_kv_heads=2, head_dim=64, batch=1, dtype="f32",
        tau=0.1, num_focal=2, warmup_steps=4, steps=16, n_prompt=(32, 32), grid=(16, 16),
        n_img_range=None, window=(3, 3), jump_every=0, focal_band=None,
        planted_layers=(1, 3), alpha_hi=4.0, alpha_lo=0.5, sigma=0.5, seed=1000),
    # Qwen2.5-VL-7B-like shapes, one sequence.
    "7b-b1": Workload(
        name="7b-b1",
        description="Qwen2.5-VL-7B-like decode attention: B=1, 28 layers, 28 q / 4 kv heads, "
        "d=128, bf16 KV, 6400 image (80x80) + 64 prompt + 1024 decode tokens, tau=0.05",
        num_layers=28, num_q_heads=28, num_kv_heads=4, head_dim=128, batch=1, dtype="bf16",
        tau=0.05, num_focal=4, warmup_steps=8, steps=1024, n_prompt=(64, 64), grid=(80, 80),
        n_img_range=None, window=(3, 5), jump_every=0, focal_band=(14, 22),
        planted_layers=None, alpha_hi=4.0, alpha_lo=None, sigma=0.5, seed=1001),
    # Same shapes, 16 ragged sequences.
    "7b-b16-ragged": Workload(
        name="7b-b16-ragged",
        description="Qwen2.5-VL-7B-like decode attention: B=16 ragged, image tokens "
        "U{2048..8192} (near-square grids), prompt U{64..256}, 512 decode steps, tau=0.05",
        num_layers=28, num_q_heads=28, num_kv_heads=4, head_dim=128, batch=16, dtype="bf16",
        tau=0.05, num_focal=4, warmup_steps=8, steps=512, n_prompt=(64, 256), grid=None,
        n_img_range=(2048, 8192), window=(3, 5), jump_every=0, focal_band=(14, 22),
        planted_layers=None, alpha_hi=4.0, alpha_lo=None, sigma=0.5, seed=1002),
    # 32B-like long dense page with line jumps.
    "32b-b4-longpage": Workload(
        name="32b-b4-longpage",
        description="32B-like long dense page: B=4, 64 layers, 40 q / 8 kv heads, d=128, "
        "16384 image (128x128) + 128 prompt + 4096 decode tokens, 3x7 window with a "
        "line jump every 128 steps, |C|=6, tau=0.05",
        num_layers=64, num_q_heads=40, num_kv_heads=8, head_dim=128, batch=4, dtype="bf16",
        tau=0.05, num_focal=6, warmup_steps=8, steps=4096, n_prompt=(128, 128),
        grid=(128, 128), n_img_range=None, window=(3, 7), jump_every=128,
        focal_band=_band(64), planted_layers=None, alpha_hi=4.0, alpha_lo=None,
        sigma=0.5, seed=1003),
    # 72B-like sweep (tau and sigma are swept by the caller).
    "72b-b8-sweep": Workload(
        name="72b-b8-sweep",
        description="72B-like sweep: B=8, 80 layers, 64 q / 8 kv heads, d=128, 12800 image "
        "(80x160) + 128 prompt + 2048 decode tokens, |C|=8, tau in {.02,.05,.1,.2,1}, "
        "sigma in {.25,.5,1}",
        num_layers=80, num_q_heads=64, num_kv_heads=8, head_dim=128, batch=8, dtype="bf16",
        tau=0.05, num_focal=8, warmup_steps=8, steps=2048, n_prompt=(128, 128),
        grid=(80, 160), n_img_range=None, window=(3, 5), jump_every=0,
        focal_band=_band(80), planted_layers=None, alpha_hi=4.0, alpha_lo=None,
        sigma=0.5, seed=1004),
}

SIGMA_SWEEP = (0.25, 0.5, 1.0)
TAU_SWEEP = (0.02, 0.05, 0.1, 0.2, 1.0)


def get_workload(name: str, **overrides) -> Workload:
    """Return a named workload, optionally with fields replaced.

    For the 72B-like sweep, overriding ``sigma`` also moves the seed by
    10 * (index of sigma in the sweep), so every sigma has its own inputs while
    every tau sees identical inputs.
    """
    wl = WORKLOADS[name]
    if name == "72b-b8-sweep" and "sigma" in overrides and "seed" not in overrides:
        overrides["seed"] = wl.seed + 10 * SIGMA_SWEEP.index(overrides["sigma"])
    return wl.with_overrides(**overrides) if overrides else wl


# --------------------------------------------------------------------------
# Per-workload structure (everything except the big tensors)
# --------------------------------------------------------------------------


@dataclass
class Structure:
    n_img: np.ndarray  # [B] int
    n_prompt: np.ndarray  # [B] int
    grid_w: np.ndarray  # [B] columns of each page grid
    grid_h: np.ndarray  # [B] rows of each page grid
    centre: np.ndarray  # [T, B] window centre cell (image-token index)
    alpha: np.ndarray  # [L] float32, query alignment of each layer
    max_seq_len: int  # cache row stride S_max
    windows: List[List[np.ndarray]] = field(default_factory=list)  # [B][T] token ids
    alpha_late: Optional[np.ndarray] = None  # [L] alpha from drift_step on (drifting workloads)
    drift_step: int = 0
    spans: Optional[List[List[Tuple[int, int]]]] = None  # [B] (start, count) of each page
    image_rows: Optional[List[np.ndarray]] = None  # [B] cache row of image token j

    def image_row(self, b: int, j: np.ndarray) -> np.ndarray:
        """Cache rows of image tokens j of sequence b."""
        return np.asarray(j) if self.image_rows is None else self.image_rows[b][np.asarray(j)]

    def alpha_at(self, l: int, steps) -> np.ndarray:
        """[len(steps)] float32: query alignment of layer l at each step."""
        steps = np.asarray(list(steps), dtype=np.int64)
        a = np.full(len(steps), self.alpha[l], dtype=np.float32)
        if self.alpha_late is not None:
            a[steps >= self.drift_step] = self.alpha_late[l]
        return a

    def lens(self, t: int) -> np.ndarray:
        """[B, 2] int32: (image tokens, valid cache rows) at decode step t.

        The current token's key/value is already in the cache, hence the +1.
        """
        out = np.empty((len(self.n_img), 2), dtype=np.int32)
        out[:, 0] = self.n_img
        out[:, 1] = self.n_img + self.n_prompt + t + 1
        return out


def _window_tokens(centre: int, n_img: int, W: int, win: Tuple[int, int]) -> np.ndarray:
    r0, c0 = divmod(int(centre), W)
    hr, hc = win[0] // 2, win[1] // 2
    H = -(-n_img // W)
    ids = []
    for r in range(max(0, r0 - hr), min(H, r0 + hr + 1)):
        for c in range(max(0, c0 - hc), min(W, c0 + hc + 1)):
            j = r * W + c
            if j < n_img:
                ids.append(j)
    return np.asarray(ids, dtype=np.int64)


def _seeds(wl: Workload):
    root = np.random.SeedSequence(wl.seed)
    meta, alpha_ss, layers_ss = root.spawn(3)
    return meta, alpha_ss, layers_ss.spawn(wl.num_layers)


def make_structure(wl: Workload) -> Structure:
    meta, alpha_ss, _ = _seeds(wl)
    rng = np.random.Generator(np.random.PCG64(meta))
    B, T = wl.batch, wl.steps
    if wl.grid is not None:
        H, W = wl.grid
        n_img = np.full(B, H * W, dtype=np.int64)
        grid_w = np.full(B, W, dtype=np.int64)
    else:
        lo, hi = wl.n_img_range
        n_img = rng.integers(lo, hi + 1, size=B).astype(np.int64)
        grid_w = np.array([math.ceil(math.sqrt(n)) for n in n_img], dtype=np.int64)
    grid_h = np.array([-(-int(n) // int(w)) for n, w in zip(n_img, grid_w)], dtype=np.int64)
    lo, hi = wl.n_prompt
    n_prompt = (np.full(B, lo, dtype=np.int64) if lo == hi
                else rng.integers(lo, hi + 1, size=B).astype(np.int64))
    if B == 1:
        start = np.zeros(1, dtype=np.int64)
    else:
        start = np.array([rng.integers(0, n) for n in n_img], dtype=np.int64)

    centre = np.empty((T, B), dtype=np.int64)
    for b in range(B):
        cell = int(start[b])
        W = int(grid_w[b])
        H = int(grid_h[b])
        n = int(n_img[b])
        for t in range(T):
            if t > 0:
                if wl.jump_every and t % wl.jump_every == 0:
                    r = (cell // W + 1) % H
                    c = int(rng.integers(0, W))
                    cell = min(r * W + c, n - 1)
                else:
                    cell = (cell + 1) % n
            centre[t, b] = cell

    arng = np.random.Generator(np.random.PCG64(alpha_ss))
    L = wl.num_layers
    if wl.alpha_lo is not None:
        alpha = np.full(L, wl.alpha_lo, dtype=np.float64)
    else:
        alpha = arng.uniform(0.3, 1.0, size=L)
    if wl.planted_layers is not None:
        for l in wl.planted_layers:
            alpha[l] = wl.alpha_hi
    if wl.focal_band is not None:
        alpha[wl.focal_band[0]: wl.focal_band[1] + 1] = wl.alpha_hi
    alpha_late = None
    if wl.drift is not None:
        low = (np.full(L, wl.alpha_lo, dtype=np.float64) if wl.alpha_lo is not None
               else arng.uniform(0.3, 1.0, size=L))
        alpha_late = np.where(alpha == wl.alpha_hi, low, alpha)
        for l in wl.drift[1]:
            alpha_late[l] = wl.alpha_hi
        alpha_late = alpha_late.astype(np.float32)
    s_max = int(np.max(n_img + n_prompt)) + T
    st = Structure(n_img=n_img, n_prompt=n_prompt, grid_w=grid_w, grid_h=grid_h,
                   centre=centre, alpha=alpha.astype(np.float32), max_seq_len=s_max,
                   alpha_late=alpha_late, drift_step=0 if wl.drift is None else int(wl.drift[0]))
    st.windows = [[_window_tokens(centre[t, b], int(n_img[b]), int(grid_w[b]), wl.window)
                   for t in range(T)] for b in range(B)]
    if wl.pages > 1 or wl.page_text != (0, 0):
        pre, gap = wl.page_text
        st.spans, st.image_rows = [], []
        for b in range(B):
            m = int(n_img[b]) // wl.pages
            assert m * wl.pages == int(n_img[b]), "pages must split the image evenly"
            assert int(n_prompt[b]) >= pre + gap * (wl.pages - 1), "n_prompt counts the text around pages"
            sp = [(pre + i * (m + gap), m) for i in range(wl.pages)]
            st.spans.append(sp)
            st.image_rows.append(np.concatenate([np.arange(a, a + c) for a, c in sp]).astype(np.int64))
    return st


# --------------------------------------------------------------------------
# Tensors
# --------------------------------------------------------------------------


def _to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


class Generator:
    """Produces the tensors of one workload, layer by layer.

    ``layer_kv(l)``  -> K, V float32 [B, Hkv, S_max, d] (values representable
                        in the workload dtype)
    ``layer_queries(l, steps)`` -> q float32 [len(steps), B, Hq, d]
    """

    def __init__(self, wl: Workload, structure: Optional[Structure] = None):
        self.wl = wl
        self.st = structure if structure is not None else make_structure(wl)
        _, _, self._layer_ss = _seeds(wl)
        self._kv_cache: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}

    def _streams(self, l: int):
        k_ss, v_ss, q_ss = self._layer_ss[l].spawn(3)
        return k_ss, v_ss, q_ss

    def layer_kv(self, l: int, keep: bool = False) -> Tuple[np.ndarray, np.ndarray]:
        if l in self._kv_cache:
            return self._kv_cache[l]
        wl = self.wl
        shape = (wl.batch, wl.num_kv_heads, self.st.max_seq_len, wl.head_dim)
        k_ss, v_ss, _ = self._streams(l)
        K = np.random.Generator(np.random.PCG64(k_ss)).standard_normal(shape, dtype=np.float32)
        V = np.random.Generator(np.random.PCG64(v_ss)).standard_normal(shape, dtype=np.float32)
        K = _to_dtype(K, wl.dtype)
        V = _to_dtype(V, wl.dtype)
        if keep:
            self._kv_cache[l] = (K, V)
        return K, V

    def layer_queries(self, l: int, steps: Optional[Sequence[int]] = None,
                      K: Optional[np.ndarray] = None) -> np.ndarray:
        """Queries of layer l for the given steps (default: all T steps)."""
        wl, st = self.wl, self.st
        T, B, Hq, Hkv, d = wl.steps, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
        g = Hq // Hkv
        steps = np.arange(T) if steps is None else np.asarray(list(steps), dtype=np.int64)
        if K is None:
            K, _ = self.layer_kv(l)
        _, _, q_ss = self._streams(l)
        # The noise of all T steps is drawn in one block so that any subset of
        # steps sees the same numbers.
        eps = np.random.Generator(np.random.PCG64(q_ss)).standard_normal(
            (T, B, Hq, d), dtype=np.float32)[steps]
        q = np.empty((len(steps), B, Hq, d), dtype=np.float32)
        for b in range(B):
            wins = [st.windows[b][int(t)] for t in steps]
            wmax = max(len(w) for w in wins)
            idx = np.zeros((len(steps), wmax), dtype=np.int64)
            wgt = np.zeros((len(steps), wmax), dtype=np.float32)
            for i, w in enumerate(wins):
                idx[i, :len(w)] = w
                wgt[i, :len(w)] = 1.0 / len(w)
            gathered = K[b][:, st.image_row(b, idx), :]  # [Hkv, S, wmax, d]
            mean = np.einsum("hswd,sw->shd", gathered, wgt, optimize=True)  # [S, Hkv, d]
            mean_q = np.repeat(mean, g, axis=1)  # [S, Hq, d], head h -> kv head h // g
            q[:, b] = st.alpha_at(l, steps)[:, None, None] * mean_q + np.float32(wl.sigma) * eps[:, b]
        return _to_dtype(q, wl.dtype)


# --------------------------------------------------------------------------
# Device-side generation for the large workloads
# --------------------------------------------------------------------------


class DeviceGenerator:
    """The same workload drawn on the GPU with torch's seeded generator.

    Host generation of the 32B/72B-like caches (tens of GB) would take
    minutes, so these tensors are drawn on the device: keys and values
    N(0, 1) per (layer, tensor) stream, queries alpha * window-mean key +
    sigma * N(0, I).  Values are produced in float32 and rounded to the
    workload dtype.  The structure (lengths, windows, alphas) is the same as
    the host generator's; only the random numbers differ.  Anything checked
    on the CPU is read back from these device tensors.
    """

    def __init__(self, wl: Workload, structure: Optional[Structure] = None, device="cuda:0"):
        import torch

        self.torch = torch
        self.wl = wl
        self.st = structure if structure is not None else make_structure(wl)
        self.device = torch.device(device)
        self.io_dtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        _, _, self._layer_ss = _seeds(wl)

    def _seed(self, l: int, which: int) -> int:
        return int(self._layer_ss[l].spawn(3)[which].generate_state(1, dtype=np.uint64)[0] % (2**63))

    def _normal(self, shape, seed: int):
        g = self.torch.Generator(device=self.device)
        g.manual_seed(seed)
        return self.torch.randn(shape, generator=g, device=self.device, dtype=self.torch.float32)

    def layer_kv(self, l: int):
        wl = self.wl
        shape = (wl.batch, wl.num_kv_heads, self.st.max_seq_len, wl.head_dim)
        K = self._normal(shape, self._seed(l, 0)).to(self.io_dtype)
        V = self._normal(shape, self._seed(l, 1)).to(self.io_dtype)
        return K, V

    def layer_queries(self, l: int, steps: Sequence[int], K):
        """Queries of layer l at the given steps, [len(steps), B, Hq, d] on the device."""
        torch = self.torch
        wl, st = self.wl, self.st
        steps = list(steps)
        T, B, Hq, Hkv, d = wl.steps, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
        g_ = Hq // Hkv
        # the noise of all T steps is one block, so any subset sees the same numbers
        eps = self._normal((T, B, Hq, d), self._seed(l, 2))[steps]
        q = torch.empty((len(steps), B, Hq, d), dtype=torch.float32, device=self.device)
        for b in range(B):
            wins = [st.windows[b][int(t)] for t in steps]
            wmax = max(len(w) for w in wins)
            idx = np.zeros((len(steps), wmax), dtype=np.int64)
            wgt = np.zeros((len(steps), wmax), dtype=np.float32)
            for i, w in enumerate(wins):
                idx[i, :len(w)] = w
                wgt[i, :len(w)] = 1.0 / len(w)
            idx_t = torch.from_numpy(st.image_row(b, idx)).to(self.device)
            wgt_t = torch.from_numpy(wgt).to(self.device)
            Kb = K[b].float()  # [Hkv, S, d]
            gathered = Kb[:, idx_t.reshape(-1)].reshape(Hkv, len(steps), wmax, d)
            mean = (gathered * wgt_t[None, :, :, None]).sum(dim=2)  # [Hkv, S, d]
            mean_q = mean.permute(1, 0, 2).repeat_interleave(g_, dim=1)  # [S, Hq, d]
            a_t = torch.from_numpy(st.alpha_at(l, steps)).to(self.device)[:, None, None]
            q[:, b] = a_t * mean_q + float(wl.sigma) * eps[:, b]
        return q.to(self.io_dtype)
