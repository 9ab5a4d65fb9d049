"""Workload table: the five synthetic workloads the path is measured and tested on.

Each entry states shapes, the token layout (latent grid, text length, the
reorder to apply), the mask-selection knobs and the generator seed.  The
shapes stand in for the workloads the source pages describe (their models and
datasets are not available):

* ``tiny``   -- 4 frames of a 4x4 grid, N=64, d=64, fp32 (the teaching video of
  the SparseAttn article, section 3.3), predicted mask at b=16, tau=0.9,
  theta=0.5.
* ``image``  -- an image DiT at 64x64 latent, B=2, 24 heads, N=4096, d=128, block
  128, sparsity 0.6, TopCdf tau=0.9 (the MindIE-SD "sparse" page's image example
  and its default sparsity for image tasks).
* ``video``  -- a video DiT latent [16,32,48] with 226 text tokens prepended,
  [4,8,4] window reorder, first frame and text as sink blocks, sparsity 0.8
  (RainFusion2.0 on the MindIE-SD page).
* ``long_video`` -- latent [28,30,53], N=44520, Hilbert reorder, b_q=128 / b_k=64,
  tau=0.95, theta=0.6, lambda=-8, sparsity 0.8 (SpargeAttn reading notes,
  sections 2.2-2.5).
* ``causal_long`` -- GQA 32/8 heads, N=131072, causal, sliding window 4096,
  4 sink tokens, TopCdf tau=0.9, block 128 (the long-context row of the
  SpargeAttn speed table; the sliding-window definition of the "Local Sliding
  and Sparse Attention" page).
"""

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

ORDER_IDENTITY = 0
ORDER_WINDOW = 1
ORDER_HILBERT = 2


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    latent: Tuple[int, int, int]  # (t, h, w) of the video tokens
    txt_len: int                  # text tokens, prepended in the original layout
    D: int
    dtype: str                    # "f32" or "bf16": the dtype handed to the permute step
    order: int                    # ORDER_*
    window: Tuple[int, int, int] = (1, 1, 1)  # [t,h,w] reorder window (ORDER_WINDOW)
    first_frame_sink: bool = False
    block_q: int = 128
    block_k: int = 128
    causal: bool = False
    window_tokens: int = 0        # causal sliding window W in tokens (0 = off)
    sink_front: int = 0           # tokens at the front of the permuted order kept as sinks
    sink_back: int = 0            # tokens at the back of the permuted order kept as sinks
    sink_rows: int = 0            # tokens at the front whose query blocks keep their whole row
    tile: Optional[Tuple[int, int, int]] = None  # 3-D tile windows forced as blocks (None = off)
    tile_radius: Tuple[int, int, int] = (0, 0, 0)  # their reach in tiles along t, h, w
    latent_k: Optional[Tuple[int, int, int]] = None  # keys/values on their own grid (None: the latent)
    txt_len_k: Optional[int] = None               # text tokens among the keys (None: txt_len)
    tau: Optional[float] = None   # TopCdf cumulative mass (None = unset)
    theta: Optional[float] = None  # self-similarity guard (None = off)
    sparsity: Optional[float] = None  # keep floor (None = unset)
    lam: Optional[float] = None   # PV-skip threshold (None = off)
    seed: int = 0
    sweep: Tuple[float, ...] = field(default_factory=tuple)

    @property
    def N(self) -> int:
        t, h, w = self.latent
        return self.txt_len + t * h * w

    @property
    def N_k(self) -> int:
        t, h, w = self.latent if self.latent_k is None else self.latent_k
        return (self.txt_len if self.txt_len_k is None else self.txt_len_k) + t * h * w

    def with_sparsity(self, s: Optional[float]) -> "Workload":
        return replace(self, sparsity=s)


CONFIGS = {
    "tiny": Workload(
        name="tiny", B=1, Hq=1, Hkv=1, latent=(4, 4, 4), txt_len=0, D=64,
        dtype="f32", order=ORDER_IDENTITY, block_q=16, block_k=16,
        tau=0.9, theta=0.5, seed=1),
    "image": Workload(
        name="image", B=2, Hq=24, Hkv=24, latent=(1, 64, 64), txt_len=0, D=128,
        dtype="bf16", order=ORDER_IDENTITY, block_q=128, block_k=128,
        tau=0.9, sparsity=0.6, seed=2),
    "video": Workload(
        name="video", B=1, Hq=24, Hkv=24, latent=(16, 32, 48), txt_len=226, D=128,
        dtype="bf16", order=ORDER_WINDOW, window=(4, 8, 4), first_frame_sink=True,
        block_q=128, block_k=128, sink_front=32 * 48, sink_back=226,
        sparsity=0.8, seed=3),
    "long_video": Workload(
        name="long_video", B=1, Hq=24, Hkv=24, latent=(28, 30, 53), txt_len=0, D=128,
        dtype="bf16", order=ORDER_HILBERT, block_q=128, block_k=64,
        tau=0.95, theta=0.6, lam=-8.0, sparsity=0.8, seed=4, sweep=(0.5, 0.8, 0.9)),
    "causal_long": Workload(
        name="causal_long", B=1, Hq=32, Hkv=8, latent=(1, 1, 131072), txt_len=0, D=128,
        dtype="bf16", order=ORDER_IDENTITY, block_q=128, block_k=128, causal=True,
        window_tokens=4096, sink_front=4, tau=0.9, seed=5),
}


def get_config(name: str) -> Workload:
    return CONFIGS[name]
