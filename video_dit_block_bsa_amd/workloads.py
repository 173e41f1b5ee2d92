"""The five BSA workloads: latent grids, heads and selection rules.

Grids follow the token counts of the pages' stages (WAN2.1 VAE 4x8x8 and a
1x2x2 patchify give a 4x16x16 pixel-to-token reduction): a 480p coarse
stage, the 720p x 93-frame refinement stage, a long 215K-token sequence,
and a video-continuation case with condition frames and CDF selection.
Heads = 32 and head_dim = 128 come from the DiT's 4096 hidden size.
"""

from __future__ import annotations

from dataclasses import dataclass, field


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    W: int
    heads: int
    head_dim: int = 128
    batch: int = 1
    kind: str = "field"
    seed: int = 0
    mode: str = "topk"
    k: int = 1
    p: float = 0.9
    k_min: int = 1
    k_max: int = 64
    cond_frames: int = 0
    chunk: tuple = (4, 4, 8)
    key_chunk: tuple = ()  # empty: the same as chunk
    note: str = field(default="", compare=False)

    @property
    def seq_len(self) -> int:
        return self.T * self.H * self.W

    @property
    def num_blocks(self) -> int:
        """Query blocks per (batch, head). Counts are ceilings: a chunk that
        does not divide the grid leaves a partial block at the far edge."""
        ct, ch, cw = self.chunk
        return _cdiv(self.T, ct) * _cdiv(self.H, ch) * _cdiv(self.W, cw)

    @property
    def cond_blocks(self) -> int:
        """Leading condition query blocks (cond_frames is a multiple of ct)."""
        ct, ch, cw = self.chunk
        return (self.cond_frames // ct) * _cdiv(self.H, ch) * _cdiv(self.W, cw)

    @property
    def block_tokens(self) -> int:
        ct, ch, cw = self.chunk
        return ct * ch * cw

    @property
    def kchunk(self) -> tuple:
        return tuple(self.key_chunk) if self.key_chunk else tuple(self.chunk)

    @property
    def key_block_tokens(self) -> int:
        a, b, c = self.kchunk
        return a * b * c

    @property
    def num_key_blocks(self) -> int:
        a, b, c = self.kchunk
        return _cdiv(self.T, a) * _cdiv(self.H, b) * _cdiv(self.W, c)

    @property
    def stride(self) -> int:
        return self.k if self.mode == "topk" else self.k_max


WORKLOADS = {
    "tiny": Workload("tiny", 4, 8, 16, heads=2, kind="iid", seed=0, k=2,
                     note="512 tokens, 4 blocks; k=4 is the dense check"),
    "480p": Workload("480p", 12, 32, 56, heads=32, seed=1, k=11,
                     note="21,504 tokens, 168 blocks, ~93.5% sparsity"),
    "720p": Workload("720p", 24, 48, 80, heads=32, seed=2, k=45,
                     note="92,160 tokens, 720 blocks, 93.75% sparsity"),
    "long": Workload("long", 56, 48, 80, heads=32, seed=3, k=105,
                     note="215,040 tokens, 1,680 blocks, 93.75% sparsity"),
    "vc": Workload("vc", 16, 48, 80, heads=32, seed=4, mode="cdf", p=0.90,
                   k_min=4, k_max=64, cond_frames=4,
                   note="61,440 tokens, 4 condition frames, CDF 0.90 in [4, 64]"),
    # Decoupled key blocks on the 215K grid at the refinement ratio r = N_k/16.
    "long_k64": Workload("long_k64", 56, 48, 80, heads=32, seed=3, k=210, key_chunk=(2, 4, 8),
                         note="215,040 tokens, 128-token query blocks, 3,360 key blocks of 64"),
    "long_k256": Workload("long_k256", 56, 48, 80, heads=32, seed=3, k=52, key_chunk=(4, 8, 8),
                          note="215,040 tokens, 128-token query blocks, 840 key blocks of 256"),
    "long_q64": Workload("long_q64", 56, 48, 80, heads=32, seed=3, k=105, chunk=(2, 4, 8),
                         key_chunk=(4, 4, 8),
                         note="215,040 tokens, 3,360 query blocks of 64, 1,680 key blocks of 128"),
}


def effective_flops(w: Workload, total_kept_blocks: int) -> float:
    """4 * n_q * kept_keys * d summed over heads: two matmuls of 2 flop/MAC,
    counted only over kept (query block, key block) pairs."""
    return 4.0 * w.block_tokens * w.key_block_tokens * w.head_dim * float(total_kept_blocks)
