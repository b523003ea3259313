"""Seeded synthetic inputs for the fused attention forward.

This module is shared by the tests, the benchmark and the smoke check. It holds
only input generation (random draws, document lengths, per-head ALiBi slopes and
the workload table); it computes nothing of attention itself, so that the GPU
path and the CPU oracle stay independent of each other.

The pages name the variants (sliding window, document packing, ALiBi,
soft-capping: Neuron FA4 explainer, "PyTorch Gets the Upgrade Too"; NextVector
FlexAttention article, "What Happened?") but give no shapes and no data set; the
shapes, seeds and distributions below are synthetic stand-ins of the workloads
the method is benchmarked on (workloads limited by arithmetic rather than
memory traffic: PyTorch FlexAttention FA4-backend post).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    """One attention-forward problem: shapes, dtype, variant and seeds."""

    name: str
    B: int
    H: int          # query heads
    Hkv: int        # key/value heads (GQA when Hkv < H)
    S: int          # Skv, and Sq unless `sq` is set
    D: int          # head dimension
    dtype: str      # "bf16" or "fp32" element type of Q/K/V/O
    causal: bool = False
    window: int = 0             # 0 = no sliding window; else q - k < window
    documents: bool = False     # document-packing mask
    doc_len_range: tuple = (512, 4096)
    mod: str = "none"           # "none" | "alibi" | "softcap" | "relbias"
    softcap: float = 30.0
    seed: int = 0
    doc_seed: int = 0
    q_offset: int = 0           # query row i sits at key position i + q_offset
    prefix: int | None = None   # prefix-LM boundary (with causal), or None
    sq: int = 0                 # > 0: query rows, when fewer than the keys
    rel_max: int = 0            # clip distance R of the relative-bias table (mod "relbias")
    decode: bool = False        # run through the decode entry point (packed heads, split keys)
    split: bool = False         # run through the split-KV entry point (split key lists, merged)

    @property
    def Sq(self) -> int:
        return self.sq or self.S

    @property
    def Skv(self) -> int:
        return self.S

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five problem families (tiny parity case, dense, causal GQA, packed
# documents with a sliding window, long-context score modifications).
WORKLOADS = {
    "tiny_causal": Workload("tiny_causal", B=1, H=2, Hkv=2, S=128, D=64, dtype="fp32",
                            causal=True, seed=0),
    "dense": Workload("dense", B=4, H=16, Hkv=16, S=4096, D=128, dtype="bf16", seed=1),
    "causal_gqa": Workload("causal_gqa", B=2, H=32, Hkv=8, S=8192, D=128, dtype="bf16",
                           causal=True, seed=2),
    # one GPU's share of causal_gqa when the heads are split over 8 GPUs
    # (whole GQA groups: 1 key/value head and its 4 query heads per GPU)
    "causal_gqa_shard8": Workload("causal_gqa_shard8", B=2, H=4, Hkv=1, S=8192, D=128,
                                  dtype="bf16", causal=True, seed=2),
    # the same shard through the split-KV entry point: 256 query tiles for 256
    # CUs, each tile's key list split and the parts merged
    "causal_gqa_shard8_split": Workload("causal_gqa_shard8_split", B=2, H=4, Hkv=1, S=8192, D=128,
                                        dtype="bf16", causal=True, seed=2, split=True),
    "doc_swa": Workload("doc_swa", B=1, H=16, Hkv=16, S=16384, D=128, dtype="bf16",
                        causal=True, window=1024, documents=True, seed=3, doc_seed=3),
    "alibi_d64": Workload("alibi_d64", B=1, H=32, Hkv=32, S=32768, D=64, dtype="bf16",
                          causal=True, mod="alibi", seed=4),
    "alibi_d128": Workload("alibi_d128", B=1, H=32, Hkv=32, S=32768, D=128, dtype="bf16",
                           causal=True, mod="alibi", seed=5),
    "softcap_d64": Workload("softcap_d64", B=1, H=32, Hkv=32, S=32768, D=64, dtype="bf16",
                            causal=True, mod="softcap", seed=4),
    "softcap_d128": Workload("softcap_d128", B=1, H=32, Hkv=32, S=32768, D=128, dtype="bf16",
                             causal=True, mod="softcap", seed=5),
    # further variants: prefix-LM (a bidirectional 2048-token prompt, then
    # causal) on the causal GQA shape, and a 4096-token prefill chunk after
    # 28672 cached keys (query row i at key position 28672 + i)
    "prefix_lm": Workload("prefix_lm", B=2, H=32, Hkv=8, S=8192, D=128, dtype="bf16",
                          causal=True, prefix=2048, seed=6),
    "chunked_prefill": Workload("chunked_prefill", B=1, H=32, Hkv=8, S=32768, sq=4096,
                                q_offset=28672, D=128, dtype="bf16", causal=True, seed=7),
    # relative-position bias (a per-head table over distances clipped to
    # +-1023) on the causal GQA shape
    "relbias": Workload("relbias", B=2, H=32, Hkv=8, S=8192, D=128, dtype="bf16", causal=True,
                        mod="relbias", rel_max=1023, seed=8),
    # head dimension 256 on the causal GQA shape
    "causal_gqa_d256": Workload("causal_gqa_d256", B=2, H=16, Hkv=8, S=8192, D=256, dtype="bf16",
                                causal=True, seed=10),
    # one decoding step: 16 sequences, each one new query row per head after
    # 32767 cached keys (GQA 32 query / 8 key-value heads)
    "decode": Workload("decode", B=16, H=32, Hkv=8, S=32768, sq=1, q_offset=32767, D=128,
                       dtype="bf16", causal=True, decode=True, seed=9),
}


def draw_qkv(B: int, H: int, Hkv: int, Sq: int, Skv: int, D: int, seed: int):
    """Q, K, V as float32 N(0, 1) on the CPU, drawn in that order from one
    torch CPU generator seeded with `seed`."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, H, Sq, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, Skv, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, Skv, D), generator=g, dtype=torch.float32)
    return q, k, v


def draw_dout(B: int, H: int, Sq: int, D: int, seed: int) -> torch.Tensor:
    """The output gradient dO for backward tests and benches: float32 N(0, 1)
    on the CPU from a torch CPU generator seeded with `seed` + 1000."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 1000)
    return torch.randn((B, H, Sq, D), generator=g, dtype=torch.float32)


def rel_bias_table(H: int, R: int, seed: int) -> np.ndarray:
    """Relative-bias table [H, 2R + 1] as float32: N(0, 1) from a torch CPU
    generator seeded with `seed` + 2000."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 2000)
    return torch.randn((H, 2 * R + 1), generator=g, dtype=torch.float32).numpy()


def as_element_type(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Cast a float32 CPU tensor to the workload's element type (bf16 uses
    round-to-nearest-even, which is what torch's cast does)."""
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "fp32":
        return x.contiguous()
    raise ValueError(f"unknown element type {dtype!r}")


def bf16_values(x: torch.Tensor) -> np.ndarray:
    """The exact values a bf16 consumer sees, as float64 (round-to-nearest-even
    from float32 when `x` is not already bf16)."""
    return x.to(torch.bfloat16).to(torch.float64).numpy()


def document_lengths(S: int, seed: int, lo: int = 512, hi: int = 4096) -> list[int]:
    """Document lengths drawn uniformly from the inclusive range [lo, hi] with
    numpy's default_rng(seed) until they cover S positions; the last document is
    cut to fit (so it may be shorter than lo)."""
    rng = np.random.default_rng(int(seed))
    out: list[int] = []
    total = 0
    while total < S:
        n = int(rng.integers(lo, hi, endpoint=True))
        n = min(n, S - total)
        out.append(n)
        total += n
    return out


def document_ids(lengths: list[int]) -> np.ndarray:
    """Per-position document label (0, 0, ..., 1, 1, ...) as int32."""
    return np.repeat(np.arange(len(lengths), dtype=np.int32),
                     np.asarray(lengths, dtype=np.int64)).astype(np.int32)


def alibi_slopes(H: int) -> np.ndarray:
    """Per-head ALiBi slopes as float32, the geometric sequence 2^(-8 i / H) for
    1-based head number i (head 0 gets 2^(-8/H))."""
    i = np.arange(1, H + 1, dtype=np.float64)
    return np.exp2(-8.0 * i / H).astype(np.float32)


@dataclass
class Inputs:
    """Host-side inputs of one workload."""

    wl: Workload
    q: torch.Tensor             # element type of the workload, CPU
    k: torch.Tensor
    v: torch.Tensor
    doc_ids: np.ndarray | None  # int32 [B, S] or None
    slopes: np.ndarray | None   # float32 [H] or None
    extra: dict = field(default_factory=dict)
    rel_bias: np.ndarray | None = None   # float32 [H, 2R + 1] or None


def make_inputs(wl: Workload) -> Inputs:
    q, k, v = draw_qkv(wl.B, wl.H, wl.Hkv, wl.Sq, wl.Skv, wl.D, wl.seed)
    q, k, v = (as_element_type(t, wl.dtype) for t in (q, k, v))
    doc = None
    if wl.documents:
        # batch row b draws its document layout from seed doc_seed + b
        doc = np.stack([document_ids(document_lengths(max(wl.Sq + wl.q_offset, wl.Skv), wl.doc_seed + b,
                                                      *wl.doc_len_range))
                        for b in range(wl.B)]).astype(np.int32)
    slopes = alibi_slopes(wl.H) if wl.mod == "alibi" else None
    rel = rel_bias_table(wl.H, wl.rel_max, wl.seed) if wl.mod == "relbias" else None
    return Inputs(wl, q, k, v, doc, slopes, rel_bias=rel)
