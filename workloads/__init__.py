"""Seeded synthetic inputs for sharded paged decode attention.

This module only draws and encodes input data: sequence lengths, a paged
block pool with a scattered block table, queries and cached K/V or latent
rows. It holds none of the attention arithmetic, so the CPU oracle and the
HIP path can both consume its output without sharing any method code.

Workloads follow the shapes the pages describe for Decode Context
Parallelism ("Efficient Decode Context Parallelism with vLLM for Long Context
Workloads", section A4: agentic trace with median input about 67K, 53 % above
64K, about 8 % above 128K, 3-4 % above 256K, a tail near 1M, and 18 % below
8K).  The trace itself is not available; its length statistics are stood in
for by stratified quantiles of a log-linear CDF through those points.

Every random draw comes from ``numpy.random.default_rng([seed, stream, i])``
with a fixed stream id per tensor, so each group of blocks can be regenerated
on its own and threads can fill disjoint groups in parallel.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

KI = 1024

# (CDF value, context length in tokens).  The 18 % knot reads "18 % of all
# requests are shorter than 8K"; the median knot is 67K; the tail ends at 1M.
BIMODAL_KNOTS = (
    (0.0, 1 * KI),
    (0.18, 8 * KI),
    (0.47, 64 * KI),
    (0.50, 67 * KI),
    (0.92, 128 * KI),
    (0.965, 256 * KI),
    (1.0, 1024 * KI),
)

# Stream ids for the independent random draws of one workload.
_S_LENGTH_SHUFFLE = 1
_S_BLOCK_PERM = 2
_S_Q = 3
_S_K = 4
_S_V = 5
_S_SCALE = 6

F8_E4M3_MAX = 448.0


@dataclass(frozen=True)
class Spec:
    """Shape of one decode-attention workload (one layer, one decode step)."""

    name: str
    kind: str  # "gqa": separate K and V per KV head; "mla": one shared latent row
    batch: int
    num_q_heads: int
    num_kv_heads: int
    qk_dim: int
    v_dim: int
    block_size: int
    num_shards: int
    kv_dtype: str  # "f32", "bf16" or "fp8" (OCP e4m3 with one fp32 scale per token)
    lengths: object  # an int (every sequence that long) or "bimodal"
    softmax_scale: float
    seed: int
    len_div: int = 1  # divides every length (scaled-down twin of a workload)
    q_len: int = 1  # query tokens per sequence (multi-token decode when > 1)

    @property
    def q_dtype(self) -> str:
        return "f32" if self.kv_dtype == "f32" else "bf16"

    def kv_bytes_per_token(self) -> int:
        """Bytes of cached K/V (or latent, plus scale) one token occupies."""
        if self.kind == "gqa":
            elt = 4 if self.kv_dtype == "f32" else 2
            return self.num_kv_heads * (self.qk_dim + self.v_dim) * elt
        if self.kv_dtype == "fp8":
            return self.qk_dim + 4
        return self.qk_dim * (4 if self.kv_dtype == "f32" else 2)


SPECS = {
    s.name: s
    for s in (
        Spec("gqa_f32_b1_L256", "gqa", 1, 4, 1, 64, 64, 16, 2, "f32", 256, 1.0 / 8.0, 1),
        Spec("gqa_bf16_b32_L32k", "gqa", 32, 64, 8, 128, 128, 16, 4, "bf16", 32 * KI,
             1.0 / math.sqrt(128.0), 2),
        Spec("mla_bf16_b64_bimodal", "mla", 64, 64, 1, 576, 512, 64, 8, "bf16", "bimodal",
             1.0 / math.sqrt(576.0), 3),
        Spec("mla_fp8_b128_bimodal", "mla", 128, 64, 1, 576, 512, 64, 8, "fp8", "bimodal",
             1.0 / math.sqrt(576.0), 4),
        Spec("mla_bf16_b8_L1m", "mla", 8, 64, 1, 576, 512, 64, 8, "bf16", 1024 * KI,
             1.0 / math.sqrt(576.0), 5),
    )
}

# The headline workload: absorbed-MLA bf16, batch 64, bimodal lengths, D = 8.
HEADLINE = "mla_bf16_b64_bimodal"


def scaled(spec: Spec, batch_div: int = 8, len_div: int = 64) -> Spec:
    """A smaller twin of ``spec``: batch / batch_div, every length / len_div."""
    return replace(
        spec,
        name=f"{spec.name}_div{batch_div}x{len_div}",
        batch=max(1, spec.batch // batch_div),
        len_div=spec.len_div * len_div,
    )


def bimodal_lengths(batch: int, seed: int, knots=BIMODAL_KNOTS) -> np.ndarray:
    """Stratified inverse-CDF lengths: L_b = F^-1((b + 1/2) / B), then shuffled.

    F is log-linear in length between the knots, so the realised fractions
    above 64K / 128K / 256K match the knots up to 1/B.
    """
    u = (np.arange(batch, dtype=np.float64) + 0.5) / batch
    cdf = np.array([c for c, _ in knots])
    logl = np.log(np.array([l for _, l in knots], dtype=np.float64))
    lengths = np.rint(np.exp(np.interp(u, cdf, logl))).astype(np.int64)
    np.random.default_rng([seed, _S_LENGTH_SHUFFLE]).shuffle(lengths)
    return lengths


def seq_lengths(spec: Spec) -> np.ndarray:
    if spec.lengths == "bimodal":
        lens = bimodal_lengths(spec.batch, spec.seed)
    else:
        lens = np.full(spec.batch, int(spec.lengths), dtype=np.int64)
    if spec.len_div > 1:
        lens = np.maximum(1, lens // spec.len_div)
    return lens.astype(np.int32)


@dataclass
class Workload:
    """Host-side arrays for one workload.

    Layouts (all C-contiguous):
      q           [B, q_len * Hq, qk_dim]     float32, or uint16 bf16 bit patterns
                  (token-major: row t * Hq + h is head h of query token t)
      k_cache     gqa: [num_blocks, bs, Hkv, qk_dim]; mla: latent [num_blocks, bs, qk_dim]
      v_cache     gqa: [num_blocks, bs, Hkv, v_dim];  mla: None (V is latent[..., :v_dim])
      kv_scale    fp8 only: float32 [num_blocks, bs], one scale per cached token
      seq_lens    int32 [B]
      block_table int32 [B, max_blocks], logical block j of sequence b -> physical
                  block id; entries past ceil(L_b / bs) are -1
    Cached values are float32, uint16 (bf16 bits) or uint8 (e4m3 codes).
    """

    spec: Spec
    seq_lens: np.ndarray
    block_table: np.ndarray
    num_blocks: int
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: Optional[np.ndarray]
    kv_scale: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]

    def kv_bytes(self) -> int:
        """Bytes of cached data the sequences actually cover (one read each)."""
        return int(self.seq_lens.astype(np.int64).sum()) * self.spec.kv_bytes_per_token()


def build_block_table(seq_lens: np.ndarray, block_size: int, seed: int):
    """Scatter every sequence's logical blocks over a seeded permutation of the pool."""
    nb = (seq_lens.astype(np.int64) + block_size - 1) // block_size
    num_blocks = int(nb.sum())
    perm = np.random.default_rng([seed, _S_BLOCK_PERM]).permutation(num_blocks).astype(np.int32)
    max_blocks = int(max(1, nb.max(initial=0)))
    table = np.full((len(seq_lens), max_blocks), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nb):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, num_blocks


def _threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    n = int(env) if env and env.isdigit() else (os.cpu_count() or 1)
    return max(1, min(16, n))


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (torch's cast)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3 ("fn") codes, saturating at +-448, round-to-nearest-even."""
    import torch

    x = np.clip(x, -F8_E4M3_MAX, F8_E4M3_MAX)
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return encode_bf16(x)
    if dtype == "fp8":
        return encode_e4m3(x)
    raise ValueError(dtype)


_NP_STORE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}


def fill_blocks(seed: int, stream: int, num_blocks: int, block_shape, dtype: str,
                draw: str = "normal", lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    """Per-block random data, generated in independent groups of blocks.

    Group g covers blocks [g*G, (g+1)*G) and is drawn from
    default_rng([seed, stream, g]); G depends only on the block shape.
    """
    per_block = int(np.prod(block_shape))
    group = max(1, (1 << 20) // per_block)
    out = np.empty((num_blocks,) + tuple(block_shape), dtype=_NP_STORE[dtype])
    ngroups = (num_blocks + group - 1) // group

    def work(g):
        b0 = g * group
        b1 = min(num_blocks, b0 + group)
        rng = np.random.default_rng([seed, stream, g])
        shape = (b1 - b0,) + tuple(block_shape)
        if draw == "normal":
            x = rng.standard_normal(shape, dtype=np.float32)
        else:
            x = rng.uniform(lo, hi, shape).astype(np.float32)
        out[b0:b1] = _encode(x, dtype)

    if ngroups <= 1:
        for g in range(ngroups):
            work(g)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(ngroups)))
    return out


def _build(spec: Spec, lens: np.ndarray) -> Workload:
    s = spec.seed
    table, num_blocks = build_block_table(lens, spec.block_size, s)
    q32 = np.random.default_rng([s, _S_Q]).standard_normal(
        (spec.batch, spec.q_len * spec.num_q_heads, spec.qk_dim), dtype=np.float32)
    q = _encode(q32, spec.q_dtype)
    bs = spec.block_size
    scale = None
    if spec.kind == "gqa":
        k = fill_blocks(s, _S_K, num_blocks, (bs, spec.num_kv_heads, spec.qk_dim), spec.kv_dtype)
        v = fill_blocks(s, _S_V, num_blocks, (bs, spec.num_kv_heads, spec.v_dim), spec.kv_dtype)
    else:
        k = fill_blocks(s, _S_K, num_blocks, (bs, spec.qk_dim), spec.kv_dtype)
        v = None
        if spec.kv_dtype == "fp8":
            scale = fill_blocks(s, _S_SCALE, num_blocks, (bs,), "f32", draw="uniform", lo=0.5, hi=2.0)
    return Workload(spec, lens, table, num_blocks, q, k, v, scale)


def make(spec, seed: Optional[int] = None) -> Workload:
    """Build the host arrays of ``spec`` (a Spec or a name in SPECS)."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    if seed is not None:
        spec = replace(spec, seed=seed)
    return _build(spec, seq_lengths(spec))


def custom(kind: str, seq_lens, *, num_q_heads: int, num_kv_heads: int = 1, qk_dim: int,
           v_dim: int, block_size: int, num_shards: int, kv_dtype: str, softmax_scale=None,
           seed: int = 0, name: str = "custom", q_len: int = 1) -> Workload:
    """A workload with explicit per-sequence lengths (edge cases, ragged tails)."""
    lens = np.asarray(seq_lens, dtype=np.int32).reshape(-1)
    spec = Spec(name, kind, len(lens), num_q_heads, num_kv_heads, qk_dim, v_dim, block_size,
                num_shards, kv_dtype, "explicit",
                softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(qk_dim), seed,
                q_len=q_len)
    return _build(spec, lens)


def to_torch(w: Workload, device="cuda"):
    """Device tensors of a workload (plain copies; bf16 bit patterns become torch.bfloat16,
    e4m3 codes stay uint8). Returns a namespace with q, k_cache, v_cache, kv_scale,
    block_table and seq_lens."""
    import torch
    from types import SimpleNamespace

    def dev(x, bf16=False):
        if x is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(x))
        if bf16:
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(device)

    bf = w.spec.kv_dtype == "bf16"
    return SimpleNamespace(
        q=dev(w.q, w.spec.q_dtype == "bf16"),
        k_cache=dev(w.k_cache, bf),
        v_cache=dev(w.v_cache, bf),
        kv_scale=dev(w.kv_scale),
        block_table=dev(w.block_table),
        seq_lens=dev(w.seq_lens),
    )
