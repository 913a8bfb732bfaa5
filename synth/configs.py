"""The five synthetic workloads of the sparse-attention path and their inputs.

Fixed dimensions (all workloads): indexer keys 128-d (bf16 in, int8 once
pooled), 32 indexer heads, groups of 4 tokens, a budget of 512 groups (2048
tokens), 64 attention heads over a 512-d MLA latent, softmax scale 1/sqrt(512).
Pages: 256 tokens of keys / latent rows, which is 64 pooled groups; one logical
page id addresses the key, latent and pooled pools alike.

Workloads (seed = workload index):
  0  decode, B=1,  L=8192
  1  decode, B=64, L=131072 each
  2  decode, B=8,  L=1,048,576 each
  3  prefill chunk: 2048 queries at positions 1,046,528..1,048,575 of one
     1,048,576-token sequence
  4  ragged decode, B=32, L_b = floor(512 * 2^(11 u_b)) (log-uniform on
     [512, 2^20)), pages placed at a seeded random permutation of the pool

Input recipe (tensor ids of the generator in parentheses):
  indexer keys (1)      N(0,1) -> bf16, logical [sum L, 128], element
                        (token_offset(b) + t) * 128 + d
  pooling logits (2)    4 x N(0,1) in double; weights = softmax -> fp32
  indexer query (3)     int8 uniform [-127, 127], [rows, 32, 128]
  head weights (4)      int8 uniform [0, 64], [rows, 32]
  latent cache (5)      N(0,1) -> bf16, logical [sum L, 512]
  attention query (6)   N(0,1) -> bf16, [rows, 64, 512]
  lengths (7)           uniform double u_b (workload 4 only)
  page permutation (8)  Fisher-Yates with j = draw_i mod (i + 1) (workload 4 only)

Linear-attention (KDA) decode steps, n (sequence, head) units, step s (each
tensor drawn at element offset s * its size per step):
  query (32)            N(0,1) -> bf16, [n, 128]
  key (33)              N(0,1) in double, scaled to unit length per unit, -> bf16 (nearest even)
  value (34)            N(0,1) -> bf16, [n, 128]
  decay (35)            0.9 + 0.1 u, fp32 [n, 128]
  gate (36)             u, fp32 [n]
  initial state (37)    N(0,1) -> bf16, [n, 128, 128] (step 0 only)

Layers that share one selection (IndexShare): layer 0 uses the tensors above;
layer l >= 1 has its own attention query (tensor id 16 + l, same layout) and a
latent cache equal to layer 0's with the sign bit flipped on the channels whose
bit l - 1 is set -- still N(0,1) per element, a different cache per layer, and
cheap to build on the device without generating a new 8 GiB pool.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from . import normal_bf16, normal_f64, raw_u64, uniform_f64, uniform_i8

IDX_DIM = 128
IDX_HEADS = 32
GROUP = 4
TOPK_GROUPS = 512
ATT_HEADS = 64
LAT_DIM = 512
PAGE_TOKENS = 256
PAGE_GROUPS = PAGE_TOKENS // GROUP
SM_SCALE = 1.0 / math.sqrt(LAT_DIM)

T_KEYS, T_POOLW, T_QIDX, T_HEADW, T_LATENT, T_QATT, T_LENS, T_PERM = 1, 2, 3, 4, 5, 6, 7, 8
T_QATT_LAYER = 16  # attention query of layer l >= 1: tensor id 16 + l


T_KDA_Q, T_KDA_K, T_KDA_V, T_KDA_ALPHA, T_KDA_BETA, T_KDA_STATE = 32, 33, 34, 35, 36, 37
KDA_DIM = 128


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of float32 values, as bits (input plumbing)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def kda_inputs(seed: int, n: int, step: int):
    """Per-step inputs of n KDA units: (q, k, v) bf16 bits [n,128], alpha fp32
    [n,128], beta fp32 [n]."""
    D = KDA_DIM
    off = step * n * D
    q = normal_bf16(seed, T_KDA_Q, (n, D), start=off)
    kd = normal_f64(seed, T_KDA_K, (n, D), start=off)
    k = _to_bf16_bits((kd / np.linalg.norm(kd, axis=1, keepdims=True)).astype(np.float32))
    v = normal_bf16(seed, T_KDA_V, (n, D), start=off)
    alpha = (0.9 + 0.1 * uniform_f64(seed, T_KDA_ALPHA, (n, D), start=off)).astype(np.float32)
    beta = uniform_f64(seed, T_KDA_BETA, (n,), start=step * n).astype(np.float32)
    return q, k, v, alpha, beta


def kda_state(seed: int, n: int) -> np.ndarray:
    """Initial bf16 state bits [n, 128, 128]."""
    return normal_bf16(seed, T_KDA_STATE, (n, KDA_DIM, KDA_DIM))


def layer_flip_view(bits, layer: int):
    """The channels of layer `layer` (>= 1) whose latent sign bit is flipped
    relative to layer 0, as a strided view of a [..., 512] array of bf16 bits
    (numpy or torch, int16/uint16): channels c with bit layer-1 of c set.
    XOR-ing 0x8000 into the view in place turns layer 0's cache into layer
    `layer`'s, and back."""
    w = 1 << (layer - 1)
    return bits.reshape(-1, LAT_DIM // (2 * w), 2, w)[:, :, 1, :]


@dataclass
class Workload:
    index: int
    name: str
    seed: int
    kind: str                      # "decode" | "prefill"
    lens: List[int]
    paged_random: bool = False     # random physical page placement
    q_pos: Optional[np.ndarray] = None
    description: str = ""
    _perm: Optional[np.ndarray] = field(default=None, repr=False)

    # ---- shape helpers -------------------------------------------------
    @property
    def batch(self) -> int:
        return len(self.lens)

    @property
    def rows(self) -> int:
        return self.batch if self.kind == "decode" else int(len(self.q_pos))

    def groups(self, b: int) -> int:
        return (self.lens[b] + GROUP - 1) // GROUP

    def pages(self, b: int) -> int:
        return (self.lens[b] + PAGE_TOKENS - 1) // PAGE_TOKENS

    @property
    def max_pages(self) -> int:
        return max(self.pages(b) for b in range(self.batch))

    @property
    def num_pages(self) -> int:
        return sum(self.pages(b) for b in range(self.batch))

    @property
    def token_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lens)]).astype(np.int64)

    @property
    def page_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum([self.pages(b) for b in range(self.batch)])]).astype(np.int64)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lens))

    def row_seq(self) -> np.ndarray:
        if self.kind == "decode":
            return np.arange(self.batch, dtype=np.int32)
        return np.zeros(self.rows, dtype=np.int32)

    def row_pos(self) -> np.ndarray:
        if self.kind == "decode":
            return np.array([L - 1 for L in self.lens], dtype=np.int32)
        return self.q_pos.astype(np.int32)

    # ---- page placement ------------------------------------------------
    def page_perm(self) -> np.ndarray:
        """Physical page id of logical page p (pages of all sequences in order)."""
        if self._perm is None:
            n = self.num_pages
            if not self.paged_random:
                self._perm = np.arange(n, dtype=np.int64)
            else:
                r = raw_u64(self.seed, T_PERM, (n,))
                perm = np.arange(n, dtype=np.int64)
                for i in range(n - 1, 0, -1):
                    j = int(r[n - 1 - i] % np.uint64(i + 1))
                    perm[i], perm[j] = perm[j], perm[i]
                self._perm = perm
        return self._perm

    def block_table(self) -> np.ndarray:
        bt = np.full((self.batch, self.max_pages), -1, dtype=np.int32)
        perm = self.page_perm()
        po = self.page_offsets
        for b in range(self.batch):
            bt[b, : self.pages(b)] = perm[po[b]: po[b + 1]]
        return bt

    # ---- inputs ----------------------------------------------------------
    def keys_logical(self, b: Optional[int] = None) -> np.ndarray:
        """bf16 bits, [L_b,128] for one sequence or [sum L,128] for all."""
        if b is None:
            return normal_bf16(self.seed, T_KEYS, (self.total_tokens, IDX_DIM))
        t0 = int(self.token_offsets[b])
        return normal_bf16(self.seed, T_KEYS, (self.lens[b], IDX_DIM), start=t0 * IDX_DIM)

    def latent_logical(self, b: Optional[int] = None, t0: int = 0, n: Optional[int] = None) -> np.ndarray:
        """bf16 bits of latent rows: all sequences, or rows [t0, t0+n) of sequence b."""
        if b is None:
            return normal_bf16(self.seed, T_LATENT, (self.total_tokens, LAT_DIM))
        n = self.lens[b] - t0 if n is None else n
        start = (int(self.token_offsets[b]) + t0) * LAT_DIM
        return normal_bf16(self.seed, T_LATENT, (n, LAT_DIM), start=start)

    def pool_weights(self) -> np.ndarray:
        logits = normal_f64(self.seed, T_POOLW, (GROUP,))
        e = np.exp(logits - logits.max())
        return (e / e.sum()).astype(np.float32)

    def q_idx(self, r0: int = 0, n: Optional[int] = None) -> np.ndarray:
        n = self.rows - r0 if n is None else n
        return uniform_i8(self.seed, T_QIDX, (n, IDX_HEADS, IDX_DIM), -127, 127,
                          start=r0 * IDX_HEADS * IDX_DIM)

    def head_w(self, r0: int = 0, n: Optional[int] = None) -> np.ndarray:
        n = self.rows - r0 if n is None else n
        return uniform_i8(self.seed, T_HEADW, (n, IDX_HEADS), 0, 64, start=r0 * IDX_HEADS)

    def q_attn(self, r0: int = 0, n: Optional[int] = None, layer: int = 0) -> np.ndarray:
        n = self.rows - r0 if n is None else n
        tid = T_QATT if layer == 0 else T_QATT_LAYER + layer
        return normal_bf16(self.seed, tid, (n, ATT_HEADS, LAT_DIM), start=r0 * ATT_HEADS * LAT_DIM)

    # ---- paged pools built from logical arrays (host side plumbing) --------
    def scatter_pages(self, logical: np.ndarray, per_page_rows: int, pad_value) -> np.ndarray:
        """Place logical rows [sum L, D] into a page pool [num_pages, per_page_rows, D]."""
        D = logical.shape[1]
        pool = np.full((self.num_pages, per_page_rows, D), pad_value, dtype=logical.dtype)
        perm = self.page_perm()
        po = self.page_offsets
        to = self.token_offsets
        for b in range(self.batch):
            L = self.lens[b]
            for j in range(self.pages(b)):
                a = j * per_page_rows
                e = min(L, a + per_page_rows)
                pool[perm[po[b] + j], : e - a] = logical[to[b] + a: to[b] + e]
        return pool

    def is_identity_dense(self) -> bool:
        return (not self.paged_random) and all(L % PAGE_TOKENS == 0 for L in self.lens)


def _loguniform_lens(seed: int, n: int) -> List[int]:
    u = uniform_f64(seed, T_LENS, (n,))
    return [int(math.floor(512.0 * 2.0 ** (11.0 * float(x)))) for x in u]


def workload(i: int) -> Workload:
    if i == 0:
        return Workload(0, "decode_b1_L8192", 0, "decode", [8192],
                        description="single decode query, L=8192")
    if i == 1:
        return Workload(1, "decode_b64_L131072", 1, "decode", [131072] * 64,
                        description="decode batch 64 x 131,072 tokens")
    if i == 2:
        return Workload(2, "decode_b8_L1048576", 2, "decode", [1 << 20] * 8,
                        description="decode batch 8 x 1,048,576 tokens")
    if i == 3:
        return Workload(3, "prefill_q2048_L1048576", 3, "prefill", [1 << 20],
                        q_pos=np.arange(1046528, 1048576, dtype=np.int64),
                        description="prefill chunk of 2048 queries at the end of a 1,048,576-token sequence")
    if i == 4:
        return Workload(4, "ragged_paged_b32", 4, "decode", _loguniform_lens(4, 32), paged_random=True,
                        description="ragged paged decode batch of 32, L log-uniform on [512, 2^20)")
    raise ValueError(i)


def custom(name: str, seed: int, lens, kind: str = "decode", q_pos=None, paged_random: bool = False) -> Workload:
    """A small workload with the same dims, for tests (ragged tails, dense fallback, ...)."""
    return Workload(-1, name, seed, kind, [int(x) for x in lens], paged_random=paged_random,
                    q_pos=None if q_pos is None else np.asarray(q_pos, dtype=np.int64))
