"""Seeded synthetic inputs for the drafter step (shared by the oracle side and the GPU side).

This module holds no arithmetic of the method itself: it only draws the inputs (weights, target activations, the
shared K=V cache, rotary tables, token ids) that both the CPU oracle and the HIP path consume.

Random values come from a counter-based generator so that any element, or any subset of rows, can be regenerated
bit-identically on the CPU (for the oracle) and on the GPU (for the large tables that would take too long to build on
the host): element i of tensor t under seed s is a pure function of (s, t, i) built from 32-bit integer hashing
(Chris Wellons' "lowbias32" mixer) and exactly-rounded fp32 arithmetic only, so CPU and GPU give the same bits.

The value distribution approximates N(0, 1) by the Irwin-Hall sum of four independent 16-bit uniforms (mean 0,
variance 1, tails bounded at about 3.46 sigma). Values are scaled in fp32 and rounded to bf16 with
round-to-nearest-even on the fp32 bit pattern.

Workloads (shapes from the pages' variant descriptions, sizes as stated per workload):
  * E2B-shaped drafter (backbone 1536), E4B-shaped drafter (backbone 2560): hidden 256, 4 layers (3 sliding, 1 full),
    4 query heads of 256, one shared K=V head, GeGLU FFN 1024, vocab 262144, 2048 centroids, top 32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

# ----------------------------------------------------------------------------------------------------------------
# configuration


@dataclasses.dataclass(frozen=True)
class DrafterShape:
    backbone: int = 1536
    hidden: int = 256
    n_layer: int = 4
    n_head: int = 4
    n_kv_head: int = 1
    head_dim: int = 256
    ffn: int = 1024
    vocab: int = 262144
    n_centroids: int = 2048
    top_k: int = 32
    swa_window: int = 512
    full_attn_layers: int = 0b1000  # bit l set => layer l reads the full-attention cache
    rms_eps: float = 1e-6
    attn_scale: float = 1.0 / 16.0
    embed_scale: float = 1.0
    rope_theta_sliding: float = 1.0e4
    rope_theta_full: float = 1.0e6

    @property
    def vsc(self) -> int:
        """Tokens per cluster of the masked head (0 for the dense tied head, n_centroids == 0)."""
        return self.vocab // self.n_centroids if self.n_centroids else 0

    @property
    def dense_head(self) -> bool:
        return self.n_centroids == 0

    @property
    def q_dim(self) -> int:
        return self.n_head * self.head_dim

    def is_full(self, layer: int) -> bool:
        return bool((self.full_attn_layers >> layer) & 1)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: DrafterShape
    batch: int
    context: int  # keys in each sequence's shared cache (both types)
    n_steps: int  # draft_block length
    ragged: bool = False  # per-row lengths context - 37*b instead of all equal
    seed: int = 0
    shared_kv: bool = False  # one cache per type read by every row (rows of one sequence), else one per row

    def lens(self) -> List[int]:
        if self.ragged:
            return [max(1, self.context - 37 * b) for b in range(self.batch)]
        return [self.context] * self.batch


E2B = DrafterShape(backbone=1536)
E4B = DrafterShape(backbone=2560)
# 26B-A4B-shaped drafter with the dense tied head (no centroids): backbone 2816, hidden 1024, 8 query heads of 256
# over one shared K=V head, FFN 4096, sliding window 1024
E26B = DrafterShape(backbone=2816, hidden=1024, n_head=8, n_kv_head=1, head_dim=256, ffn=4096, n_centroids=0, top_k=1,
                    swa_window=1024)

WORKLOADS: Dict[str, Workload] = {
    # E2B-shaped drafter, one step, batch 1, shared KV context 256
    "e2b_b1_ctx256_step1": Workload("e2b_b1_ctx256_step1", E2B, batch=1, context=256, n_steps=1),
    # E2B-shaped drafter, draft_block of 4 at a constant position, batch 1, context 4096
    "e2b_b1_ctx4096_block4": Workload("e2b_b1_ctx4096_block4", E2B, batch=1, context=4096, n_steps=4),
    # E4B-shaped drafter, batch 16 independent sequences, context 8192 each, draft_block 4
    "e4b_b16_ctx8192_block4": Workload("e4b_b16_ctx8192_block4", E4B, batch=16, context=8192, n_steps=4),
    # the same with two KV heads (two query heads per kv head): twice the cache bytes
    "e4b_nkv2_b16_ctx8192_block4": Workload("e4b_nkv2_b16_ctx8192_block4", dataclasses.replace(E4B, n_kv_head=2),
                                            batch=16, context=8192, n_steps=4),
    # 26B-A4B-shaped drafter with the dense head, batch 32, context 32768 each, draft_block 4
    "e26b_b32_ctx32768_block4": Workload("e26b_b32_ctx32768_block4", E26B, batch=32, context=32768, n_steps=4),
    # verify width: 256 query rows of one sequence sharing one cache of 131072 keys (window 1024), one drafter step
    "e4b_verify256_ctx131072": Workload("e4b_verify256_ctx131072", dataclasses.replace(E4B, swa_window=1024),
                                        batch=256, context=131072, n_steps=1, shared_kv=True),
}

# small shapes for fast CPU checks and multi-tile / ragged GPU parity cases
TINY = DrafterShape(backbone=64, hidden=32, n_layer=4, n_head=4, n_kv_head=1, head_dim=64, ffn=64, vocab=1024,
                    n_centroids=8, top_k=2, swa_window=16)
TINY_DENSE = dataclasses.replace(TINY, n_centroids=0, top_k=1)

# ----------------------------------------------------------------------------------------------------------------
# counter-based generator

_M32 = 0xFFFFFFFF
IH4_MEAN = 4 * 32767.5  # Irwin-Hall(4) mean of four uniforms on {0..65535}
IH4_SD = math.sqrt(4 * (65536.0 ** 2 - 1.0) / 12.0)

# tensor ids: one stream per tensor; per-layer tensors use 100 + 16*layer + k
TID = {
    "pre_proj": 1, "post_proj": 2, "output_norm": 3, "token_embd": 4, "centroids": 5, "ordering": 6,
    "target_embd": 7, "target_hidden": 8, "last_token": 9, "kv_sliding": 10, "kv_full": 11, "v_sliding": 12,
    "v_full": 13, "h_probe": 14,
}
LAYER_TID = {"attn_q": 0, "attn_q_norm": 1, "attn_output": 2, "attn_norm": 3, "post_attention_norm": 4,
             "ffn_norm": 5, "post_ffw_norm": 6, "ffn_gate": 7, "ffn_up": 8, "ffn_down": 9, "layer_output_scale": 10}


def layer_tid(layer: int, name: str) -> int:
    return 100 + 16 * layer + LAYER_TID[name]


def _mul32(x: torch.Tensor, m: int) -> torch.Tensor:
    """(x * m) mod 2^32 for int64 x in [0, 2^32), without int64 overflow."""
    lo, hi = m & 0xFFFF, m >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _M32


def hash32(x: torch.Tensor) -> torch.Tensor:
    """lowbias32 integer mixer on int64 tensors holding values in [0, 2^32)."""
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _key(seed: int, tid: int) -> int:
    k = torch.tensor([(seed * 0x9E3779B1 + tid * 0x85EBCA77 + 0x165667B1) & _M32], dtype=torch.int64)
    return int(hash32(hash32(k))[0])


def std_normal_f32(seed: int, tid: int, idx: torch.Tensor) -> torch.Tensor:
    """Approximately N(0,1) fp32 values for int64 element indices `idx` (any device)."""
    key = _key(seed, tid)
    h1 = hash32((idx & _M32) ^ key)
    h2 = hash32(h1 ^ 0x68E31DA4)
    s = (h1 & 0xFFFF) + (h1 >> 16) + (h2 & 0xFFFF) + (h2 >> 16)
    # 2*(s - mean) is an exact integer (|.| < 2^24), scaled by 1/(2*sd) with one exactly-rounded fp32 multiply
    z = (s * 2 - int(2 * IH4_MEAN)).to(torch.float32)
    return z * torch.tensor(1.0 / (2.0 * IH4_SD), dtype=torch.float32, device=idx.device)


def uniform_u32(seed: int, tid: int, idx: torch.Tensor) -> torch.Tensor:
    return hash32((idx & _M32) ^ _key(seed, tid))


def f32_to_bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 bit pattern (int16 tensor), round to nearest even, via integer ops (inputs are finite)."""
    b = x.contiguous().view(torch.int32).to(torch.int64) & _M32
    r = ((b >> 16) & 1) + 0x7FFF
    out = ((b + r) >> 16) & 0xFFFF
    return (out - ((out >> 15) << 16)).to(torch.int16)  # reinterpret the low 16 bits as signed


def gen_bf16(seed: int, tid: int, shape, std: float, mean: float = 0.0, device="cpu", chunk: int = 1 << 24,
             row_index: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 bit patterns (int16) of N(mean, std^2)-like values.

    With `row_index` (int64 tensor of rows of a 2-D `shape`), only those rows are produced, identical to the same rows
    of the full tensor.
    """
    shape = tuple(int(s) for s in shape)
    std_t = torch.tensor(std, dtype=torch.float32, device=device)
    mean_t = torch.tensor(mean, dtype=torch.float32, device=device)
    if row_index is not None:
        assert len(shape) == 2
        ncol = shape[1]
        rows = row_index.to(device=device, dtype=torch.int64)
        idx = rows[:, None] * ncol + torch.arange(ncol, device=device, dtype=torch.int64)[None, :]
        v = std_normal_f32(seed, tid, idx.reshape(-1)) * std_t
        if mean != 0.0:
            v = v + mean_t
        return f32_to_bf16_bits(v).reshape(len(rows), ncol)
    n = 1
    for s in shape:
        n *= s
    out = torch.empty(n, dtype=torch.int16, device=device)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        idx = torch.arange(a, b, device=device, dtype=torch.int64)
        v = std_normal_f32(seed, tid, idx) * std_t
        if mean != 0.0:
            v = v + mean_t
        out[a:b] = f32_to_bf16_bits(v)
    return out.reshape(shape)


def permutation(seed: int, tid: int, n: int) -> torch.Tensor:
    """Random permutation of range(n) (int32, CPU): argsort of unique hashed keys."""
    idx = torch.arange(n, dtype=torch.int64)
    keys = (uniform_u32(seed, tid, idx) << 20) | idx  # n <= 2^20: unique keys
    assert n <= (1 << 20)
    return torch.argsort(keys).to(torch.int32)


def rope_tables(shape: DrafterShape, positions: List[int]) -> np.ndarray:
    """cos/sin tables [B][2 types][2][head_dim/2] fp32 for each row's constant position (type 0 sliding, 1 full).

    Half-split rotary frequencies inv_freq_i = theta^(-2i/head_dim), angle = pos * inv_freq_i, computed in fp64.
    """
    half = shape.head_dim // 2
    out = np.zeros((len(positions), 2, 2, half), dtype=np.float32)
    i = np.arange(half, dtype=np.float64)
    for t, theta in enumerate((shape.rope_theta_sliding, shape.rope_theta_full)):
        inv = theta ** (-2.0 * i / shape.head_dim)
        for b, p in enumerate(positions):
            ang = float(p) * inv
            out[b, t, 0] = np.cos(ang).astype(np.float32)
            out[b, t, 1] = np.sin(ang).astype(np.float32)
    return out


# ----------------------------------------------------------------------------------------------------------------
# weights and inputs


def make_weights(shape: DrafterShape, seed: int = 0, device="cpu") -> Dict[str, object]:
    """All drafter weights as bf16 bit tensors ([out][in] row-major) + int32 ordering + float layer scales."""
    H, Bb, F, Q = shape.hidden, shape.backbone, shape.ffn, shape.q_dim
    w: Dict[str, object] = {
        "pre_proj": gen_bf16(seed, TID["pre_proj"], (H, 2 * Bb), 1.0 / math.sqrt(2 * Bb), device=device),
        "post_proj": gen_bf16(seed, TID["post_proj"], (Bb, H), 1.0 / math.sqrt(H), device=device),
        "output_norm": gen_bf16(seed, TID["output_norm"], (H,), 0.1, 1.0, device=device),
        "token_embd": gen_bf16(seed, TID["token_embd"], (shape.vocab, H), 0.02, device=device),
    }
    if not shape.dense_head:
        w["centroids"] = gen_bf16(seed, TID["centroids"], (shape.n_centroids, H), 1.0 / math.sqrt(H), device=device)
        w["token_ordering"] = permutation(seed, TID["ordering"], shape.vocab).to(device)
    layers = []
    for l in range(shape.n_layer):
        t = lambda n: layer_tid(l, n)  # noqa: E731
        lw = {
            "attn_q": gen_bf16(seed, t("attn_q"), (Q, H), 1.0 / math.sqrt(H), device=device),
            "attn_q_norm": gen_bf16(seed, t("attn_q_norm"), (shape.head_dim,), 0.1, 1.0, device=device),
            "attn_output": gen_bf16(seed, t("attn_output"), (H, Q), 1.0 / math.sqrt(Q), device=device),
            "attn_norm": gen_bf16(seed, t("attn_norm"), (H,), 0.1, 1.0, device=device),
            "post_attention_norm": gen_bf16(seed, t("post_attention_norm"), (H,), 0.1, 1.0, device=device),
            "ffn_norm": gen_bf16(seed, t("ffn_norm"), (H,), 0.1, 1.0, device=device),
            "post_ffw_norm": gen_bf16(seed, t("post_ffw_norm"), (H,), 0.1, 1.0, device=device),
            "ffn_gate": gen_bf16(seed, t("ffn_gate"), (F, H), 1.0 / math.sqrt(H), device=device),
            "ffn_up": gen_bf16(seed, t("ffn_up"), (F, H), 1.0 / math.sqrt(H), device=device),
            "ffn_down": gen_bf16(seed, t("ffn_down"), (H, F), 1.0 / math.sqrt(F), device=device),
        }
        s = std_normal_f32(seed, t("layer_output_scale"), torch.zeros(1, dtype=torch.int64))
        lw["layer_output_scale"] = float(np.float32(1.0) + np.float32(0.1) * np.float32(float(s[0])))
        layers.append(lw)
    w["layers"] = layers
    return w


def make_inputs(wl: Workload, device="cpu", with_target_embd: bool = True, distinct_v: bool = False) -> Dict[str, object]:
    """Per-call inputs: target hidden [B][Bb], last token [B], shared K(=V) caches [B][n_kv][cap][hd] per type,
    lengths, rope tables, and (optionally, full size) the target's input embedding table [V][Bb]."""
    sh, B = wl.shape, wl.batch
    KB = 1 if wl.shared_kv else B  # cache rows
    cap = wl.context
    lens = wl.lens()
    d: Dict[str, object] = {
        "target_hidden": gen_bf16(wl.seed, TID["target_hidden"], (B, sh.backbone), 1.0, device=device),
        "last_token": (uniform_u32(wl.seed, TID["last_token"], torch.arange(B, dtype=torch.int64)) % sh.vocab)
        .to(torch.int32).to(device),
        "k_sliding": gen_bf16(wl.seed, TID["kv_sliding"], (KB, sh.n_kv_head, cap, sh.head_dim), 1.0, device=device),
        "k_full": gen_bf16(wl.seed, TID["kv_full"], (KB, sh.n_kv_head, cap, sh.head_dim), 1.0, device=device),
        "len_sliding": list(lens),
        "len_full": list(lens),
        "positions": list(lens),
    }
    if distinct_v:
        d["v_sliding"] = gen_bf16(wl.seed, TID["v_sliding"], (KB, sh.n_kv_head, cap, sh.head_dim), 1.0, device=device)
        d["v_full"] = gen_bf16(wl.seed, TID["v_full"], (KB, sh.n_kv_head, cap, sh.head_dim), 1.0, device=device)
    d["rope"] = torch.from_numpy(rope_tables(sh, d["positions"])).to(device)
    if with_target_embd:
        d["target_embd"] = gen_bf16(wl.seed, TID["target_embd"], (sh.vocab, sh.backbone), 1.0, device=device)
    return d


class LazyRows:
    """Row provider for the target's input embedding table [V][Bb] that generates only requested rows (CPU)."""

    def __init__(self, seed: int, shape: DrafterShape):
        self.seed, self.shape = seed, shape
        self._cache: Dict[int, np.ndarray] = {}

    def __getitem__(self, row: int) -> np.ndarray:
        row = int(row)
        if row not in self._cache:
            t = gen_bf16(self.seed, TID["target_embd"], (self.shape.vocab, self.shape.backbone), 1.0,
                         row_index=torch.tensor([row], dtype=torch.int64))
            self._cache[row] = t[0].numpy().view(np.uint16)
        return self._cache[row]


def to_numpy_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint16)
