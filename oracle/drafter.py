"""CPU oracle of the Gemma 4 assistant (MTP drafter) draft step.

TEST INFRASTRUCTURE ONLY. This module is the slow, plain, obviously-correct definition that the HIP path is checked
against. Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may import it; the product
path never calls it and shares no code with it (it uses NumPy only: no torch, no ctypes, nothing from the package).

Arithmetic: IEEE fp64 everywhere. The only quantisation inside a step is the one the interface fixes: the
post-projected hidden state handed back to the caller (and fed to the next drafted step) is bf16 like every other
stored activation of the target (fp64 -> fp32 round-to-nearest -> bf16 round-to-nearest-even). Stored inputs are bf16
(weights, embeddings, K/V, target hidden), the token ordering int32, the rotary tables fp32. Integer decisions
(top-k of the centroid scores, argmax of the logits row) are taken on fp32 values, the precision the GPU takes them in.

Pages cited (by title; sections as headed on each page):
  [MTP doc]    "Gemma 4 Multi-Token Prediction (MTP) drafter" (llama.cpp fork, gemma4-assistant.md)
  [Inventory]  "Gemma 4 Assistant (MTP drafter) - tensor inventory (Stage 0)"
  [Guide]      "Gemma 4 Assistant 使用指南：用 MTP 投机解码与 KV Sharing 加速 Gemma 4 推理" (gitcode blog)
  [Explained]  "Gemma 4 drafter explained" (techtwitter)

Readings where the pages are silent or disagree (each also listed in the design notes):
  * concat order: target hidden first, token embedding second ([MTP doc] "What it is": "2x backbone input");
  * SWA key set under the flipped mask at one query: the last min(window, len) keys; full attention: all len keys;
  * GQA: query head h reads kv head floor(h * n_kv / n_head);
  * RMSNorm(v, w) = v / sqrt(mean(v^2) + eps) * w (weight used as stored);
  * GeGLU = gelu_tanh(gate) * up; layer_scalar multiplies the residual stream after the FFN residual add;
  * rotary: half-split pairs (i, i + d/2) with per-row fp32 cos/sin tables for the constant position;
  * top-k order: descending fp32 score, ties to the lower centroid index; argmax ties to the lowest token id;
  * mask value: fp32(-1e30) ([Inventory] "Centroid / ordered embeddings LM head", step 5);
  * precision: the configurations state bf16 weights with fp32 accumulation and nothing about rounding activations,
    so activations stay unrounded (fp64 here, fp32 on the GPU) and only stored tensors are bf16;
  * sampling at temperature T > 0: p = softmax(row / T) over the scored tokens (the -1e30 entries have p = 0),
    drawn by inverse CDF with a caller-supplied uniform u in [0, 1), the CDF running in the head table's row order
    (masked head: selected clusters by ascending index, each cluster's ids in ordering order; dense head: token
    order), so that the draw does not depend on how near-equal centroid scores are ranked.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

NEG_FILL_F32 = np.float32(-1e30)  # [Inventory] "Centroid / ordered embeddings LM head", step 5: -1e30f fill


# ----------------------------------------------------------------------------------------------------------------
# number formats


def bf16_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16 / int16 array) to fp64: a bf16 is the high half of an fp32."""
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_bits(x) -> np.ndarray:
    """fp64 -> fp32 (round to nearest) -> bf16 bit pattern (round to nearest, ties to even), as uint16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


def round_bf16(x) -> np.ndarray:
    """Value of x after rounding to bf16 (fp64 -> fp32 -> bf16), returned as fp64."""
    return bf16_to_f64(bf16_bits(x))


# ----------------------------------------------------------------------------------------------------------------
# elementary operations


def rmsnorm(v: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMS normalisation over the last axis, scaled by the stored weight (sandwich norms, q_norm and output norm of
    the [MTP doc] "Tensor schema": attn_norm, post_attention_norm, ffn_norm, post_ffw_norm, attn_q_norm, output_norm)."""
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * w


def gelu_tanh(a: np.ndarray) -> np.ndarray:
    """Tanh-approximated GELU: 0.5 a (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3)))."""
    a = np.asarray(a, dtype=np.float64)
    return 0.5 * a * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (a + 0.044715 * a ** 3)))


def rope_rotate(q: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate the pairs (q[i], q[i + d/2]) by the angle whose cos/sin are given for pair i."""
    d2 = q.shape[-1] // 2
    a, b = q[..., :d2], q[..., d2:]
    c, s = np.asarray(cos, np.float64), np.asarray(sin, np.float64)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def key_window(length: int, window: int, full: bool):
    """Keys one query attends to in the shared cache, as [start, stop).

    [Guide] section 2(4): with a single query the full-attention mask is the same as a bidirectional one, so a
    full-attention layer reads every valid key; the sliding mask is flipped from the future to the past, so a
    sliding layer reads the most recent `window` keys.
    """
    if full:
        return 0, length
    return length - min(window, length), length


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Single-query attention: softmax(scale * K q) weighted sum of the rows of V (explicit softmax, fp64)."""
    s = scale * (K @ q)
    p = np.exp(s - np.max(s))
    p = p / np.sum(p)
    return p @ V


def topk_desc(scores32: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest fp32 scores in descending order, ties to the lower index (k rounds of selection:
    take the first maximum, remove it)."""
    s = np.asarray(scores32, dtype=np.float32).astype(np.float64).copy()
    out = np.empty(k, dtype=np.int64)
    for j in range(k):
        i = int(np.argmax(s))  # first occurrence: lowest index among equal maxima
        out[j] = i
        s[i] = -np.inf
    return out


# ----------------------------------------------------------------------------------------------------------------
# model description


@dataclasses.dataclass
class Config:
    backbone: int
    hidden: int
    n_layer: int
    n_head: int
    n_kv_head: int
    head_dim: int
    ffn: int
    vocab: int
    n_centroids: int
    top_k: int
    swa_window: int
    full_attn_layers: int
    rms_eps: float = 1e-6
    attn_scale: float = 1.0 / 16.0
    embed_scale: float = 1.0

    @property
    def vsc(self) -> int:
        """Tokens per cluster of the masked head; 0 for the dense tied head (n_centroids == 0)."""
        return self.vocab // self.n_centroids if self.n_centroids else 0

    @property
    def dense(self) -> bool:
        return self.n_centroids == 0

    def is_full(self, l: int) -> bool:
        return bool((self.full_attn_layers >> l) & 1)


def config_from(shape) -> Config:
    names = [f.name for f in dataclasses.fields(Config)]
    return Config(**{n: getattr(shape, n) for n in names})


def check_head_invariants(cfg: Config, ordering: np.ndarray) -> None:
    """Structural checks the [Inventory] "GGUF / converter layout" verification names: n_vocab divisible by
    n_centroids, an I32 ordering of length n_vocab; plus: every token listed exactly once, and values below 2^18 so
    the F32 storage of [MTP doc] "Tensor schema" is lossless."""
    o = np.asarray(ordering)
    if cfg.vocab % cfg.n_centroids != 0:
        raise ValueError("n_vocab % n_centroids != 0")
    if not (0 < cfg.top_k <= cfg.n_centroids):
        raise ValueError("top_k out of range")
    if o.shape != (cfg.vocab,):
        raise ValueError("token_ordering length != n_vocab")
    if o.min() < 0 or o.max() >= cfg.vocab or np.any(np.bincount(o, minlength=cfg.vocab) != 1):
        raise ValueError("token_ordering is not a permutation of the vocabulary")


class Model:
    """Drafter weights decoded to fp64 once (the head table stays bf16 and is decoded per gathered row)."""

    def __init__(self, cfg: Config, w: Dict[str, object]):
        self.cfg = cfg
        d = lambda t: bf16_to_f64(_np16(t))  # noqa: E731
        self.pre = d(w["pre_proj"]).reshape(cfg.hidden, 2 * cfg.backbone)
        self.post = d(w["post_proj"]).reshape(cfg.backbone, cfg.hidden)
        self.out_norm = d(w["output_norm"])
        self.head_bits = _np16(w["token_embd"]).reshape(cfg.vocab, cfg.hidden)
        if cfg.dense:  # dense tied head: every token scored, no centroids or ordering
            self.cen = None
            self.ordering = None
        else:
            self.cen = d(w["centroids"]).reshape(cfg.n_centroids, cfg.hidden)
            self.ordering = np.asarray(_np32(w["token_ordering"]), dtype=np.int64)
            check_head_invariants(cfg, self.ordering)
        self.layers = []
        for lw in w["layers"]:
            self.layers.append({
                "q": d(lw["attn_q"]).reshape(cfg.n_head * cfg.head_dim, cfg.hidden),
                "q_norm": d(lw["attn_q_norm"]),
                "o": d(lw["attn_output"]).reshape(cfg.hidden, cfg.n_head * cfg.head_dim),
                "attn_norm": d(lw["attn_norm"]),
                "post_attn_norm": d(lw["post_attention_norm"]),
                "ffn_norm": d(lw["ffn_norm"]),
                "post_ffw_norm": d(lw["post_ffw_norm"]),
                "gate": d(lw["ffn_gate"]).reshape(cfg.ffn, cfg.hidden),
                "up": d(lw["ffn_up"]).reshape(cfg.ffn, cfg.hidden),
                "down": d(lw["ffn_down"]).reshape(cfg.hidden, cfg.ffn),
                "scale": float(np.float32(lw["layer_output_scale"])),
            })


def _np16(t) -> np.ndarray:
    if hasattr(t, "detach"):
        t = t.detach().cpu().contiguous().numpy()
    return np.asarray(t).view(np.uint16)


def _np32(t) -> np.ndarray:
    if hasattr(t, "detach"):
        t = t.detach().cpu().contiguous().numpy()
    return np.asarray(t)


@dataclasses.dataclass
class SharedKV:
    """The target's last-layer caches per attention type ([MTP doc] "Runtime implementation", piece 1;
    [Guide] section 2(4): shared_kv_states {full_attention, sliding_attention} -> (key, value)).

    k[t], v[t]: [B][n_kv][cap][head_dim] bf16 bits (v may be the same array as k: K = V);
    lens[t]: valid keys per row; rope: [B][2 types][2 (cos, sin)][head_dim/2] fp32. Type index 0 = sliding, 1 = full.
    shared[t] (optional, default False): one cache [1][n_kv][cap][head_dim] read by every row (rows of one sequence
    scored together, each with its own length and position).
    first[t] (optional, default 0): slot of each row's oldest valid key. Row b's valid keys, oldest first, are slots
    (first + i) mod cap for i < len: a left-padded batch ([Guide] section 2 "create_attention_masks" and
    padding_side="left") starts at its padding width, a ring-buffer cache at its oldest slot.
    """
    k: Sequence[np.ndarray]
    v: Sequence[np.ndarray]
    lens: Sequence[Sequence[int]]
    rope: np.ndarray
    first: Optional[Sequence[Sequence[int]]] = None
    shared: Optional[Sequence[bool]] = None

    def row(self, t: int, b: int) -> int:
        """Cache row that batch row b reads."""
        return 0 if (self.shared is not None and self.shared[t]) else b

    def slots(self, t: int, b: int, a0: int, a1: int) -> np.ndarray:
        """Cache slots of the row's valid keys a0 .. a1 - 1 (oldest first)."""
        cap = self.k[t].shape[2]
        f = 0 if self.first is None else int(self.first[t][b])
        if not (0 <= f < cap and 0 <= a0 <= a1 <= int(self.lens[t][b]) <= cap):
            raise ValueError("cache window outside the cache")
        return (f + np.arange(a0, a1)) % cap


# ----------------------------------------------------------------------------------------------------------------
# the step


def decoder_layer(m: Model, l: int, x: np.ndarray, b: int, kv: SharedKV) -> np.ndarray:
    """One Q-only decoder layer on the residual stream x (fp64 [hidden]) of row b.

    [MTP doc] "What it is" (Q-only attention over the target's last-layer K/V of the matching type; per-layer
    scalar); "Tensor schema" (q, q_norm, output, the four sandwich norms, gate/up/down, layer_output_scale);
    [Inventory] "Notes for llama.cpp port" 2 (V taken from K); [Guide] section 2(2) (constant position).
    """
    cfg, L = m.cfg, m.layers[l]
    t = 1 if cfg.is_full(l) else 0
    r = x
    u = rmsnorm(x, L["attn_norm"], cfg.rms_eps)
    q = (L["q"] @ u).reshape(cfg.n_head, cfg.head_dim)
    cos, sin = kv.rope[b, t, 0], kv.rope[b, t, 1]
    length = int(kv.lens[t][b])
    a0, a1 = key_window(length, cfg.swa_window, t == 1)
    o = np.empty((cfg.n_head, cfg.head_dim))
    for h in range(cfg.n_head):
        g = h * cfg.n_kv_head // cfg.n_head
        qh = rope_rotate(rmsnorm(q[h], L["q_norm"], cfg.rms_eps), cos, sin)
        sl = kv.slots(t, b, a0, a1)
        cb = kv.row(t, b)
        K = bf16_to_f64(kv.k[t][cb, g, sl])
        V = K if kv.v[t] is kv.k[t] else bf16_to_f64(kv.v[t][cb, g, sl])
        o[h] = attend(qh, K, V, cfg.attn_scale)
    x = r + rmsnorm(L["o"] @ o.reshape(-1), L["post_attn_norm"], cfg.rms_eps)
    r = x
    u = rmsnorm(x, L["ffn_norm"], cfg.rms_eps)
    mm = gelu_tanh(L["gate"] @ u) * (L["up"] @ u)
    x = (r + rmsnorm(L["down"] @ mm, L["post_ffw_norm"], cfg.rms_eps)) * L["scale"]
    return x


def masked_head_row(m: Model, h: np.ndarray, want_row: bool = False) -> Dict[str, object]:
    """Centroid-clustered masked LM head for one normed hidden state h [hidden].

    [Inventory] "Centroid / ordered embeddings LM head": centroid logits = centroids . h; top_k of them; the
    ordering viewed as [n_centroids][vsc] lists each centroid's vsc token ids; those rows of the token embedding
    table dotted with h give the sparse logits; the full row is -1e30 except at the selected ids.
    [Guide] section 5 (use_ordered_embeddings): the head computes logits only for top_k * (vocab / n_centroids)
    tokens. [Explained] "The Efficient Embedder".
    """
    cfg = m.cfg
    sc = m.cen @ h
    sc32 = sc.astype(np.float32)
    sel = topk_desc(sc32, cfg.top_k)
    ids = m.ordering.reshape(cfg.n_centroids, cfg.vsc)[sel].reshape(-1)
    z = bf16_to_f64(m.head_bits[ids]) @ h
    z32 = z.astype(np.float32)
    row = np.full(cfg.vocab, NEG_FILL_F32, dtype=np.float32)
    row[ids] = z32
    nxt = int(np.argmax(row))
    srt = np.sort(sc32.astype(np.float64))[::-1]
    zs = np.sort(z32.astype(np.float64))[::-1]
    out = {
        "scores": sc32, "sel": sel, "ids": ids, "z": z32, "next": nxt,
        "cgap": float(srt[cfg.top_k - 1] - srt[cfg.top_k]) if cfg.top_k < cfg.n_centroids else np.inf,
        "margin": float(zs[0] - zs[1]),
    }
    if want_row:
        out["row"] = row
    return out


def dense_head_row(m: Model, h: np.ndarray, chunk: int = 16384) -> np.ndarray:
    """Dense tied head: logits over the whole vocabulary, token_embd . h for every token (the
    use_ordered_embeddings=false form: [Guide] section 5; [MTP doc] "Variants supported": the large drafters tie
    the full embedding as their head). Decoded in row chunks to bound host memory."""
    out = np.empty(m.cfg.vocab, dtype=np.float32)
    for a in range(0, m.cfg.vocab, chunk):
        out[a:a + chunk] = (bf16_to_f64(m.head_bits[a:a + chunk]) @ h).astype(np.float32)
    return out


def dense_head_result(m: Model, h: np.ndarray) -> Dict[str, object]:
    """The dense head's outputs in the form of masked_head_row's: the full fp32 row, its argmax (first occurrence:
    lowest token id on ties) and the top-1 minus top-2 margin."""
    row = dense_head_row(m, h)
    nxt = int(np.argmax(row))
    top2 = np.partition(row.astype(np.float64), -2)[-2:]
    return {"scores": None, "sel": [], "ids": [], "z": [], "next": nxt, "cgap": np.inf,
            "margin": float(top2[1] - top2[0]), "row": row}


def head_order(m: Model, sel: Optional[np.ndarray]) -> np.ndarray:
    """The scored tokens in the head table's row order: for the masked head the selected clusters by ascending
    cluster index, each cluster's vsc ids as the ordering lists them ([Inventory] "Centroid / ordered embeddings LM
    head", step 3); for the dense head every token in id order."""
    if m.cfg.dense:
        return np.arange(m.cfg.vocab, dtype=np.int64)
    return m.ordering.reshape(m.cfg.n_centroids, m.cfg.vsc)[np.sort(np.asarray(sel))].reshape(-1)


def sample_row(values: np.ndarray, order: np.ndarray, temperature: float, u: float) -> Dict[str, object]:
    """Draw one token from p = softmax(values / temperature) by inverse CDF at u in [0, 1).

    `values` are the fp32 logits of the tokens in `order` (the head table's row order). The token is the first one
    whose cumulative probability exceeds u (the last token with p > 0 if rounding leaves the total below u).
    Returns the token, its probability, and the distance from u to the nearer end of the token's CDF interval (how
    far u is from selecting a neighbour)."""
    z = np.asarray(values, dtype=np.float32).astype(np.float64)
    e = np.exp((z - np.max(z)) / temperature)
    p = e / np.sum(e)
    c = np.cumsum(p)
    above = np.nonzero(c > u)[0]
    j = int(above[0]) if above.size else int(np.nonzero(p > 0)[0][-1])
    lo = c[j] - p[j]
    return {"token": int(order[j]), "prob": float(p[j]), "cdf_margin": float(min(u - lo, c[j] - u))}


def drafter_step(m: Model, target_hidden, last_token, target_embd, kv: SharedKV, want_rows: bool = False,
                 rows: Optional[Sequence[int]] = None, temperature: Optional[float] = None,
                 uniforms: Optional[Sequence[float]] = None) -> Dict[str, object]:
    """One drafter forward for every batch row (or the listed `rows`).

    With a temperature > 0 the token is drawn by `sample_row` at uniforms[b] over the row's scored tokens instead of
    taken by argmax, and its draft probability is returned ("prob"), as stochastic acceptance needs.

    Input: [target_last_hidden ; embed(last_token)] with the token embedded by the target's input table
    ([MTP doc] "What it is": 2x backbone input; [Explained] "Target Activations": the input embedding table is
    shared with the target). pre_projection to hidden, the decoder layers, output norm, post_projection back to the
    backbone width (the next step's hidden input, [Guide] section 6: last_hidden_state is post-projected), and the
    masked head on the normed hidden state.
    """
    cfg = m.cfg
    th = _np16(target_hidden).reshape(-1, cfg.backbone)
    tok = np.asarray(_np32(last_token)).reshape(-1)
    B = th.shape[0]
    rows = list(range(B)) if rows is None else list(rows)
    res = {"hidden_out": np.zeros((len(rows), cfg.backbone), np.uint16), "next": np.zeros(len(rows), np.int64),
           "sel": [], "ids": [], "z": [], "scores": [], "cgap": [], "margin": [], "h": [], "rows": rows}
    if want_rows:
        res["row"] = []
    for i, b in enumerate(rows):
        e = cfg.embed_scale * bf16_to_f64(target_embd[int(tok[b])])
        x0 = np.concatenate([bf16_to_f64(th[b]), e])
        x = m.pre @ x0
        for l in range(cfg.n_layer):
            x = decoder_layer(m, l, x, b, kv)
        h = rmsnorm(x, m.out_norm, cfg.rms_eps)
        res["hidden_out"][i] = bf16_bits(m.post @ h)  # handed back in bf16, the target's activation format
        hd = dense_head_result(m, h) if cfg.dense else masked_head_row(m, h, want_row=want_rows or bool(temperature))
        if temperature:
            order = head_order(m, hd["sel"])
            smp = sample_row(hd["row"][order], order, temperature, float(uniforms[b]))
            hd["next"] = smp["token"]
            res.setdefault("prob", []).append(smp["prob"])
            res.setdefault("cdf_margin", []).append(smp["cdf_margin"])
        res["next"][i] = hd["next"]
        for k in ("sel", "ids", "z", "scores", "cgap", "margin"):
            res[k].append(hd[k])
        res["h"].append(h)
        if want_rows:
            res["row"].append(hd["row"])
    return res


def draft_block(m: Model, n: int, target_hidden, last_token, target_embd, kv: SharedKV,
                forced_tokens: Optional[np.ndarray] = None, rows: Optional[Sequence[int]] = None,
                temperature: Optional[float] = None, uniforms: Optional[np.ndarray] = None) -> List[Dict]:
    """n chained drafter steps at the constant position over the same shared cache.

    Step i+1 takes step i's post-projected hidden state and drafted token ([Explained] "Target Activations": the
    drafter's own projected activations replace the target's in later rounds; [Guide] section 2(3): within a draft
    round the last-seen token is the drafter's own). With `forced_tokens` [n][B], step i+1 is fed
    forced_tokens[i] instead of the oracle's own token (teacher forcing for parity across near-ties).
    """
    cfg = m.cfg
    th = _np16(target_hidden).reshape(-1, cfg.backbone).copy()
    tok = np.asarray(_np32(last_token)).reshape(-1).astype(np.int64).copy()
    B = th.shape[0]
    rows = list(range(B)) if rows is None else list(rows)
    out = []
    for i in range(n):
        r = drafter_step(m, th, tok, target_embd, kv, rows=rows, temperature=temperature,
                         uniforms=None if uniforms is None else uniforms[i])
        out.append(r)
        for j, b in enumerate(rows):
            th[b] = r["hidden_out"][j]
            tok[b] = r["next"][j] if forced_tokens is None else int(forced_tokens[i][b])
    return out
