"""Python face of the C ABI: builds the ABI structs from torch device tensors, allocates outputs and the workspace,
and calls mtpd_drafter_step / mtpd_draft_block / mtpd_masked_head on torch's current stream.

torch is used for device memory and streams only; all arithmetic runs in libmtpd.so.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import abi


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def stream_read(buf: torch.Tensor, sink: torch.Tensor, key: int = 0x5EED5EED) -> None:
    """Measurement aid (mtpd_stream_read): one streaming read of the whole contiguous device tensor `buf` on torch's
    current stream; `sink` is a device int32/uint32 tensor of at least one element."""
    if not (buf.is_cuda and buf.is_contiguous() and sink.is_cuda and sink.numel() >= 1):
        raise ValueError("stream_read needs a contiguous device buffer and a device sink")
    nbytes = buf.numel() * buf.element_size()
    abi.check(abi.lib().mtpd_stream_read(buf.data_ptr(), nbytes - nbytes % 16, key & 0xFFFFFFFF, sink.data_ptr(),
                                         _stream()))


class SharedKV:
    """The two target caches ([batch][n_kv][cap][head_dim] bf16 device tensors, v may be k), HOST per-row lengths,
    optional HOST per-row first slots (left padding, ring buffers), and the rotary table [batch][2][2][head_dim/2]
    fp32 on the device."""

    def __init__(self, k_sliding, k_full, len_sliding: Sequence[int], len_full: Sequence[int], rope,
                 v_sliding=None, v_full=None, first_sliding: Optional[Sequence[int]] = None,
                 first_full: Optional[Sequence[int]] = None, shared: bool = False):
        self.k = (k_sliding, k_full)
        self.v = (k_sliding if v_sliding is None else v_sliding, k_full if v_full is None else v_full)
        self.lens = ([int(x) for x in len_sliding], [int(x) for x in len_full])
        self.first = tuple(None if f is None else [int(x) for x in f] for f in (first_sliding, first_full))
        self.shared = bool(shared)  # both caches are one [1][n_kv][cap][head_dim] cache read by every row
        self.rope = rope

    def struct(self):
        arrs = [(C.c_int32 * len(l))(*l) for l in self.lens]
        firsts = [None if f is None else (C.c_int32 * len(f))(*f) for f in self.first]
        kvs = []
        for t in range(2):
            kvs.append(abi.mtpd_kv(k=_ptr(self.k[t]), v=_ptr(self.v[t]), cap=int(self.k[t].shape[2]),
                                   shared=1 if self.shared else 0, len=C.cast(arrs[t], abi.i32p),
                                   first=None if firsts[t] is None else C.cast(firsts[t], abi.i32p)))
        s = abi.mtpd_shared_kv(sliding=kvs[0], full=kvs[1], rope=_ptr(self.rope))
        return s, (arrs, firsts)  # keep the host arrays alive for the call


class Drafter:
    """A handle over borrowed device weights (dict as produced by fixtures.synth.make_weights, on the device)."""

    def __init__(self, shape, weights: Dict[str, object], max_batch: int = abi.MTPD_MAX_BATCH,
                 options: Optional[Dict[int, int]] = None):
        """options: {abi.MTPD_OPT_*: value} applied right after creation (see include/mtpd.h)."""
        L = abi.lib()
        self.shape = shape
        self.weights = weights  # keep the tensors alive: the handle borrows them
        cfg = abi.mtpd_config(backbone=shape.backbone, hidden=shape.hidden, n_layer=shape.n_layer,
                              n_head=shape.n_head, n_kv_head=shape.n_kv_head, head_dim=shape.head_dim,
                              ffn=shape.ffn, vocab=shape.vocab, n_centroids=shape.n_centroids, top_k=shape.top_k,
                              swa_window=shape.swa_window, full_attn_layers=shape.full_attn_layers,
                              rms_eps=shape.rms_eps, attn_scale=shape.attn_scale, embed_scale=shape.embed_scale)
        layers = (abi.mtpd_layer * shape.n_layer)()
        for i, lw in enumerate(weights["layers"]):
            for name in ("attn_q", "attn_q_norm", "attn_output", "attn_norm", "post_attention_norm", "ffn_norm",
                         "post_ffw_norm", "ffn_gate", "ffn_up", "ffn_down"):
                setattr(layers[i], name, _ptr(lw[name]))
            layers[i].layer_output_scale = float(lw["layer_output_scale"])
        w = abi.mtpd_weights(pre_proj=_ptr(weights["pre_proj"]), post_proj=_ptr(weights["post_proj"]),
                             output_norm=_ptr(weights["output_norm"]), token_embd=_ptr(weights["token_embd"]),
                             centroids=_ptr(weights.get("centroids")),  # absent with the dense head
                             token_ordering=_ptr(weights.get("token_ordering")),
                             layers=layers)
        self._cfg, self._layers, self._w = cfg, layers, w
        h = C.c_void_p()
        abi.check(L.mtpd_create(C.byref(cfg), C.byref(w), int(max_batch), C.byref(h)))
        self.handle = h
        self.max_batch = max_batch
        self._ws: Dict[int, torch.Tensor] = {}
        for k, v in (options or {}).items():
            self.set_option(k, v)

    def set_option(self, option: int, value: int) -> None:
        abi.check(abi.lib().mtpd_set_option(self.handle, int(option), int(value)))

    def fault_status(self, clear: bool = False) -> int:
        """0 if every persistent-kernel launch finished its waits normally (see mtpd_fault_status)."""
        st = int(abi.lib().mtpd_fault_status(self.handle, 1 if clear else 0))
        if st < 0:
            abi.check(st)
        return st

    def close(self):
        if getattr(self, "handle", None):
            abi.lib().mtpd_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def timing(self, enable: bool) -> None:
        """Switch per-kernel timing records on (clearing them) or off (keeping them for timing_records)."""
        abi.check(abi.lib().mtpd_timing_enable(self.handle, 1 if enable else 0))

    def timing_records(self) -> List[Tuple[str, float]]:
        """(launch-site label, duration in ms) of every launch recorded since timing was switched on."""
        L = abi.lib()
        cap = abi.MTPD_MAX_TIMED
        names = (C.c_char_p * cap)()
        ms = (C.c_float * cap)()
        n = int(L.mtpd_timing_read(self.handle, cap, names, ms))
        if n < 0:
            abi.check(n)
        return [(names[i].decode(), float(ms[i])) for i in range(min(n, cap))]

    def workspace_bytes(self, batch: int) -> int:
        return int(abi.lib().mtpd_workspace_bytes(self.handle, int(batch)))

    def workspace(self, batch: int) -> torch.Tensor:
        n = self.workspace_bytes(batch)
        if n == 0:
            raise ValueError(f"bad batch {batch}")
        ws = self._ws.get(batch)
        if ws is None:
            ws = torch.empty(n, dtype=torch.uint8, device="cuda")
            self._ws[batch] = ws
        return ws

    def drafter_step(self, target_hidden, last_token, target_embd, kv: SharedKV, want_logits: bool = False,
                     want_sparse: bool = False, out: Optional[Dict[str, torch.Tensor]] = None,
                     workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
        sh = self.shape
        B = int(target_hidden.shape[0])
        dev = target_hidden.device
        o = out if out is not None else {}
        if "next" not in o:
            o["next"] = torch.empty(B, dtype=torch.int32, device=dev)
            o["hidden_out"] = torch.empty(B, sh.backbone, dtype=torch.int16, device=dev)
            if want_logits:
                o["logits"] = torch.empty(B, sh.vocab, dtype=torch.float32, device=dev)
            if want_sparse:
                if sh.n_centroids == 0:
                    raise ValueError("the dense head has no per-cluster outputs")
                kv_n = sh.top_k * sh.vocab // sh.n_centroids
                o["sel"] = torch.empty(B, sh.top_k, dtype=torch.int32, device=dev)
                o["ids"] = torch.empty(B, kv_n, dtype=torch.int32, device=dev)
                o["z"] = torch.empty(B, kv_n, dtype=torch.float32, device=dev)
        ws = workspace if workspace is not None else self.workspace(B)
        s, keep = kv.struct()
        abi.check(abi.lib().mtpd_drafter_step(
            self.handle, _stream(), _ptr(ws), B, _ptr(target_hidden), _ptr(last_token), _ptr(target_embd),
            C.byref(s), _ptr(o.get("logits")), _ptr(o["next"]), _ptr(o["hidden_out"]), _ptr(o.get("sel")),
            _ptr(o.get("ids")), _ptr(o.get("z"))))
        return o

    def drafter_step_noalloc(self, target_hidden, last_token, target_embd, kv: SharedKV,
                             out: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
        """mtpd_drafter_step_noalloc into caller-allocated outputs `out` (the keys drafter_step returns: next,
        hidden_out, optionally logits, sel, ids, z); allocates nothing."""
        B = int(target_hidden.shape[0])
        s, keep = kv.struct()
        abi.check(abi.lib().mtpd_drafter_step_noalloc(
            self.handle, _stream(), B, _ptr(target_hidden), _ptr(last_token), _ptr(target_embd), C.byref(s),
            _ptr(out.get("logits")), _ptr(out["next"]), _ptr(out["hidden_out"]), _ptr(out.get("sel")),
            _ptr(out.get("ids")), _ptr(out.get("z"))))
        return out

    def draft_block(self, n: int, target_hidden, last_token, target_embd, kv: SharedKV, want_logits: bool = False,
                    out: Optional[Dict[str, torch.Tensor]] = None,
                    workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
        sh = self.shape
        B = int(target_hidden.shape[0])
        dev = target_hidden.device
        o = out if out is not None else {}
        if "tokens" not in o:
            o["tokens"] = torch.empty(B, n, dtype=torch.int32, device=dev)
            o["hidden_out"] = torch.empty(B, sh.backbone, dtype=torch.int16, device=dev)
            if want_logits:
                o["logits"] = torch.empty(n, B, sh.vocab, dtype=torch.float32, device=dev)
        ws = workspace if workspace is not None else self.workspace(B)
        s, keep = kv.struct()
        abi.check(abi.lib().mtpd_draft_block(
            self.handle, _stream(), _ptr(ws), B, int(n), _ptr(target_hidden), _ptr(last_token), _ptr(target_embd),
            C.byref(s), _ptr(o["tokens"]), _ptr(o.get("logits")), _ptr(o["hidden_out"])))
        return o

    def draft_block_sampled(self, n: int, target_hidden, last_token, target_embd, kv: SharedKV, temperature: float,
                            uniforms, want_logits: bool = False, out: Optional[Dict[str, torch.Tensor]] = None,
                            workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
        """draft_block(n) drawing each step's token at `temperature` with uniforms [n][B] (fp32 device, in [0, 1));
        returns tokens [B][n], their draft probabilities probs [B][n], hidden_out and optionally logits."""
        sh = self.shape
        B = int(target_hidden.shape[0])
        dev = target_hidden.device
        o = out if out is not None else {}
        if "tokens" not in o:
            o["tokens"] = torch.empty(B, n, dtype=torch.int32, device=dev)
            o["probs"] = torch.empty(B, n, dtype=torch.float32, device=dev)
            o["hidden_out"] = torch.empty(B, sh.backbone, dtype=torch.int16, device=dev)
            if want_logits:
                o["logits"] = torch.empty(n, B, sh.vocab, dtype=torch.float32, device=dev)
        ws = workspace if workspace is not None else self.workspace(B)
        s, keep = kv.struct()
        abi.check(abi.lib().mtpd_draft_block_sampled(
            self.handle, _stream(), _ptr(ws), B, int(n), _ptr(target_hidden), _ptr(last_token), _ptr(target_embd),
            C.byref(s), float(temperature), _ptr(uniforms), _ptr(o["tokens"]), _ptr(o["probs"]), _ptr(o.get("logits")),
            _ptr(o["hidden_out"])))
        return o

    def sample_head(self, h, temperature: float, uniforms, want_logits: bool = False) -> Dict[str, torch.Tensor]:
        """The head alone on fp32 normed states h [m][hidden] with a token drawn per row at uniforms [m]."""
        sh = self.shape
        m = int(h.shape[0])
        dev = h.device
        o = {"token": torch.empty(m, dtype=torch.int32, device=dev), "prob": torch.empty(m, dtype=torch.float32,
                                                                                          device=dev)}
        if want_logits:
            o["logits"] = torch.empty(m, sh.vocab, dtype=torch.float32, device=dev)
        ws = self.workspace(m)
        abi.check(abi.lib().mtpd_sample_head(self.handle, _stream(), _ptr(ws), m, _ptr(h), float(temperature),
                                             _ptr(uniforms), _ptr(o["token"]), _ptr(o["prob"]), _ptr(o.get("logits"))))
        return o

    def masked_head(self, h, want_logits: bool = False, want_sparse: Optional[bool] = None) -> Dict[str, torch.Tensor]:
        """The LM head alone on fp32 normed states h [m][hidden]; with n_centroids == 0 the dense tied head (no
        per-cluster outputs; want_sparse defaults to True for the masked head only)."""
        sh = self.shape
        if want_sparse is None:
            want_sparse = sh.n_centroids > 0
        if want_sparse and sh.n_centroids == 0:
            raise ValueError("the dense head has no per-cluster outputs")
        m = int(h.shape[0])
        dev = h.device
        o = {"argmax": torch.empty(m, dtype=torch.int32, device=dev)}
        if want_logits:
            o["logits"] = torch.empty(m, sh.vocab, dtype=torch.float32, device=dev)
        if want_sparse:
            kv_n = sh.top_k * sh.vocab // sh.n_centroids
            o["sel"] = torch.empty(m, sh.top_k, dtype=torch.int32, device=dev)
            o["ids"] = torch.empty(m, kv_n, dtype=torch.int32, device=dev)
            o["z"] = torch.empty(m, kv_n, dtype=torch.float32, device=dev)
        ws = self.workspace(m)
        abi.check(abi.lib().mtpd_masked_head(
            self.handle, _stream(), _ptr(ws), m, _ptr(h), _ptr(o.get("logits")), _ptr(o["argmax"]),
            _ptr(o.get("sel")), _ptr(o.get("ids")), _ptr(o.get("z"))))
        return o
