"""Shared helpers of the GPU parity tests: build one case's inputs for both sides from the seeded generators, and
compare the HIP outputs with the oracle under the parity rules.

Parity rules:
  * selected-centroid sets identical on every row where the oracle's 32nd-33rd fp32 score gap exceeds 1e-3;
  * drafted tokens identical where that holds and the oracle's top-1 minus top-2 logit margin exceeds 1e-3;
  * floating outputs (sparse logits, hidden_out) within |gpu - ref| <= 2e-2 * max(|ref|, rms(ref row));
  * every non-selected logit has exactly the bit pattern of fp32(-1e30).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle as O
from fixtures import synth

GAP = 1e-3
RTOL = 2e-2
NEG_BITS = 0xF149F2CA


def to_dev(w, device="cuda"):
    if isinstance(w, torch.Tensor):
        return w.to(device)
    if isinstance(w, dict):
        return {k: to_dev(v, device) for k, v in w.items()}
    if isinstance(w, list):
        return [to_dev(v, device) for v in w]
    return w


class Case:
    """Inputs of one parity case on both sides. Everything except the target's input embedding table is generated
    on one device and copied to the other; that table is generated on the GPU and row-wise on the CPU by the same
    counter-based generator (bit-identity of the two is itself tested)."""

    def __init__(self, shape, batch: int, context: int, ragged: bool = False, seed: int = 0,
                 distinct_v: bool = False, lens: Optional[Sequence[int]] = None, max_batch: Optional[int] = None,
                 gen_device: str = "cpu", shared_kv: bool = False, swa_window: Optional[int] = None,
                 options: Optional[Dict[int, int]] = None):
        """gen_device "cuda" runs the (bit-identical) generators on the GPU and copies the results to the host, for
        shapes whose tables take the CPU generator too long."""
        from mtp_drafter_step_amd import Drafter, SharedKV
        self.shape, self.batch = shape, batch
        if swa_window is not None:
            shape = dataclasses.replace(shape, swa_window=swa_window)
            self.shape = shape
        wl = synth.Workload("case", shape, batch=batch, context=context, n_steps=1, ragged=ragged, seed=seed,
                            shared_kv=shared_kv)
        self.w = to_dev(synth.make_weights(shape, seed=seed, device=gen_device), "cpu")
        inp = synth.make_inputs(wl, device=gen_device, with_target_embd=False, distinct_v=distinct_v)
        inp = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        if lens is not None:
            inp["len_sliding"] = list(lens)
            inp["len_full"] = list(lens)
            inp["positions"] = list(lens)
            inp["rope"] = torch.from_numpy(synth.rope_tables(shape, list(lens)))
        self.inp = inp
        self.model = O.Model(O.config_from(shape), self.w)
        ks = [inp["k_sliding"].numpy().view(np.uint16), inp["k_full"].numpy().view(np.uint16)]
        vs = ks if not distinct_v else [inp["v_sliding"].numpy().view(np.uint16), inp["v_full"].numpy().view(np.uint16)]
        self.kv_cpu = O.SharedKV(k=ks, v=vs, lens=[inp["len_sliding"], inp["len_full"]], rope=inp["rope"].numpy(),
                                 shared=[shared_kv, shared_kv])
        self.temb_cpu = synth.LazyRows(seed, shape)
        # device side
        self.wg = to_dev(self.w)
        self.temb = synth.gen_bf16(seed, synth.TID["target_embd"], (shape.vocab, shape.backbone), 1.0, device="cuda")
        self.th = inp["target_hidden"].cuda()
        self.tok = inp["last_token"].cuda()
        kd = [inp["k_sliding"].cuda(), inp["k_full"].cuda()]
        vd = [None, None] if not distinct_v else [inp["v_sliding"].cuda(), inp["v_full"].cuda()]
        self.kv = SharedKV(kd[0], kd[1], inp["len_sliding"], inp["len_full"], inp["rope"].cuda(), vd[0], vd[1],
                           shared=shared_kv)
        self.drafter = Drafter(shape, self.wg, max_batch=max_batch or max(batch, 1), options=options)

    def oracle_step(self, rows=None, want_rows=False, th=None, tok=None):
        th = self.inp["target_hidden"].numpy().view(np.uint16) if th is None else th
        tok = self.inp["last_token"].numpy() if tok is None else tok
        return O.drafter_step(self.model, th, tok, self.temb_cpu, self.kv_cpu, want_rows=want_rows, rows=rows)


def rel_ratio(got: np.ndarray, ref: np.ndarray, rtol: float = RTOL) -> float:
    """Largest |gpu - ref| over its bound rtol * max(|ref|, rms(ref)): the float rule holds when this is <= 1."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    floor = np.sqrt(np.mean(ref * ref))
    bound = rtol * np.maximum(np.abs(ref), floor)
    err = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    return float(np.max(r))


def rel_ok(got: np.ndarray, ref: np.ndarray, rtol: float = RTOL) -> bool:
    return rel_ratio(got, ref, rtol) <= 1.0


@dataclasses.dataclass
class Tally:
    rows: int = 0
    sel_checked: int = 0
    tok_checked: int = 0
    worst: float = 0.0  # largest observed error over the float bound (sparse logits, hidden_out)

    def note(self, ratio: float) -> float:
        self.worst = max(self.worst, ratio)
        return ratio

    def summary(self):
        return (f"rows={self.rows} sel_checked={self.sel_checked} tok_checked={self.tok_checked} "
                f"max_err/bound={self.worst:.4f} (bound {RTOL} relative)")


def compare_head_row(tally: Tally, cfg, ref: Dict, r: int, sel: np.ndarray, ids: Optional[np.ndarray],
                     z: Optional[np.ndarray], nxt: int, row: Optional[np.ndarray] = None, where: str = ""):
    """Compare one row's head outputs (GPU arrays) with oracle result `ref` (row index r in the oracle's lists)."""
    tally.rows += 1
    ref_sel = np.asarray(ref["sel"][r])
    if ref["cgap"][r] > GAP:
        tally.sel_checked += 1
        assert set(sel.tolist()) == set(ref_sel.tolist()), f"{where} row {r}: selected centroids differ"
        # order: descending, and equal to the oracle's where adjacent gaps are clear
        if ids is not None:
            ref_map = dict(zip(np.asarray(ref["ids"][r]).tolist(), np.asarray(ref["z"][r]).tolist()))
            got_map = dict(zip(ids.tolist(), z.tolist()))
            assert set(got_map) == set(ref_map), f"{where} row {r}: candidate ids differ"
            keys = sorted(ref_map)
            ratio = tally.note(rel_ratio([got_map[k] for k in keys], [ref_map[k] for k in keys]))
            assert ratio <= 1.0, f"{where} row {r}: sparse logits off by {ratio:.3f} of the bound"
        if ref["margin"][r] > GAP:
            tally.tok_checked += 1
            assert nxt == ref["next"][r], f"{where} row {r}: next token {nxt} != {ref['next'][r]}"
    if row is not None:
        finite = row.view(np.uint32) != NEG_BITS
        assert int(finite.sum()) == cfg.top_k * cfg.vsc, f"{where} row {r}: finite count {int(finite.sum())}"
        if ids is not None:
            assert set(np.nonzero(finite)[0].tolist()) == set(ids.tolist())
            assert np.array_equal(row[ids], z), f"{where} row {r}: scattered values differ from sparse logits"
        assert nxt == int(np.argmax(row)), f"{where} row {r}: next is not the argmax of the row"
    # the drafted token must always be one of the candidate ids and their maximum
    if ids is not None:
        assert nxt in set(ids.tolist())
        zmax = z.max()
        assert nxt == int(ids[z == zmax].min())


# Dense head on identical fp32 inputs: fp32 accumulation of H <= 1024 products (H * 2^-24 < 6.2e-5) plus the
# kernel's bf16 hi + lo split of h (|h - hi - lo| <= 2^-17 |h|, under 7.7e-6) bound |gpu - exact| by 7e-5 times
# sum_k |E[v][k] h[k]|; the oracle's own fp32 rounding adds 6e-8 of |row|.
DENSE_TOL = 1e-4


def dense_abs_bound(head_bits: np.ndarray, h: np.ndarray, chunk: int = 16384) -> np.ndarray:
    """sum_k |E[v][k]| |h[k]| for every row v (the scale of the dense-head tolerance)."""
    out = np.empty(head_bits.shape[0])
    ah = np.abs(np.asarray(h, np.float64))
    for a in range(0, head_bits.shape[0], chunk):
        out[a:a + chunk] = np.abs(O.bf16_to_f64(head_bits[a:a + chunk])) @ ah
    return out


def compare_dense_row(tally: Tally, ref_row: np.ndarray, ref_next: int, ref_margin: float, nxt: int,
                      row: Optional[np.ndarray], bound: Optional[np.ndarray] = None, where: str = ""):
    """One row of the dense head: the full row within DENSE_TOL * bound when both sides saw the same h (else
    within the step tolerance), the token equal to the oracle's where its top-1 minus top-2 margin exceeds GAP,
    and always equal to the first maximum of the GPU's own row."""
    tally.rows += 1
    if row is not None:
        if ref_row is not None and bound is not None:
            err = np.abs(row.astype(np.float64) - ref_row.astype(np.float64))
            worst = int(np.argmax(err - DENSE_TOL * bound))
            assert np.all(err <= DENSE_TOL * bound), f"{where}: logit {worst} off by {err[worst]:.3g}"
        elif ref_row is not None:
            assert rel_ok(row, ref_row), f"{where}: logits"
        assert nxt == int(np.argmax(row)), f"{where}: next is not the first maximum of the row"
    if ref_margin > GAP:
        tally.tok_checked += 1
        assert nxt == ref_next, f"{where}: next token {nxt} != {ref_next}"


def compare_step(case: Case, out: Dict[str, torch.Tensor], ref: Dict, rows: Sequence[int], where: str = "step") -> Tally:
    cfg = case.model.cfg
    tally = Tally()
    nxt = out["next"].cpu().numpy()
    hid = out["hidden_out"].cpu().numpy().view(np.uint16)
    sel = out["sel"].cpu().numpy() if "sel" in out else None
    ids = out["ids"].cpu().numpy() if "ids" in out else None
    z = out["z"].cpu().numpy() if "z" in out else None
    logits = out.get("logits")
    for i, b in enumerate(rows):
        row = logits[b].cpu().numpy() if logits is not None else None
        if cfg.dense:
            compare_dense_row(tally, ref["row"][i] if "row" in ref else None, ref["next"][i], ref["margin"][i],
                              int(nxt[b]), row, where=f"{where} row {b}")
        elif sel is not None:
            compare_head_row(tally, cfg, ref, i, sel[b], ids[b], z[b], int(nxt[b]), row, where)
        ratio = tally.note(rel_ratio(O.bf16_to_f64(hid[b]), O.bf16_to_f64(ref["hidden_out"][i])))
        assert ratio <= 1.0, f"{where} row {b}: hidden_out off by {ratio:.3f} of the bound"
    return tally
