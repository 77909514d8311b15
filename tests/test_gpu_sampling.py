"""GPU parity of temperature sampling (draft_block_sampled, sample_head) through the C ABI.

The draw is checked on identical inputs: the oracle's sampler runs on the logits row the GPU produced (the rows
themselves are checked against the oracle by the other parity tests), and the GPU's token must equal the oracle's
wherever u lies more than SAMPLE_TOL (in probability) from the ends of the drawn token's CDF interval; its probability
within relative 1e-4. SAMPLE_TOL covers fp32 sums of up to 262144 positive terms (tile sums in a fixed tree order,
then at most 64 sequential tile additions: under 5e-6 relative) and exp2 rounding."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from fixtures import synth
from parity import GAP, Case

pytestmark = pytest.mark.gpu
SAMPLE_TOL = 2e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mtp_drafter_step_amd import abi
    abi.lib()


def scored_order(case, row):
    """The head table order of the tokens the GPU row scored (for the masked head: its finite entries' clusters)."""
    m = case.model
    if m.cfg.dense:
        return O.head_order(m, None)
    ids = np.nonzero(row.view(np.uint32) != np.uint32(0xF149F2CA))[0]
    inv = np.empty_like(m.ordering)
    inv[m.ordering] = np.arange(m.ordering.size)
    sel = np.unique(inv[ids] // m.cfg.vsc)
    assert sel.size == m.cfg.top_k
    return O.head_order(m, sel)


def check_draw(row, order, T, u, tok, prob, where):
    smp = O.sample_row(row[order], order, T, float(u))
    checked = smp["cdf_margin"] > SAMPLE_TOL
    if checked:
        assert tok == smp["token"], f"{where}: token {tok} != {smp['token']} (margin {smp['cdf_margin']:.2e})"
        assert abs(prob - smp["prob"]) <= 1e-4 * smp["prob"], f"{where}: prob {prob} != {smp['prob']}"
    assert row[tok] > -1e29, f"{where}: drew a masked token"
    return checked


HEAD_CASES = {  # (shape, temperature, rows)
    "e4b_masked": (synth.E4B, 1.0, 32),
    "e4b_masked_cold": (synth.E4B, 0.05, 32),
    # 64 rows x top 32 = every cluster's worth: the head runs grouped by cluster
    "e4b_masked_grouped": (synth.E4B, 0.7, 64),
    "dense_h256": (None, 0.3, 32),  # E2B-shaped with a dense 8208-token head (two tiles, a ragged second)
    "e26b_dense": (synth.E26B, 0.05, 32),
}


@pytest.mark.parametrize("name", list(HEAD_CASES))
def test_sample_head_draws_match_the_oracle_sampler(name):
    import dataclasses
    shape, T, m = HEAD_CASES[name]
    if shape is None:
        shape = dataclasses.replace(synth.E2B, n_centroids=0, top_k=1, vocab=8208)
    say(f"sample_head {name} T={T}")
    case = Case(shape, batch=1, context=16, max_batch=m, gen_device="cuda")
    g = torch.Generator().manual_seed(300)
    h = torch.randn(m, shape.hidden, generator=g, dtype=torch.float32)
    u = torch.rand(m, generator=g, dtype=torch.float32)
    out = case.drafter.sample_head(h.cuda(), T, u.cuda(), want_logits=True)
    torch.cuda.synchronize()
    lg = out["logits"].cpu().numpy()
    tok = out["token"].cpu().numpy()
    pr = out["prob"].cpu().numpy()
    checked = 0
    for r in range(m):
        checked += check_draw(lg[r], scored_order(case, lg[r]), T, u[r], int(tok[r]), float(pr[r]), f"{name} row {r}")
    say(f"checked {checked}/{m}")
    assert checked >= m // 2
    # the whole pipeline from h: where u is far from any interval end, the oracle's own logits give the same draw
    for r in (0, 7, m - 1):
        hr = h[r].numpy().astype(np.float64)
        ref = O.dense_head_result(case.model, hr) if shape.n_centroids == 0 else \
            O.masked_head_row(case.model, hr, want_row=True)
        order = O.head_order(case.model, None if shape.n_centroids == 0 else ref["sel"])
        smp = O.sample_row(ref["row"][order], order, T, float(u[r]))
        if smp["cdf_margin"] > 1e-3 and (shape.n_centroids == 0 or ref["cgap"] > GAP):
            assert int(tok[r]) == smp["token"], f"{name} row {r}: pipeline draw"


BLOCK_CASES = {
    "e4b_b16_ctx8192_block4": (synth.E4B, 16, 8192, 0.7),
    "e26b_b32_ctx32768_block4": (synth.E26B, 32, 32768, 0.1),
}


@pytest.mark.parametrize("name", list(BLOCK_CASES))
def test_draft_block_sampled(name):
    """Each step's draw against the oracle sampler on that step's GPU logits row; the block equals chained one-step
    sampled blocks bit for bit (so step i+1 read step i's drawn token and hidden state); repeated calls agree."""
    shape, B, ctx, T = BLOCK_CASES[name]
    say(f"draft_block_sampled {name} T={T}")
    case = Case(shape, batch=B, context=ctx, gen_device="cuda")
    n = 4
    g = torch.Generator().manual_seed(301)
    u = torch.rand(n, B, generator=g, dtype=torch.float32).cuda()
    d = case.drafter
    blk = d.draft_block_sampled(n, case.th, case.tok, case.temb, case.kv, T, u, want_logits=True)
    blk = {k: v.clone() for k, v in blk.items()}
    again = d.draft_block_sampled(n, case.th, case.tok, case.temb, case.kv, T, u, want_logits=True)
    torch.cuda.synchronize()
    for k in blk:
        assert torch.equal(again[k], blk[k]), f"repeat: {k}"
    th, tok = case.th.clone(), case.tok.clone()
    checked = 0
    for i in range(n):
        st = d.draft_block_sampled(1, th, tok, case.temb, case.kv, T, u[i:i + 1].contiguous(), want_logits=True)
        st = {k: v.clone() for k, v in st.items()}
        torch.cuda.synchronize()
        assert torch.equal(st["tokens"][:, 0], blk["tokens"][:, i]), f"step {i}: chained tokens"
        assert torch.equal(st["logits"][0], blk["logits"][i]), f"step {i}: chained logits"
        lg = blk["logits"][i].cpu().numpy()
        toks = blk["tokens"][:, i].cpu().numpy()
        prs = blk["probs"][:, i].cpu().numpy()
        uu = u[i].cpu().numpy()
        for b in range(B):
            checked += check_draw(lg[b], scored_order(case, lg[b]), T, uu[b], int(toks[b]), float(prs[b]),
                                  f"{name} step {i} row {b}")
        th, tok = st["hidden_out"], st["tokens"][:, 0].contiguous()
    assert torch.equal(th, blk["hidden_out"])
    say(f"checked {checked}/{n * B}")
    assert checked >= n * B // 2


def test_sampling_at_tiny_temperature_is_the_argmax_block():
    case = Case(synth.E4B, batch=8, context=3000, ragged=True)
    d = case.drafter
    ref = d.draft_block(4, case.th, case.tok, case.temb, case.kv, want_logits=True)
    ref = {k: v.clone() for k, v in ref.items()}
    u = torch.rand(4, 8, generator=torch.Generator().manual_seed(302), dtype=torch.float32).cuda()
    got = d.draft_block_sampled(4, case.th, case.tok, case.temb, case.kv, 1e-5, u, want_logits=True)
    torch.cuda.synchronize()
    parted = set()  # rows after a near-tie, where the two chains may part
    for i in range(4):
        lg = ref["logits"][i].cpu().numpy()
        for b in range(8):
            if b in parted:
                continue
            top2 = np.sort(lg[b])[-2:]
            if top2[1] - top2[0] > 1e-3:
                assert int(got["tokens"][b, i]) == int(ref["tokens"][b, i]), (i, b)
                assert float(got["probs"][b, i]) == 1.0
            else:
                parted.add(b)
    assert len(parted) < 8
