"""GPU parity of the dense tied head (n_centroids == 0, the large drafters' head): the HIP path through the C ABI
against the CPU oracle, for the head alone on identical fp32 inputs and inside whole drafter steps."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle as O
from fixtures import synth
from parity import GAP, Case, Tally, compare_dense_row, compare_step, dense_abs_bound

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mtp_drafter_step_amd import abi
    abi.lib()


def dense(base, **over):
    return dataclasses.replace(base, n_centroids=0, top_k=1, **over)


HEAD_CASES = {
    # hidden 256, vocab 4112 = 257 tiles of 16: the last 32-row group is half outside the table
    "h256_v4112": (dense(synth.E2B, vocab=4112), [1, 16, 17, 33, 64]),
    "h512_v2064": (dense(synth.E2B, hidden=512, vocab=2064), [5, 32]),
    "h768_v1040": (dense(synth.E2B, hidden=768, vocab=1040), [3, 40]),
    # the 26B-A4B-shaped head: 262144 x 1024
    "e26b": (synth.E26B, [32]),
}


@pytest.mark.parametrize("name", list(HEAD_CASES))
def test_dense_head_parity(name):
    shape, ms = HEAD_CASES[name]
    case = Case(shape, batch=1, context=16, max_batch=64, gen_device="cuda")
    E = case.model.head_bits
    for m in ms:
        say(f"dense head {name} m={m}")
        g = torch.Generator().manual_seed(200 + m)
        h = torch.randn(m, shape.hidden, generator=g, dtype=torch.float32)
        out = case.drafter.masked_head(h.cuda(), want_logits=True)
        torch.cuda.synchronize()
        assert "sel" not in out
        logits = out["logits"].cpu().numpy()
        am = out["argmax"].cpu().numpy()
        # every row: the argmax is the first maximum of the row the kernel wrote
        assert np.array_equal(am, np.argmax(logits, axis=1))
        rows = list(range(m)) if shape.vocab <= 8192 else [0, m // 2, m - 1]
        tally = Tally()
        for r in rows:
            hr = h[r].numpy().astype(np.float64)
            ref = O.dense_head_result(case.model, hr)
            compare_dense_row(tally, ref["row"], ref["next"], ref["margin"], int(am[r]), logits[r],
                              bound=dense_abs_bound(E, hr), where=f"{name} m={m} row {r}")
        say(tally.summary())
        assert tally.tok_checked >= len(rows) // 2


def test_dense_head_exact_ties_go_to_lowest_id():
    """Table rows 100, 4000 and 4100 are one row copied: their logits tie exactly (same terms in the same order),
    h points along that row so they are the row maximum, and the lowest id (100) must win, in every batch column
    and across the blocks and waves that hold the copies."""
    from mtp_drafter_step_amd import Drafter
    shape = dense(synth.E2B, vocab=4112)
    case = Case(shape, batch=1, context=16, max_batch=64, gen_device="cuda")
    E = case.wg["token_embd"].clone()
    E[[100, 4000, 4100]] = E[2000].clone()
    wg = dict(case.wg)
    wg["token_embd"] = E
    d = Drafter(shape, wg, max_batch=64)
    u = O.bf16_to_f64(E[2000].cpu().numpy().view(np.uint16))
    h = torch.from_numpy(np.tile(50.0 * u, (33, 1)).astype(np.float32))
    out = d.masked_head(h.cuda(), want_logits=True)
    torch.cuda.synchronize()
    assert out["argmax"].cpu().tolist() == [100] * 33
    lg = out["logits"].cpu().numpy()
    assert np.all(lg[:, 100] == lg[:, 2000]) and np.all(lg[:, 4000] == lg[:, 2000])


STEP_CASES = {
    # 26B-A4B-shaped drafter, ragged context around a full sliding window
    "e26b_b4_ragged1500": dict(shape=synth.E26B, batch=4, context=1500, ragged=True),
    # the full workload shape: batch 32, context 32768 (rows sampled for the oracle)
    "e26b_b32_ctx32768": dict(shape=synth.E26B, batch=32, context=32768),
}


@pytest.mark.parametrize("name", list(STEP_CASES))
def test_dense_drafter_step_parity(name):
    say(f"dense drafter_step case={name}")
    kw = STEP_CASES[name]
    case = Case(**kw, gen_device="cuda")
    out = case.drafter.drafter_step(case.th, case.tok, case.temb, case.kv, want_logits=True)
    torch.cuda.synchronize()
    B = kw["batch"]
    rows = list(range(B)) if B <= 4 else [0, 13, B - 1]
    ref = case.oracle_step(rows=rows, want_rows=True)
    tally = compare_step(case, out, ref, rows, where=name)
    say(tally.summary())
    assert tally.tok_checked >= len(rows) // 2
    nxt = out["next"].cpu().numpy()
    assert np.array_equal(nxt, np.argmax(out["logits"].cpu().numpy(), axis=1))


def test_dense_draft_block_parity_stepwise():
    """draft_block(4) with the dense head on the full 26B-shaped workload: the block equals chained drafter_step
    calls bit for bit, and each step matches the oracle on that step's exact inputs (sampled rows)."""
    say("dense draft_block e26b_b32_ctx32768_block4")
    case = Case(synth.E26B, batch=32, context=32768, gen_device="cuda")
    n = 4
    blk = case.drafter.draft_block(n, case.th, case.tok, case.temb, case.kv, want_logits=True)
    blk = {k: v.clone() for k, v in blk.items()}
    torch.cuda.synchronize()
    th, tok = case.th.clone(), case.tok.clone()
    rows = [0, 31]
    tallies = []
    for i in range(n):
        st = case.drafter.drafter_step(th, tok, case.temb, case.kv, want_logits=True)
        st = {k: v.clone() for k, v in st.items()}
        torch.cuda.synchronize()
        assert torch.equal(st["next"], blk["tokens"][:, i].contiguous()), f"step {i}: block tokens"
        assert torch.equal(st["logits"], blk["logits"][i]), f"step {i}: block logits"
        ref = case.oracle_step(rows=rows, want_rows=True, th=th.cpu().numpy().view(np.uint16), tok=tok.cpu().numpy())
        tallies.append(compare_step(case, st, ref, rows, where=f"step {i}"))
        th, tok = st["hidden_out"], st["next"]
    torch.cuda.synchronize()
    assert torch.equal(th, blk["hidden_out"])
    say(" | ".join(t.summary() for t in tallies))
    assert sum(t.tok_checked for t in tallies) >= n * len(rows) // 2
