"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle as O
from fixtures import synth
from parity import Case, Tally, compare_head_row, compare_step, rel_ok

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mtp_drafter_step_amd import abi
    abi.lib()  # fails loudly if the library is missing


def test_generator_identical_on_gpu_and_cpu():
    shape = synth.E2B
    rows = torch.tensor([0, 1, 77777, 262143], dtype=torch.int64)
    full_gpu = synth.gen_bf16(0, synth.TID["target_embd"], (shape.vocab, shape.backbone), 1.0, device="cuda")
    got = full_gpu[rows.cuda()].cpu()
    want = synth.gen_bf16(0, synth.TID["target_embd"], (shape.vocab, shape.backbone), 1.0, row_index=rows)
    assert torch.equal(got, want)
    w_cpu = synth.gen_bf16(3, 5, (512, 256), 0.0625)
    w_gpu = synth.gen_bf16(3, 5, (512, 256), 0.0625, device="cuda").cpu()
    assert torch.equal(w_cpu, w_gpu)


@pytest.mark.parametrize("m,scale", [(1, 1.0), (16, 1.0), (64, 1.0), (64, 0.1)])
def test_masked_head_parity(m, scale):
    """Centroid scores ~ N(0, scale^2). At scale 1 the top-ranked scores share their leading key byte with a few
    dozen others; at scale 0.1 a couple of hundred scores share it, so the selection takes more than one radix
    pass."""
    say(f"masked_head m={m} scale={scale}")
    case = Case(synth.E4B, batch=1, context=16, max_batch=64)
    g = torch.Generator().manual_seed(100 + m)
    h = torch.randn(m, 256, generator=g, dtype=torch.float32) * scale
    out = case.drafter.masked_head(h.cuda(), want_logits=True, want_sparse=True)
    torch.cuda.synchronize()
    tally = Tally()
    for r in range(m):
        ref = O.masked_head_row(case.model, h[r].numpy().astype(np.float64))
        refl = {k: [ref[k]] for k in ("sel", "ids", "z", "cgap", "margin", "next")}
        compare_head_row(tally, case.model.cfg, refl, 0, out["sel"][r].cpu().numpy(), out["ids"][r].cpu().numpy(),
                         out["z"][r].cpu().numpy(), int(out["argmax"][r]), out["logits"][r].cpu().numpy(),
                         where=f"head m={m}")
    say(tally.summary())
    assert tally.sel_checked >= m // 2


HEAD_SHAPES = {
    # 40 clusters of 48 ids, top 7: a cluster count that is no power of two, an odd top_k
    "c40_v48_k7": dataclasses.replace(synth.E4B, vocab=1920, n_centroids=40, top_k=7),
    # 16 clusters of 1024 ids (the largest cluster the ABI takes), top 3
    "c16_v1024_k3": dataclasses.replace(synth.E4B, vocab=16384, n_centroids=16, top_k=3),
    # 4096 clusters of 16 ids, top 64 (the largest cluster count and top_k)
    "c4096_v16_k64": dataclasses.replace(synth.E4B, vocab=65536, n_centroids=4096, top_k=64),
    # hidden 512: 64 clusters of 32 ids, top 5
    "h512_c64_v32_k5": dataclasses.replace(synth.E4B, hidden=512, vocab=2048, n_centroids=64, top_k=5),
    # hidden 1024 (one id tile per wave at a time, the rows reloaded per group of tiles): 32 clusters of 128, top 4
    "h1024_c32_v128_k4": dataclasses.replace(synth.E4B, hidden=1024, vocab=4096, n_centroids=32, top_k=4),
}


@pytest.mark.parametrize("m", [3, 64])
@pytest.mark.parametrize("name", list(HEAD_SHAPES))
def test_masked_head_shapes(name, m):
    """The masked head at the edges of its shape limits. At 3 rows the head runs one block per (row, slot); at 64
    rows (64 top_k at least the cluster count) it runs the per-row top-k, the grouping by cluster and one block per
    selected cluster."""
    shape = HEAD_SHAPES[name]
    say(f"masked_head {name} m={m}")
    case = Case(shape, batch=1, context=16, max_batch=64)
    g = torch.Generator().manual_seed(300 + m)
    h = torch.randn(m, shape.hidden, generator=g, dtype=torch.float32)
    out = case.drafter.masked_head(h.cuda(), want_logits=True, want_sparse=True)
    torch.cuda.synchronize()
    tally = Tally()
    for r in range(m):
        ref = O.masked_head_row(case.model, h[r].numpy().astype(np.float64))
        refl = {k: [ref[k]] for k in ("sel", "ids", "z", "cgap", "margin", "next")}
        compare_head_row(tally, case.model.cfg, refl, 0, out["sel"][r].cpu().numpy(), out["ids"][r].cpu().numpy(),
                         out["z"][r].cpu().numpy(), int(out["argmax"][r]), out["logits"][r].cpu().numpy(),
                         where=f"head {name} m={m}")
        # the slots are in descending score order
        sc = np.asarray(ref["scores"]) if ref.get("scores") is not None else None
        if sc is not None and ref["cgap"] > 1e-3:
            got = sc[out["sel"][r].cpu().numpy()]
            assert np.all(np.diff(got) <= 1e-3), f"{name} row {r}: slots out of order"
    say(tally.summary())
    assert tally.sel_checked >= m // 2


@pytest.mark.parametrize("batch", [1, 64, 65, 256])
@pytest.mark.parametrize("ntie", [20, 40, 100])
def test_masked_head_exact_ties(ntie, batch):
    """Centroid rows 0 .. ntie-1 are copies of row ntie and h points along that row, so those ntie + 1 scores tie
    exactly (identical terms in the same order) and lie far above every other score. Ties go to the lower index, so
    the first slots must be centroids 0, 1, 2, ... in order. With 20 ties the rest of the slots come from the
    untied scores; 40 tied members are ordered by the small in-wave sort of the one-row-per-block head, 100 by its
    rank-by-index path. From batch 64 every row is the same and the head takes its per-row selection and per-cluster
    scoring, each cluster then serving every row: one 64-entry tile per cluster at 64 rows, two (64 + 1) at 65 and
    four at 256. Every row is compared."""
    from mtp_drafter_step_amd import Drafter
    say(f"masked_head ties={ntie} batch={batch}")
    case = Case(synth.E4B, batch=1, context=16, max_batch=batch)
    w = dict(case.w)
    cen = case.w["centroids"].clone()
    cen[:ntie] = cen[ntie]
    w["centroids"] = cen
    model = O.Model(O.config_from(case.shape), w)
    wg = dict(case.wg)
    wg["centroids"] = cen.cuda()
    d = Drafter(case.shape, wg, max_batch=batch)
    u = O.bf16_to_f64(cen[ntie].numpy().view(np.uint16))
    h = torch.from_numpy((50.0 * u).astype(np.float32)).reshape(1, -1).repeat(batch, 1).contiguous()
    out = d.masked_head(h.cuda(), want_logits=True, want_sparse=True)
    torch.cuda.synchronize()
    k = case.shape.top_k
    ref = O.masked_head_row(model, h[0].numpy().astype(np.float64))
    lead = min(ntie + 1, k)
    assert list(ref["sel"])[:lead] == list(range(lead))
    tally = Tally()
    refl = {key: [ref[key]] for key in ("sel", "ids", "z", "cgap", "margin", "next")}
    for r in range(batch):
        sel = out["sel"][r].cpu().numpy()
        assert sel[:lead].tolist() == list(range(lead)), f"row {r}"
        if lead == k:  # every slot tied: the order is fixed by index alone
            assert sel.tolist() == list(ref["sel"]), f"row {r}"
            assert out["ids"][r].cpu().tolist() == list(np.asarray(ref["ids"])), f"row {r}"
            assert rel_ok(out["z"][r].cpu().numpy(), ref["z"])
        compare_head_row(tally, case.model.cfg, refl, 0, sel, out["ids"][r].cpu().numpy(), out["z"][r].cpu().numpy(),
                         int(out["argmax"][r]), out["logits"][r].cpu().numpy(), where=f"ties row {r}")
    say(tally.summary())


STEP_CASES = {
    # E2B-shaped, batch 1, shared context 256 (shorter than the sliding window: sliding == full)
    "e2b_b1_ctx256": dict(shape=synth.E2B, batch=1, context=256),
    # E4B-shaped, batch 16, context 8192 per sequence
    "e4b_b16_ctx8192": dict(shape=synth.E4B, batch=16, context=8192),
    # ragged lengths 700 - 37 b: windows partly full, several key tiles and a ragged last tile per row
    "e4b_b6_ragged700": dict(shape=synth.E4B, batch=6, context=700, ragged=True),
    # E4B with two KV heads, batch 16, K = V: the two-kv-head workload's shapes at a shorter, ragged context
    "e4b_nkv2_b16_ragged1500": dict(shape=dataclasses.replace(synth.E4B, n_kv_head=2), batch=16, context=1500,
                                    ragged=True),
    # E4B with two KV heads (the variant table's E4B), distinct V caches
    "e4b_nkv2_distinct_v": dict(shape=dataclasses.replace(synth.E4B, n_kv_head=2), batch=3, context=1000,
                                distinct_v=True),
    # window 1 and a row with a single key
    "e2b_window1_len1": dict(shape=dataclasses.replace(synth.E2B, swa_window=1), batch=3, context=64,
                             lens=[64, 1, 33]),
    # more than one 64-row group of blocks
    "e2b_b64_ctx300": dict(shape=synth.E2B, batch=64, context=300, ragged=True),
    # the largest batch the ABI takes, per-row caches
    "e2b_b256_ctx200": dict(shape=synth.E2B, batch=256, context=200, ragged=True),
    # hidden 512 and 768 (the small-batch kernels' wider prologues)
    "e2b_h512_b3_ragged600": dict(shape=dataclasses.replace(synth.E2B, hidden=512), batch=3, context=600, ragged=True),
    "e2b_h768_b5_ragged600": dict(shape=dataclasses.replace(synth.E2B, hidden=768), batch=5, context=600, ragged=True),
    # head_dim 128 and 64 (the vector-ALU attention): 2 and 8 query heads per kv head
    "e2b_hd128_g2": dict(shape=dataclasses.replace(synth.E2B, head_dim=128, n_head=8, n_kv_head=4), batch=3,
                         context=700, ragged=True),
    "e2b_hd64_g8": dict(shape=dataclasses.replace(synth.E2B, head_dim=64, n_head=16, n_kv_head=2), batch=2,
                        context=600, ragged=True),
}


@pytest.mark.parametrize("name", list(STEP_CASES))
def test_drafter_step_parity(name):
    say(f"drafter_step case={name}")
    kw = STEP_CASES[name]
    case = Case(**kw)
    out = case.drafter.drafter_step(case.th, case.tok, case.temb, case.kv, want_logits=True, want_sparse=True)
    torch.cuda.synchronize()
    B = kw["batch"]
    rows = list(range(B)) if B <= 16 else list(range(0, B, 7)) + [B - 1]
    ref = case.oracle_step(rows=rows)
    tally = compare_step(case, out, ref, rows, where=name)
    say(tally.summary())
    assert tally.sel_checked >= len(rows) // 2


def test_vector_alu_attention_at_head_dim_256():
    """The vector-ALU attention (selected by the handle option MTPD_OPT_ATTN_VALU, else used only for head_dim 64 / 128)
    on head_dim 256 with 4 and 8 query heads per kv head, split over several key ranges."""
    from mtp_drafter_step_amd import Drafter, abi
    for shape in (synth.E4B, synth.E26B):
        say(f"valu attention {shape.n_head}/{shape.n_kv_head} heads")
        case = Case(shape, batch=3, context=2500, ragged=True, gen_device="cuda")
        d = Drafter(shape, case.wg, max_batch=3, options={abi.MTPD_OPT_ATTN_VALU: 1, abi.MTPD_OPT_PERSISTENT: 0})
        want_sparse = shape.n_centroids > 0
        out = d.drafter_step(case.th, case.tok, case.temb, case.kv, want_logits=True, want_sparse=want_sparse)
        torch.cuda.synchronize()
        rows = [0, 1, 2]
        ref = case.oracle_step(rows=rows, want_rows=not want_sparse)
        tally = compare_step(case, out, ref, rows, where=f"valu {shape.n_head}")
        say(tally.summary())
        assert tally.tok_checked >= 1


def test_left_padded_and_ring_buffer_caches():
    """The same keys in a left-padded batch (both caches, junk before each row's keys) and in a ring-buffer
    sliding cache (capacity 700 >= window 512, position p in slot p mod 700, rows wrapping past the end) give
    outputs bit-identical to the linear caches (same keys in the same order and splits), and match the oracle."""
    from mtp_drafter_step_amd import SharedKV, abi
    case = Case(synth.E4B, batch=4, context=1500, ragged=True)
    B = 4
    ref = case.drafter.drafter_step(case.th, case.tok, case.temb, case.kv, want_logits=True, want_sparse=True)
    ref = {k: v.clone() for k, v in ref.items()}
    lens = case.kv.lens
    g = torch.Generator(device="cuda").manual_seed(5)
    # left padding
    pads = [0, 17, 64, 3]
    padded = []
    for t in range(2):
        k = case.kv.k[t]
        big = torch.randint(-32768, 32767, (B, k.shape[1], k.shape[2] + 64, k.shape[3]), generator=g, device="cuda",
                            dtype=torch.int32).to(torch.int16)
        for b in range(B):
            big[b, :, pads[b]:pads[b] + lens[t][b]] = k[b, :, :lens[t][b]]
        padded.append(big)
    kvp = SharedKV(padded[0], padded[1], lens[0], lens[1], case.kv.rope, first_sliding=pads, first_full=pads)
    say("left-padded caches")
    got = case.drafter.drafter_step(case.th, case.tok, case.temb, kvp, want_logits=True, want_sparse=True)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(got[k], ref[k]), f"left padding: {k}"
    # ring-buffer sliding cache
    C = 700
    ks = case.kv.k[0]
    ring = torch.randint(-32768, 32767, (B, ks.shape[1], C, ks.shape[3]), generator=g, device="cuda",
                         dtype=torch.int32).to(torch.int16)
    rlen, rfirst = [], []
    for b in range(B):
        L = lens[0][b]
        n = min(L, C)
        pos = torch.arange(L - n, L, device="cuda")
        ring[b, :, pos % C] = ks[b, :, L - n:L]
        rlen.append(n)
        rfirst.append((L - n) % C)
    assert any(f + n > C for f, n in zip(rfirst, rlen))
    kvr = SharedKV(ring, case.kv.k[1], rlen, lens[1], case.kv.rope, first_sliding=rfirst)
    say("ring-buffer sliding cache")
    got = case.drafter.drafter_step(case.th, case.tok, case.temb, kvr, want_logits=True, want_sparse=True)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(got[k], ref[k]), f"ring buffer: {k}"
    # the oracle on the ring layout
    ring_np = ring.cpu().numpy().view(np.uint16)
    okv = O.SharedKV(k=[ring_np, case.kv_cpu.k[1]], v=[ring_np, case.kv_cpu.k[1]], lens=[rlen, lens[1]],
                     rope=case.kv_cpu.rope, first=[rfirst, [0] * B])
    oref = O.drafter_step(case.model, case.inp["target_hidden"].numpy().view(np.uint16), case.inp["last_token"].numpy(),
                          case.temb_cpu, okv)
    tally = compare_step(case, got, oref, list(range(B)), where="ring")
    say(tally.summary())
    # a first slot outside the cache is rejected before anything runs
    bad = SharedKV(ring, case.kv.k[1], rlen, lens[1], case.kv.rope, first_sliding=[C, 0, 0, 0])
    with pytest.raises(abi.MtpdError) as ei:
        case.drafter.drafter_step(case.th, case.tok, case.temb, bad)
    assert "first" in str(ei.value)


SHARED_CASES = {
    # 4 query heads per kv head: 32 rows per block of the multi-query kernel, 8 live; ragged windows
    "e4b_b8_ragged3000": dict(shape=synth.E4B, batch=8, context=3000, ragged=True),
    # two kv heads (2 query heads each), two 64-row blocks
    "e4b_nkv2_b80": dict(shape=dataclasses.replace(synth.E4B, n_kv_head=2), batch=80, context=1200, ragged=True),
    # 8 query heads per kv head (16 rows per block), dense head
    "e26b_b5_ragged1500": dict(shape=synth.E26B, batch=5, context=1500, ragged=True, gen_device="cuda"),
}


@pytest.mark.parametrize("name", list(SHARED_CASES))
def test_shared_cache_rows(name):
    """Rows of one sequence reading one shared cache (own lengths, tokens and positions; the multi-query attention)
    against the oracle; the same call with per-row copies of the cache (the per-row attention) too."""
    from mtp_drafter_step_amd import SharedKV
    kw = SHARED_CASES[name]
    say(f"shared cache {name}")
    case = Case(**kw, shared_kv=True)
    dense = case.shape.n_centroids == 0
    B = kw["batch"]
    out = case.drafter.drafter_step(case.th, case.tok, case.temb, case.kv, want_logits=True, want_sparse=not dense)
    out = {k: v.clone() for k, v in out.items()}
    rows = list(range(B)) if B <= 8 else list(range(0, B, 9)) + [B - 1]
    ref = case.oracle_step(rows=rows, want_rows=dense)
    tally = compare_step(case, out, ref, rows, where=f"shared {name}")
    say(tally.summary())
    assert tally.tok_checked >= len(rows) // 2
    copies = [t.expand(B, -1, -1, -1).contiguous() for t in case.kv.k]
    kvc = SharedKV(copies[0], copies[1], case.kv.lens[0], case.kv.lens[1], case.kv.rope)
    got = case.drafter.drafter_step(case.th, case.tok, case.temb, kvc, want_logits=True, want_sparse=not dense)
    torch.cuda.synchronize()
    tally = compare_step(case, got, ref, rows, where=f"copies {name}")
    assert tally.tok_checked >= len(rows) // 2


def test_verify_width_step():
    """The verify-width workload: 256 rows of one sequence sharing one cache of 131072 keys (window 1024), the
    largest batch the ABI takes. Rows 0 .. 63 repeat row 0's target hidden state and token, so each of their clusters
    is chosen by 64 rows (one full tile of the grouped head per cluster); 16 rows against the oracle: four of the
    repeated group and twelve spread over the rest, and the repeated rows equal to each other bit for bit."""
    say("verify width: 256 rows, shared 131072-key cache")
    case = Case(synth.E4B, batch=256, context=131072, gen_device="cuda", shared_kv=True, swa_window=1024)
    th = case.th.clone()
    tok = case.tok.clone()
    th[1:64] = th[0]
    tok[1:64] = tok[0]
    out = case.drafter.drafter_step(th, tok, case.temb, case.kv, want_logits=True, want_sparse=True)
    torch.cuda.synchronize()
    for k in ("next", "hidden_out", "sel", "ids", "z", "logits"):
        assert torch.equal(out[k][1:64], out[k][0:1].expand_as(out[k][1:64])), k
    rows = [0, 1, 31, 63] + list(range(64, 256, 17))[:11] + [255]
    thn = th.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = case.oracle_step(rows=rows, th=thn, tok=tok.cpu().numpy())
    tally = compare_step(case, out, ref, rows, where="verify")
    say(tally.summary())
    assert tally.rows == 16 and tally.sel_checked >= 12


def test_verify_width_head_shared_clusters():
    """The grouped head at verify width on rows that share most of their clusters: 8 distinct fp32 states, each
    repeated over 32 rows with a small per-row perturbation; all 256 rows against the oracle's head on the same
    input."""
    say("verify width head: 256 rows in 8 groups of near-identical states")
    case = Case(synth.E4B, batch=1, context=16, max_batch=256)
    g = torch.Generator().manual_seed(7)
    base = torch.randn(8, case.shape.hidden, generator=g, dtype=torch.float32) * 3.0
    h = base.repeat_interleave(32, dim=0) + 0.01 * torch.randn(256, case.shape.hidden, generator=g)
    out = case.drafter.masked_head(h.cuda(), want_logits=True, want_sparse=True)
    torch.cuda.synchronize()
    tally = Tally()
    shared = 0
    for r in range(256):
        ref = O.masked_head_row(case.model, h[r].numpy().astype(np.float64))
        refl = {key: [ref[key]] for key in ("sel", "ids", "z", "cgap", "margin", "next")}
        sel = out["sel"][r].cpu().numpy()
        if r % 32:
            shared += len(set(sel.tolist()) & set(out["sel"][r - r % 32].cpu().numpy().tolist()))
        compare_head_row(tally, case.model.cfg, refl, 0, sel, out["ids"][r].cpu().numpy(), out["z"][r].cpu().numpy(),
                         int(out["argmax"][r]), out["logits"][r].cpu().numpy(), where=f"shared row {r}")
    frac = shared / (248 * case.shape.top_k)
    say(tally.summary() + f" clusters shared with the group's first row: {frac:.2f}")
    assert frac > 0.7 and tally.sel_checked >= 128


GEMM_PATH_CASES = {
    # 32+ rows take the matrix-core dense stages by default: run both paths on the same inputs
    "e4b_b40_ragged2000": dict(shape=synth.E4B, batch=40, context=2000, ragged=True),
    "e26b_b32_ctx4000": dict(shape=synth.E26B, batch=32, context=4000, ragged=True, gen_device="cuda"),
    # hidden 768 at 33 rows: three 16-row tiles, the last with one row
    "e2b_h768_b33_ragged900": dict(shape=dataclasses.replace(synth.E2B, hidden=768), batch=33, context=900, ragged=True),
    # and the matrix-core path forced on a small batch (one 16-row pass with ragged columns)
    "e4b_b5_forced": dict(shape=synth.E4B, batch=5, context=900, ragged=True),
    # one long row among short ones: the full layer takes the most key-range splits (32), so both split merges
    # (k_merge on the large-batch path, k_oproj's prologue on the small one) run their widest form
    "e4b_b32_one_long_row": dict(shape=synth.E4B, batch=32, context=4096, lens=[4096] + [40] * 31),
}


@pytest.mark.parametrize("name", list(GEMM_PATH_CASES))
def test_dense_stage_paths(name):
    """The large-batch path (residual + norm kernels, matrix-core GEMMs with K-split partials, separate attention
    merge) and the small-batch path (fused prologues), each forced on a fresh handle, both against the oracle."""
    from mtp_drafter_step_amd import Drafter, abi
    kw = GEMM_PATH_CASES[name]
    case = Case(**kw)
    dense = case.shape.n_centroids == 0
    B = kw["batch"]
    rows = list(range(B)) if B <= 8 else list(range(0, B, 6)) + [B - 1]
    ref = case.oracle_step(rows=rows, want_rows=dense)
    for flag in (2, 1):
        say(f"dense stages {name} MTPD_OPT_DENSE_PATH={flag}")
        d = Drafter(case.shape, case.wg, max_batch=B,
                    options={abi.MTPD_OPT_DENSE_PATH: flag, abi.MTPD_OPT_PERSISTENT: 0})
        out = d.drafter_step(case.th, case.tok, case.temb, case.kv, want_logits=True, want_sparse=not dense)
        torch.cuda.synchronize()
        tally = compare_step(case, out, ref, rows, where=f"{name} path {flag}")
        say(tally.summary())
        assert tally.tok_checked >= len(rows) // 2


def test_drafter_step_is_deterministic():
    case = Case(synth.E4B, batch=4, context=2000, ragged=True)
    a = case.drafter.drafter_step(case.th, case.tok, case.temb, case.kv, want_logits=True, want_sparse=True)
    a = {k: v.clone() for k, v in a.items()}
    b = case.drafter.drafter_step(case.th, case.tok, case.temb, case.kv, want_logits=True, want_sparse=True)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


BLOCK_CASES = {
    "e2b_b1_ctx4096_block4": dict(shape=synth.E2B, batch=1, context=4096, n=4),
    "e4b_b16_ctx8192_block4": dict(shape=synth.E4B, batch=16, context=8192, n=4),
    # the two-kv-head workload at its full size
    "e4b_nkv2_b16_ctx8192_block4": dict(shape=dataclasses.replace(synth.E4B, n_kv_head=2), batch=16, context=8192,
                                        n=4),
}


@pytest.mark.parametrize("name", list(BLOCK_CASES))
def test_draft_block_parity_stepwise(name):
    """draft_block(n) against the oracle one step at a time on identical inputs.

    The block is replayed as chained drafter_step calls, which must reproduce its tokens and logits bit for bit;
    the oracle is then given each step's exact inputs (the GPU's bf16 hidden_out and token of the previous step).
    Chaining the oracle on its own hidden states is not a parity test: one-ulp bf16 differences in hidden_out
    grow through the steps (a few flips move centroid scores by about 1e-2 three steps later), so agreement
    after the first step would depend on rounding luck rather than on the arithmetic."""
    say(f"draft_block case={name}")
    kw = dict(BLOCK_CASES[name])
    n = kw.pop("n")
    case = Case(**kw)
    blk = case.drafter.draft_block(n, case.th, case.tok, case.temb, case.kv, want_logits=True)
    blk = {k: v.clone() for k, v in blk.items()}
    torch.cuda.synchronize()
    B = kw["batch"]
    th, tok = case.th.clone(), case.tok.clone()
    rows = list(range(B))
    tallies = []
    for i in range(n):
        st = case.drafter.drafter_step(th, tok, case.temb, case.kv, want_logits=True, want_sparse=True)
        st = {k: v.clone() for k, v in st.items()}
        torch.cuda.synchronize()
        assert torch.equal(st["next"], blk["tokens"][:, i].contiguous()), f"step {i}: block tokens"
        assert torch.equal(st["logits"], blk["logits"][i]), f"step {i}: block logits"
        ref = case.oracle_step(rows=rows, th=th.cpu().numpy().view(np.uint16), tok=tok.cpu().numpy())
        tallies.append(compare_step(case, st, ref, rows, where=f"step {i}"))
        th, tok = st["hidden_out"], st["next"]
    torch.cuda.synchronize()
    assert torch.equal(th, blk["hidden_out"])
    say(" | ".join(t.summary() for t in tallies))
    assert sum(t.sel_checked for t in tallies) >= (n * B) // 2


def test_draft_block_equals_chained_steps():
    case = Case(synth.E4B, batch=5, context=1500, ragged=True)
    n = 3
    blk = case.drafter.draft_block(n, case.th, case.tok, case.temb, case.kv, want_logits=True)
    blk = {k: v.clone() for k, v in blk.items()}
    th, tok = case.th.clone(), case.tok.clone()
    for i in range(n):
        s = case.drafter.drafter_step(th, tok, case.temb, case.kv, want_logits=True)
        assert torch.equal(s["next"], blk["tokens"][:, i].contiguous()), i
        assert torch.equal(s["logits"], blk["logits"][i]), i
        th, tok = s["hidden_out"].clone(), s["next"].clone()
    torch.cuda.synchronize()
    assert torch.equal(th, blk["hidden_out"])


def test_graph_replays_match_direct_launches():
    """The same call replayed from a captured graph, interleaved with other work and synchronisations, gives
    bit-identical results to direct launches (graphs disabled) every time."""
    from mtp_drafter_step_amd import Drafter, abi
    case = Case(synth.E4B, batch=4, context=1200, ragged=True, options={abi.MTPD_OPT_PERSISTENT: 0})
    direct = Drafter(case.shape, case.wg, max_batch=4,
                     options={abi.MTPD_OPT_GRAPHS: 0, abi.MTPD_OPT_PERSISTENT: 0})
    ref = direct.draft_block(3, case.th, case.tok, case.temb, case.kv, want_logits=True)
    ref = {k: v.clone() for k, v in ref.items()}
    for rep in range(4):
        out = case.drafter.draft_block(3, case.th, case.tok, case.temb, case.kv, want_logits=True)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(out[k], ref[k]), (rep, k)
        # unrelated eager work between replays
        other = case.drafter.drafter_step(case.th, case.tok, case.temb, case.kv, want_sparse=True)
        torch.cuda.synchronize()
        assert other["next"].shape[0] == 4


@pytest.mark.parametrize("name,shape,batch", [("e4b_b4_small_path", synth.E4B, 4), ("e2b_b48_gemm_path", synth.E2B, 48)])
def test_caller_graph_capture_replays(name, shape, batch):
    """A caller captures draft_block into its own graph (the library then launches straight into the caller's
    capture instead of replaying its own graphs): every replay, with eager work and synchronisations between them,
    reproduces the eager call bit for bit. At 48 rows the step takes the matrix-core dense stages and the grouped
    head."""
    say(f"caller capture {name}")
    case = Case(shape, batch=batch, context=900, ragged=True, max_batch=batch)
    d = case.drafter
    ws = d.workspace(batch)
    ref = d.draft_block(2, case.th, case.tok, case.temb, case.kv, want_logits=True, workspace=ws)
    ref = {k: v.clone() for k, v in ref.items()}
    out = {"tokens": torch.empty_like(ref["tokens"]), "hidden_out": torch.empty_like(ref["hidden_out"]),
           "logits": torch.empty_like(ref["logits"])}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture's stream kind, outside the capture
        d.draft_block(2, case.th, case.tok, case.temb, case.kv, want_logits=True, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.draft_block(2, case.th, case.tok, case.temb, case.kv, want_logits=True, out=out, workspace=ws)
    for rep in range(3):
        for v in out.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(out[k], ref[k]), (name, rep, k)
        other = d.drafter_step(case.th, case.tok, case.temb, case.kv, want_sparse=False)  # eager work between
        torch.cuda.synchronize()
        assert other["next"].shape[0] == batch


@pytest.mark.parametrize("persistent", [0, 1])
def test_kernel_timing_records_every_launch_and_keeps_results(persistent):
    """Timing records: one per kernel launch of the call, in launch order, with positive durations; the results
    equal those of the graph-replayed (per-stage kernels) or plain (persistent kernel) call."""
    from mtp_drafter_step_amd import abi
    case = Case(synth.E4B, batch=4, context=1200, ragged=True, options={abi.MTPD_OPT_PERSISTENT: persistent})
    d = case.drafter
    ref = d.draft_block(2, case.th, case.tok, case.temb, case.kv, want_logits=True)
    ref = {k: v.clone() for k, v in ref.items()}
    d.timing(True)
    out = d.draft_block(2, case.th, case.tok, case.temb, case.kv, want_logits=True)
    torch.cuda.synchronize()
    d.timing(False)
    recs = d.timing_records()
    for k in ref:
        assert torch.equal(out[k], ref[k]), k
    names = [r[0] for r in recs]
    if persistent:  # every step of the call in one launch
        assert names == ["team"], names
        assert recs[0][1] > 0.0
        return
    L = case.shape.n_layer
    per_step = ["pre"] + ["qproj", "attn", "o_proj", "ffn", "down"] * L + ["post", "head"]
    got = [("attn" if n.startswith("attn_") and "merge" not in n else n) for n in names if "merge" not in n]
    assert got == per_step * 2 + ["final"], names
    assert all(ms > 0.0 for _, ms in recs)
    # after switching off, calls replay graphs again and add no records
    d.draft_block(2, case.th, case.tok, case.temb, case.kv, want_logits=True)
    torch.cuda.synchronize()
    assert len(d.timing_records()) == len(recs)
