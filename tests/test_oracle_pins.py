"""Pins of the CPU oracle to facts fixed outside itself: hand-computed values, closed forms, invariants, special cases
that reduce to a library routine, and brute force on tiny inputs. CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import softmax as sp_softmax

import oracle as O
from fixtures import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- number formats


def test_bf16_hand_values():
    # 1.0 = 0x3F80; 1 + 2^-8 is exactly halfway between 1.0 and 1 + 2^-7 -> ties to even -> 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (0x3F81, odd) and 1 + 2^-6 (0x3F82, even) -> 0x3F82
    vals = [1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.0, 0.0, 1.0 + 2.0 ** -7, 3.140625, -0.5]
    want = [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x0000, 0x3F81, 0x4049, 0xBF00]
    assert list(O.bf16_bits(np.array(vals))) == want
    assert np.array_equal(O.bf16_to_f64(np.array(want, dtype=np.uint16)),
                          np.array([1.0, 1.0, 1.0 + 2.0 ** -6, -2.0, 0.0, 1.0 + 2.0 ** -7, 3.140625, -0.5]))


def test_bf16_matches_torch_conversion():
    # torch's own fp32 -> bf16 conversion (round to nearest even) is an independent implementation
    x = rng(1).standard_normal(200000).astype(np.float32) * np.float32(3.0)
    ours = O.bf16_bits(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = torch.from_numpy(theirs.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_to_f64(theirs), back)


def test_mask_value_bits():
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    bits = int(g["mask_value_f32_bits"]["value"], 16)
    assert int(np.array([O.NEG_FILL_F32], np.float32).view(np.uint32)[0]) == bits
    assert float(O.NEG_FILL_F32) == pytest.approx(-1e30, rel=1e-7)


# ---------------------------------------------------------------- elementary ops


def test_rmsnorm_hand_and_closed_form():
    out = O.rmsnorm(np.array([3.0, 4.0]), np.ones(2), 0.0)  # mean square 12.5
    assert np.allclose(out, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    v = rng(2).standard_normal((5, 256)) * 7.0
    y = O.rmsnorm(v, np.ones(256), 1e-6)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-7)
    w = rng(3).standard_normal(256)
    assert np.allclose(O.rmsnorm(v, w, 1e-6), y * w)
    assert np.array_equal(O.rmsnorm(np.zeros(8), np.ones(8), 1e-6), np.zeros(8))


def test_gelu_tanh_against_exact_gelu():
    a = np.linspace(-8, 8, 4001)
    exact = np.array([0.5 * t * (1.0 + math.erf(t / math.sqrt(2.0))) for t in a])
    g = O.gelu_tanh(a)
    assert np.max(np.abs(g - exact)) < 1e-3       # the tanh form approximates the erf form to ~5e-4
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert abs(O.gelu_tanh(np.array([20.0]))[0] - 20.0) < 1e-12
    assert abs(O.gelu_tanh(np.array([-20.0]))[0]) < 1e-12
    # torch's tanh-approximate gelu (independent implementation)
    tg = torch.nn.functional.gelu(torch.from_numpy(a), approximate="tanh").numpy()
    assert np.allclose(g, tg, rtol=0, atol=1e-12)


def test_rope_is_complex_rotation():
    r = rng(4)
    q = r.standard_normal(64)
    ang = r.uniform(-10, 10, 32)
    out = O.rope_rotate(q, np.cos(ang), np.sin(ang))
    z = (q[:32] + 1j * q[32:]) * np.exp(1j * ang)
    assert np.allclose(out[:32], z.real) and np.allclose(out[32:], z.imag)
    assert np.allclose(O.rope_rotate(q, np.ones(32), np.zeros(32)), q)  # position 0 is the identity
    pair_norm = lambda v: v[:32] ** 2 + v[32:] ** 2  # noqa: E731
    assert np.allclose(pair_norm(out), pair_norm(q))


def test_key_window_cases():
    assert O.key_window(256, 512, False) == (0, 256)     # window wider than context: sliding == full
    assert O.key_window(4096, 512, False) == (3584, 4096)
    assert O.key_window(4096, 512, True) == (0, 4096)
    assert O.key_window(10, 1, False) == (9, 10)


def test_attention_closed_forms():
    r = rng(5)
    K = r.standard_normal((50, 16))
    V = r.standard_normal((50, 16))
    # q = 0: uniform weights -> mean of V
    assert np.allclose(O.attend(np.zeros(16), K, V, 0.25), V.mean(axis=0))
    # identical keys -> uniform weights
    Kc = np.tile(K[:1], (50, 1))
    assert np.allclose(O.attend(r.standard_normal(16), Kc, V, 0.25), V.mean(axis=0))
    # one key: that value
    assert np.allclose(O.attend(r.standard_normal(16), K[:1], V[:1], 0.25), V[0])
    # against scipy's softmax
    q = r.standard_normal(16)
    p = sp_softmax(0.25 * (K @ q))
    assert np.allclose(O.attend(q, K, V, 0.25), p @ V)
    # permutation of the key/value rows does not change the result
    perm = r.permutation(50)
    assert np.allclose(O.attend(q, K[perm], V[perm], 0.25), O.attend(q, K, V, 0.25))
    # a dominating key: the result tends to its value
    Kd = K.copy()
    Kd[17] = q * 100.0
    assert np.allclose(O.attend(q, Kd, V, 1.0), V[17], atol=1e-9)


def test_topk_matches_stable_sort_with_ties():
    r = rng(6)
    for trial in range(20):
        s = r.standard_normal(2048).astype(np.float32)
        # plant ties at the selection boundary and inside the selection
        order = np.argsort(-s, kind="stable")
        s[order[33]] = s[order[31]]
        s[order[5]] = s[order[4]]
        s = s.astype(np.float32)
        want = np.argsort(-s.astype(np.float64), kind="stable")[:32]
        assert np.array_equal(O.topk_desc(s, 32), want)


# ---------------------------------------------------------------- head


def _tiny_model(seed=0, **over):
    shape = synth.TINY
    if over:
        import dataclasses
        shape = dataclasses.replace(shape, **over)
    w = synth.make_weights(shape, seed=seed)
    return O.Model(O.config_from(shape), w), w, shape


def test_masked_head_invariants_and_dense_equality():
    m, w, shape = _tiny_model()
    cfg = m.cfg
    r = rng(7)
    for t in range(10):
        h = O.round_bf16(r.standard_normal(cfg.hidden))
        out = O.masked_head_row(m, h, want_row=True)
        row = out["row"]
        finite = row != O.NEG_FILL_F32
        assert finite.sum() == cfg.top_k * cfg.vsc
        assert np.all(row.view(np.uint32)[~finite] == 0xF149F2CA)
        blocks = np.asarray(w["token_ordering"]).reshape(cfg.n_centroids, cfg.vsc)[out["sel"]]
        assert set(np.nonzero(finite)[0].tolist()) == set(blocks.reshape(-1).tolist())
        assert len(set(out["ids"].tolist())) == len(out["ids"])
        # sparse logits equal the brute-force dense product at the selected ids
        dense = np.array([sum(float(a) * float(b) for a, b in zip(O.bf16_to_f64(m.head_bits[i]), h))
                          for i in range(cfg.vocab)])
        assert np.allclose(row[finite], dense[finite].astype(np.float32), rtol=1e-6, atol=1e-7)
        assert out["next"] == int(np.argmax(np.where(finite, dense, -np.inf)))
        # the selected clusters are the top-k by brute-force centroid scores
        cs = np.array([np.dot(O.bf16_to_f64(np.asarray(w["centroids"]).view(np.uint16)[c]), h)
                       for c in range(cfg.n_centroids)]).astype(np.float32)
        assert set(out["sel"].tolist()) == set(np.argsort(-cs.astype(np.float64), kind="stable")[:cfg.top_k].tolist())


def test_masked_head_all_clusters_equals_dense_argmax():
    m, w, shape = _tiny_model(top_k=8)  # k == n_centroids: every token is scored
    r = rng(8)
    for t in range(10):
        h = O.round_bf16(r.standard_normal(m.cfg.hidden))
        out = O.masked_head_row(m, h, want_row=True)
        dense = O.dense_head_row(m, h)
        assert np.array_equal(out["row"], dense)
        assert out["next"] == int(np.argmax(dense))


def test_head_invariant_checks_reject_bad_inputs():
    m, w, shape = _tiny_model()
    cfg = m.cfg
    bad = np.asarray(w["token_ordering"]).copy()
    bad[3] = bad[4]
    with pytest.raises(ValueError):
        O.check_head_invariants(cfg, bad)
    import dataclasses
    with pytest.raises(ValueError):
        O.check_head_invariants(dataclasses.replace(cfg, n_centroids=7), np.asarray(w["token_ordering"]))
    with pytest.raises(ValueError):
        O.check_head_invariants(dataclasses.replace(cfg, top_k=9), np.asarray(w["token_ordering"]))


def test_argmax_tie_goes_to_lowest_token():
    m, w, shape = _tiny_model()
    cfg = m.cfg
    # make every head row identical: all selected logits tie; the lowest selected token id must win
    m.head_bits = np.tile(m.head_bits[:1], (cfg.vocab, 1))
    h = O.round_bf16(rng(9).standard_normal(cfg.hidden))
    out = O.masked_head_row(m, h)
    assert out["next"] == int(np.min(out["ids"]))


# ---------------------------------------------------------------- sampling


def test_sample_row_closed_form_weights():
    """Logits T*log(w) at temperature T give p = w / sum(w) exactly in the limit of exact arithmetic (softmax of
    log-weights): with w = 1, 2, 3, 4 the CDF steps are at 0.1, 0.3, 0.6, 1.0, so u picks the token whose interval
    holds it, in the given order."""
    order = np.array([907, 3, 55, 12])
    for T in (0.5, 1.0, 3.0):
        vals = (T * np.log([1.0, 2.0, 3.0, 4.0])).astype(np.float32)
        for u, want, pw in ((0.0, 907, 0.1), (0.05, 907, 0.1), (0.15, 3, 0.2), (0.35, 55, 0.3), (0.65, 12, 0.4),
                            (0.999999, 12, 0.4)):
            r = O.sample_row(vals, order, T, u)
            assert r["token"] == want and abs(r["prob"] - pw) < 1e-6
        r = O.sample_row(vals, order, T, 0.3 + 1e-3)
        assert r["token"] == 55 and abs(r["cdf_margin"] - 1e-3) < 1e-6


def test_sample_row_uniform_and_peaked_limits():
    order = np.arange(100, 140)
    flat = np.full(40, 0.37, np.float32)
    for u in (0.0, 0.013, 0.51, 0.987, 0.99999):  # off the CDF steps at multiples of 1/40
        r = O.sample_row(flat, order, 0.8, u)
        assert r["token"] == order[int(u * 40)] and abs(r["prob"] - 1 / 40) < 1e-12
    # a tiny temperature puts all mass on the maximum (lowest position on ties) for any u
    vals = rng(40).standard_normal(40).astype(np.float32)
    for u in (0.0, 0.5, 0.999999):
        r = O.sample_row(vals, order, 1e-6, u)
        assert r["token"] == order[int(np.argmax(vals))] and r["prob"] == 1.0
    # masked entries (-1e30) are never drawn, whatever u
    vals2 = vals.copy()
    vals2[::2] = O.NEG_FILL_F32
    for u in np.linspace(0, 0.999999, 50):
        assert (O.sample_row(vals2, order, 1.0, u)["token"] - 100) % 2 == 1


def test_sample_frequencies_match_probabilities_on_a_grid():
    """Inverse-CDF sampling over a fine grid of u reproduces each token's probability to within the grid step."""
    vals = rng(41).standard_normal(12).astype(np.float32)
    order = np.arange(12)
    N = 20000
    counts = np.zeros(12)
    probs = {}
    for k in range(N):
        r = O.sample_row(vals, order, 0.9, (k + 0.5) / N)
        counts[r["token"]] += 1
        probs[r["token"]] = r["prob"]
    for t, pr in probs.items():
        assert abs(counts[t] / N - pr) <= 1.0 / N + 1e-12
    assert abs(sum(probs.values()) - 1.0) < 1e-12 and len(probs) == 12


def test_head_order_masked_and_dense():
    m, w, shape = _tiny_model()
    sel = np.array([5, 1, 6])
    order = O.head_order(m, sel)
    blocks = np.asarray(w["token_ordering"]).reshape(shape.n_centroids, shape.vsc)
    assert np.array_equal(order, np.concatenate([blocks[1], blocks[5], blocks[6]]))
    md, _, _ = _tiny_model(n_centroids=0, top_k=1)
    assert np.array_equal(O.head_order(md, None), np.arange(shape.vocab))


def test_sampled_step_at_tiny_temperature_is_the_argmax_step():
    m, w, shape = _tiny_model()
    wl, d, kv = _tiny_inputs(shape, batch=3)
    th = d["target_hidden"].numpy().view(np.uint16)
    emb = d["target_embd"].numpy().view(np.uint16)
    tok = d["last_token"].numpy()
    ref = O.drafter_step(m, th, tok, emb, kv)
    got = O.drafter_step(m, th, tok, emb, kv, temperature=1e-6, uniforms=[0.3, 0.9, 0.0])
    for b in range(3):
        if ref["margin"][b] > 1e-3:
            assert got["next"][b] == ref["next"][b] and got["prob"][b] == 1.0
    assert np.array_equal(got["hidden_out"], ref["hidden_out"])


# ---------------------------------------------------------------- whole step


def _tiny_inputs(shape, batch=3, context=40, ragged=True, seed=0):
    wl = synth.Workload("tiny", shape, batch=batch, context=context, n_steps=3, ragged=ragged, seed=seed)
    d = synth.make_inputs(wl)
    kv = O.SharedKV(k=[d["k_sliding"].numpy().view(np.uint16), d["k_full"].numpy().view(np.uint16)],
                    v=None, lens=[d["len_sliding"], d["len_full"]], rope=d["rope"].numpy())
    kv.v = kv.k
    return wl, d, kv


def test_layer_scalar_zero_branch_closed_form():
    """With attn_output = ffn_down = 0 every branch adds RMSNorm(0) = 0, so the residual stream leaving the last
    layer is pre_projection(x0) times the product of the per-layer scalars."""
    m, w, shape = _tiny_model()
    for L in m.layers:
        L["o"][:] = 0.0
        L["down"][:] = 0.0
    wl, d, kv = _tiny_inputs(shape)
    th = d["target_hidden"].numpy().view(np.uint16)
    emb = d["target_embd"].numpy().view(np.uint16)
    b = 1
    x0 = np.concatenate([O.bf16_to_f64(th[b]), O.bf16_to_f64(emb[int(d["last_token"][b])])])
    x = m.pre @ x0
    want = x * np.prod([L["scale"] for L in m.layers])
    for l in range(m.cfg.n_layer):
        x = O.decoder_layer(m, l, x, b, kv)
    assert np.allclose(x, want, rtol=1e-13, atol=0)


def test_gqa_head_mapping_through_the_layer():
    """n_kv = 2, n_head = 4: query heads 0-1 read kv head 0 and heads 2-3 kv head 1. Kv head 1 holds one repeated key
    (K = V), so heads 2 and 3 return that key whatever their query, while kv head 0 keeps random keys. With the
    columns of attn_output that read heads 0-1 set to zero and the FFN branch zeroed, decoder_layer must equal the
    closed form (x + RMSNorm(W_o [.. ; c ; c], post_attention_norm)) * s for every layer and row; a head mapping
    that sent head 2 or 3 to kv head 0 would read random keys there."""
    m, w, shape = _tiny_model(n_kv_head=2)
    wl, d, kv = _tiny_inputs(shape)
    cfg = m.cfg
    for t in range(2):
        kv.k[t][:, 1] = kv.k[t][:, 1, :1]
    kv.v = kv.k
    hd = cfg.head_dim
    x = rng(10).standard_normal(cfg.hidden)
    for l in range(cfg.n_layer):
        L = m.layers[l]
        L["down"][:] = 0.0
        L["o"][:, :2 * hd] = 0.0
        t = 1 if cfg.is_full(l) else 0
        for b in range(3):
            c = O.bf16_to_f64(kv.k[t][b, 1, 0])
            o = np.concatenate([np.zeros(2 * hd), c, c])
            want = (x + O.rmsnorm(L["o"] @ o, L["post_attn_norm"], cfg.rms_eps)) * L["scale"]
            assert np.allclose(O.decoder_layer(m, l, x, b, kv), want, rtol=1e-12, atol=1e-12), (l, b)


def test_window_one_returns_last_key():
    m, w, shape = _tiny_model(swa_window=1)
    wl, d, kv = _tiny_inputs(shape)
    b = 2
    a0, a1 = O.key_window(kv.lens[0][b], 1, False)
    K = O.bf16_to_f64(kv.k[0][b, 0, a0:a1])
    assert K.shape[0] == 1
    o = O.attend(rng(11).standard_normal(shape.head_dim), K, K, 0.125)
    assert np.array_equal(o, O.bf16_to_f64(kv.k[0][b, 0, kv.lens[0][b] - 1]))


def test_concat_order_metamorphic():
    """Swapping the two input halves together with the two column blocks of pre_projection leaves the step
    unchanged: the hidden state is paired with the first backbone-wide block of pre_projection's input."""
    m, w, shape = _tiny_model()
    wl, d, kv = _tiny_inputs(shape, batch=2)
    th = d["target_hidden"].numpy().view(np.uint16)
    emb = d["target_embd"].numpy().view(np.uint16)
    tok = d["last_token"].numpy()
    ref = O.drafter_step(m, th, tok, emb, kv)
    Bb = shape.backbone
    m2 = O.Model(m.cfg, w)
    m2.pre = np.concatenate([m.pre[:, Bb:], m.pre[:, :Bb]], axis=1)
    emb2 = emb.copy()
    th2 = th.copy()
    for b in range(2):  # token b's embedding row becomes the hidden input and vice versa
        emb2[int(tok[b])] = th[b]
        th2[b] = emb[int(tok[b])]
    got = O.drafter_step(m2, th2, tok, emb2, kv)
    assert np.array_equal(got["hidden_out"], ref["hidden_out"])
    assert np.array_equal(got["next"], ref["next"])


def test_draft_block_equals_chained_steps():
    m, w, shape = _tiny_model()
    wl, d, kv = _tiny_inputs(shape)
    th = d["target_hidden"].numpy().view(np.uint16)
    emb = d["target_embd"].numpy().view(np.uint16)
    tok = d["last_token"].numpy()
    blk = O.draft_block(m, 3, th, tok, emb, kv)
    cur_h, cur_t = th.copy(), tok.copy()
    for i in range(3):
        s = O.drafter_step(m, cur_h, cur_t, emb, kv)
        assert np.array_equal(s["hidden_out"], blk[i]["hidden_out"])
        assert np.array_equal(s["next"], blk[i]["next"])
        cur_h, cur_t = s["hidden_out"], s["next"]


def test_left_padded_and_ring_caches_equal_the_linear_cache():
    """The same keys stored left-padded (row b's keys after pad_b junk slots) or in a ring-buffer sliding cache
    (capacity 24 >= window, position p in slot p mod 24, oldest slot first) give bit-identical steps: only the slot
    of each key changes, and the keys are gathered oldest first."""
    m, w, shape = _tiny_model()
    wl, d, kv = _tiny_inputs(shape, batch=3, context=40, ragged=True)
    th = d["target_hidden"].numpy().view(np.uint16)
    emb = d["target_embd"].numpy().view(np.uint16)
    tok = d["last_token"].numpy()
    ref = O.drafter_step(m, th, tok, emb, kv)
    r = rng(30)
    B, nkv, cap, hd = kv.k[0].shape
    # left padding: pad_b junk slots, then the row's keys; both caches
    pads = [5, 0, 11]
    padded, firsts = [], []
    for t in range(2):
        big = r.integers(0, 1 << 16, size=(B, nkv, cap + 11, hd), dtype=np.uint16)
        for b in range(B):
            L = int(kv.lens[t][b])
            big[b, :, pads[b]:pads[b] + L] = kv.k[t][b, :, :L]
        padded.append(big)
        firsts.append(pads)
    kvp = O.SharedKV(k=padded, v=padded, lens=kv.lens, rope=kv.rope, first=firsts)
    got = O.drafter_step(m, th, tok, emb, kvp)
    assert np.array_equal(got["hidden_out"], ref["hidden_out"]) and np.array_equal(got["next"], ref["next"])
    # ring-buffer sliding cache of 24 slots holding the last 24 positions of each row
    C = 24
    ring = r.integers(0, 1 << 16, size=(B, nkv, C, hd), dtype=np.uint16)
    rlen, rfirst = [], []
    for b in range(B):
        L = int(kv.lens[0][b])
        n = min(L, C)
        for p in range(L - n, L):
            ring[b, :, p % C] = kv.k[0][b, :, p]
        rlen.append(n)
        rfirst.append((L - n) % C)
    kvr = O.SharedKV(k=[ring, kv.k[1]], v=[ring, kv.k[1]], lens=[rlen, kv.lens[1]], rope=kv.rope,
                     first=[rfirst, [0] * B])
    got = O.drafter_step(m, th, tok, emb, kvr)
    assert any(f + n > C for f, n in zip(rfirst, rlen))  # at least one row wraps around the end
    assert np.array_equal(got["hidden_out"], ref["hidden_out"]) and np.array_equal(got["next"], ref["next"])
    with pytest.raises(ValueError):
        O.SharedKV(k=[ring, kv.k[1]], v=[ring, kv.k[1]], lens=[[C + 1] * B, kv.lens[1]], rope=kv.rope).slots(0, 0, 0, 3)


def test_shared_cache_equals_per_row_copies():
    """One cache read by every row (each row with its own length, token and position) gives exactly the step of
    per-row caches that are all copies of that cache."""
    m, w, shape = _tiny_model()
    wl, d, kv = _tiny_inputs(shape, batch=3, context=40, ragged=True)
    th = d["target_hidden"].numpy().view(np.uint16)
    emb = d["target_embd"].numpy().view(np.uint16)
    tok = d["last_token"].numpy()
    one = [kv.k[t][:1].copy() for t in range(2)]
    copies = [np.repeat(one[t], 3, axis=0) for t in range(2)]
    ref = O.drafter_step(m, th, tok, emb, O.SharedKV(k=copies, v=copies, lens=kv.lens, rope=kv.rope))
    got = O.drafter_step(m, th, tok, emb, O.SharedKV(k=one, v=one, lens=kv.lens, rope=kv.rope, shared=[True, True]))
    assert np.array_equal(got["hidden_out"], ref["hidden_out"]) and np.array_equal(got["next"], ref["next"])
    # and it differs from the rows' own caches (rows 1, 2 read row 0's keys)
    own = O.drafter_step(m, th, tok, emb, kv)
    assert not np.array_equal(own["hidden_out"][1:], got["hidden_out"][1:])


def test_step_rows_are_independent():
    m, w, shape = _tiny_model()
    wl, d, kv = _tiny_inputs(shape)
    th = d["target_hidden"].numpy().view(np.uint16)
    emb = d["target_embd"].numpy().view(np.uint16)
    tok = d["last_token"].numpy()
    full = O.drafter_step(m, th, tok, emb, kv)
    one = O.drafter_step(m, th, tok, emb, kv, rows=[2])
    assert np.array_equal(one["hidden_out"][0], full["hidden_out"][2])
    assert one["next"][0] == full["next"][2]


def test_dense_step_equals_masked_step_with_every_cluster():
    """The dense tied head scores every token; the masked head with top_k = n_centroids also scores every token
    (no -1e30 entries), so on the same weights the two steps must agree in hidden state, token and whole row."""
    shape_m = __import__("dataclasses").replace(synth.TINY, top_k=synth.TINY.n_centroids)
    wm = synth.make_weights(shape_m, seed=3)
    wd = synth.make_weights(synth.TINY_DENSE, seed=3)
    assert "centroids" not in wd and "token_ordering" not in wd
    for k in wd:
        if k != "layers":
            assert torch.equal(wd[k], wm[k]), k
    mm, md = O.Model(O.config_from(shape_m), wm), O.Model(O.config_from(synth.TINY_DENSE), wd)
    wl, d, kv = _tiny_inputs(synth.TINY_DENSE, batch=4)
    th = d["target_hidden"].numpy().view(np.uint16)
    emb = d["target_embd"].numpy().view(np.uint16)
    tok = d["last_token"].numpy()
    a = O.drafter_step(mm, th, tok, emb, kv, want_rows=True)
    b = O.drafter_step(md, th, tok, emb, kv, want_rows=True)
    assert np.array_equal(a["hidden_out"], b["hidden_out"])
    assert np.array_equal(a["next"], b["next"])
    for ra, rb, mg in zip(a["row"], b["row"], b["margin"]):
        assert np.array_equal(ra, rb)
        srt = np.sort(rb.astype(np.float64))
        assert mg == srt[-1] - srt[-2]
    assert all(len(x) == 0 for x in b["sel"]) and all(len(x) == 0 for x in b["ids"])


def test_dense_head_one_hot_table_closed_form():
    """Head row i = unit vector e_(i mod H): the logit of token i is h[i mod H]. The argmax is the first index of
    max(h) (it recurs every H tokens; the lowest token id wins) and the top-1 minus top-2 margin is 0."""
    m, w, shape = _tiny_model(n_centroids=0, top_k=1)
    H, V = m.cfg.hidden, m.cfg.vocab
    bits = np.zeros((V, H), np.uint16)
    bits[np.arange(V), np.arange(V) % H] = 0x3F80  # bf16 1.0
    m.head_bits = bits
    for t in range(5):
        h = O.round_bf16(rng(20 + t).standard_normal(H))
        out = O.dense_head_result(m, h)
        assert np.array_equal(out["row"], h[np.arange(V) % H].astype(np.float32))
        assert out["next"] == int(np.argmax(h)) and out["next"] < H
        assert out["margin"] == 0.0


# ---------------------------------------------------------------- shapes named on the pages


def _param_count(shape):
    H, Bb, F, Q, hd = shape.hidden, shape.backbone, shape.ffn, shape.q_dim, shape.head_dim
    per_layer = Q * H + hd + H * Q + 4 * H + 3 * F * H + 1
    return 2 * Bb * H + H * Bb + H + shape.vocab * H + shape.n_centroids * H + shape.n_layer * per_layer


def test_page_constants_against_workload_shapes():
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    for shape in (synth.E2B, synth.E4B):
        assert shape.vocab == g["vocab"]["value"]
        assert shape.n_centroids == g["n_centroids"]["value"]
        assert shape.top_k == g["top_k"]["value"]
        assert shape.hidden == g["hidden"]["value"]
        assert shape.n_layer == g["n_layer"]["value"]
        assert shape.top_k * shape.vsc == 4096  # finite logits per row
        # the pages quote about 76-78 M parameters; our FFN width (1024) gives ~74-75 M
        assert abs(_param_count(shape) - g["params_approx_e2b_e4b"]["value"]) < 0.06 * g["params_approx_e2b_e4b"]["value"]
    assert synth.E26B.backbone == g["backbone_26b"]["value"]
    assert synth.E26B.vocab == g["vocab"]["value"] and synth.E26B.n_layer == g["n_layer"]["value"]
    assert synth.E26B.dense_head and synth.E26B.q_dim == 8 * 256
    assert synth.E2B.backbone == g["backbone_e2b"]["value"]
    assert synth.E4B.backbone == g["backbone_e4b"]["value"]


def test_full_size_ordering_and_head_row():
    shape = synth.E4B
    perm = synth.permutation(0, synth.TID["ordering"], shape.vocab).numpy()
    cfg = O.config_from(shape)
    O.check_head_invariants(cfg, perm)
    assert perm.max() < (1 << 18)
    assert np.array_equal(perm.astype(np.float32).astype(np.int64), perm)  # exact in F32


# ---------------------------------------------------------------- the input generator (shared with the GPU side)


def test_generator_rows_match_full_tensor_and_distribution():
    full = synth.gen_bf16(0, 77, (64, 96), 1.0)
    rows = torch.tensor([3, 0, 63, 17])
    part = synth.gen_bf16(0, 77, (64, 96), 1.0, row_index=rows)
    assert torch.equal(part, full[rows])
    v = O.bf16_to_f64(synth.gen_bf16(0, 78, (1 << 18,), 2.0).numpy())
    assert abs(v.mean()) < 0.02 and abs(v.std() - 2.0) < 0.02


# ---------------------------------------------------------------- structure of the decoder layer


def test_sandwich_norm_scale_invariance():
    """The sandwich norms make a layer's output independent of the scale of q_proj (q_norm), o_proj
    (post_attention_norm), ffn_down (post_ffw_norm) and, since GeGLU is linear in the up branch, of ffn_up. With
    eps = 0 and a factor of 2 (exact in bf16) the invariance is exact. A dropped norm, or gelu applied to the up branch
    instead of the gate branch, breaks it."""
    m, w, shape = _tiny_model(rms_eps=0.0)
    wl, d, kv = _tiny_inputs(shape)
    x = rng(12).standard_normal(shape.hidden)
    for l in range(shape.n_layer):
        ref = O.decoder_layer(m, l, x, 1, kv)
        for key in ("q", "o", "down", "up"):
            saved = m.layers[l][key].copy()
            m.layers[l][key] = saved * 2.0
            got = O.decoder_layer(m, l, x, 1, kv)
            m.layers[l][key] = saved
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), (l, key)
        # the gate branch is not scale invariant (gelu is not homogeneous): a check that the test can fail
        saved = m.layers[l]["gate"].copy()
        m.layers[l]["gate"] = saved * 2.0
        assert not np.allclose(O.decoder_layer(m, l, x, 1, kv), ref, rtol=1e-6)
        m.layers[l]["gate"] = saved


def test_attention_branch_closed_form_with_identical_keys():
    """If every key of a kv head equals k (K = V), each query head reading it returns k whatever its query. With the
    FFN branch zeroed, a layer then maps x to (x + RMSNorm(W_o [o_0;..;o_{n-1}], post_attention_norm)) * s with
    o_h the constant key of head h's kv head: this pins the head-to-kv mapping, the head concatenation order and the
    post-attention norm weight."""
    m, w, shape = _tiny_model(n_kv_head=2)
    wl, d, kv = _tiny_inputs(shape)
    cfg = m.cfg
    for t in range(2):
        kv.k[t][:, 0] = kv.k[t][:, 0, :1]
        kv.k[t][:, 1] = kv.k[t][:, 1, :1]
    kv.v = kv.k
    x = rng(13).standard_normal(cfg.hidden)
    for l in range(cfg.n_layer):
        m.layers[l]["down"][:] = 0.0
        t = 1 if cfg.is_full(l) else 0
        b = 2
        k0 = O.bf16_to_f64(kv.k[t][b, 0, 0])
        k1 = O.bf16_to_f64(kv.k[t][b, 1, 0])
        o = np.concatenate([k0, k0, k1, k1])  # heads 0,1 -> kv 0; heads 2,3 -> kv 1
        L = m.layers[l]
        want = (x + O.rmsnorm(L["o"] @ o, L["post_attn_norm"], cfg.rms_eps)) * L["scale"]
        got = O.decoder_layer(m, l, x, b, kv)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12), l


# ---------------------------------------------------------------- the query path, the softmax scale and the norm roles
# Metamorphic relations through decoder_layer / drafter_step: each transforms an input in a way the method's
# definition says must (or must not) change the result, with factors of 2 and quarter turns that are exact in bf16
# and fp64, so that equalities are exact.


def _distinct_v_inputs(shape, batch=3, context=40, seed=0):
    """Tiny inputs whose caches carry a V distinct from K (the attention output then shows what was read as V)."""
    wl = synth.Workload("tiny", shape, batch=batch, context=context, n_steps=1, ragged=True, seed=seed)
    d = synth.make_inputs(wl, distinct_v=True)
    u16 = lambda t: t.numpy().view(np.uint16).copy()  # noqa: E731
    kv = O.SharedKV(k=[u16(d["k_sliding"]), u16(d["k_full"])], v=[u16(d["v_sliding"]), u16(d["v_full"])],
                    lens=[d["len_sliding"], d["len_full"]], rope=d["rope"].numpy().copy())
    return d, kv


def _quarter_turn_tables(B, half, seed):
    """Per-row, per-type rotary tables whose angles are multiples of pi/2 (cos, sin in {0, +1, -1}, so a rotation of
    bf16 values is exact), different for the sliding and the full type."""
    r = rng(seed)
    k = r.integers(0, 4, size=(B, 2, half))
    while np.array_equal(k[:, 0], k[:, 1]) or np.all(k % 2 == 0):
        k = r.integers(0, 4, size=(B, 2, half))
    tab = np.zeros((B, 2, 2, half), np.float32)
    tab[:, :, 0] = np.array([1, 0, -1, 0], np.float32)[k]  # cos(k pi/2)
    tab[:, :, 1] = np.array([0, 1, 0, -1], np.float32)[k]  # sin(k pi/2)
    return tab


def _rotate_back_bits(bits, cos, sin):
    """bf16 keys rotated by minus the angle of (cos, sin) on the half-split pairs (i, i + d/2): (a, b) ->
    (a cos + b sin, b cos - a sin). With cos, sin in {0, +-1} every output is +-a or +-b, so the result is exact."""
    v = O.bf16_to_f64(bits)
    d2 = v.shape[-1] // 2
    a, b = v[..., :d2], v[..., d2:]
    c, s = cos.astype(np.float64), sin.astype(np.float64)
    out = np.concatenate([a * c + b * s, b * c - a * s], axis=-1)
    res = O.bf16_bits(out)
    assert np.array_equal(O.bf16_to_f64(res), out)
    return res


def test_rope_rotates_the_normed_query_with_its_type_table():
    """The score of a query rotated by R(theta) against key k equals the unrotated query against R(-theta) k. So a
    layer whose rotary tables hold angles theta (one table per attention type, per row) must equal the same layer
    with identity tables (cos 1, sin 0) over keys rotated by -theta of their type, V unchanged. This pins that RoPE is
    applied (to q only), after q_norm (the q_norm weight is not symmetric between the two halves of a pair, so norming
    the rotated query differs), and with the table of the layer's own type (the two types' angles differ)."""
    m, w, shape = _tiny_model()
    d, kv = _distinct_v_inputs(shape)
    cfg = m.cfg
    B, half = 3, cfg.head_dim // 2
    for L in m.layers:
        assert not np.allclose(L["q_norm"][:half], L["q_norm"][half:])
    kv.rope = _quarter_turn_tables(B, half, seed=31)
    ident = np.zeros_like(kv.rope)
    ident[:, :, 0] = 1.0
    rot = []
    for t in range(2):
        kt = kv.k[t].copy()
        for b in range(B):
            kt[b] = _rotate_back_bits(kv.k[t][b], kv.rope[b, t, 0], kv.rope[b, t, 1])
        rot.append(kt)
    kv_b = O.SharedKV(k=rot, v=kv.v, lens=kv.lens, rope=ident)
    kv_c = O.SharedKV(k=kv.k, v=kv.v, lens=kv.lens, rope=ident)
    x = rng(32).standard_normal(cfg.hidden)
    for l in range(cfg.n_layer):
        for b in range(B):
            a_ = O.decoder_layer(m, l, x, b, kv)
            b_ = O.decoder_layer(m, l, x, b, kv_b)
            assert np.allclose(a_, b_, rtol=1e-12, atol=1e-12), (l, b)
            # control: the rotation does change the layer (the relation is not vacuous) wherever the window holds
            # more than one key (a single key is returned whatever the query)
            if kv.lens[1 if cfg.is_full(l) else 0][b] > 1:
                assert not np.allclose(a_, O.decoder_layer(m, l, x, b, kv_c), rtol=1e-6), (l, b)


def test_softmax_scale_multiplies_the_scores():
    """Doubling every key (exact in bf16) and halving attn_scale leaves each score, and so the layer, bit for bit
    unchanged (V distinct from K, so V is not doubled); changing attn_scale alone changes the layer."""
    m, w, shape = _tiny_model()
    d, kv = _distinct_v_inputs(shape)
    cfg = m.cfg
    k2 = [O.bf16_bits(2.0 * O.bf16_to_f64(kv.k[t])) for t in range(2)]
    kv2 = O.SharedKV(k=k2, v=kv.v, lens=kv.lens, rope=kv.rope)
    import dataclasses
    m_half = O.Model(dataclasses.replace(cfg, attn_scale=cfg.attn_scale / 2), w)
    m_dbl = O.Model(dataclasses.replace(cfg, attn_scale=cfg.attn_scale * 2), w)
    x = rng(33).standard_normal(cfg.hidden)
    for l in range(cfg.n_layer):
        for b in range(3):
            ref = O.decoder_layer(m, l, x, b, kv)
            assert np.array_equal(O.decoder_layer(m_half, l, x, b, kv2), ref), (l, b)
            if kv.lens[1 if cfg.is_full(l) else 0][b] > 1:  # one key: the scale cannot matter
                assert not np.allclose(O.decoder_layer(m_dbl, l, x, b, kv), ref, rtol=1e-6), (l, b)


def test_sandwich_norm_weight_roles():
    """Which norm weight feeds which branch. With eps = 0: doubling attn_norm's weight doubles q, which q_norm
    removes exactly, so the layer is bit-identical; doubling ffn_norm's weight doubles the GeGLU inputs (gelu is not
    homogeneous), so the layer changes; doubling post_attention_norm or post_ffw_norm doubles that branch's
    contribution. Permuting attn_norm's weight (not a scalar multiple) changes q, so the layer changes."""
    m, w, shape = _tiny_model(rms_eps=0.0)
    d, kv = _distinct_v_inputs(shape)
    x = rng(34).standard_normal(shape.hidden)
    for l in range(shape.n_layer):
        L = m.layers[l]
        for b in range(3):
            ref = O.decoder_layer(m, l, x, b, kv)
            for key, same in (("attn_norm", True), ("ffn_norm", False), ("post_attn_norm", False),
                              ("post_ffw_norm", False)):
                saved = L[key].copy()
                L[key] = saved * 2.0
                got = O.decoder_layer(m, l, x, b, kv)
                L[key] = saved
                if same:
                    assert np.array_equal(got, ref), (l, b, key)
                else:
                    assert not np.allclose(got, ref, rtol=1e-6), (l, b, key)
            if kv.lens[1 if shape.is_full(l) else 0][b] > 1:  # one key: q cannot matter
                saved = L["attn_norm"].copy()
                L["attn_norm"] = saved[::-1].copy()
                assert not np.allclose(O.decoder_layer(m, l, x, b, kv), ref, rtol=1e-6), (l, b)
                L["attn_norm"] = saved


def _step_inputs(shape, batch=3):
    wl, d, kv = _tiny_inputs(shape, batch=batch)
    return (d["target_hidden"].numpy().view(np.uint16), d["last_token"].numpy(),
            d["target_embd"].numpy().view(np.uint16), kv)


def test_output_norm_feeds_post_projection_and_the_head():
    """h = RMSNorm(x, output_norm) feeds both post_projection and the head. With eps = 0, doubling the last layer's
    scalar doubles x, which the output norm removes exactly: hidden_out, the selected clusters, the ids, the sparse
    logits and the token are bit-identical. Doubling output_norm's weight doubles h: hidden_out and the sparse
    logits double exactly (bf16 and fp32 scale exactly by 2), selections and token are unchanged."""
    m, w, shape = _tiny_model(rms_eps=0.0)
    th, tok, emb, kv = _step_inputs(shape)
    ref = O.drafter_step(m, th, tok, emb, kv)
    m.layers[-1]["scale"] *= 2.0
    got = O.drafter_step(m, th, tok, emb, kv)
    m.layers[-1]["scale"] /= 2.0
    assert np.array_equal(got["hidden_out"], ref["hidden_out"])
    for b in range(3):
        for key in ("sel", "ids", "z"):
            assert np.array_equal(got[key][b], ref[key][b]), (b, key)
    assert np.array_equal(got["next"], ref["next"])
    m.out_norm = m.out_norm * 2.0
    got = O.drafter_step(m, th, tok, emb, kv)
    assert np.array_equal(O.bf16_to_f64(got["hidden_out"]), 2.0 * O.bf16_to_f64(ref["hidden_out"]))
    for b in range(3):
        assert np.array_equal(got["sel"][b], ref["sel"][b]) and np.array_equal(got["ids"][b], ref["ids"][b])
        assert np.array_equal(got["z"][b], np.float32(2.0) * ref["z"][b])
    assert np.array_equal(got["next"], ref["next"])


def test_embed_scale_multiplies_the_embedded_token():
    """embed_scale = 2 over the target table E gives the same step, bit for bit, as embed_scale = 1 over the table
    2E (exact in bf16); embed_scale = 2 alone changes the step."""
    m, w, shape = _tiny_model()
    th, tok, emb, kv = _step_inputs(shape)
    import dataclasses
    m2 = O.Model(dataclasses.replace(m.cfg, embed_scale=2.0), w)
    emb2 = O.bf16_bits(2.0 * O.bf16_to_f64(emb))
    a = O.drafter_step(m2, th, tok, emb, kv)
    b = O.drafter_step(m, th, tok, emb2, kv)
    assert np.array_equal(a["hidden_out"], b["hidden_out"]) and np.array_equal(a["next"], b["next"])
    ref = O.drafter_step(m, th, tok, emb, kv)
    assert not np.array_equal(a["hidden_out"], ref["hidden_out"])


def test_distinct_values_are_read_as_v():
    """With every key of a row equal (uniform softmax weights) and a distinct V, each head returns the mean of V
    over the row's key window (np.mean over the window's rows: the window of the layer's type); with the FFN branch
    zeroed the layer is (x + RMSNorm(W_o [o_0; ..], post_attention_norm)) * s."""
    m, w, shape = _tiny_model()
    d, kv = _distinct_v_inputs(shape)
    cfg = m.cfg
    for t in range(2):
        kv.k[t][:] = kv.k[t][:, :, :1]
    x = rng(35).standard_normal(cfg.hidden)
    for l in range(cfg.n_layer):
        L = m.layers[l]
        L["down"][:] = 0.0
        t = 1 if cfg.is_full(l) else 0
        for b in range(3):
            n = int(kv.lens[t][b])
            a0 = 0 if t == 1 else n - min(cfg.swa_window, n)
            mean_v = O.bf16_to_f64(kv.v[t][b, 0, a0:n]).mean(axis=0)
            o = np.tile(mean_v, cfg.n_head)
            want = (x + O.rmsnorm(L["o"] @ o, L["post_attn_norm"], cfg.rms_eps)) * L["scale"]
            assert np.allclose(O.decoder_layer(m, l, x, b, kv), want, rtol=1e-12, atol=1e-12), (l, b)
