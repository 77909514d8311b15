"""The allocation-free entry point (mtpd_drafter_step_noalloc) against mtpd_drafter_step on the same inputs, through
the C ABI: two calls in a row on one device, the second with a smaller batch, each bit-identical to the entry point
with a caller workspace (the same kernels run on the same inputs). Also its size limit, checked on the host."""
import sys

import numpy as np
import pytest
import torch

from fixtures import synth
from parity import Case

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


def _outputs(case, B):
    sh = case.shape
    kv_n = sh.top_k * sh.vocab // sh.n_centroids
    return {"next": torch.full((B,), -7, dtype=torch.int32, device="cuda"),
            "hidden_out": torch.zeros(B, sh.backbone, dtype=torch.int16, device="cuda"),
            "logits": torch.zeros(B, sh.vocab, dtype=torch.float32, device="cuda"),
            "sel": torch.zeros(B, sh.top_k, dtype=torch.int32, device="cuda"),
            "ids": torch.zeros(B, kv_n, dtype=torch.int32, device="cuda"),
            "z": torch.zeros(B, kv_n, dtype=torch.float32, device="cuda")}


def test_noalloc_step_matches_the_workspace_entry_point():
    from mtp_drafter_step_amd import abi
    big = Case(synth.E4B, batch=16, context=2048, ragged=True, seed=0)
    small = Case(synth.E2B, batch=5, context=700, ragged=True, seed=1)
    got = []
    for case, B in ((big, 16), (small, 5)):
        say(f"noalloc batch {B} backbone {case.shape.backbone}")
        o = _outputs(case, B)
        case.drafter.drafter_step_noalloc(case.th, case.tok, case.temb, case.kv, o)
        torch.cuda.synchronize()
        got.append({k: v.clone() for k, v in o.items()})
    for (case, B), g in zip(((big, 16), (small, 5)), got):
        ref = case.drafter.drafter_step(case.th, case.tok, case.temb, case.kv, want_logits=True, want_sparse=True)
        torch.cuda.synchronize()
        for k in ("next", "hidden_out", "sel", "ids", "z", "logits"):
            assert torch.equal(g[k].view(torch.int32) if g[k].dtype == torch.float32 else g[k],
                               ref[k].view(torch.int32) if ref[k].dtype == torch.float32 else ref[k]), (B, k)
        say(f"batch {B}: tokens {g['next'].cpu().tolist()}")
    # a batch whose workspace exceeds the scratch array is rejected on the host, before any launch
    need = big.drafter.workspace_bytes(16)
    assert need <= abi.MTPD_NOALLOC_SCRATCH_BYTES
    wide = Case(synth.E4B, batch=1, context=64, max_batch=256)
    assert wide.drafter.workspace_bytes(256) > abi.MTPD_NOALLOC_SCRATCH_BYTES
    th = torch.zeros(256, synth.E4B.backbone, dtype=torch.int16, device="cuda")
    tok = torch.zeros(256, dtype=torch.int32, device="cuda")
    kv = wide.kv
    with pytest.raises(abi.MtpdError) as ei:
        wide.drafter.drafter_step_noalloc(th, tok, wide.temb, kv, _outputs(wide, 256))
    assert ei.value.code in (abi.MTPD_ESHAPE,)
