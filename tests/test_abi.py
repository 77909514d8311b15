"""C-ABI checks that need no GPU: the library loads and exports every function include/mtpd.h declares, the ctypes
structs match the C layout, and host-side validation rejects bad arguments before any device work."""
import ctypes as C
import os
import re
import subprocess

import pytest

from mtp_drafter_step_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mtpd.h")


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"MTPD_API\s+[\w\s\*]+?\b(mtpd_\w+)\s*\(", src)))


def test_header_declares_the_bound_symbols():
    assert declared_functions() == sorted(abi.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = abi.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", abi.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (mtpd_\w+)", out))
    assert exported == set(declared_functions())
    assert L.mtpd_abi_version() == 6


def test_struct_layout_matches_c(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "mtpd.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu\\n", sizeof(mtpd_config), sizeof(mtpd_layer), sizeof(mtpd_weights), sizeof(mtpd_kv),
         sizeof(mtpd_shared_kv));
  printf("%zu %zu %zu %zu %zu\\n", offsetof(mtpd_config, embed_scale), offsetof(mtpd_layer, layer_output_scale),
         offsetof(mtpd_weights, layers), offsetof(mtpd_kv, first), offsetof(mtpd_shared_kv, rope));
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    sizes = [int(x) for x in lines[0].split()]
    offs = [int(x) for x in lines[1].split()]
    assert sizes == [C.sizeof(abi.mtpd_config), C.sizeof(abi.mtpd_layer), C.sizeof(abi.mtpd_weights),
                     C.sizeof(abi.mtpd_kv), C.sizeof(abi.mtpd_shared_kv)]
    assert offs == [abi.mtpd_config.embed_scale.offset, abi.mtpd_layer.layer_output_scale.offset,
                    abi.mtpd_weights.layers.offset, abi.mtpd_kv.first.offset, abi.mtpd_shared_kv.rope.offset]


def good_config(**over):
    c = dict(backbone=1536, hidden=256, n_layer=4, n_head=4, n_kv_head=1, head_dim=256, ffn=1024, vocab=262144,
             n_centroids=2048, top_k=32, swa_window=512, full_attn_layers=0b1000, rms_eps=1e-6, attn_scale=0.0625,
             embed_scale=1.0)
    c.update(over)
    return abi.mtpd_config(**c)


def create_rc(cfg, weights=None, max_batch=16):
    h = C.c_void_p()
    rc = abi.lib().mtpd_create(C.byref(cfg) if cfg is not None else None,
                               C.byref(weights) if weights is not None else None, max_batch, C.byref(h))
    return rc, abi.lib().mtpd_last_error().decode()


@pytest.mark.parametrize("over,code,msg", [
    (dict(vocab=262143), abi.MTPD_ESHAPE, "n_centroids"),
    (dict(top_k=4096), abi.MTPD_ESHAPE, "top_k"),
    (dict(n_head=3, n_kv_head=2), abi.MTPD_ESHAPE, "n_kv_head"),
    (dict(n_centroids=0, top_k=5), abi.MTPD_ESHAPE, "top_k must be 0 or 1"),
    (dict(n_centroids=0, top_k=1, vocab=262150), abi.MTPD_ESHAPE, "multiple of 16 with the dense head"),
    (dict(n_centroids=-1), abi.MTPD_ESHAPE, "positive"),
    (dict(head_dim=512), abi.MTPD_ESHAPE, "head_dim"),
    (dict(hidden=250), abi.MTPD_ESHAPE, "multiple of 256"),
    (dict(top_k=65, n_centroids=2048), abi.MTPD_ESHAPE, "top_k > 64"),
    (dict(swa_window=0), abi.MTPD_ESHAPE, "positive"),
    (dict(attn_scale=0.0), abi.MTPD_EINVAL, "attn_scale"),
])
def test_create_rejects_bad_config(over, code, msg):
    rc, err = create_rc(good_config(**over))
    assert rc == code and msg in err


def test_backbone_limit():
    """backbone up to 8192 passes the config checks (the first error is then the NULL weights); above, ESHAPE."""
    rc, err = create_rc(good_config(backbone=8448))
    assert rc == abi.MTPD_ESHAPE and "backbone" in err
    for bb in (4096, 4352, 8192):
        rc, err = create_rc(good_config(backbone=bb))
        assert rc == abi.MTPD_EINVAL and "weights" in err, (bb, err)


def test_stream_read_rejects_bad_arguments():
    """The measurement read checks its pointers and size on the host, before any device work."""
    L = abi.lib()
    sink = 0x2000
    assert L.mtpd_stream_read(None, 16, 0, sink, None) == abi.MTPD_EINVAL
    assert L.mtpd_stream_read(0x1008, 16, 0, sink, None) == abi.MTPD_EINVAL
    assert "aligned" in L.mtpd_last_error().decode()
    assert L.mtpd_stream_read(0x1000, 24, 0, sink, None) == abi.MTPD_EINVAL
    assert "multiple of 16" in L.mtpd_last_error().decode()
    assert L.mtpd_stream_read(0x1000, 16, 0, None, None) == abi.MTPD_EINVAL


def test_create_rejects_null_and_misaligned_weights():
    rc, err = create_rc(None)
    assert rc == abi.MTPD_EINVAL
    rc, err = create_rc(good_config())
    assert rc == abi.MTPD_EINVAL and "weights" in err
    layers = (abi.mtpd_layer * 4)()
    w = abi.mtpd_weights(pre_proj=0x1000, post_proj=0x1000, output_norm=0x1000, token_embd=0x1000, centroids=0x1000,
                         token_ordering=0x1008, layers=layers)
    rc, err = create_rc(good_config(), w)
    assert rc == abi.MTPD_EINVAL and "token_ordering" in err and "aligned" in err
    w.token_ordering = 0x1000
    rc, err = create_rc(good_config(), w)  # layer pointers are NULL
    assert rc == abi.MTPD_EINVAL and "layers[0].attn_q" in err
    rc, err = create_rc(good_config(), w, max_batch=257)
    assert rc == abi.MTPD_ESHAPE and "max_batch" in err


def test_dense_head_config_needs_no_centroids_or_ordering():
    """With n_centroids == 0 the centroid table and the ordering are not read: NULL passes their checks and the
    first rejected pointer is a layer weight."""
    layers = (abi.mtpd_layer * 4)()
    w = abi.mtpd_weights(pre_proj=0x1000, post_proj=0x1000, output_norm=0x1000, token_embd=0x1000, centroids=None,
                         token_ordering=None, layers=layers)
    for top_k in (0, 1):
        rc, err = create_rc(good_config(n_centroids=0, top_k=top_k, hidden=1024, backbone=2816, n_head=8,
                                        ffn=4096), w)
        assert rc == abi.MTPD_EINVAL and "layers[0].attn_q" in err, err
    rc, err = create_rc(good_config(), w)  # the masked head does need them
    assert rc == abi.MTPD_EINVAL and "centroids" in err


def test_calls_reject_null_handle():
    L = abi.lib()
    assert L.mtpd_workspace_bytes(None, 1) == 0
    rc = L.mtpd_drafter_step(None, None, None, 1, None, None, None, None, None, None, None, None, None, None)
    assert rc == abi.MTPD_EINVAL and "handle" in L.mtpd_last_error().decode()
    rc = L.mtpd_draft_block(None, None, None, 1, 4, None, None, None, None, None, None, None)
    assert rc == abi.MTPD_EINVAL
    rc = L.mtpd_masked_head(None, None, None, 1, None, None, None, None, None, None)
    assert rc == abi.MTPD_EINVAL
    rc = L.mtpd_draft_block_sampled(None, None, None, 1, 4, None, None, None, None, 1.0, None, None, None, None, None)
    assert rc == abi.MTPD_EINVAL
    rc = L.mtpd_sample_head(None, None, None, 1, None, 1.0, None, None, None, None)
    assert rc == abi.MTPD_EINVAL
    L.mtpd_destroy(None)


def test_timing_calls_reject_null_handle():
    import ctypes as C
    L = abi.lib()
    assert L.mtpd_timing_enable(None, 1) == abi.MTPD_EINVAL
    names = (C.c_char_p * 4)()
    ms = (C.c_float * 4)()
    assert L.mtpd_timing_read(None, 4, names, ms) == abi.MTPD_EINVAL
