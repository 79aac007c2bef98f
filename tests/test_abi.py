"""C-ABI library on the host (no GPU needed): it loads, exports every entry
point declared in include/qsa.h, and rejects bad arguments before launching
anything.  Pointers passed here are never dereferenced: every call is refused
by host-side validation first."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_37_amd import qsa as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")

INVALID, UNSUPPORTED = 1, 2
FAKE = 0x10000  # 16-byte aligned, never dereferenced by a rejected call


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_four_path_calls():
    names = declared_functions()
    for n in ("qsa_compress_keys", "qsa_index_topk", "qsa_sparse_attn_prefill",
              "qsa_sparse_attn_decode"):
        assert n in names


def test_library_exports_every_declared_symbol(qsa_lib):
    for name in declared_functions():
        assert hasattr(qsa_lib, name), f"{name} not exported"
        assert name in Q.SIGNATURES, f"{name} has no binding signature"
    assert qsa_lib.qsa_version() >= 10000


def _err():
    return Q.lib().qsa_last_error().decode()


def test_compress_validation(qsa_lib):
    L = qsa_lib
    assert L.qsa_compress_keys(FAKE, None, FAKE, 1, 64, 48, 16, 1, None) == UNSUPPORTED
    assert "d_idx" in _err()
    assert L.qsa_compress_keys(FAKE, None, FAKE, -1, 64, 64, 16, 1, None) == INVALID
    assert L.qsa_compress_keys(FAKE, None, FAKE, 1, 64, 64, 0, 1, None) == INVALID
    assert L.qsa_compress_keys(None, None, FAKE, 1, 64, 64, 16, 1, None) == INVALID
    assert "ik" in _err()
    assert L.qsa_compress_keys(FAKE + 2, None, FAKE, 1, 64, 64, 16, 1, None) == INVALID
    assert "aligned" in _err()
    assert L.qsa_compress_keys(FAKE, None, FAKE, 1, 64, 64, 16, 7, None) == INVALID
    # nothing to do is not an error: no complete block
    assert L.qsa_compress_keys(FAKE, None, FAKE, 1, 10, 64, 16, 1, None) == 0
    assert L.qsa_compress_keys(FAKE, None, FAKE, 0, 64, 64, 16, 1, None) == 0


def test_index_validation(qsa_lib):
    L = qsa_lib
    args = lambda **kw: [kw.get("iq", FAKE), FAKE, kw.get("kvl", None), kw.get("sel", FAKE), None,
                         kw.get("batch", 1), kw.get("n_q", 256), kw.get("h_idx", 4),
                         kw.get("d_idx", 64), kw.get("max_blocks", 16), kw.get("block", 16),
                         kw.get("top_k", 4), 1, None]
    assert L.qsa_index_topk(*args(top_k=0)) == INVALID
    assert "top_k" in _err()
    assert L.qsa_index_topk(*args(max_blocks=15)) == INVALID  # < n_q / block
    assert L.qsa_index_topk(*args(top_k=257)) == UNSUPPORTED
    assert L.qsa_index_topk(*args(d_idx=96)) == UNSUPPORTED
    assert L.qsa_index_topk(*args(max_blocks=5000, n_q=1)) == UNSUPPORTED
    assert L.qsa_index_topk(*args(sel=None)) == INVALID
    assert L.qsa_index_topk(*args(n_q=0)) == 0


def test_index_decode_validation(qsa_lib):
    L = qsa_lib
    def call(**kw):
        a = dict(iq=FAKE, ik=FAKE, cmp=FAKE, kvl=FAKE, sel=FAKE, sc=None, batch=4, max_len=1024,
                 h_idx=4, d_idx=64, max_blocks=16, block=64, top_k=4, dt=1)
        a.update(kw)
        return L.qsa_index_topk_decode(a["iq"], a["ik"], a["cmp"], a["kvl"], a["sel"], a["sc"],
                                       a["batch"], a["max_len"], a["h_idx"], a["d_idx"],
                                       a["max_blocks"], a["block"], a["top_k"], a["dt"], None)
    assert call(kvl=None) == INVALID
    assert "kv_lens" in _err()
    assert call(ik=None) == INVALID
    assert "ik_cache" in _err()
    assert call(top_k=0) == INVALID
    assert call(max_len=0) == INVALID
    assert call(d_idx=96) == UNSUPPORTED
    assert call(top_k=300) == UNSUPPORTED
    assert call(max_blocks=5000) == UNSUPPORTED
    assert call(cmp=FAKE + 4) == INVALID
    assert call(batch=0) == 0


def test_prefill_validation(qsa_lib):
    L = qsa_lib
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, sel=FAKE, out=FAKE, lse=None, batch=1, seq=128, h_q=8,
                 h_kv=2, d=128, block=16, top_k=4, scale=0.1, dt=1)
        a.update(kw)
        return L.qsa_sparse_attn_prefill(a["q"], a["k"], a["v"], a["sel"], a["out"], a["lse"],
                                         a["batch"], a["seq"], a["h_q"], a["h_kv"], a["d"],
                                         a["block"], a["top_k"], a["scale"], a["dt"], None)
    assert call(h_q=6, h_kv=4) == INVALID
    assert "multiple" in _err()
    assert call(top_k=0) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(top_k=300) == UNSUPPORTED
    assert call(scale=float("nan")) == INVALID
    assert call(q=None) == INVALID
    assert call(lse=FAKE + 4) == INVALID
    assert call(h_q=48, h_kv=1) == UNSUPPORTED  # group 48 not built for bf16
    assert call(seq=0) == 0
    # head dim 256: accepted; no head dim keeps selection rows in LDS, so any top_k <= 256
    assert call(d=256, seq=0) == 0
    assert call(d=192) == UNSUPPORTED
    chunk = lambda n_q, kv_len: L.qsa_sparse_attn_prefill_chunk(
        FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, n_q, kv_len, 8, 2, 128, 16, 4, 0.1, 1, None)
    assert chunk(200, 100) == INVALID
    assert "kv_len" in _err()
    assert chunk(-1, 100) == INVALID
    assert chunk(0, 100) == 0
    varlen = lambda kvl, n_q, max_len: L.qsa_sparse_attn_prefill_varlen(
        FAKE, FAKE, FAKE, kvl, FAKE, FAKE, None, 2, n_q, max_len, 8, 2, 128, 16, 4, 0.1, 1, None)
    assert varlen(None, 10, 100) == INVALID
    assert "kv_lens" in _err()
    assert varlen(FAKE, 200, 100) == INVALID
    assert varlen(None, 0, 100) == 0


def test_decode_validation(qsa_lib):
    L = qsa_lib
    n = ctypes.c_size_t(0)
    assert L.qsa_sparse_attn_decode_workspace_size(8, 32, 4, 128, 64, 32, ctypes.byref(n)) == 0
    need = n.value
    assert need > 0  # 32 (sequence, KV head) pairs on 256 CUs -> split work -> workspace
    assert L.qsa_sparse_attn_decode_workspace_size(8, 32, 4, 128, 64, 32, None) == INVALID
    def call(**kw):
        a = dict(q=FAKE, kc=FAKE, vc=FAKE, kvl=FAKE, sel=FAKE, out=FAKE, lse=None, batch=8,
                 max_len=32768, h_q=32, h_kv=4, d=128, block=64, top_k=32, scale=0.1, ws=FAKE,
                 wsb=need, dt=1)
        a.update(kw)
        return L.qsa_sparse_attn_decode(a["q"], a["kc"], a["vc"], a["kvl"], a["sel"], a["out"],
                                        a["lse"], a["batch"], a["max_len"], a["h_q"], a["h_kv"],
                                        a["d"], a["block"], a["top_k"], a["scale"], a["ws"],
                                        a["wsb"], a["dt"], None)
    assert call(wsb=need - 1) == INVALID
    assert "workspace" in _err()
    assert call(ws=None) == INVALID
    assert call(kvl=None) == INVALID
    assert call(h_q=30) == INVALID
    assert call(h_q=64, h_kv=2) == UNSUPPORTED  # group 32 > 16 not built for bf16 decode
    assert call(batch=0) == 0
    assert call(d=256, batch=0) == 0
    assert call(d=192) == UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        Q.compress_keys(x, 16)


def test_calibration_library_exports_its_header():
    """libqsa_calib.so (the measurement kernels, not the QSA path) exports every function
    include/qsa_calibrate.h declares, and its host checks refuse bad arguments."""
    from block_sparse_attention_37_amd import calibrate as C
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "qsa_calibrate.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(qsa_calib_[a-z_0-9]+)\s*\(", text)))
    assert names
    lib = C.lib()
    for name in names:
        assert hasattr(lib, name) and name in C.SIGNATURES, name
    assert lib.qsa_calib_stream_read(None, 1024, FAKE, 1, None) == 1
    assert lib.qsa_calib_stream_read(FAKE, 1000, FAKE, 1, None) == 1  # not a multiple of 16
    assert lib.qsa_calib_mfma_bf16(0, 1, FAKE, None, None) == 1
    assert lib.qsa_calib_mfma_sink_floats(2) == 1024
