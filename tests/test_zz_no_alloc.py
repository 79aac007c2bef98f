"""qsa_sparse_attn_decode_noalloc (the decode call that takes no workspace and allocates
nothing) against qsa_sparse_attn_decode with a caller workspace, through the C ABI: two
calls in a row, the second with a smaller input, each bit-identical to the workspace call
(same kernels, same split count) and within tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle.qsa_oracle as O
from block_sparse_attention_37_amd import qsa as Q
from block_sparse_attention_37_amd import synth as S
from parity import LSE_ATOL, OUT_ATOL, max_abs

pytestmark = pytest.mark.gpu


def _case(dev, name, batch, max_len, block, top_k, h_q, h_kv, d, lens, seed):
    w = S.Workload(name, seed=seed, kind="decode", dtype="bf16", batch=batch, max_len=max_len,
                   block=block, top_k=top_k, h_q=h_q, h_kv=h_kv, d=d, h_idx=2, d_idx=32)
    lens = np.array(lens, dtype=np.int32)
    kc = torch.zeros(batch, max_len, h_kv, d, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    ik = torch.zeros(batch, max_len, w.d_idx, dtype=torch.bfloat16, device=dev)
    q = torch.zeros(batch, h_q, d, dtype=torch.bfloat16, device=dev)
    iq = torch.zeros(batch, 1, w.h_idx, w.d_idx, dtype=torch.bfloat16, device=dev)
    host = {}
    for b, s in S.decode_sequences(w, lens):
        L = int(lens[b])
        kc[b, :L] = S.to_torch(s["k"], dev)
        vc[b, :L] = S.to_torch(s["v"], dev)
        ik[b, :L] = S.to_torch(s["ik"], dev)
        q[b] = S.to_torch(s["q"], dev)
        iq[b, 0] = S.to_torch(s["iq"], dev)
        host[b] = s
    kvl = torch.from_numpy(lens).to(dev)
    cmp = Q.compress_keys(ik, block, kv_lens=kvl)
    sel = Q.index_topk(iq, cmp, block, top_k, kv_lens=kvl).reshape(batch, top_k).contiguous()
    return w, lens, q, kc, vc, kvl, sel, host


def _check(dev, case):
    w, lens, q, kc, vc, kvl, sel, host = case
    ws_bytes = Q.decode_workspace_bytes(w.batch, w.h_q, w.h_kv, w.d, w.block, w.top_k)
    ref, ref_lse = Q.sparse_attn_decode(q, kc, vc, kvl, sel, w.block, w.sm_scale, return_lse=True)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((w.batch, w.h_q), float("nan"), dtype=torch.float32, device=dev)
    Q.sparse_attn_decode_noalloc(q, kc, vc, kvl, sel, w.block, w.sm_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), f"{w.name}: output differs from the workspace call"
    assert torch.equal(lse, ref_lse), f"{w.name}: lse differs from the workspace call"
    sel_n, out_n, lse_n = sel.cpu().numpy(), out.float().cpu().numpy(), lse.cpu().numpy()
    for b, s in host.items():
        L = int(lens[b])
        toks = O.token_set([j for j in sel_n[b] if j >= 0], L - 1, w.block)
        o, l_ = O.attend(S.to_f64(s["q"]), S.to_f64(s["k"]), S.to_f64(s["v"]), toks, w.sm_scale)
        assert max_abs(out_n[b], o) <= OUT_ATOL["bf16"], f"{w.name} seq {b}"
        assert max_abs(lse_n[b], l_) <= LSE_ATOL["bf16"], f"{w.name} seq {b}"
    return ws_bytes


def test_noalloc_decode_matches_workspace_call_twice(gpu):
    dev = gpu
    # first call: 3 sequences, 64 chunks each -> several splits, scratch in use
    big = _case(dev, "noalloc_big", batch=3, max_len=4200, block=64, top_k=48, h_q=16, h_kv=2,
                d=128, lens=[4200, 3100, 4097], seed=301)
    nbytes = _check(dev, big)
    assert nbytes > 0, "the first case must use the scratch array"
    # second call, smaller: fewer sequences, shorter, another head dim and split count; it
    # reuses the scratch the first call left behind
    small = _case(dev, "noalloc_small", batch=2, max_len=700, block=32, top_k=8, h_q=16,
                  h_kv=2, d=256, lens=[700, 333], seed=302)
    _check(dev, small)
    # a call with a single split uses no scratch at all
    one = _case(dev, "noalloc_one_split", batch=64, max_len=300, block=16, top_k=4, h_q=8,
                h_kv=4, d=64, lens=[300 - (i % 7) for i in range(64)], seed=303)
    assert Q.decode_workspace_bytes(64, 8, 4, 64, 16, 4) == 0
    _check(dev, one)


def test_noalloc_decode_rejects_sizes_beyond_its_scratch(gpu):
    # 300 sequences x 16 heads x 4 splits x 257 floats > 8 MiB: refused before any launch
    need = Q.decode_workspace_bytes(300, 16, 1, 256, 64, 32)
    assert need > 8 << 20
    z = torch.zeros(16, dtype=torch.bfloat16, device=gpu)  # never dereferenced
    with pytest.raises(Q.QSAError) as e:
        st = Q.lib().qsa_sparse_attn_decode_noalloc(
            z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(),
            None, 300, 8, 16, 1, 256, 64, 32, 0.0625, Q.QSA_BF16, None)
        if st != 0:
            raise Q.QSAError(st, "qsa_sparse_attn_decode_noalloc",
                             Q.lib().qsa_last_error().decode())
    assert e.value.status == 2 and "scratch" in str(e.value)
