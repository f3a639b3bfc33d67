"""GPU: export / import of blocks' K/V data (dec_kv_export, dec_kv_import; "Candle model runner"
section 4, KvPool export/import and test kv_pool_exports_and_imports_rust_owned_blocks). A
prompt is prefilled into blocks handed out by the block manager; its blocks are exported, imported
into other blocks, and the pool's bytes must match; a decode step that reads the imported
blocks must give the same logits, bit for bit, as one that reads the originals."""

import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import dataclasses

from synthetic import MODELS, WORKLOADS, make_prompts, make_weights


@pytest.mark.parametrize("kv", ["f16", "f32"])
def test_exported_blocks_resume_decoding_identically(kv):
    from decoder_forward_pass_amd import binding as B
    from decoder_forward_pass_amd.session import Session
    shape = dataclasses.replace(MODELS["tiny_f32"], name=f"tiny_kv_{kv}", weight_dtype="bf16", kv_dtype=kv)
    s = Session(shape, make_weights(shape), max_context=128, n_blocks=24, max_rows=128, max_seqs=4)
    bp = B.BlockPool(24, shape.block_tokens)
    try:
        prompt = make_prompts(WORKLOADS["tiny_f32_t16"])[0]
        T = 40
        toks = np.resize(prompt, T).astype(np.int32)
        nb = math.ceil((T + 1) / shape.block_tokens)
        src = bp.alloc(nb)
        tbl_src = np.array([src], np.int32)
        s.prefill([0], [T], toks, tbl_src, B.DEC_LOGITS_NONE)
        fills = [min(shape.block_tokens, T - i * shape.block_tokens) for i in range(nb)]
        for b, f in zip(src, fills):
            bp.set_fill(b, f)
        torch.cuda.synchronize()
        blob = B.dec_kv_export(s.ctx, s.stream, src, fills)
        assert len(blob) == B._lib.dec_kv_export_bytes(s.ctx, nb)
        dst = bp.alloc(nb)
        got_fills = B.dec_kv_import(s.ctx, s.stream, blob, dst)
        assert got_fills == fills
        pool = s.pool.view(torch.uint8).reshape(shape.n_layers, 2, 24, -1).cpu().numpy()
        for a, b in zip(src, dst):
            assert np.array_equal(pool[:, :, a], pool[:, :, b])
        # decode one token on each copy: same logits, bit for bit
        nxt = np.array([int(prompt[0])], np.int32)
        la = s.decode_step([T], tbl_src, tokens_host=nxt).clone()
        lb = s.decode_step([T], np.array([dst], np.int32), tokens_host=nxt).clone()
        torch.cuda.synchronize()
        assert torch.equal(la, lb)
        # an envelope from another block format is refused
        bad = bytearray(blob)
        bad[8:12] = (shape.n_layers + 1).to_bytes(4, "little")
        with pytest.raises(B.DecError) as e:
            B.dec_kv_import(s.ctx, s.stream, bytes(bad), dst)
        assert e.value.code == B.DEC_E_UNSUPPORTED
    finally:
        bp.close()
        s.close()
