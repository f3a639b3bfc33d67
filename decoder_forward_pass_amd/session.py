"""A decoder bound to torch-allocated device memory, and a host block allocator.

``Session`` allocates the weights blob, KV pool and workspace as torch uint8
tensors, uploads the packed weights, and calls the C ABI through
``binding``. ``BlockAllocator`` hands out pool blocks to sequences (in a
shuffled order by default, so paging is never accidentally contiguous) and
builds the [n_seqs, max_blocks] tables the calls take ("Candle model runner"
section 4: forward writes K and V into the blocks its table names; the caller
allocates the blocks). Every step of the forward pass runs in the library.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from .blob import pack_blob

_WDT = {"f32": B.DEC_F32, "bf16": B.DEC_BF16, "uint4": B.DEC_UINT4_G32, "int4sym": B.DEC_INT4_SYM_G32}
_KVT = {"f32": B.DEC_F32, "f16": B.DEC_F16}


def make_config(shape, *, max_context: int, n_blocks: int, max_rows: int, max_seqs: int,
                block_tokens: int | None = None) -> B.dec_config:
    c = B.dec_config()
    c.n_layers, c.d_model, c.n_heads = shape.n_layers, shape.d_model, shape.n_heads
    c.n_kv_heads, c.head_dim, c.ff_hidden, c.vocab = shape.n_kv_heads, shape.head_dim, shape.ff_hidden, shape.vocab
    c.max_context = max_context
    c.rms_eps = shape.rms_eps
    c.rope_base = shape.rope_base
    c.rope_split = c.qk_norm = c.tie_embeddings = 1
    c.weight_dtype = _WDT[shape.weight_dtype]
    c.kv_dtype = _KVT[shape.kv_dtype]
    c.block_tokens = block_tokens or shape.block_tokens
    c.n_blocks, c.max_rows, c.max_seqs = n_blocks, max_rows, max_seqs
    return c


class BlockAllocator:
    def __init__(self, n_blocks: int, block_tokens: int, seed: int | None = 0):
        order = np.arange(n_blocks, dtype=np.int32)
        if seed is not None:
            np.random.default_rng(seed).shuffle(order)
        self.free = list(order[::-1])
        self.B = block_tokens
        self.tables: dict = {}

    def ensure(self, seq, length: int) -> list:
        """Give ``seq`` enough blocks for positions 0 .. length-1; returns its table."""
        t = self.tables.setdefault(seq, [])
        need = (length + self.B - 1) // self.B
        while len(t) < need:
            if not self.free:
                raise RuntimeError("KV pool exhausted")
            t.append(int(self.free.pop()))
        return t

    def table_array(self, seqs, width: int | None = None) -> np.ndarray:
        rows = [self.tables[s] for s in seqs]
        w = width or max(1, max(len(r) for r in rows))
        out = np.zeros((len(rows), w), dtype=np.int32)
        for i, r in enumerate(rows):
            out[i, :len(r)] = r
        return out


class Session:
    def __init__(self, shape, weights, *, max_context: int, n_blocks: int, max_rows: int, max_seqs: int,
                 device: str = "cuda", blob=None):
        """``weights`` are packed into the blob; or ``blob`` (a host uint8 array, e.g. from
        dec_load_safetensors) is uploaded as it is and ``weights`` is ignored."""
        self.shape = shape
        self.cfg = make_config(shape, max_context=max_context, n_blocks=n_blocks, max_rows=max_rows,
                               max_seqs=max_seqs)
        B.dec_check_config(self.cfg)
        if blob is None:
            blob = pack_blob(self.cfg, weights)
        self.weights = torch.from_numpy(blob).to(device)
        del blob
        self.pool = torch.empty(B.dec_kv_pool_bytes(self.cfg), dtype=torch.uint8, device=device)
        self.workspace = torch.empty(B.dec_workspace_bytes(self.cfg), dtype=torch.uint8, device=device)
        self.stream = torch.cuda.current_stream().cuda_stream
        self.ctx = B.dec_init(self.cfg, self.weights.data_ptr(), self.weights.numel(), self.pool.data_ptr(),
                              self.pool.numel(), self.workspace.data_ptr(), self.workspace.numel(), self.stream)
        self.device = device

    def close(self) -> None:
        if self.ctx:
            torch.cuda.synchronize()
            B.dec_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def vocab(self) -> int:
        return self.cfg.vocab

    def prefill(self, start, n_new, tokens, block_tables, mode: int = B.DEC_LOGITS_ALL, logits=None,
                next_tokens=None):
        """One dec_prefill call; returns the logits tensor (allocated if not given)."""
        n_out = int(np.sum(n_new)) if mode == B.DEC_LOGITS_ALL else (len(n_new) if mode == B.DEC_LOGITS_LAST else 0)
        if logits is None and n_out:
            logits = torch.empty((n_out, self.vocab), dtype=torch.float32, device=self.device)
        B.dec_prefill(self.ctx, self.stream, start, n_new, tokens, block_tables, mode,
                      logits.data_ptr() if n_out else 0,
                      next_tokens.data_ptr() if next_tokens is not None else 0)
        return logits

    def decode_step(self, positions, block_tables, *, tokens_host=None, tokens_device=None, logits=None,
                    next_tokens=None, static: bool = False):
        """One dec_decode_step call (dec_decode_step_static with ``static``); returns the logits."""
        n = len(positions)
        if logits is None:
            logits = torch.empty((n, self.vocab), dtype=torch.float32, device=self.device)
        B.dec_decode_step(self.ctx, self.stream, positions, block_tables, logits.data_ptr(),
                          next_tokens.data_ptr() if next_tokens is not None else 0, tokens_host=tokens_host,
                          tokens_device=tokens_device.data_ptr() if tokens_device is not None else 0,
                          static=static)
        return logits

    def sample(self, logits, params, history, ids, rng, next_ids=None, logprob=None):
        """One dec_sample call over the rows of ``logits`` (device float32 [n, ld]).

        params: list of dec_sampling; history: list of dec_history ranges into ``ids`` (device
        int32, or None); rng: device uint64 tensor [n, 2] (advanced in place). Returns
        (next ids int32 [n], logprobs float64 [n]) on the device.
        """
        n = logits.shape[0]
        if logits.dim() != 2 or logits.stride(1) != 1:
            raise ValueError("logits must be [n, ld] with unit column stride")
        # (torch reports stride 0 for a dimension of size 1)
        ld = logits.stride(0) if n > 1 else logits.shape[1]
        if next_ids is None:
            next_ids = torch.empty(n, dtype=torch.int32, device=self.device)
        if logprob is None:
            logprob = torch.empty(n, dtype=torch.float64, device=self.device)
        n_ids = ids.numel() if ids is not None else 0
        B.dec_sample(self.ctx, self.stream, logits.data_ptr(), ld, params, history,
                     ids.data_ptr() if n_ids else 0, n_ids, rng.data_ptr(), next_ids.data_ptr(), logprob.data_ptr())
        return next_ids, logprob

    def dequant(self, index: int) -> torch.Tensor:
        e = B.dec_weight_entry(self.cfg, index)
        out = torch.empty((e.rows, e.cols), dtype=torch.float32, device=self.device)
        B.dec_debug_dequant(self.ctx, self.stream, index, out.data_ptr())
        return out

    def pool_view(self) -> torch.Tensor:
        """The KV pool as [layers, 2, n_blocks, H_kv, B, D] (float32, or f16 bit patterns as int16)."""
        c = self.cfg
        dt = torch.float32 if c.kv_dtype == B.DEC_F32 else torch.int16
        return self.pool.view(dt).view(c.n_layers, 2, c.n_blocks, c.n_kv_heads, c.block_tokens, c.head_dim)
