"""Device staging of a prefill batch: host arrays -> GPU tensors -> library calls.

``DeviceBatch`` uploads the descriptor arrays of a batch and builds the
``minipic_batch`` struct that points at them. ``DeviceWorkload`` additionally
owns the paged caches, the query/output buffers, the cos/sin table and the
workspace for a layout object exposing the attributes of a generated
workload (block tables, logical positions, span ids, flags, token values and
their slots). torch is used for device memory and the stream only; all
computation runs in libminipic.so.
"""
import ctypes

import numpy as np
import torch

from ._binding import (MINIPIC_BF16, MINIPIC_F32, minipic_batch, minipic_get_launch_info,
                       minipic_prefill_attn, minipic_prefill_plan, minipic_prefill_run,
                       minipic_reference_prerotated, minipic_rope_table,
                       minipic_workspace_size, minipic_write_kv, minipic_decode_attn,
                       minipic_decode_prerotated, minipic_decode_workspace_size)


def _dev(a, device, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def _values(a, dtype_name, device):
    """float32 array or bf16 bit pattern (uint16) -> device tensor of the element type."""
    a = np.ascontiguousarray(a)
    if dtype_name == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)


class DeviceBatch:
    def __init__(self, *, q_indptr, q_ctx_idx, ctx_len, block_table, logical_pos, span_id, blk_flags,
                 num_q_heads, num_kv_heads, head_dim, block_size=16, max_q_len=None, max_ctx_len=None,
                 device="cuda"):
        self.q_indptr = _dev(np.asarray(q_indptr, np.int32), device)
        self.q_ctx_idx = _dev(np.asarray(q_ctx_idx, np.int32), device)
        self.ctx_len = _dev(np.asarray(ctx_len, np.int32), device)
        self.block_table = _dev(np.asarray(block_table, np.int32), device)
        self.logical_pos = _dev(np.asarray(logical_pos, np.int32), device)
        self.span_id = _dev(np.asarray(span_id, np.int32), device)
        self.blk_flags = _dev(np.asarray(blk_flags, np.uint8), device)
        qi = np.asarray(q_indptr, np.int64)
        R = len(qi) - 1
        mb = int(np.asarray(block_table).shape[1])
        self.struct = minipic_batch(
            num_reqs=R, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
            block_size=block_size, max_blocks_per_req=mb, total_q=int(qi[-1]) if R else 0,
            max_q_len=int(max_q_len if max_q_len is not None else (np.diff(qi).max() if R else 0)),
            max_ctx_len=int(max_ctx_len if max_ctx_len is not None else (np.max(ctx_len) if R else 0)),
            q_indptr=self.q_indptr.data_ptr(), q_ctx_idx=self.q_ctx_idx.data_ptr(),
            ctx_len=self.ctx_len.data_ptr(), block_table=self.block_table.data_ptr(),
            logical_pos=self.logical_pos.data_ptr(), span_id=self.span_id.data_ptr(),
            blk_flags=self.blk_flags.data_ptr())


class DeviceWorkload:
    """A generated prefill batch resident on the GPU.

    After construction the tokens that are cached before the step are already
    in the paged cache; ``write_new`` stores this step's new tokens and
    ``attend`` runs the attention of the step.
    """

    def __init__(self, w, device="cuda", rope_table=True, flags=0, cache_fill=0.0):
        self.w = w
        self.device = device
        self.dtype_code = MINIPIC_BF16 if w.dtype == "bf16" else MINIPIC_F32
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        Hkv, D, B = w.num_kv_heads, w.head_dim, w.block_size
        self.batch = DeviceBatch(q_indptr=w.q_indptr, q_ctx_idx=w.q_ctx_idx, ctx_len=w.ctx_len,
                                 block_table=w.block_table, logical_pos=w.logical_pos, span_id=w.span_id,
                                 blk_flags=w.blk_flags, num_q_heads=w.num_q_heads, num_kv_heads=Hkv,
                                 head_dim=D, block_size=B, device=device)
        self.num_blocks = int(w.num_blocks)
        # cache_fill: the value of every slot no token is written to (NaN
        # stands for unwritten or recycled memory)
        self.k_cache = torch.full((self.num_blocks, Hkv, B, D), cache_fill, dtype=tdt, device=device)
        self.v_cache = torch.full((self.num_blocks, Hkv, D, B), cache_fill, dtype=tdt, device=device)
        self.q = _values(w.q, w.dtype, device)
        self.out = torch.zeros_like(self.q)
        self.k_new = _values(w.k_tok[w.new_tok], w.dtype, device)
        self.v_new = _values(w.v_tok[w.new_tok], w.dtype, device)
        self.slot_new = _dev(w.tok_slot[w.new_tok].astype(np.int64), device)
        self.max_pos = int(w.max_pos)
        self.cos_sin = torch.empty((self.max_pos, D), dtype=torch.float32, device=device)
        if rope_table:
            minipic_rope_table(self.cos_sin, self.max_pos, D, w.rope_theta)
        ws = minipic_workspace_size(self.batch.struct, self.dtype_code)
        self.workspace = torch.zeros(max(ws, 256), dtype=torch.uint8, device=device)
        self.flags = flags
        # tokens cached before the step
        if len(w.setup_tok):
            ks = _values(w.k_tok[w.setup_tok], w.dtype, device)
            vs = _values(w.v_tok[w.setup_tok], w.dtype, device)
            ss = _dev(w.tok_slot[w.setup_tok].astype(np.int64), device)
            self._write(ks, vs, ss)
            del ks, vs, ss

    def _write(self, k, v, slots):
        minipic_write_kv(k, v, slots, self.k_cache, self.v_cache, num_kv_heads=self.w.num_kv_heads,
                         head_dim=self.w.head_dim, block_size=self.w.block_size, num_blocks=self.num_blocks)

    def launch_info(self):
        return minipic_get_launch_info(self.batch.struct, self.dtype_code)

    def write_new(self):
        self._write(self.k_new, self.v_new, self.slot_new)

    def attend(self, out=None, flags=None, q=None):
        minipic_prefill_attn(self.q if q is None else q, self.k_cache, self.v_cache, self.num_blocks,
                             self.batch.struct, self.cos_sin, self.max_pos, self.out if out is None else out,
                             self.workspace, flags=self.flags if flags is None else flags)

    def plan(self, flags=None):
        """The planning kernels only: the plan in the workspace serves run() calls."""
        minipic_prefill_plan(self.num_blocks, self.batch.struct, self.cos_sin, self.max_pos, self.workspace,
                             dtype_code=self.dtype_code, flags=self.flags if flags is None else flags)

    def run(self, out=None, flags=None, q=None, k_cache=None, v_cache=None):
        """Attention and merge on the plan made by plan() (as attend(), without planning)."""
        minipic_prefill_run(self.q if q is None else q, self.k_cache if k_cache is None else k_cache,
                            self.v_cache if v_cache is None else v_cache, self.num_blocks, self.batch.struct,
                            self.cos_sin, self.max_pos, self.out if out is None else out, self.workspace,
                            flags=self.flags if flags is None else flags)

    def attend_prerotated(self, out=None, flags=None, k_cache=None, q=None):
        minipic_reference_prerotated(self.q if q is None else q, self.k_cache if k_cache is None else k_cache,
                                     self.v_cache, self.num_blocks, self.batch.struct,
                                     self.out if out is None else out, self.workspace, cos_sin=self.cos_sin,
                                     max_pos=self.max_pos, flags=self.flags if flags is None else flags)

    def _decode_ws(self):
        if getattr(self, "decode_workspace", None) is None:
            n = minipic_decode_workspace_size(self.batch.struct, self.dtype_code)
            self.decode_workspace = torch.zeros(max(n, 256), dtype=torch.uint8, device=self.device)
        return self.decode_workspace

    def decode(self, out=None, q=None):
        """Decode attention: the batch must hold one query row per request."""
        minipic_decode_attn(self.q if q is None else q, self.k_cache, self.v_cache, self.num_blocks,
                            self.batch.struct, self.cos_sin, self.max_pos, self.out if out is None else out,
                            self._decode_ws())

    def decode_prerotated(self, out=None, k_cache=None, q=None):
        minipic_decode_prerotated(self.q if q is None else q, self.k_cache if k_cache is None else k_cache,
                                  self.v_cache, self.num_blocks, self.batch.struct,
                                  self.out if out is None else out, self._decode_ws())

    def decode_error_word(self) -> int:
        return int(self._decode_ws()[:4].view(torch.int32).item())

    def step(self):
        """One pass of the hot path: write this step's K~/V, then attend."""
        self.write_new()
        self.attend()

    def error_word(self) -> int:
        return int(self.workspace[:4].view(torch.int32).item())
