"""Device buffers for the library, allocated with PyTorch (plumbing only).

``Engine`` sizes and allocates the packed-weight buffer, the workspace and the
KV pool through the C ABI's sizing calls, creates the model and KV handles,
and forwards the round's calls with the current HIP stream.
"""
import math

import torch

from . import binding as B


class Engine:
    def __init__(self, cfg, max_rows=64, max_seqs=8, max_ctx=8192, n_blocks=None, max_blocks_per_seq=None,
                 device="cuda:0"):
        if not torch.cuda.is_available():
            raise RuntimeError("the verify-step library needs a GPU")
        B.lib()  # fails loudly if libvstep.so is missing
        self.cfg, self.device = cfg, torch.device(device)
        self.max_rows, self.max_seqs, self.max_ctx = max_rows, max_seqs, max_ctx
        if max_blocks_per_seq is None:
            max_blocks_per_seq = math.ceil((max_ctx + 2 * B.VS_MAX_ROWS) / 16)
        if n_blocks is None:
            n_blocks = max_blocks_per_seq * max_seqs
        self.n_blocks, self.bps = n_blocks, max_blocks_per_seq
        wb = B.vs_weight_bytes(cfg)
        ws = B.vs_workspace_bytes(cfg, max_rows, max_seqs, max_ctx)
        kb = B.vs_kv_bytes(cfg, n_blocks, max_seqs, max_blocks_per_seq)
        if not (wb and ws and kb):
            raise ValueError(f"unsupported shape: {cfg}")
        self.weights = torch.empty(wb, dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.device)
        self.kvbuf = torch.zeros(kb, dtype=torch.uint8, device=self.device)
        self.model = B.vs_model_create(cfg, self.weights.data_ptr(), self.workspace.data_ptr(), max_rows, max_seqs,
                                       max_ctx, self.stream)
        self.kv = B.vs_kv_create(self.model, self.kvbuf.data_ptr(), n_blocks, max_seqs, max_blocks_per_seq,
                                 self.stream)
        self.result = torch.zeros((max_seqs, B.VS_RESULT_INTS), dtype=torch.int32, device=self.device)

    @property
    def stream(self):
        return torch.cuda.current_stream(self.device).cuda_stream

    def close(self):
        if getattr(self, "kv", None):
            B.vs_kv_destroy(self.kv)
            self.kv = None
        if getattr(self, "model", None):
            B.vs_model_destroy(self.model)
            self.model = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- weights ----
    def set_tensor(self, tensor_id, layer, src_bf16):
        """src_bf16: device tensor (int16/uint16/bfloat16) in canonical layout."""
        assert src_bf16.is_cuda and src_bf16.element_size() == 2 and src_bf16.is_contiguous()
        B.vs_model_set_tensor(self.model, tensor_id, layer, src_bf16.data_ptr(), self.stream)

    # ---- state ----
    def open(self, max_len):
        return B.vs_seq_open(self.kv, max_len, self.stream)

    def state(self):
        """(P, pending, committed) as host lists (synchronises)."""
        return [_view(self.kvbuf, ptr, self.max_seqs * 4).view(torch.int32).cpu().tolist()
                for ptr in B.vs_kv_state(self.kv)]

    def kv_layer(self, layer):
        """Views of layer `layer`: K [blocks][Hkv][hd/8][16][8] (each block's K tile is cut
        into 8-dim pieces, piece-major), V [blocks][Hkv][hd][16], block table."""
        k, v, bt = B.vs_kv_layer(self.kv, layer)
        c = self.cfg
        n = self.n_blocks * c.n_kv_heads * 16 * c.head_dim
        kt = _view(self.kvbuf, k, n * 2).view(torch.bfloat16).view(self.n_blocks, c.n_kv_heads, c.head_dim // 8, 16, 8)
        vt = _view(self.kvbuf, v, n * 2).view(torch.bfloat16).view(self.n_blocks, c.n_kv_heads, c.head_dim, 16)
        btt = _view(self.kvbuf, bt, self.max_seqs * self.bps * 4).view(torch.int32).view(self.max_seqs, self.bps)
        return kt, vt, btt

    def sync(self):
        B.vs_kv_sync(self.kv, self.stream)


def _view(buf, ptr, nbytes):
    off = ptr - buf.data_ptr()
    assert 0 <= off and off + nbytes <= buf.numel()
    return buf[off:off + nbytes]

