"""Thin ctypes binding of libvstep.so: the C ABI of include/vstep.h under the
same names.  Arguments are marshalled only; every step runs in the library.
Device pointers are plain ints (e.g. ``tensor.data_ptr()``), streams are
``torch.cuda.current_stream().cuda_stream``; host arrays are sequences of int.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvstep.so")

VS_OK, VS_E_INVAL, VS_E_SHAPE, VS_E_NOKV, VS_E_STATE, VS_E_DEVICE = 0, -1, -2, -3, -4, -5
VS_GREEDY, VS_SAMPLE = 0, 1
VS_MAX_ROWS, VS_MAX_SEQS, VS_MAX_K, VS_N_UNIFORMS, VS_RESULT_INTS = 64, 64, 16, 48, 24
VS_MAX_PASS_ROWS = 1088
VS_DYNK_MAX_WINDOW = 256
(VS_T_EMBED, VS_T_ATTN_NORM, VS_T_WQ, VS_T_WK, VS_T_WV, VS_T_WO, VS_T_FFN_NORM, VS_T_W_GATE, VS_T_W_UP, VS_T_W_DOWN,
 VS_T_FINAL_NORM, VS_T_HEAD) = range(12)

EXPORTS = [
    "vs_last_error", "vs_weight_bytes", "vs_workspace_bytes", "vs_kv_bytes", "vs_model_create", "vs_model_set_tensor",
    "vs_model_destroy", "vs_model_set_attn_split", "vs_model_attn_split", "vs_kv_create", "vs_kv_destroy", "vs_seq_open", "vs_seq_assume", "vs_seq_rewind", "vs_seq_close", "vs_kv_state", "vs_kv_layer",
    "vs_kv_sync", "vs_prefill", "vs_forward_layers", "vs_head", "vs_draft", "vs_draft_tree", "vs_verify", "vs_accept", "vs_accept_top_p", "vs_accept_noalloc", "vs_commit",
    "vs_step", "vs_confidence", "vs_sched_init", "vs_sched_update", "vs_step_sched", "vs_dynk_init",
    "vs_dynk_update", "vs_ngram_propose", "vs_step_ngram", "vs_stats_enable", "vs_stats_read",
    "vs_stats_reset", "vs_read_probe",
]


class vs_model_cfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("d_ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("exit_layer", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float)]

    @classmethod
    def of(cls, c):
        return cls(c.n_layers, c.d_model, c.n_heads, c.n_kv_heads, c.head_dim, c.d_ffn, c.vocab, c.exit_layer,
                   c.rms_eps, c.rope_theta)


class vs_batch(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("seq", ctypes.POINTER(ctypes.c_int32)),
                ("n_rows", ctypes.POINTER(ctypes.c_int32)), ("d_depth", ctypes.c_void_p),
                ("d_mask", ctypes.c_void_p)]


class vs_sched_cfg(ctypes.Structure):
    _fields_ = [("min_k", ctypes.c_int32), ("max_k", ctypes.c_int32), ("low", ctypes.c_double),
                ("high", ctypes.c_double)]


class vs_spec_state(ctypes.Structure):
    _fields_ = [("ema", ctypes.c_double), ("k", ctypes.c_int32), ("rounds", ctypes.c_int32),
                ("last_a", ctypes.c_int32)]


class vs_dynk_cfg(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("min_k", ctypes.c_int32), ("max_k", ctypes.c_int32),
                ("up", ctypes.c_double), ("down", ctypes.c_double)]


class vs_dynk_state(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("n", ctypes.c_int32), ("head", ctypes.c_int32),
                ("a", ctypes.c_int32 * VS_DYNK_MAX_WINDOW), ("drafted", ctypes.c_int32 * VS_DYNK_MAX_WINDOW),
                ("alpha", ctypes.c_double)]


class vs_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("bytes", ctypes.c_double)]


class VsError(RuntimeError):
    def __init__(self, name, code, msg):
        super().__init__(f"{name} failed ({code}): {msg}")
        self.code = code


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, VP, F, D, SZ = ctypes.POINTER, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
        pcfg, pI = P(vs_model_cfg), P(I32)
        sig = {
            "vs_last_error": (ctypes.c_char_p, []),
            "vs_weight_bytes": (SZ, [pcfg]),
            "vs_workspace_bytes": (SZ, [pcfg, I32, I32, I32]),
            "vs_kv_bytes": (SZ, [pcfg, I32, I32, I32]),
            "vs_model_create": (I32, [pcfg, VP, VP, I32, I32, I32, VP, P(VP)]),
            "vs_model_set_tensor": (I32, [VP, I32, I32, VP, VP]),
            "vs_model_destroy": (None, [VP]),
            "vs_model_set_attn_split": (I32, [VP, I32]),
            "vs_model_attn_split": (I32, [VP]),
            "vs_kv_create": (I32, [VP, VP, I32, I32, I32, VP, P(VP)]),
            "vs_kv_destroy": (None, [VP]),
            "vs_seq_open": (I32, [VP, I32, VP, pI]),
            "vs_seq_assume": (I32, [VP, I32, I32, I32, VP]),
            "vs_seq_rewind": (I32, [VP, I32, I32, I32, VP]),
            "vs_seq_close": (I32, [VP, I32]),
            "vs_kv_state": (I32, [VP, P(VP), P(VP), P(VP)]),
            "vs_kv_layer": (I32, [VP, I32, P(VP), P(VP), P(VP)]),
            "vs_kv_sync": (I32, [VP, VP]),
            "vs_prefill": (I32, [VP, VP, I32, VP, I32, I32, F, VP, VP, VP]),
            "vs_forward_layers": (I32, [VP, VP, P(vs_batch), I32, I32, VP, VP, VP, VP]),
            "vs_head": (I32, [VP, I32, VP, VP, VP]),
            "vs_draft": (I32, [VP, VP, I32, pI, pI, I32, F, VP, VP, VP, VP, VP]),
            "vs_draft_tree": (I32, [VP, VP, I32, I32, I32, I32, F, VP, VP, VP, VP, VP, VP, VP]),
            "vs_verify": (I32, [VP, VP, P(vs_batch), I32, VP, VP, VP, VP]),
            "vs_accept": (I32, [VP, P(vs_batch), I32, F, VP, VP, VP, VP, VP, VP]),
            "vs_accept_top_p": (I32, [VP, P(vs_batch), F, D, VP, VP, VP, VP, VP, VP]),
            "vs_accept_noalloc": (I32, [I32, P(vs_batch), I32, F, VP, VP, VP, VP, VP, VP]),
            "vs_commit": (I32, [VP, VP, P(vs_batch), VP, VP]),
            "vs_step": (I32, [VP, VP, I32, pI, pI, I32, F, VP, VP, VP, VP]),
            "vs_confidence": (I32, [VP, P(vs_batch), F, VP, VP, VP]),
            "vs_sched_init": (I32, [P(vs_sched_cfg), I32, P(vs_spec_state)]),
            "vs_sched_update": (I32, [P(vs_sched_cfg), P(vs_spec_state), I32, D, D]),
            "vs_step_sched": (I32, [VP, VP, I32, pI, P(vs_sched_cfg), P(vs_spec_state), VP, VP, pI, P(D), VP]),
            "vs_dynk_init": (I32, [P(vs_dynk_cfg), I32, P(vs_dynk_state)]),
            "vs_ngram_propose": (I32, [pI, I32, I32, I32, I32, I32, pI, pI]),
            "vs_step_ngram": (I32, [VP, VP, I32, pI, I32, I32, I32, I32, I32, VP, VP, pI, pI, VP]),
            "vs_dynk_update": (I32, [P(vs_dynk_cfg), P(vs_dynk_state), I32, I32, D, pI]),
            "vs_stats_enable": (I32, [VP, I32]),
            "vs_stats_read": (I32, [VP, P(vs_kernel_stat), I32, pI]),
            "vs_stats_reset": (I32, [VP]),
            "vs_read_probe": (I32, [VP, SZ, VP, VP]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _i32(xs):
    xs = [int(x) for x in xs]
    return (ctypes.c_int32 * max(1, len(xs)))(*xs)


def _check(name, rc):
    if rc != VS_OK:
        raise VsError(name, rc, lib().vs_last_error().decode())


def vs_last_error():
    return lib().vs_last_error().decode()


def vs_weight_bytes(cfg):
    return lib().vs_weight_bytes(ctypes.byref(vs_model_cfg.of(cfg)))


def vs_workspace_bytes(cfg, max_rows, max_seqs, max_ctx):
    return lib().vs_workspace_bytes(ctypes.byref(vs_model_cfg.of(cfg)), max_rows, max_seqs, max_ctx)


def vs_kv_bytes(cfg, n_blocks, max_seqs, max_blocks_per_seq):
    return lib().vs_kv_bytes(ctypes.byref(vs_model_cfg.of(cfg)), n_blocks, max_seqs, max_blocks_per_seq)


def vs_model_create(cfg, d_weights, d_workspace, max_rows, max_seqs, max_ctx, stream):
    out = ctypes.c_void_p()
    _check("vs_model_create", lib().vs_model_create(ctypes.byref(vs_model_cfg.of(cfg)), d_weights, d_workspace,
                                                    max_rows, max_seqs, max_ctx, stream, ctypes.byref(out)))
    return out.value


def vs_model_set_tensor(model, tensor, layer, d_src, stream):
    _check("vs_model_set_tensor", lib().vs_model_set_tensor(model, tensor, layer, d_src, stream))


def vs_model_destroy(model):
    lib().vs_model_destroy(model)


def vs_model_set_attn_split(model, keys):
    _check("vs_model_set_attn_split", lib().vs_model_set_attn_split(model, keys))


def vs_model_attn_split(model):
    return lib().vs_model_attn_split(model)


def vs_kv_create(model, d_kv, n_blocks, max_seqs, max_blocks_per_seq, stream):
    out = ctypes.c_void_p()
    _check("vs_kv_create", lib().vs_kv_create(model, d_kv, n_blocks, max_seqs, max_blocks_per_seq, stream,
                                              ctypes.byref(out)))
    return out.value


def vs_kv_destroy(kv):
    lib().vs_kv_destroy(kv)


def vs_seq_open(kv, max_len, stream):
    sid = ctypes.c_int32()
    _check("vs_seq_open", lib().vs_seq_open(kv, max_len, stream, ctypes.byref(sid)))
    return sid.value


def vs_seq_assume(kv, seq, P, pending, stream):
    _check("vs_seq_assume", lib().vs_seq_assume(kv, seq, P, pending, stream))


def vs_seq_rewind(kv, seq, P, pending, stream):
    _check("vs_seq_rewind", lib().vs_seq_rewind(kv, seq, P, pending, stream))


def vs_seq_close(kv, seq):
    _check("vs_seq_close", lib().vs_seq_close(kv, seq))


def vs_kv_state(kv):
    a, b, c = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
    _check("vs_kv_state", lib().vs_kv_state(kv, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def vs_kv_layer(kv, layer):
    k, v, bt = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
    _check("vs_kv_layer", lib().vs_kv_layer(kv, layer, ctypes.byref(k), ctypes.byref(v), ctypes.byref(bt)))
    return k.value, v.value, bt.value


def vs_kv_sync(kv, stream):
    _check("vs_kv_sync", lib().vs_kv_sync(kv, stream))


def vs_prefill(model, kv, seq, d_tokens, n, mode, temp, d_u, d_logits_last, stream):
    _check("vs_prefill", lib().vs_prefill(model, kv, seq, d_tokens, n, mode, temp, d_u, d_logits_last, stream))


def make_batch(seqs, n_rows, d_depth=None, d_mask=None):
    """A vs_batch (keeps its host arrays alive on the returned object)."""
    b = vs_batch()
    b._seq, b._rows = _i32(seqs), _i32(n_rows)
    b.n_seq = len(seqs)
    b.seq = ctypes.cast(b._seq, ctypes.POINTER(ctypes.c_int32))
    b.n_rows = ctypes.cast(b._rows, ctypes.POINTER(ctypes.c_int32))
    b.d_depth = d_depth
    b.d_mask = d_mask
    return b


def vs_forward_layers(model, kv, batch, start, end, d_tokens, d_hidden_in, d_hidden_out, stream):
    _check("vs_forward_layers", lib().vs_forward_layers(model, kv, ctypes.byref(batch), start, end, d_tokens,
                                                        d_hidden_in, d_hidden_out, stream))


def vs_head(model, M, d_hidden, d_logits, stream):
    _check("vs_head", lib().vs_head(model, M, d_hidden, d_logits, stream))


def vs_draft(model, kv, seqs, ks, mode, temp, d_u, d_tokens, d_hidden_L, d_draft_logits, stream):
    _check("vs_draft", lib().vs_draft(model, kv, len(seqs), _i32(seqs), _i32(ks), mode, temp, d_u, d_tokens,
                                      d_hidden_L, d_draft_logits, stream))


def vs_draft_tree(model, kv, seq, topk, depth, keep, temp, d_tokens, d_depth, d_mask, d_parent, d_hidden_L,
                  d_level_logits, stream):
    _check("vs_draft_tree", lib().vs_draft_tree(model, kv, seq, topk, depth, keep, temp, d_tokens, d_depth, d_mask,
                                                d_parent, d_hidden_L, d_level_logits, stream))


def vs_verify(model, kv, batch, start_layer, d_tokens, d_hidden_in, d_logits, stream):
    _check("vs_verify", lib().vs_verify(model, kv, ctypes.byref(batch), start_layer, d_tokens, d_hidden_in, d_logits,
                                        stream))


def vs_accept(model, batch, mode, temp, d_tokens, d_logits, d_draft_logits, d_u, d_result, stream):
    _check("vs_accept", lib().vs_accept(model, ctypes.byref(batch), mode, temp, d_tokens, d_logits, d_draft_logits,
                                        d_u, d_result, stream))


def vs_accept_top_p(model, batch, temp, top_p, d_tokens, d_logits, d_draft_logits, d_u, d_result, stream):
    _check("vs_accept_top_p", lib().vs_accept_top_p(model, ctypes.byref(batch), temp, top_p, d_tokens, d_logits,
                                                    d_draft_logits, d_u, d_result, stream))


def vs_accept_noalloc(vocab, batch, mode, temp, d_tokens, d_logits, d_draft_logits, d_u, d_result, stream):
    _check("vs_accept_noalloc", lib().vs_accept_noalloc(vocab, ctypes.byref(batch), mode, temp, d_tokens, d_logits,
                                                        d_draft_logits, d_u, d_result, stream))


def vs_commit(model, kv, batch, d_result, stream):
    _check("vs_commit", lib().vs_commit(model, kv, ctypes.byref(batch), d_result, stream))


def vs_step(model, kv, seqs, ks, mode, temp, d_u, d_tokens, d_result, stream):
    _check("vs_step", lib().vs_step(model, kv, len(seqs), _i32(seqs), _i32(ks), mode, temp, d_u, d_tokens, d_result,
                                    stream))


def vs_confidence(model, batch, temp, d_logits, d_conf, stream):
    _check("vs_confidence", lib().vs_confidence(model, ctypes.byref(batch), temp, d_logits, d_conf, stream))


def sched_cfg(min_k=2, max_k=16, low=0.3, high=0.7):
    return vs_sched_cfg(min_k, max_k, low, high)


def vs_sched_init(cfg, k0):
    s = vs_spec_state()
    _check("vs_sched_init", lib().vs_sched_init(ctypes.byref(cfg), k0, ctypes.byref(s)))
    return s


def vs_sched_update(cfg, state, a, avg_top1, avg_gap):
    """Updates `state` (a vs_spec_state) in place; returns the next k."""
    _check("vs_sched_update", lib().vs_sched_update(ctypes.byref(cfg), ctypes.byref(state), a, avg_top1, avg_gap))
    return state.k


def vs_step_sched(model, kv, seqs, cfg, states, d_tokens, d_result, stream):
    """One scheduled round; `states` is a ctypes array of vs_spec_state,
    updated in place.  Returns (results [n][VS_RESULT_INTS], conf [n][2])."""
    n = len(seqs)
    h_res = (ctypes.c_int32 * (n * VS_RESULT_INTS))()
    h_conf = (ctypes.c_double * (2 * n))()
    _check("vs_step_sched", lib().vs_step_sched(model, kv, n, _i32(seqs), ctypes.byref(cfg), states, d_tokens,
                                                d_result, h_res, h_conf, stream))
    res = [list(h_res[i * VS_RESULT_INTS:(i + 1) * VS_RESULT_INTS]) for i in range(n)]
    conf = [(h_conf[2 * i], h_conf[2 * i + 1]) for i in range(n)]
    return res, conf


def dynk_cfg(window=64, min_k=2, max_k=8, up=0.85, down=0.7):
    return vs_dynk_cfg(window, min_k, max_k, up, down)


def vs_dynk_init(cfg, k0):
    s = vs_dynk_state()
    _check("vs_dynk_init", lib().vs_dynk_init(ctypes.byref(cfg), k0, ctypes.byref(s)))
    return s


def vs_dynk_update(cfg, state, a, k_used, c_draft=0.0):
    """Updates `state` in place; returns the next round's draft length (0 =
    a plain decoding step)."""
    kn = ctypes.c_int32()
    _check("vs_dynk_update", lib().vs_dynk_update(ctypes.byref(cfg), ctypes.byref(state), a, k_used, c_draft,
                                                  ctypes.byref(kn)))
    return kn.value


def vs_ngram_propose(tokens, search_len, min_ngram, max_ngram, k_max):
    out = (ctypes.c_int32 * max(1, k_max))()
    n = ctypes.c_int32()
    _check("vs_ngram_propose", lib().vs_ngram_propose(_i32(tokens), len(tokens), search_len, min_ngram, max_ngram,
                                                      k_max, out, ctypes.byref(n)))
    return list(out[:n.value])


def vs_step_ngram(model, kv, seq, history, search_len, min_ngram, max_ngram, k_max, d_tokens, d_result, stream):
    """One n-gram round; returns (result row, k)."""
    h_res = (ctypes.c_int32 * VS_RESULT_INTS)()
    k = ctypes.c_int32()
    _check("vs_step_ngram", lib().vs_step_ngram(model, kv, seq, _i32(history), len(history), search_len, min_ngram,
                                                max_ngram, k_max, d_tokens, d_result, h_res, ctypes.byref(k),
                                                stream))
    return list(h_res), k.value


STAT_FAMILIES = ["gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "gemm_head", "attention", "small"]


def vs_stats_enable(model, mask):
    """mask: int bitmask over STAT_FAMILIES, True for all, False/0 for none."""
    if mask is True:
        mask = -1
    _check("vs_stats_enable", lib().vs_stats_enable(model, int(mask)))


def vs_stats_reset(model):
    _check("vs_stats_reset", lib().vs_stats_reset(model))


def vs_stats_read(model):
    arr = (vs_kernel_stat * 16)()
    n = ctypes.c_int32()
    _check("vs_stats_read", lib().vs_stats_read(model, arr, 16, ctypes.byref(n)))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms, arr[i].bytes) for i in range(n.value)}


def vs_read_probe(d_src, nbytes, d_sink, stream):
    _check("vs_read_probe", lib().vs_read_probe(d_src, nbytes, d_sink, stream))
