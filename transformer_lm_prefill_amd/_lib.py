"""ctypes view of libqwen3_prefill.so: structs and prototypes mirroring include/qwen3_prefill.h."""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqwen3_prefill.so")

QWEN3_F32 = 0
QWEN3_BF16 = 1
QWEN3_F16 = 2
QWEN3_F16_TILED = 3
STATUS = {0: "QWEN3_OK", 1: "QWEN3_ERR_INVALID_ARG", 2: "QWEN3_ERR_UNSUPPORTED",
          3: "QWEN3_ERR_WORKSPACE", 4: "QWEN3_ERR_HIP"}

# Every symbol the header declares.
EXPORTS = ("qwen3_layer_workspace_bytes", "qwen3_layer_prefill", "qk_norm_mrope",
           "gqa_causal_attention", "gqa_bidirectional_attention", "vision_rope_tables",
           "apply_rope_tables", "swiglu_ffn", "swiglu_ffn_workspace_bytes", "rms_norm_rows",
           "qwen3_model_workspace_bytes", "qwen3_model_prefill_logits_last",
           "kv_cache_write", "qwen3_layer_prefill_kv", "gqa_decode_attention",
           "gqa_decode_attention_workspace_bytes", "gqa_decode_attention_noalloc", "qwen3_layer_decode",
           "qwen3_layer_decode_workspace_bytes", "dequantize_matrix",
           "qwen3_layer_quant_workspace_bytes", "qwen3_layer_prefill_quant", "qwen3_layer_decode_quant",
           "qwen3_model_prefill_logits_last_kv", "qwen3_model_decode_workspace_bytes", "qwen3_model_decode_logits",
           "qwen3_last_error", "qwen3_timing_enable", "qwen3_timing_collect", "qwen3_mfma_probe",
           "qwen3_tile_weights")


class LayerCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("mrope_section", ctypes.c_int32 * 3),
                ("wdtype", ctypes.c_int), ("act_dtype", ctypes.c_int),
                ("resid_dtype", ctypes.c_int)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm",
                                               "wo", "ffn_norm", "w_gate", "w_up", "w_down")]


class QMatrix(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int), ("data", ctypes.c_void_p), ("row_scale", ctypes.c_void_p)]


class LayerQWeights(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("wq", QMatrix), ("wk", QMatrix), ("wv", QMatrix),
                ("q_norm", ctypes.c_void_p), ("k_norm", ctypes.c_void_p), ("wo", QMatrix),
                ("ffn_norm", ctypes.c_void_p), ("w_gate", QMatrix), ("w_up", QMatrix), ("w_down", QMatrix)]


W_DENSE, W_Q4_0, W_Q8_ROW = 0, 1, 2


class ModelCfg(ctypes.Structure):
    _fields_ = [("layer", LayerCfg), ("n_layers", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_deepstack_layers", ctypes.c_int32)]


class ModelWeights(ctypes.Structure):
    _fields_ = [("token_embd", ctypes.c_void_p), ("layers", ctypes.POINTER(LayerWeights)),
                ("output_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double), ("median_ms", ctypes.c_double)]


class Qwen3Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load():
    """Load the HIP library; raises if it has not been built (there is no other path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m transformer_lm_prefill_amd.build_lib`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.qwen3_layer_workspace_bytes.argtypes = [ctypes.POINTER(LayerCfg), i32]
    lib.qwen3_layer_workspace_bytes.restype = sz
    lib.qwen3_layer_prefill.argtypes = [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerWeights),
                                        vp, vp, i32, vp, vp, i32, vp, vp, sz, vp]
    lib.qwen3_layer_prefill.restype = ctypes.c_int
    lib.qk_norm_mrope.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, f32, vp, f32,
                                  ctypes.POINTER(i32), ctypes.c_int, ctypes.c_int, vp]
    lib.qk_norm_mrope.restype = ctypes.c_int
    lib.gqa_causal_attention.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f32, ctypes.c_int, vp]
    lib.gqa_causal_attention.restype = ctypes.c_int
    lib.gqa_bidirectional_attention.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f32, ctypes.c_int, vp]
    lib.gqa_bidirectional_attention.restype = ctypes.c_int
    lib.vision_rope_tables.argtypes = [i32, i32, i32, i32, i32, f32, i32, vp, vp, vp]
    lib.vision_rope_tables.restype = ctypes.c_int
    lib.apply_rope_tables.argtypes = [vp, i32, i32, i32, ctypes.c_int64, vp, vp, i32, ctypes.c_int, vp]
    lib.apply_rope_tables.restype = ctypes.c_int
    lib.swiglu_ffn.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, vp, sz, vp]
    lib.swiglu_ffn.restype = ctypes.c_int
    lib.swiglu_ffn_workspace_bytes.argtypes = [i32, i32, ctypes.c_int]
    lib.swiglu_ffn_workspace_bytes.restype = sz
    lib.rms_norm_rows.argtypes = [vp, vp, vp, i32, i32, f32, ctypes.c_int, ctypes.c_int, vp]
    lib.rms_norm_rows.restype = ctypes.c_int
    lib.qwen3_model_workspace_bytes.argtypes = [ctypes.POINTER(ModelCfg), i32]
    lib.qwen3_model_workspace_bytes.restype = sz
    lib.qwen3_model_prefill_logits_last.argtypes = [ctypes.POINTER(ModelCfg), ctypes.POINTER(ModelWeights),
                                                    ctypes.POINTER(i32), i32, vp, vp, i32,
                                                    ctypes.POINTER(vp), vp, vp, sz, vp]
    lib.qwen3_model_prefill_logits_last.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.kv_cache_write.argtypes = [vp, vp, i64, i64, i32, i32, i32, ctypes.c_int, vp, vp, ctypes.c_int, i32, i32, vp]
    lib.kv_cache_write.restype = ctypes.c_int
    lib.qwen3_layer_prefill_kv.argtypes = [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerWeights),
                                           vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, vp, sz, vp]
    lib.qwen3_layer_prefill_kv.restype = ctypes.c_int
    lib.gqa_decode_attention.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, f32, ctypes.c_int, vp, vp, sz, vp]
    lib.gqa_decode_attention.restype = ctypes.c_int
    lib.gqa_decode_attention_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.gqa_decode_attention_workspace_bytes.restype = sz
    lib.gqa_decode_attention_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, f32, ctypes.c_int, vp, vp]
    lib.gqa_decode_attention_noalloc.restype = ctypes.c_int
    lib.qwen3_mfma_probe.argtypes = [i32, i32, vp, vp, vp]
    lib.qwen3_mfma_probe.restype = ctypes.c_int
    lib.qwen3_tile_weights.argtypes = [vp, ctypes.c_int, i32, i32, vp, vp]
    lib.qwen3_tile_weights.restype = ctypes.c_int
    lib.qwen3_layer_decode.argtypes = [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerWeights),
                                       vp, vp, vp, vp, vp, i32, i32, vp, sz, vp]
    lib.qwen3_layer_decode.restype = ctypes.c_int
    lib.qwen3_layer_decode_workspace_bytes.argtypes = [ctypes.POINTER(LayerCfg), i32]
    lib.qwen3_layer_decode_workspace_bytes.restype = sz
    lib.dequantize_matrix.argtypes = [ctypes.POINTER(QMatrix), i32, i32, ctypes.c_int, vp, vp]
    lib.dequantize_matrix.restype = ctypes.c_int
    lib.qwen3_layer_quant_workspace_bytes.argtypes = [ctypes.POINTER(LayerCfg), i32]
    lib.qwen3_layer_quant_workspace_bytes.restype = sz
    lib.qwen3_layer_prefill_quant.argtypes = [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerQWeights),
                                              vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, vp, sz, vp]
    lib.qwen3_layer_prefill_quant.restype = ctypes.c_int
    lib.qwen3_layer_decode_quant.argtypes = [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerQWeights),
                                             vp, vp, vp, vp, vp, i32, i32, vp, sz, vp]
    lib.qwen3_layer_decode_quant.restype = ctypes.c_int
    lib.qwen3_model_prefill_logits_last_kv.argtypes = [ctypes.POINTER(ModelCfg), ctypes.POINTER(ModelWeights),
                                                       vp, i32, vp, vp, i32, vp, vp, vp, i32, vp, vp, sz, vp]
    lib.qwen3_model_prefill_logits_last_kv.restype = ctypes.c_int
    lib.qwen3_model_decode_workspace_bytes.argtypes = [ctypes.POINTER(ModelCfg), i32]
    lib.qwen3_model_decode_workspace_bytes.restype = sz
    lib.qwen3_model_decode_logits.argtypes = [ctypes.POINTER(ModelCfg), ctypes.POINTER(ModelWeights), i32, vp, vp,
                                              vp, i32, i32, vp, vp, sz, vp]
    lib.qwen3_model_decode_logits.restype = ctypes.c_int
    lib.qwen3_last_error.argtypes = []
    lib.qwen3_last_error.restype = ctypes.c_char_p
    lib.qwen3_timing_enable.argtypes = [ctypes.c_int]
    lib.qwen3_timing_enable.restype = ctypes.c_int
    lib.qwen3_timing_collect.argtypes = [ctypes.POINTER(KernelTime), i32, ctypes.POINTER(i32)]
    lib.qwen3_timing_collect.restype = ctypes.c_int
    _lib = lib
    return lib


def check(status):
    if status != 0:
        msg = load().qwen3_last_error().decode(errors="replace")
        raise Qwen3Error(status, msg)
