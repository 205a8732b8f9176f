"""MI355X-native TurboQuant packed-key encode/score path.

The compute runs in libtq.so (hand-written HIP kernels for gfx950 behind the C
ABI in include/tq.h); this package is its thin Python binding. Using any
binding name raises ImportError if the library has not been built
(``python -m kv_cache_inner_amd.build``); there is no fallback path.
"""
import importlib

_BINDING = (
    "EXPORTS", "LIB_PATH", "TQ_APPEND_PREPARED", "TQ_BF16", "TQ_ERR_ARG", "TQ_ERR_DEVICE", "TQ_ERR_UNSUPPORTED",
    "TQ_ERR_WORKSPACE", "TQ_F16", "TQ_F32", "TQ_OK", "TQ_OP_ATTEND", "TQ_OP_ENCODE", "TQ_OP_SCORE", "TQ_OP_TOPK", "Bank",
    "Params", "TQError", "attend_workspace", "make_params", "score_workspace", "tq_attend", "tq_bank", "tq_copy",
    "tq_decode", "tq_encode", "tq_encode_append", "tq_encode_append_noalloc", "tq_fp32_logits", "tq_make_codebook", "tq_make_codebook_sphere",
    "tq_make_rotation", "tq_make_rotation_hadamard", "tq_params", "tq_prepare_queries", "tq_score",
    "tq_score_prepared", "tq_status_string", "tq_topk", "_lib",
)


def __getattr__(name):
    if name in _BINDING:
        mod = importlib.import_module("._lib", __name__)
        return mod if name == "_lib" else getattr(mod, name)
    raise AttributeError(name)
