"""ctypes binding of liblps (include/lps.h): same names, argument marshalling only.

Every function here forwards to the C entry point of the same name and raises
LpsError on a negative status, with the library's own error text.  Loading
fails loudly when liblps.so has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# LPS_LIB_PATH selects another build of the same library (the host-sanitizer build)
LIB_PATH = os.environ.get("LPS_LIB_PATH") or os.path.join(_HERE, "liblps.so")

LPS_OK, LPS_EINVAL, LPS_ERANGE, LPS_ESTATE, LPS_EHIP, LPS_ENOMEM, LPS_EUNSUP = 0, -1, -2, -3, -4, -5, -6
LPS_F32, LPS_BF16, LPS_MXFP4 = 0, 1, 2
LPS_EPI_STORE, LPS_EPI_ADD, LPS_EPI_SWIGLU = 0, 1, 2
KINDS = {"qkv": 1, "attn": 2, "oproj": 3, "gateup": 4, "down": 5, "head": 6}
MOE_KINDS = {"moe_gateup": 7, "moe_down": 8, "moe_gemm1": 9, "moe_gemm2": 10}
LPS_FFN_DENSE, LPS_FFN_MOE = 0, 1
DTYPES = {"f32": LPS_F32, "bf16": LPS_BF16, "mxfp4": LPS_MXFP4}


class LpsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class LayerDesc(C.Structure):
    _fields_ = [
        ("d", C.c_int32), ("nq", C.c_int32), ("nkv", C.c_int32), ("hd", C.c_int32),
        ("ff", C.c_int32), ("wdtype", C.c_int32), ("kvdtype", C.c_int32), ("ctx_max", C.c_int32),
        ("eps", C.c_float), ("rope_base", C.c_float),
        ("g_attn", C.c_void_p),
        ("w_qkv", C.c_void_p), ("s_qkv", C.c_void_p),
        ("w_o", C.c_void_p), ("s_o", C.c_void_p),
        ("g_ffn", C.c_void_p),
        ("w_gu", C.c_void_p), ("s_gu", C.c_void_p),
        ("w_d", C.c_void_p), ("s_d", C.c_void_p),
        ("k_cache", C.c_void_p), ("v_cache", C.c_void_p), ("rope_cs", C.c_void_p),
        ("ffn_kind", C.c_int32), ("moe", C.c_void_p),
    ]


class HeadDesc(C.Structure):
    _fields_ = [("d", C.c_int32), ("vocab", C.c_int32), ("wdtype", C.c_int32), ("eps", C.c_float),
                ("g_out", C.c_void_p), ("w_lm", C.c_void_p)]


class HostRing(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("tok", C.c_void_p), ("slots", C.c_int32)]


class MoEDesc(C.Structure):
    _fields_ = [("d", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32), ("ff", C.c_int32),
                ("remote_from", C.c_int32), ("eps", C.c_float),
                ("g_ffn", C.c_void_p), ("w_r", C.c_void_p), ("w_gu_e", C.c_void_p),
                ("w_d_e", C.c_void_p), ("w_gu_s", C.c_void_p), ("w_d_s", C.c_void_p)]


class Counters(C.Structure):
    _fields_ = [("stage_walks", C.c_int64), ("boundary_sends", C.c_int64),
                ("boundary_recvs", C.c_int64), ("pieces", C.c_int64), ("drains", C.c_int64),
                ("prefill_walks", C.c_int64), ("act_pieces", C.c_int64)]


P = C.c_void_p
I32, I64, F32, SZ = C.c_int32, C.c_int64, C.c_float, C.c_size_t
PI32 = C.POINTER(C.c_int32)
PI64 = C.POINTER(C.c_int64)
PP = C.POINTER(C.c_void_p)

STREAM_SINK = 2048   # LPS_STREAM_SINK: uint32 entries lps_hbm_stream_read writes

# name: (restype, argtypes, checked)  -- checked: raise on a negative int status
SIGS = {
    "lps_last_error": (C.c_char_p, [], False),
    "lps_version": (C.c_char_p, [], False),
    "lps_stage_plan": (C.c_int, [I32, I32, PI32, I32, PI32], True),
    "lps_stage_plan_counts": (C.c_int, [I32, I32, PI32, PI32], True),
    "lps_stage_of": (C.c_int, [PI32, I32, I32], True),
    "lps_stage_solve": (C.c_int, [I32, I32, PI64, PI64, PI64, PI64, I64, PI32, PI64], True),
    "lps_layer_scratch_bytes": (SZ, [C.POINTER(LayerDesc)], False),
    "lps_layer_forward": (C.c_int, [C.POINTER(LayerDesc), P, I32, P, SZ, P], True),
    "lps_model_create": (C.c_int, [C.POINTER(LayerDesc), I32, PP], True),
    "lps_model_destroy": (C.c_int, [P], True),
    "lps_model_scratch_bytes": (SZ, [P], False),
    "lps_stage_forward": (C.c_int, [P, PI32, I32, I32, P, I32, P, SZ, P], True),
    "lps_stage_forward_dpos": (C.c_int, [P, PI32, I32, I32, P, P, P, SZ, P], True),
    "lps_stage_forward_static": (C.c_int, [P, PI32, I32, I32, P, I32, P], True),
    "lps_row_at_step": (C.c_int, [P, P, I64, P, I64, I32, I32, P], True),
    "lps_boundary_hop": (C.c_int, [P, P, P, I64, P], True),
    "lps_stage_forward_dpos_hop": (C.c_int, [P, PI32, I32, I32, P, P, P, SZ, P, P, I64, P], True),
    "lps_step_finish": (C.c_int, [P, P, P, P, I32, P, I32, P, P, I32, P, I32, P, P, P, P, SZ, P], True),
    "lps_prefill_scratch_bytes": (SZ, [P, I32], False),
    "lps_stage_prefill": (C.c_int, [P, PI32, I32, I32, P, I32, I32, P, SZ, P], True),
    "lps_embed_rows": (C.c_int, [P, I32, I32, I32, P, I32, P, P], True),
    "lps_rope_table": (C.c_int, [I32, F32, I32, P], True),
    "lps_step_advance": (C.c_int, [P, I32, P, P, P, I32, P, I32, P, I32, P, P], True),
    "lps_graph_begin": (C.c_int, [P], True),
    "lps_graph_end": (C.c_int, [P, PP, I32, PP], True),
    "lps_graph_launch": (C.c_int, [P, P], True),
    "lps_graph_destroy": (C.c_int, [P], True),
    "lps_embed": (C.c_int, [P, I32, I32, I32, P, P, P], True),
    "lps_head_scratch_bytes": (SZ, [C.POINTER(HeadDesc)], False),
    "lps_head_forward": (C.c_int, [C.POINTER(HeadDesc), P, P, P, P, SZ, P], True),
    "lps_rmsnorm": (C.c_int, [P, P, F32, I32, P, P], True),
    "lps_gemv": (C.c_int, [I32, P, P, I32, I32, P, P, F32, P, I32, P], True),
    "lps_qkv_rope_append": (C.c_int, [C.POINTER(LayerDesc), P, I32, P, P], True),
    "lps_attention_scratch_bytes": (SZ, [I32, I32, I32, I32], False),
    "lps_attention_decode": (C.c_int, [I32, I32, I32, I32, P, P, I32, I32, P, P, P, SZ, P], True),
    "lps_boundary_create": (C.c_int, [I32, P, P, PP], True),
    "lps_boundary_send": (C.c_int, [P, P, I64, P], True),
    "lps_boundary_recv": (C.c_int, [P, P, I64, P], True),
    "lps_boundary_destroy": (C.c_int, [P], True),
    "lps_copy_f32": (C.c_int, [P, P, I64, P], True),
    "lps_hbm_stream_read": (C.c_int, [P, I64, P, P], True),
    "lps_logits_defer": (C.c_int, [P, P, I32, P, P, P, P, PP], True),
    "lps_pending_mark": (C.c_int, [P, PP], True),
    "lps_pending_order": (C.c_int, [P, P], True),
    "lps_pending_wait": (C.c_int, [P], True),
    "lps_pending_drop": (C.c_int, [P], True),
    "lps_moe_route_scratch_bytes": (SZ, [C.POINTER(MoEDesc), I32], False),
    "lps_moe_route": (C.c_int, [C.POINTER(MoEDesc), P, I32, P, P, P, SZ, P], True),
    "lps_moe_combine": (C.c_int, [P, P, P, P, P, P, I32, I32, I32, P, P], True),
    "lps_f32_to_f16": (C.c_int, [P, P, I64, P], True),
    "lps_moe_prefill_scratch_bytes": (SZ, [C.POINTER(MoEDesc), I32], False),
    "lps_moe_prefill": (C.c_int, [C.POINTER(MoEDesc), P, I32, I32, P, SZ, P, P], True),
    "lps_moe_layer_scratch_bytes": (SZ, [C.POINTER(MoEDesc)], False),
    "lps_moe_layer_decode": (C.c_int, [C.POINTER(MoEDesc), P, P, SZ, P], True),
    "lps_counters": (C.c_int, [C.POINTER(Counters)], True),
    "lps_timer_start": (C.c_int, [I32, I32], True),
    "lps_timer_stop": (C.c_int, [C.POINTER(C.c_float), I32, PI32], True),
    "lps_counters_reset": (C.c_int, [], True),
}

_lib = None


def load() -> C.CDLL:
    """Load liblps.so (built in-tree by layer_pipeline_stage_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m layer_pipeline_stage_amd.build` (no fallback exists)")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args, _) in SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def last_error() -> str:
    return load().lps_last_error().decode()


def _wrap(name):
    res, _, checked = SIGS[name]

    def call(*args):
        r = getattr(load(), name)(*args)
        if checked and r < 0:
            raise LpsError(r, load().lps_last_error().decode())
        return r
    call.__name__ = name
    return call


for _n in SIGS:
    globals()[_n] = _wrap(_n)


def i32_array(vals):
    arr = (C.c_int32 * max(1, len(vals)))(*vals)
    return arr


def stage_plan(n_layers, n_stages, cuts=None):
    fence = (C.c_int32 * (n_stages + 1))()
    if cuts is None:
        lps_stage_plan(n_layers, n_stages, None, 0, fence)  # noqa: F821
    else:
        lps_stage_plan(n_layers, n_stages, i32_array(cuts), len(cuts), fence)  # noqa: F821
    return list(fence)


def stage_plan_counts(n_layers, counts):
    fence = (C.c_int32 * (len(counts) + 1))()
    lps_stage_plan_counts(n_layers, len(counts), i32_array(counts), fence)  # noqa: F821
    return list(fence)


def stage_of(fence, layer):
    return lps_stage_of(i32_array(fence), len(fence) - 1, layer)  # noqa: F821


def timer_stop(cap=1 << 16):
    buf = (C.c_float * cap)()
    n = C.c_int32()
    lps_timer_stop(buf, cap, C.byref(n))  # noqa: F821
    return [buf[i] for i in range(n.value)]


def rope_table(hd, base, n_pos):
    """lps_rope_table -> numpy f32 [n_pos, hd/2, 2] (host only)."""
    import numpy as np
    out = np.zeros((n_pos, hd // 2, 2), dtype=np.float32)
    lps_rope_table(hd, base, n_pos, out.ctypes.data)  # noqa: F821
    return out


def stage_solve(free, overhead, fixed, kv, n_stages, max_groups):
    """lps_stage_solve with Python lists -> (fence, page groups)."""
    L = len(fixed)
    A = C.c_int64 * max(1, n_stages)
    B = C.c_int64 * max(1, L)
    fence = (C.c_int32 * (n_stages + 1))()
    g = C.c_int64(0)
    lib = load()
    rc = lib.lps_stage_solve(L, n_stages, A(*free), A(*overhead), B(*fixed), B(*kv), max_groups,
                             fence, C.byref(g))
    if rc < 0:
        raise LpsError(rc, lib.lps_last_error().decode())
    return list(fence), g.value


def counters() -> dict:
    c = Counters()
    lps_counters(C.byref(c))  # noqa: F821
    return {k: getattr(c, k) for k, _ in Counters._fields_}
