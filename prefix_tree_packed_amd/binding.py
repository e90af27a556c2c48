"""Python binding of libtreeattn.so (include/tree_attn.h), same names as the C ABI.

Argument marshalling only: every step of the hot path runs in the library's
host code and HIP kernels. PyTorch provides device memory and the current HIP
stream. The binding checks tensor dtypes, devices, contiguity and shapes
against the plan before any pointer reaches the library (the C ABI sees only
pointers, so this is where a short buffer is caught). There is no fallback: if
the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtreeattn.so")

TA_OK = 0
STATUS_NAMES = {0: "TA_OK", 1: "TA_ERR_INVALID_ARGUMENT", 2: "TA_ERR_INVALID_TREE",
                3: "TA_ERR_LIMIT", 4: "TA_ERR_HIP", 5: "TA_ERR_WORKSPACE"}
TA_F16, TA_F32 = 0, 1

EXPORTED = ("tree_attn_plan", "tree_attn_plan_info", "tree_attn_plan_upload",
            "tree_attn_plan_export", "tree_attn_plan_schedule", "tree_attn_plan_masks",
            "tree_attn_plan_set_max_workgroups",
            "tree_attn_plan_workgroups", "tree_attn_plan_destroy", "tree_attn_forward",
            "tree_attn_forward_chunked", "tree_attn_cache_write", "tree_attn_rope_cache_write",
            "tree_attn_forward_cached",
            "tree_pack", "tree_pack_info", "tree_pack_export", "tree_pack_destroy",
            "tree_request_cost", "tree_form_batches", "readout_mlp_workspace_size", "readout_mlp",
            "readout_mlp_noalloc", "readout_pack_gate_up",
            "letter_logits", "decision_readout", "tree_attn_mfma_peak_probe", "tree_attn_last_error")


class TreeAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class _TreeDesc(ctypes.Structure):
    _fields_ = [("num_rows", ctypes.c_int32),
                ("row_block_indptr", ctypes.POINTER(ctypes.c_int32)),
                ("block_parent", ctypes.POINTER(ctypes.c_int32)),
                ("block_len", ctypes.POINTER(ctypes.c_int32)),
                ("row_q_begin", ctypes.POINTER(ctypes.c_int32)),
                ("row_q_end", ctypes.POINTER(ctypes.c_int32))]


class _AttnCfg(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("scale", ctypes.c_float),
                ("out_dtype", ctypes.c_int), ("write_lse", ctypes.c_int32),
                ("batch_invariant", ctypes.c_int32)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [("num_q_tokens", ctypes.c_int64), ("num_kv_tokens", ctypes.c_int64),
                ("useful_pairs", ctypes.c_int64), ("cost_packed", ctypes.c_int64),
                ("cost_separate", ctypes.c_int64), ("num_rows", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("num_leaves", ctypes.c_int32),
                ("max_depth", ctypes.c_int32), ("num_q_tiles", ctypes.c_int32),
                ("num_work_items", ctypes.c_int32), ("num_key_tiles", ctypes.c_int64),
                ("num_masked_key_tiles", ctypes.c_int64), ("q_tile_tokens", ctypes.c_int32),
                ("one_shot", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t),
                ("num_segments", ctypes.c_int64), ("batch_invariant", ctypes.c_int32),
                ("mask_words_per_tile", ctypes.c_int32), ("num_mask_words", ctypes.c_int64)]


class _PackInfo(ctypes.Structure):
    _fields_ = [("num_prompts", ctypes.c_int64), ("num_rows", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("num_tokens", ctypes.c_int64),
                ("separate_tokens", ctypes.c_int64)]


_lib = None


class _MlpWeights(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("eps", ctypes.c_float),
                ("pad0", ctypes.c_int32), ("norm_w", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p)]


def load_library(path: str = LIB_PATH):
    """Load libtreeattn.so once. torch is imported first so that the library
    binds to the HIP runtime torch already loaded (one runtime per process)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads torch's HIP runtime before ours)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m prefix_tree_packed_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    p32 = ctypes.POINTER(ctypes.c_int32)
    lib.tree_attn_plan.argtypes = [ctypes.POINTER(_TreeDesc), ctypes.POINTER(_AttnCfg), ctypes.POINTER(vp)]
    lib.tree_attn_plan_info.argtypes = [vp, ctypes.POINTER(_PlanInfo)]
    lib.tree_attn_plan_upload.argtypes = [vp, vp, ctypes.c_size_t, vp]
    lib.tree_attn_plan_export.argtypes = [vp, p32, p32, p32, p32, p32, p32]
    lib.tree_attn_plan_schedule.argtypes = [vp, p32, p32, p32, p32, p32]
    lib.tree_attn_plan_masks.argtypes = [vp, vp]
    lib.tree_attn_plan_set_max_workgroups.argtypes = [vp, i32]
    lib.tree_attn_plan_workgroups.argtypes = [vp, i32, p32, p32]
    lib.tree_attn_plan_destroy.argtypes = [vp]
    lib.tree_attn_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.tree_attn_forward_chunked.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, vp, vp]
    lib.tree_attn_cache_write.argtypes = [vp, vp, vp, vp, vp, i64, vp]
    lib.tree_attn_rope_cache_write.argtypes = [vp, vp, vp, vp, vp, vp, i32, ctypes.c_int, vp, vp,
                                               i64, vp]
    lib.tree_attn_forward_cached.argtypes = [vp, vp, vp, vp, i64, vp, vp, vp]
    lib.decision_readout.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, vp, vp, vp]
    p64 = ctypes.POINTER(ctypes.c_int64)
    lib.tree_pack.argtypes = [p32, p64, p32, p64, i32, i32, i32, ctypes.POINTER(vp)]
    lib.tree_pack_info.argtypes = [vp, ctypes.POINTER(_PackInfo)]
    lib.tree_pack_export.argtypes = [vp, p32, p32, p32, p32, p32, p32, p32]
    lib.tree_pack_destroy.argtypes = [vp]
    lib.tree_request_cost.argtypes = [p32, p64, i32, i32, p64]
    lib.tree_form_batches.argtypes = [p64, i32, i64, p32]
    lib.readout_mlp_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.readout_mlp.argtypes = [vp, i64, vp, i32, ctypes.POINTER(_MlpWeights), vp, ctypes.c_size_t, vp, vp]
    lib.readout_mlp_noalloc.argtypes = [vp, i64, vp, i32, ctypes.POINTER(_MlpWeights), vp, vp]
    lib.readout_pack_gate_up.argtypes = [vp, vp, i32, i32, vp, vp]
    lib.tree_attn_mfma_peak_probe.argtypes = [i32, i32, vp, ctypes.POINTER(ctypes.c_int64), vp]
    lib.letter_logits.argtypes = [vp, i32, i32, vp, ctypes.c_float, vp, i32, vp, vp, i32, vp, vp]
    for name in EXPORTED[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    lib.tree_attn_last_error.restype = ctypes.c_char_p
    lib.tree_attn_last_error.argtypes = []
    _lib = lib
    return lib


def tree_attn_last_error() -> str:
    return load_library().tree_attn_last_error().decode()


def _check(status: int):
    if status != TA_OK:
        raise TreeAttnError(status, tree_attn_last_error())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr32(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """Owns a ta_plan_t; freed by tree_attn_plan_destroy (or on garbage collection)."""

    def __init__(self, handle: int, arrays, cfg: dict):
        self.handle = ctypes.c_void_p(handle)
        self._arrays = arrays  # keep host arrays alive for the call's duration
        self.cfg = cfg
        self.workspace = None
        self._info = None

    @property
    def info(self) -> dict:
        if self._info is None:
            self._info = tree_attn_plan_info(self)
        return self._info

    def __del__(self):
        try:
            tree_attn_plan_destroy(self)
        except Exception:
            pass


def tree_attn_plan(tree, num_q_heads: int, num_kv_heads: int, head_dim: int, scale: float,
                   out_dtype: str = "f16", write_lse: bool = False,
                   batch_invariant: bool = False) -> Plan:
    """Build a plan from a tree description (any object with the fields
    row_block_indptr, block_parent, block_len, row_q_begin, row_q_end)."""
    lib = load_library()
    indptr = _i32(tree.row_block_indptr)
    parent = _i32(tree.block_parent)
    lens = _i32(tree.block_len)
    qb = None if getattr(tree, "row_q_begin", None) is None else _i32(tree.row_q_begin)
    qe = None if getattr(tree, "row_q_end", None) is None else _i32(tree.row_q_end)
    # The C planner reads these arrays up to the sizes indptr implies; a short
    # array would be read past its end, so the lengths are checked here.
    if indptr.ndim != 1 or indptr.shape[0] < 1 or int(indptr[0]) != 0:
        raise ValueError("row_block_indptr must be a 1-D array starting at 0")
    if np.any(np.diff(indptr) < 0):
        raise ValueError("row_block_indptr must be non-decreasing")
    n_rows, n_blocks = int(indptr.shape[0]) - 1, int(indptr[-1])
    if parent.shape != (n_blocks,) or lens.shape != (n_blocks,):
        raise ValueError(f"block_parent and block_len need {n_blocks} entries (row_block_indptr[-1]), "
                         f"got {parent.shape} and {lens.shape}")
    for name, a in (("row_q_begin", qb), ("row_q_end", qe)):
        if a is not None and a.shape != (n_rows,):
            raise ValueError(f"{name} needs {n_rows} entries (one per row), got {a.shape}")
    desc = _TreeDesc(int(indptr.shape[0]) - 1, _ptr32(indptr), _ptr32(parent), _ptr32(lens),
                     _ptr32(qb), _ptr32(qe))
    od = {"f16": TA_F16, "f32": TA_F32}[out_dtype]
    cfg = _AttnCfg(int(num_q_heads), int(num_kv_heads), int(head_dim), float(scale), od,
                   1 if write_lse else 0, 1 if batch_invariant else 0)
    out = ctypes.c_void_p()
    _check(lib.tree_attn_plan(ctypes.byref(desc), ctypes.byref(cfg), ctypes.byref(out)))
    return Plan(out.value, (indptr, parent, lens, qb, qe),
                {"num_q_heads": int(num_q_heads), "num_kv_heads": int(num_kv_heads),
                 "head_dim": int(head_dim), "scale": float(scale), "out_dtype": out_dtype,
                 "write_lse": bool(write_lse), "batch_invariant": bool(batch_invariant)})


def tree_attn_plan_info(plan: Plan) -> dict:
    info = _PlanInfo()
    _check(load_library().tree_attn_plan_info(plan.handle, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in _PlanInfo._fields_}


def tree_attn_plan_upload(plan: Plan, workspace=None, stream=None):
    """Upload the plan's device tables. Allocates a torch uint8 workspace on the
    current device when none is given; returns the workspace (kept on the plan)."""
    import torch
    need = plan.info["workspace_bytes"]
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load_library().tree_attn_plan_upload(plan.handle, ctypes.c_void_p(workspace.data_ptr()),
                                                nbytes, _stream_handle(stream)))
    plan.workspace = workspace
    return workspace


def tree_attn_plan_export(plan: Plan) -> dict:
    info = plan.info
    nq, nl = info["num_q_tokens"], info["num_leaves"]
    out = {k: np.zeros(nq, np.int32) for k in ("pos_id", "tok_row", "tok_block", "tok_offset")}
    out["leaf_block"] = np.zeros(nl, np.int32)
    out["leaf_readout_tok"] = np.zeros(nl, np.int32)
    _check(load_library().tree_attn_plan_export(
        plan.handle, _ptr32(out["pos_id"]), _ptr32(out["tok_row"]), _ptr32(out["tok_block"]),
        _ptr32(out["tok_offset"]), _ptr32(out["leaf_block"]), _ptr32(out["leaf_readout_tok"])))
    return out


def tree_attn_plan_schedule(plan: Plan) -> dict:
    """Host copy of the block-sparse schedule (query tiles, key tiles with their
    visibility interval and segments, work items longest first, per-token
    pre-order positions and subtree ends)."""
    info = plan.info
    out = {"q_tiles": np.zeros((info["num_q_tiles"], 5), np.int32),
           "key_tiles": np.zeros((info["num_key_tiles"], 8), np.int32),
           "work": np.zeros(info["num_work_items"], np.int32),
           "tok_anc": np.zeros((info["num_kv_tokens"], 2), np.int32),
           "segments": np.zeros((info["num_segments"], 2), np.int32)}
    _check(load_library().tree_attn_plan_schedule(
        plan.handle, _ptr32(out["q_tiles"]), _ptr32(out["key_tiles"]), _ptr32(out["work"]),
        _ptr32(out["tok_anc"]), _ptr32(out["segments"])))
    return out


def tree_attn_plan_masks(plan: Plan) -> np.ndarray:
    """Host copy of the visibility bits of the flagged key tiles, reshaped to
    [blocks, mask_words_per_tile] (uint32)."""
    info = plan.info
    out = np.zeros(info["num_mask_words"], np.uint32)
    _check(load_library().tree_attn_plan_masks(plan.handle, out.ctypes.data_as(ctypes.c_void_p)))
    return out.reshape(-1, info["mask_words_per_tile"])


def key_tile_rows(sch: dict, i: int) -> np.ndarray:
    """Row-space keys of key tile i of an exported schedule, in slot order."""
    k0, n, _, _, _, nseg, seg, _ = (int(x) for x in sch["key_tiles"][i])
    if nseg == 1:
        return np.arange(k0, k0 + n)
    segs = sch["segments"][seg:seg + nseg]
    out = np.empty(n, np.int64)
    for k, (slot0, row0) in enumerate(segs):
        slot1 = segs[k + 1][0] if k + 1 < nseg else n
        out[slot0:slot1] = np.arange(row0, row0 + slot1 - slot0)
    return out


def tree_attn_plan_set_max_workgroups(plan: Plan, max_workgroups: int) -> None:
    """Cap the persistent grid of later uploads (0: no cap)."""
    _check(load_library().tree_attn_plan_set_max_workgroups(plan.handle, int(max_workgroups)))


def tree_attn_plan_workgroups(plan: Plan, n_wg: int) -> dict:
    """Host copy of the split of the work items over n_wg persistent workgroups:
    workgroup w runs wg_items[wg_ptr[w]:wg_ptr[w + 1]]."""
    out = {"wg_ptr": np.zeros(max(int(n_wg), 0) + 1, np.int32),
           "wg_items": np.zeros(plan.info["num_work_items"], np.int32)}
    _check(load_library().tree_attn_plan_workgroups(plan.handle, int(n_wg), _ptr32(out["wg_ptr"]),
                                                    _ptr32(out["wg_items"])))
    return out


def tree_attn_plan_destroy(plan: Plan) -> None:
    if plan.handle is not None and plan.handle.value:
        _check(load_library().tree_attn_plan_destroy(plan.handle))
        plan.handle = ctypes.c_void_p(None)


def _expect(t, name, shape, dtype):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _vp(t):
    return ctypes.c_void_p(None if t is None else t.data_ptr())


def _attn_io_checks(plan, q, o, lse):
    import torch
    info, cfg = plan.info, plan.cfg
    nq, hq, hkv, d = info["num_q_tokens"], cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"]
    _expect(q, "q", (nq, hq, d), torch.float16)
    _expect(o, "o", (nq, hq, d), torch.float32 if cfg["out_dtype"] == "f32" else torch.float16)
    if lse is not None:
        _expect(lse, "lse", (hq, nq), torch.float32)
    return nq, hkv, d


def tree_attn_forward(plan: Plan, q, k, v, o, lse=None, stream=None) -> None:
    import torch
    nq, hkv, d = _attn_io_checks(plan, q, o, lse)
    _expect(k, "k", (nq, hkv, d), torch.float16)
    _expect(v, "v", (nq, hkv, d), torch.float16)
    _check(load_library().tree_attn_forward(plan.handle, _vp(q), _vp(k), _vp(v), _vp(o), _vp(lse),
                                            _stream_handle(stream)))


def tree_attn_forward_chunked(plan: Plan, q, k_new, v_new, k_cache, v_cache, o, lse=None,
                              stream=None) -> None:
    import torch
    nq, hkv, d = _attn_io_checks(plan, q, o, lse)
    _expect(k_new, "k_new", (nq, hkv, d), torch.float16)
    _expect(v_new, "v_new", (nq, hkv, d), torch.float16)
    ct = k_cache.shape[0]
    _expect(k_cache, "k_cache", (ct, hkv, d), torch.float16)
    _expect(v_cache, "v_cache", (ct, hkv, d), torch.float16)
    _check(load_library().tree_attn_forward_chunked(
        plan.handle, _vp(q), _vp(k_new), _vp(v_new), _vp(k_cache), _vp(v_cache), int(ct), _vp(o),
        _vp(lse), _stream_handle(stream)))


def tree_attn_cache_write(plan: Plan, k_new, v_new, k_cache, v_cache, stream=None) -> None:
    import torch
    info, cfg = plan.info, plan.cfg
    nq, hkv, d = info["num_q_tokens"], cfg["num_kv_heads"], cfg["head_dim"]
    _expect(k_new, "k_new", (nq, hkv, d), torch.float16)
    _expect(v_new, "v_new", (nq, hkv, d), torch.float16)
    ct = k_cache.shape[0]
    _expect(k_cache, "k_cache", (ct, hkv, d), torch.float16)
    _expect(v_cache, "v_cache", (ct, hkv, d), torch.float16)
    _check(load_library().tree_attn_cache_write(plan.handle, _vp(k_new), _vp(v_new), _vp(k_cache),
                                                _vp(v_cache), int(ct), _stream_handle(stream)))


ROPE_STYLES = {"half": 0, "interleaved": 1}


def tree_attn_rope_cache_write(plan: Plan, q_in, q_out, k_new, v_new, cos_sin, k_cache, v_cache,
                               style: str = "half", stream=None) -> None:
    """Rotary embedding at the plan's position ids on Q (into q_out, which may
    be q_in) and K, with rotated K and V written into the row-space cache.
    cos_sin: float32 [max_pos, head_dim / 2, 2] table of (cos, sin)."""
    import torch
    info, cfg = plan.info, plan.cfg
    nq, hq, hkv, d = info["num_q_tokens"], cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"]
    if style not in ROPE_STYLES:
        raise ValueError(f"style must be one of {sorted(ROPE_STYLES)}")
    _expect(q_in, "q_in", (nq, hq, d), torch.float16)
    _expect(q_out, "q_out", (nq, hq, d), torch.float16)
    _expect(k_new, "k_new", (nq, hkv, d), torch.float16)
    _expect(v_new, "v_new", (nq, hkv, d), torch.float16)
    _expect(cos_sin, "cos_sin", (cos_sin.shape[0], d // 2, 2), torch.float32)
    ct = k_cache.shape[0]
    _expect(k_cache, "k_cache", (ct, hkv, d), torch.float16)
    _expect(v_cache, "v_cache", (ct, hkv, d), torch.float16)
    _check(load_library().tree_attn_rope_cache_write(
        plan.handle, _vp(q_in), _vp(q_out), _vp(k_new), _vp(v_new), _vp(cos_sin),
        int(cos_sin.shape[0]), ROPE_STYLES[style], _vp(k_cache), _vp(v_cache), int(ct),
        _stream_handle(stream)))


def tree_attn_forward_cached(plan: Plan, q, k_cache, v_cache, o, lse=None, stream=None) -> None:
    import torch
    nq, hkv, d = _attn_io_checks(plan, q, o, lse)
    ct = k_cache.shape[0]
    _expect(k_cache, "k_cache", (ct, hkv, d), torch.float16)
    _expect(v_cache, "v_cache", (ct, hkv, d), torch.float16)
    _check(load_library().tree_attn_forward_cached(plan.handle, _vp(q), _vp(k_cache), _vp(v_cache),
                                                   int(ct), _vp(o), _vp(lse), _stream_handle(stream)))


def decision_readout(logits, row1, row2, n_letters, T, p_avg, p_cal, stream=None) -> None:
    import torch
    if logits.dim() != 2:
        raise ValueError("logits must be [n_rows, ld]")
    n_rows, ld = logits.shape
    n_dec = row1.shape[0]
    _expect(logits, "logits", (n_rows, ld), torch.float32)
    for name, t, dt in (("row1", row1, torch.int32), ("row2", row2, torch.int32),
                        ("n_letters", n_letters, torch.int32), ("T", T, torch.float32)):
        _expect(t, name, (n_dec,), dt)
    _expect(p_avg, "p_avg", (n_dec, ld), torch.float32)
    _expect(p_cal, "p_cal", (n_dec, ld), torch.float32)
    _check(load_library().decision_readout(_vp(logits), int(n_rows), int(ld), _vp(row1), _vp(row2),
                                           _vp(n_letters), _vp(T), int(n_dec), _vp(p_avg), _vp(p_cal),
                                           _stream_handle(stream)))


# ---------------------------------------------------------------------------
# readout-only last layer: MLP block at readout rows, answer-letter logits
# ---------------------------------------------------------------------------

def readout_mlp_workspace_size(n_readout: int, d_model: int, d_ff: int) -> int:
    out = ctypes.c_size_t()
    _check(load_library().readout_mlp_workspace_size(int(n_readout), int(d_model), int(d_ff),
                                                     ctypes.byref(out)))
    return int(out.value)


def readout_workspace_views(workspace, n_readout: int, d_model: int, d_ff: int):
    """(xn [n, d_model], act [n, d_ff]) f16 views of a readout_mlp workspace."""
    import torch
    b = workspace.view(torch.uint8)
    nx = n_readout * d_model * 2
    off = (nx + 255) // 256 * 256
    xn = b[:nx].view(torch.float16).view(n_readout, d_model)
    act = b[off:off + n_readout * d_ff * 2].view(torch.float16).view(n_readout, d_ff)
    return xn, act


def readout_pack_gate_up(w_gate, w_up, out=None, stream=None):
    """The interleaved [2 d_ff, d_model] gate/up matrix readout_mlp reads."""
    import torch
    ff, dm = w_gate.shape
    _expect(w_gate, "w_gate", (ff, dm), torch.float16)
    _expect(w_up, "w_up", (ff, dm), torch.float16)
    if out is None:
        out = torch.empty((2 * ff, dm), dtype=torch.float16, device=w_gate.device)
    _expect(out, "w_gate_up", (2 * ff, dm), torch.float16)
    _check(load_library().readout_pack_gate_up(_vp(w_gate), _vp(w_up), int(ff), int(dm), _vp(out),
                                               _stream_handle(stream)))
    return out


def readout_mlp(hidden, readout_tok, norm_w, w_gate_up, w_down, h_out, eps: float = 1e-5,
                workspace=None, stream=None):
    """MLP block with its residual at the readout rows of hidden [n_tokens, d_model]
    (f16): h_out [n_readout, d_model] f16. w_gate_up is readout_pack_gate_up's
    layout. Returns the workspace (uint8 tensor)."""
    import torch
    if hidden.dim() != 2:
        raise ValueError("hidden must be [n_tokens, d_model]")
    n_tok, dm = hidden.shape
    ff = w_gate_up.shape[0] // 2
    n = readout_tok.shape[0]
    _expect(hidden, "hidden", (n_tok, dm), torch.float16)
    _expect(readout_tok, "readout_tok", (n,), torch.int32)
    _expect(norm_w, "norm_w", (dm,), torch.float16)
    _expect(w_gate_up, "w_gate_up", (2 * ff, dm), torch.float16)
    _expect(w_down, "w_down", (dm, ff), torch.float16)
    _expect(h_out, "h_out", (n, dm), torch.float16)
    need = readout_mlp_workspace_size(n, dm, ff)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=hidden.device)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_cuda:
        raise ValueError("workspace must be a 1-D uint8 GPU tensor")
    w = _MlpWeights(int(dm), int(ff), float(eps), 0, norm_w.data_ptr(), w_gate_up.data_ptr(),
                    w_down.data_ptr())
    _check(load_library().readout_mlp(_vp(hidden), int(n_tok), _vp(readout_tok), int(n), ctypes.byref(w),
                                      _vp(workspace), int(workspace.numel()), _vp(h_out),
                                      _stream_handle(stream)))
    return workspace


def readout_mlp_noalloc(hidden, readout_tok, norm_w, w_gate_up, w_down, h_out, eps: float = 1e-5,
                        stream=None) -> None:
    """readout_mlp without a workspace: the library's fixed per-device scratch
    holds the intermediates (for callers that cannot allocate; calls that may
    overlap on one device race on that scratch)."""
    import torch
    if hidden.dim() != 2:
        raise ValueError("hidden must be [n_tokens, d_model]")
    n_tok, dm = hidden.shape
    ff = w_gate_up.shape[0] // 2
    n = readout_tok.shape[0]
    _expect(hidden, "hidden", (n_tok, dm), torch.float16)
    _expect(readout_tok, "readout_tok", (n,), torch.int32)
    _expect(norm_w, "norm_w", (dm,), torch.float16)
    _expect(w_gate_up, "w_gate_up", (2 * ff, dm), torch.float16)
    _expect(w_down, "w_down", (dm, ff), torch.float16)
    _expect(h_out, "h_out", (n, dm), torch.float16)
    w = _MlpWeights(int(dm), int(ff), float(eps), 0, norm_w.data_ptr(), w_gate_up.data_ptr(),
                    w_down.data_ptr())
    _check(load_library().readout_mlp_noalloc(_vp(hidden), int(n_tok), _vp(readout_tok), int(n),
                                              ctypes.byref(w), _vp(h_out), _stream_handle(stream)))


def letter_logits(h, final_norm_w, lm_head, letter_ids, n_letters, logits, eps: float = 1e-5,
                  stream=None) -> None:
    """Final RMS norm of readout rows h [n, d_model] (f16) and the logits of each
    row's letters: logits [n, ld] f32 (the layout decision_readout takes)."""
    import torch
    if h.dim() != 2 or logits.dim() != 2:
        raise ValueError("h must be [n, d_model] and logits [n, ld]")
    n, dm = h.shape
    ld = logits.shape[1]
    vocab = lm_head.shape[0]
    _expect(h, "h", (n, dm), torch.float16)
    _expect(final_norm_w, "final_norm_w", (dm,), torch.float16)
    _expect(lm_head, "lm_head", (vocab, dm), torch.float16)
    _expect(letter_ids, "letter_ids", (n, ld), torch.int32)
    _expect(n_letters, "n_letters", (n,), torch.int32)
    _expect(logits, "logits", (n, ld), torch.float32)
    _check(load_library().letter_logits(_vp(h), int(n), int(dm), _vp(final_norm_w), float(eps),
                                        _vp(lm_head), int(vocab), _vp(letter_ids), _vp(n_letters),
                                        int(ld), _vp(logits), _stream_handle(stream)))


def tree_attn_mfma_peak_probe(n_wg: int, iters: int, out, stream=None) -> int:
    """Launch the register-only MFMA probe (out: float32 GPU tensor of
    n_wg * 256 entries); returns the FLOPs it performs."""
    import torch
    _expect(out, "out", (n_wg * 256,), torch.float32)
    flops = ctypes.c_int64()
    _check(load_library().tree_attn_mfma_peak_probe(int(n_wg), int(iters), _vp(out), ctypes.byref(flops),
                                                    _stream_handle(stream)))
    return int(flops.value)


# ---------------------------------------------------------------------------
# packing tokenized prompts into prefix-tree rows, request cost, batches
# ---------------------------------------------------------------------------

def _ptr64(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _concat(prompts):
    lens = np.asarray([len(p) for p in prompts], np.int64)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    toks = (np.concatenate([np.asarray(p, np.int32) for p in prompts]).astype(np.int32)
            if len(prompts) else np.zeros(0, np.int32))
    return np.ascontiguousarray(toks), np.ascontiguousarray(indptr)


def tree_pack(prompts, parts=None, max_row_tokens: int = 32768, max_depth: int = 8) -> dict:
    """Pack tokenized prompts (sequences of token ids) into prefix-tree rows.
    parts[i] optionally lists prompt i's part lengths. Returns the rows in
    ta_tree_desc layout (row_block_indptr, block_parent, block_len), the row
    tokens and each prompt's (row, block, row-local readout index)."""
    lib = load_library()
    toks, indptr = _concat(prompts)
    pl = pi = None
    if parts is not None:
        pl, pi = _concat(parts)
    h = ctypes.c_void_p()
    _check(lib.tree_pack(_ptr32(toks), _ptr64(indptr), _ptr32(pl), _ptr64(pi), len(prompts),
                         int(max_row_tokens), int(max_depth), ctypes.byref(h)))
    try:
        info = _PackInfo()
        _check(lib.tree_pack_info(h, ctypes.byref(info)))
        out = {"row_block_indptr": np.zeros(info.num_rows + 1, np.int32),
               "block_parent": np.zeros(info.num_blocks, np.int32),
               "block_len": np.zeros(info.num_blocks, np.int32),
               "row_tokens": np.zeros(info.num_tokens, np.int32),
               "prompt_row": np.zeros(info.num_prompts, np.int32),
               "prompt_block": np.zeros(info.num_prompts, np.int32),
               "prompt_readout": np.zeros(info.num_prompts, np.int32)}
        _check(lib.tree_pack_export(h, *(_ptr32(out[k]) for k in (
            "row_block_indptr", "block_parent", "block_len", "row_tokens", "prompt_row",
            "prompt_block", "prompt_readout"))))
        out["separate_tokens"] = int(info.separate_tokens)
        return out
    finally:
        lib.tree_pack_destroy(h)


def tree_request_cost(prompts, cached_prefix: int = 0) -> int:
    lib = load_library()
    toks, indptr = _concat(prompts)
    cost = ctypes.c_int64()
    _check(lib.tree_request_cost(_ptr32(toks), _ptr64(indptr), len(prompts), int(cached_prefix),
                                 ctypes.byref(cost)))
    return int(cost.value)


def tree_form_batches(costs, limit: int = 8192) -> np.ndarray:
    lib = load_library()
    c = np.ascontiguousarray(np.asarray(costs, np.int64))
    out = np.zeros(len(c), np.int32)
    _check(lib.tree_form_batches(_ptr64(c), len(c), int(limit), _ptr32(out)))
    return out
