"""Python binding of libsv (HIP, gfx950): batched verification of draft blocks.

Argument marshalling only.  Every function below has the name and argument
order of the C entry point declared in ``include/sv.h``; tensor arguments are
torch tensors (device memory, or host memory where the header says "host"),
``None`` passes a null pointer, and ``stream`` defaults to torch's current
stream.  A nonzero return code raises :class:`SvError`.  There is no fallback:
importing this package without the built ``libsv.so`` raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsv.so")

SV_F32 = 0
SV_BF16 = 1
SV_Q_DENSE = 0
SV_Q_MIXTURE = 1
SV_OK = 0
SV_ERR_ARG = 1
SV_ERR_WORKSPACE = 2
SV_ERR_LAUNCH = 3
SV_ERR_TOO_LARGE = 4
SV_NOALLOC_SCRATCH_BYTES = 1 << 20

STATUS_BITS = {
    0x001: "BAD_TEMPERATURE", 0x002: "BAD_TOP_P", 0x004: "NONFINITE", 0x008: "BAD_SCORE",
    0x010: "BAD_TOKEN", 0x020: "BAD_OFFSETS", 0x040: "EMPTY_POSTERIOR", 0x080: "BAD_BUDGET",
    0x100: "BAD_NACC", 0x200: "BAD_BLOCK", 0x400: "BAD_TREE",
}

EXPORTS = [
    "sv_workspace_bytes", "sv_workspace_init", "sv_get_status", "sv_clear_status", "sv_status_string",
    "dvl_alloc_pack", "sv_softmax_stats", "sv_topp_threshold", "sv_mixture_q", "sv_accept",
    "sv_residual_sample", "sv_philox_uniforms", "sv_verify_rows", "sv_verify_rows_dense", "sv_accept_sample",
    "sv_selftest_exp", "sv_selftest_philox_host", "sv_selftest_rows_host", "sv_residual_sample_noalloc",
    "sv_tree_workspace_bytes", "sv_tree_verify",
]


class SvError(RuntimeError):
    pass


# torch first: its libraries load the HIP runtime it ships (by the name
# libamdhip64.so), and libsv, loaded after it, binds to that same runtime by
# soname.  Loaded the other way round, libsv would pull in the system runtime
# and torch a second one beside it, and torch's streams would be foreign to
# libsv's launches.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libsv.so not found at {LIB_PATH}; build it with `python draft_verification_sv_amd/build.py` "
        "(there is no CPU fallback)"
    )

_lib = C.CDLL(LIB_PATH)

_vp, _i32, _i64, _sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
_SIGS = {
    "sv_workspace_bytes": [_i32, _i32, _i32, _i32, C.POINTER(C.c_size_t)],
    "sv_workspace_init": [_vp, _sz, _vp],
    "sv_get_status": [_vp, _vp, C.POINTER(C.c_uint32)],
    "sv_clear_status": [_vp, _vp],
    "dvl_alloc_pack": [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sv_softmax_stats": [_vp, _i32, _i64, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sv_topp_threshold": [_vp, _i32, _i64, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          _sz, _vp],
    "sv_mixture_q": [_vp, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sv_accept": [_vp, _i32, _i64, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i64,
                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sv_residual_sample": [_vp, _i32, _i64, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i64,
                           _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sv_residual_sample_noalloc": [_vp, _i32, _i64, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _vp,
                                   _i32, _i64, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "sv_philox_uniforms": [_vp, _i32, _i32, _vp, _vp],
    "sv_tree_workspace_bytes": [_i32, _i32, _i32, C.POINTER(C.c_size_t)],
    "sv_tree_verify": [_vp, _i32, _i64, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32,
                       _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _sz, _vp],
    "sv_selftest_exp": [_vp, _vp, _i32, _vp],
    "sv_verify_rows_dense": [_vp, _i32, _i64, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                             _i64, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "sv_verify_rows": [_vp, _i32, _i64, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32,
                       _i32, _vp, _i32, _vp, _vp, _vp, _sz, _vp],
    "sv_accept_sample": [_vp, _i32, _i64, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i64,
                         _vp, _vp, _i32, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                         _vp, _sz, _vp],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _i32
_lib.sv_status_string.argtypes = [_i32]
_lib.sv_status_string.restype = C.c_char_p
_lib.sv_selftest_rows_host.restype = _i32
_lib.sv_selftest_philox_host.restype = _i32


def lib():
    return _lib


def _p(t):
    """Raw pointer of a tensor (or int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def _check(rc: int, name: str):
    if rc != SV_OK:
        err = SvError(f"{name}: {_lib.sv_status_string(rc).decode()} (code {rc})")
        err.code = rc
        raise err


def sv_status_string(code: int) -> str:
    return _lib.sv_status_string(code).decode()


def decode_status(word: int) -> list:
    return [name for bit, name in STATUS_BITS.items() if word & bit]


# ---------------------------------------------------------------- workspace
def sv_workspace_bytes(R: int, b: int, K: int, V: int) -> int:
    out = C.c_size_t(0)
    _check(_lib.sv_workspace_bytes(R, b, K, V, C.byref(out)), "sv_workspace_bytes")
    return int(out.value)


def sv_workspace_init(ws, ws_bytes: int, stream=None):
    _check(_lib.sv_workspace_init(_p(ws), ws_bytes, _stream(stream)), "sv_workspace_init")


def sv_get_status(ws, stream=None) -> int:
    out = C.c_uint32(0)
    _check(_lib.sv_get_status(_p(ws), _stream(stream), C.byref(out)), "sv_get_status")
    return int(out.value)


def sv_clear_status(ws, stream=None):
    _check(_lib.sv_clear_status(_p(ws), _stream(stream)), "sv_clear_status")


def make_workspace(R: int, b: int, K: int, V: int, device="cuda"):
    """Allocate (torch) and zero a workspace; returns (tensor, nbytes)."""
    import torch

    n = sv_workspace_bytes(R, b, K, V)
    n = (n + 255) // 256 * 256
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    sv_workspace_init(ws, n)
    return ws, n


# ---------------------------------------------------------------- entry points
def dvl_alloc_pack(a, R, b, block_len, budget, s, L, pos_off, tgt_off, ws, ws_bytes, stream=None):
    _check(_lib.dvl_alloc_pack(_p(a), R, b, _p(block_len), _p(budget), _p(s), _p(L), _p(pos_off), _p(tgt_off),
                               _p(ws), ws_bytes, _stream(stream)), "dvl_alloc_pack")


def sv_softmax_stats(logits, dtype, ld, V, row_off, row_stride, R, max_rows, temperature, row_max, row_argmax,
                     row_lse, ws, ws_bytes, stream=None):
    _check(_lib.sv_softmax_stats(_p(logits), dtype, ld, V, _p(row_off), row_stride, R, max_rows, _p(temperature),
                                 _p(row_max), _p(row_argmax), _p(row_lse), _p(ws), ws_bytes, _stream(stream)),
           "sv_softmax_stats")


def sv_topp_threshold(logits, dtype, ld, V, row_off, row_stride, R, max_rows, temperature, top_p, row_max,
                      row_argmax, row_lse, row_cut, row_kept_lse, ws, ws_bytes, stream=None):
    _check(_lib.sv_topp_threshold(_p(logits), dtype, ld, V, _p(row_off), row_stride, R, max_rows, _p(temperature),
                                  _p(top_p), _p(row_max), _p(row_argmax), _p(row_lse), _p(row_cut),
                                  _p(row_kept_lse), _p(ws), ws_bytes, _stream(stream)), "sv_topp_threshold")


def sv_mixture_q(comp_logits, dtype, ld, V, K, b, mix_logits, pos_off, R, max_pos, draft_tok, branch_tok, post_w,
                 q_at_draft, ws, ws_bytes, stream=None):
    _check(_lib.sv_mixture_q(_p(comp_logits), dtype, ld, V, K, b, _p(mix_logits), _p(pos_off), R, max_pos,
                             _p(draft_tok), _p(branch_tok), _p(post_w), _p(q_at_draft), _p(ws), ws_bytes,
                             _stream(stream)), "sv_mixture_q")


def sv_verify_rows(tgt_logits, dtype, tgt_ld, V, tgt_off, R, max_rows, temperature, top_p, row_max, row_argmax,
                   row_lse, row_cut, row_kept_lse, comp_logits, comp_ld, K, b, pos_off, max_pos, draft_tok,
                   branch_T, ws, ws_bytes, stream=None):
    _check(_lib.sv_verify_rows(_p(tgt_logits), dtype, tgt_ld, V, _p(tgt_off), R, max_rows, _p(temperature),
                               _p(top_p), _p(row_max), _p(row_argmax), _p(row_lse), _p(row_cut), _p(row_kept_lse),
                               _p(comp_logits), comp_ld, K, b, _p(pos_off), max_pos, _p(draft_tok), _p(branch_T),
                               _p(ws), ws_bytes, _stream(stream)), "sv_verify_rows")


def sv_verify_rows_dense(tgt_logits, dtype, tgt_ld, V, tgt_off, R, max_rows, temperature, top_p, row_max,
                         row_argmax, row_lse, row_cut, row_kept_lse, draft_logits, draft_dtype, draft_ld, b, pos_off,
                         max_pos, draft_tok, draft_max, draft_argmax, draft_lse, ws, ws_bytes, stream=None):
    _check(_lib.sv_verify_rows_dense(_p(tgt_logits), dtype, tgt_ld, V, _p(tgt_off), R, max_rows, _p(temperature),
                                     _p(top_p), _p(row_max), _p(row_argmax), _p(row_lse), _p(row_cut),
                                     _p(row_kept_lse), _p(draft_logits), draft_dtype, draft_ld, b, _p(pos_off),
                                     max_pos, _p(draft_tok), _p(draft_max), _p(draft_argmax), _p(draft_lse), _p(ws),
                                     ws_bytes, _stream(stream)), "sv_verify_rows_dense")


def sv_accept_sample(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut,
                     row_kept_lse, draft_tok, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, K,
                     mix_logits, comp_logits, comp_ld, branch_T, branch_tok, post_w, q_at_draft, seed, n_acc, token,
                     is_bonus, p_out, q_out, u_out, ws, ws_bytes, stream=None):
    _check(_lib.sv_accept_sample(_p(tgt_logits), dtype, tgt_ld, V, _p(tgt_off), _p(pos_off), R, b, _p(temperature),
                                 _p(row_argmax), _p(row_cut), _p(row_kept_lse), _p(draft_tok), q_mode,
                                 _p(draft_logits), draft_dtype, draft_ld, _p(draft_argmax), _p(draft_lse), K,
                                 _p(mix_logits), _p(comp_logits), comp_ld, _p(branch_T), _p(branch_tok), _p(post_w),
                                 _p(q_at_draft), _p(seed), _p(n_acc), _p(token), _p(is_bonus), _p(p_out), _p(q_out),
                                 _p(u_out), _p(ws), ws_bytes, _stream(stream)), "sv_accept_sample")


def sv_accept(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut, row_kept_lse,
              draft_tok, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, q_at_draft, seed,
              n_acc, p_out, q_out, u_out, ws, ws_bytes, stream=None):
    _check(_lib.sv_accept(_p(tgt_logits), dtype, tgt_ld, V, _p(tgt_off), _p(pos_off), R, b, _p(temperature),
                          _p(row_argmax), _p(row_cut), _p(row_kept_lse), _p(draft_tok), q_mode, _p(draft_logits),
                          draft_dtype, draft_ld, _p(draft_argmax), _p(draft_lse), _p(q_at_draft), _p(seed),
                          _p(n_acc), _p(p_out), _p(q_out), _p(u_out), _p(ws), ws_bytes, _stream(stream)),
           "sv_accept")


def sv_residual_sample(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut,
                       row_kept_lse, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, K,
                       branch_tok, post_w, seed, n_acc, token, is_bonus, ws, ws_bytes, stream=None):
    _check(_lib.sv_residual_sample(_p(tgt_logits), dtype, tgt_ld, V, _p(tgt_off), _p(pos_off), R, b,
                                   _p(temperature), _p(row_argmax), _p(row_cut), _p(row_kept_lse), q_mode,
                                   _p(draft_logits), draft_dtype, draft_ld, _p(draft_argmax), _p(draft_lse), K,
                                   _p(branch_tok), _p(post_w), _p(seed), _p(n_acc), _p(token), _p(is_bonus), _p(ws),
                                   ws_bytes, _stream(stream)), "sv_residual_sample")


def sv_residual_sample_noalloc(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax,
                               row_cut, row_kept_lse, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax,
                               draft_lse, K, branch_tok, post_w, seed, n_acc, token, is_bonus, status, stream=None):
    _check(_lib.sv_residual_sample_noalloc(_p(tgt_logits), dtype, tgt_ld, V, _p(tgt_off), _p(pos_off), R, b,
                                           _p(temperature), _p(row_argmax), _p(row_cut), _p(row_kept_lse), q_mode,
                                           _p(draft_logits), draft_dtype, draft_ld, _p(draft_argmax), _p(draft_lse),
                                           K, _p(branch_tok), _p(post_w), _p(seed), _p(n_acc), _p(token),
                                           _p(is_bonus), _p(status), _stream(stream)), "sv_residual_sample_noalloc")


def sv_tree_workspace_bytes(max_nodes, max_kids, V) -> int:
    out = C.c_size_t(0)
    _check(_lib.sv_tree_workspace_bytes(max_nodes, max_kids, V, C.byref(out)), "sv_tree_workspace_bytes")
    return int(out.value)


def sv_tree_verify(tgt_logits, dtype, tgt_ld, V, node_off, parent, token, R, b, max_nodes, max_kids, temperature,
                   row_argmax, row_cut, row_kept_lse, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse,
                   seed, n_acc, path, stop_node, token_out, is_bonus, p_out, q_out, u_out, ws, ws_bytes, tree_ws,
                   tree_ws_bytes, stream=None):
    _check(_lib.sv_tree_verify(_p(tgt_logits), dtype, tgt_ld, V, _p(node_off), _p(parent), _p(token), R, b, max_nodes,
                               max_kids, _p(temperature), _p(row_argmax), _p(row_cut), _p(row_kept_lse),
                               _p(draft_logits), draft_dtype, draft_ld, _p(draft_argmax), _p(draft_lse), _p(seed),
                               _p(n_acc), _p(path), _p(stop_node), _p(token_out), _p(is_bonus), _p(p_out), _p(q_out),
                               _p(u_out), _p(ws), ws_bytes, _p(tree_ws), tree_ws_bytes, _stream(stream)),
           "sv_tree_verify")


def sv_selftest_exp(x, out, n, stream=None):
    _check(_lib.sv_selftest_exp(_p(x), _p(out), n, _stream(stream)), "sv_selftest_exp")


def sv_philox_uniforms(seed, R, n_pos, out, stream=None):
    _check(_lib.sv_philox_uniforms(_p(seed), R, n_pos, _p(out), _stream(stream)), "sv_philox_uniforms")


def sv_selftest_philox_host() -> int:
    return int(_lib.sv_selftest_philox_host())


def sv_selftest_rows_host() -> int:
    return int(_lib.sv_selftest_rows_host())


def selftest_host() -> dict:
    """Host-side checks compiled into the library (no GPU needed)."""
    return {"rows": sv_selftest_rows_host(), "philox": sv_selftest_philox_host()}
