"""Thin ctypes binding of the ReplaySSM C ABI (include/ssm_replay.h).

Argument marshalling only: every function here has the name of the C entry point it calls, turns
torch tensors into device pointers and the current HIP stream into a hipStream_t, and raises
SSMError on a non-zero status. All computation happens in the HIP library; there is no fallback
path, and importing this module fails loudly when libssm_replay.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Mapping, Optional

import torch

# the in-tree build; SSM_REPLAY_LIB names another build of the same library (same ABI) instead
_LIB_PATH = (os.environ.get("SSM_REPLAY_LIB")
             or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssm_replay.so"))

SSM_OK, SSM_E_ARG, SSM_E_SHAPE, SSM_E_ALIGN, SSM_E_STATE, SSM_E_CAPACITY, SSM_E_UNSUPPORTED, \
    SSM_E_HIP = 0, -1, -2, -3, -4, -5, -6, -7
SSM_MAMBA2, SSM_GDN, SSM_KDA = 0, 1, 2
SSM_IN_F32, SSM_IN_BF16 = 0, 1
SSM_RC_NONE, SSM_RC_FP8_ROW, SSM_RC_FP4_B16 = 0, 1, 2
SSM_FLUSH_IF_FULL, SSM_FLUSH_ALL = 0, 1
SSM_FLAG_ACCEPT_CLAMPED = 1


class SSMError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, _lib.ssm_status_string(status).decode(),
                                                 status))


class ssm_config(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("groups", ctypes.c_int32), ("dim_p", ctypes.c_int32), ("dim_n", ctypes.c_int32),
                ("window", ctypes.c_int32), ("max_draft", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("readcopy", ctypes.c_int32),
                ("gdn_scale", ctypes.c_float), ("share_ckpt", ctypes.c_int32)]


class ssm_layout(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_uint64), ("ring_cap", ctypes.c_int32),
                ("ckpt_slots", ctypes.c_int32), ("off_ckpt", ctypes.c_uint64),
                ("off_rc_codes", ctypes.c_uint64), ("off_rc_scale", ctypes.c_uint64),
                ("off_rc_tscale", ctypes.c_uint64), ("off_ring", ctypes.c_uint64 * 5),
                ("off_ptr", ctypes.c_uint64), ("off_flags", ctypes.c_uint64),
                ("off_refcnt", ctypes.c_uint64)]


class ssm_state(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("pending", ctypes.c_int32),
                ("count_lo", ctypes.c_int32), ("count_hi", ctypes.c_int32),
                ("cfg", ssm_config), ("lay", ssm_layout), ("mem", ctypes.c_void_p),
                ("A", ctypes.c_void_p), ("D", ctypes.c_void_p), ("ring_start", ctypes.c_int32)]


class ssm_m2_in(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("dt", ctypes.c_void_p)]


class ssm_gdn_in(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("g", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libssm_replay.so is not built (run __graft_entry__.build() or "
                           "python -m ssm_decode_state_amd.build); there is no fallback path")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32
    P = ctypes.POINTER
    sig = {
        "ssm_abi_version": ([], i32),
        "ssm_status_string": ([st], ctypes.c_char_p),
        "ssm_layout_query": ([P(ssm_config), P(ssm_layout)], st),
        "ssm_ckpt_init": ([P(ssm_state), P(ssm_config), vp, ctypes.c_uint64, vp, vp, vp, vp], st),
        "ssm_replay_decode": ([P(ssm_state), vp, vp, vp], st),
        "ssm_flush": ([P(ssm_state), i32, vp], st),
        "ssm_spec_append": ([P(ssm_state), i32, vp, vp, vp], st),
        "ssm_spec_rollback": ([P(ssm_state), vp, vp], st),
        "ssm_ckpt_export": ([P(ssm_state), vp, vp], st),
        "ssm_conventional_step": ([P(ssm_config), vp, vp, vp, vp, vp, vp], st),
        "ssm_tiles_pack": ([P(ssm_config), vp, vp, vp], st),
        "ssm_tiles_unpack": ([P(ssm_config), vp, vp, vp], st),
        "ssm_debug_codec": ([i32, vp, vp, ctypes.c_int64, vp], st),
        "ssm_conventional_spec_snapshot": ([P(ssm_config), vp, vp, i32, vp, vp, vp, vp, vp], st),
        "ssm_conventional_spec_select": ([P(ssm_config), vp, vp, i32, vp, vp], st),
        "ssm_debug_flags": ([P(ssm_state), P(ctypes.c_int32), i32, vp], st),
        "ssm_restore": ([P(ssm_state), vp, vp], st),
        "ssm_fork": ([P(ssm_state), P(ctypes.c_int32), P(ctypes.c_int32), i32, vp], st),
        "ssm_debug_stream_read": ([vp, ctypes.c_uint64, vp, i32, vp], st),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


_lib = _load()
EXPORTS = ("ssm_abi_version", "ssm_status_string", "ssm_layout_query", "ssm_ckpt_init",
           "ssm_replay_decode", "ssm_flush", "ssm_spec_append", "ssm_spec_rollback",
           "ssm_ckpt_export", "ssm_conventional_step", "ssm_tiles_pack", "ssm_tiles_unpack",
           "ssm_debug_codec", "ssm_conventional_spec_snapshot", "ssm_conventional_spec_select",
           "ssm_debug_flags", "ssm_restore", "ssm_fork", "ssm_debug_stream_read")


def _st(st):
    """Accept either an ssm_state or a State that owns one."""
    return st.st if isinstance(st, State) else st


def _check(fn: str, status: int) -> None:
    if status != SSM_OK:
        raise SSMError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the ReplaySSM ABI must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def make_config(kind: int, batch: int, heads: int, groups: int, dim_p: int, dim_n: int,
                window: int, max_draft: int = 1, in_dtype: int = SSM_IN_BF16,
                readcopy: int = SSM_RC_NONE, gdn_scale: float = 1.0,
                share_ckpt: int = 0) -> ssm_config:
    return ssm_config(kind, batch, heads, groups, dim_p, dim_n, window, max_draft, in_dtype,
                      readcopy, gdn_scale, share_ckpt)


def _inputs(cfg: ssm_config, inp: Mapping[str, torch.Tensor]):
    if cfg.kind == SSM_MAMBA2:
        return ssm_m2_in(inp["x"].data_ptr(), inp["B"].data_ptr(), inp["C"].data_ptr(),
                         inp["dt"].data_ptr())
    return ssm_gdn_in(inp["q"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(),
                      inp["beta"].data_ptr(), inp["g"].data_ptr())


def ssm_abi_version() -> int:
    return _lib.ssm_abi_version()


def ssm_status_string(status: int) -> str:
    return _lib.ssm_status_string(status).decode()


def ssm_layout_query(cfg: ssm_config) -> ssm_layout:
    lay = ssm_layout()
    _check("ssm_layout_query", _lib.ssm_layout_query(ctypes.byref(cfg), ctypes.byref(lay)))
    return lay


def ssm_ckpt_init(st: ssm_state, cfg: ssm_config, mem: torch.Tensor, h0: Optional[torch.Tensor],
                  A: Optional[torch.Tensor], D: Optional[torch.Tensor], stream=None) -> None:
    _check("ssm_ckpt_init", _lib.ssm_ckpt_init(
        ctypes.byref(st), ctypes.byref(cfg), _ptr(mem), mem.numel() * mem.element_size(),
        _ptr(h0), _ptr(A), _ptr(D), _stream(stream)))


def ssm_replay_decode(st: ssm_state, inputs: Mapping[str, torch.Tensor], y: torch.Tensor,
                      stream=None) -> None:
    st = _st(st)
    inp = _inputs(st.cfg, inputs)
    _check("ssm_replay_decode", _lib.ssm_replay_decode(ctypes.byref(st), ctypes.byref(inp),
                                                       _ptr(y), _stream(stream)))


def ssm_flush(st: ssm_state, mode: int, stream=None) -> None:
    st = _st(st)
    _check("ssm_flush", _lib.ssm_flush(ctypes.byref(st), mode, _stream(stream)))


def ssm_spec_append(st: ssm_state, ndraft: int, inputs: Mapping[str, torch.Tensor],
                    y: torch.Tensor, stream=None) -> None:
    st = _st(st)
    inp = _inputs(st.cfg, inputs)
    _check("ssm_spec_append", _lib.ssm_spec_append(ctypes.byref(st), ndraft, ctypes.byref(inp),
                                                   _ptr(y), _stream(stream)))


def ssm_spec_rollback(st: ssm_state, n_accept: torch.Tensor, stream=None) -> None:
    if n_accept.dtype != torch.int32:
        raise ValueError("n_accept must be int32")
    st = _st(st)
    _check("ssm_spec_rollback", _lib.ssm_spec_rollback(ctypes.byref(st), _ptr(n_accept),
                                                       _stream(stream)))


def ssm_restore(st, n_back: torch.Tensor, stream=None) -> None:
    if n_back.dtype != torch.int32:
        raise ValueError("n_back must be int32")
    st = _st(st)
    _check("ssm_restore", _lib.ssm_restore(ctypes.byref(st), _ptr(n_back), _stream(stream)))


def ssm_fork(st, src, dst, stream=None) -> None:
    """src, dst: sequences of host ints (copied into host int32 arrays)."""
    src, dst = list(src), list(dst)
    if len(src) != len(dst):
        raise ValueError("src and dst must have the same length")
    n = len(src)
    a = (ctypes.c_int32 * max(n, 1))(*src)
    b = (ctypes.c_int32 * max(n, 1))(*dst)
    st = _st(st)
    _check("ssm_fork", _lib.ssm_fork(ctypes.byref(st), a, b, n, _stream(stream)))


def ssm_ckpt_export(st: ssm_state, h_out: torch.Tensor, stream=None) -> None:
    st = _st(st)
    _check("ssm_ckpt_export", _lib.ssm_ckpt_export(ctypes.byref(st), _ptr(h_out),
                                                   _stream(stream)))


def ssm_conventional_step(cfg: ssm_config, h: torch.Tensor, inputs: Mapping[str, torch.Tensor],
                          A: Optional[torch.Tensor], D: Optional[torch.Tensor], y: torch.Tensor,
                          stream=None) -> None:
    inp = _inputs(cfg, inputs)
    _check("ssm_conventional_step", _lib.ssm_conventional_step(
        ctypes.byref(cfg), _ptr(h), ctypes.byref(inp), _ptr(A), _ptr(D), _ptr(y),
        _stream(stream)))


def ssm_conventional_spec_snapshot(cfg: ssm_config, h: torch.Tensor, h_snap: torch.Tensor,
                                   ndraft: int, inputs: Mapping[str, torch.Tensor],
                                   A: torch.Tensor, D: torch.Tensor, y: torch.Tensor,
                                   stream=None) -> None:
    inp = _inputs(cfg, inputs)
    _check("ssm_conventional_spec_snapshot", _lib.ssm_conventional_spec_snapshot(
        ctypes.byref(cfg), _ptr(h), _ptr(h_snap), ndraft, ctypes.byref(inp), _ptr(A), _ptr(D),
        _ptr(y), _stream(stream)))


def ssm_conventional_spec_select(cfg: ssm_config, h: torch.Tensor, h_snap: torch.Tensor,
                                 ndraft: int, n_accept: torch.Tensor, stream=None) -> None:
    if n_accept.dtype != torch.int32:
        raise ValueError("n_accept must be int32")
    _check("ssm_conventional_spec_select", _lib.ssm_conventional_spec_select(
        ctypes.byref(cfg), _ptr(h), _ptr(h_snap), ndraft, _ptr(n_accept), _stream(stream)))


def ssm_debug_stream_read(src: torch.Tensor, out: torch.Tensor, blocks: int, stream=None) -> None:
    """One pass of streaming reads over the bytes of src (measurement reference); out: int32
    [>= 4 * blocks] on the device."""
    _check("ssm_debug_stream_read", _lib.ssm_debug_stream_read(
        _ptr(src), src.numel() * src.element_size(), _ptr(out), blocks, _stream(stream)))


def ssm_debug_flags(st, clear: bool = False, stream=None) -> int:
    st = _st(st)
    out = ctypes.c_int32(0)
    _check("ssm_debug_flags", _lib.ssm_debug_flags(ctypes.byref(st), ctypes.byref(out),
                                                   int(clear), _stream(stream)))
    return out.value


def ssm_tiles_pack(cfg: ssm_config, natural: torch.Tensor, tiles: torch.Tensor,
                   stream=None) -> None:
    _check("ssm_tiles_pack", _lib.ssm_tiles_pack(ctypes.byref(cfg), _ptr(natural), _ptr(tiles),
                                                 _stream(stream)))


def ssm_tiles_unpack(cfg: ssm_config, tiles: torch.Tensor, natural: torch.Tensor,
                     stream=None) -> None:
    _check("ssm_tiles_unpack", _lib.ssm_tiles_unpack(ctypes.byref(cfg), _ptr(tiles),
                                                     _ptr(natural), _stream(stream)))


# bytes of input and output per work item of each ssm_debug_codec op
_CODEC_IO = {0: (4, 1), 1: (1, 4), 2: (4, 1), 3: (1, 4), 4: (4, 1), 5: (1, 4), 6: (4, 1),
             7: (1, 4), 8: (4, 16), 9: (4, 32), 10: (16, 4), 11: (32, 4)}


def ssm_debug_codec(op: int, inp: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """n = number of work items implied by the input size; both buffers are checked to hold n
    items (the C entry point takes plain pointers and cannot check)."""
    if op not in _CODEC_IO:
        raise ValueError("unknown codec op %d" % op)
    bi, bo = _CODEC_IO[op]
    nin = inp.numel() * inp.element_size()
    n = nin // bi
    if n * bi != nin or out.numel() * out.element_size() < n * bo:
        raise ValueError("codec op %d: input of %d bytes / output of %d bytes do not match"
                         % (op, nin, out.numel() * out.element_size()))
    _check("ssm_debug_codec", _lib.ssm_debug_codec(op, _ptr(inp), _ptr(out), n, _stream(stream)))


class State:
    """Owner of one layer's device memory and its ssm_state (keeps the borrowed tensors alive)."""

    def __init__(self, cfg: ssm_config, h0: Optional[torch.Tensor] = None,
                 A: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
                 device: str = "cuda", stream=None):
        self.cfg = cfg
        self.layout = ssm_layout_query(cfg)
        self.mem = torch.empty(max(1, self.layout.total_bytes), dtype=torch.uint8, device=device)
        self.A, self.D = A, D
        self.st = ssm_state()
        ssm_ckpt_init(self.st, cfg, self.mem, h0, A, D, stream)

    def region(self, offset: int, nbytes: int) -> torch.Tensor:
        """Raw bytes of a region of the state memory (a view, for inspection in tests)."""
        return self.mem[offset:offset + nbytes]
