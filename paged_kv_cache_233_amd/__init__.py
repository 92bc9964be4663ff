"""Paged KV-cache attention for MI355X (gfx950).

A thin ctypes binding of ``libpkv.so`` (built from ``csrc/``): argument
marshalling only. Every step of the hot path runs in the library: the host
block allocator in C++, and the scatter, block copy, decode and
chunked-prefill attention in HIP kernels. PyTorch provides device memory and
the stream; tensors are passed as raw pointers with
``torch.cuda.current_stream()``.

There is no fallback: if the library cannot be built or loaded, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Dict, List, NamedTuple, Optional, Sequence, Tuple

import numpy as np

__all__ = ["Error", "Allocator", "library", "reshape_and_cache", "copy_blocks",
           "decode_workspace_size", "decode_workspace", "decode", "prefill_workspace_size",
           "prefill_workspace", "prefill_chunk",
           "F32", "BF16", "BLOCK_SIZE"]

BLOCK_SIZE = 16
F32 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")
# The host-only build of the allocator, scheduler and hashing code with
# address and undefined-behaviour sanitizers (build.build_host_sanitized()).
# With PKV_HOST_SANITIZED=1 the binding loads it instead of libpkv.so; its
# kernel entry points are absent and calling one raises AttributeError.
HOST_SANITIZED_LIB_PATH = os.path.join(_HERE, "libpkv_host_asan.so")

_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None

_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p
_c_f = ctypes.c_float
_c_sz = ctypes.c_size_t


class Stats(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("used_blocks", ctypes.c_int32),
                ("free_blocks", ctypes.c_int32), ("shared_blocks", ctypes.c_int32),
                ("logical_tokens", ctypes.c_int64), ("stored_tokens", ctypes.c_int64),
                ("utilisation", ctypes.c_double)]


_SIGNATURES = {
    "pkv_last_error": ([], ctypes.c_char_p),
    "pkv_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "pkv_version": ([], ctypes.c_int),
    "pkv_allocator_create": ([_c_i32, ctypes.POINTER(_c_p)], ctypes.c_int),
    "pkv_allocator_destroy": ([_c_p], ctypes.c_int),
    "pkv_allocator_set_free_order": ([_c_p, _c_p, _c_i32], ctypes.c_int),
    "pkv_allocator_shuffle_free_list": ([_c_p, ctypes.c_uint64], ctypes.c_int),
    "pkv_set_debug_checks": ([_c_i32], ctypes.c_int),
    "pkv_check_slot_mapping": ([_c_p, _c_i64, _c_i32], ctypes.c_int),
    "pkv_seq_add": ([_c_p, _c_i64], ctypes.c_int),
    "pkv_seq_append": ([_c_p, _c_i64, _c_i32, _c_p, _c_p, _c_i32, _c_p], ctypes.c_int),
    "pkv_batch_append": ([_c_p, _c_p, _c_p, _c_i32, _c_p, _c_p, _c_i32, _c_p], ctypes.c_int),
    "pkv_seq_fork": ([_c_p, _c_i64, _c_i64], ctypes.c_int),
    "pkv_seq_free": ([_c_p, _c_i64], ctypes.c_int),
    "pkv_seq_len": ([_c_p, _c_i64, _c_p], ctypes.c_int),
    "pkv_allocator_enable_prefix_caching": ([_c_p, _c_i32], ctypes.c_int),
    "pkv_seq_add_cached": ([_c_p, _c_i64, _c_p, _c_i32, ctypes.c_uint64, _c_i32, _c_p], ctypes.c_int),
    "pkv_stream_read": ([_c_p, _c_sz, _c_p, _c_i32, _c_p], ctypes.c_int),
    "pkv_prefix_lookup": ([_c_p, _c_p, _c_i32, ctypes.c_uint64, _c_i32, _c_p, _c_p], ctypes.c_int),
    "pkv_scheduler_create": ([_c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_p], ctypes.c_int),
    "pkv_scheduler_destroy": ([_c_p], ctypes.c_int),
    "pkv_scheduler_add_request": ([_c_p, _c_i64, _c_p, _c_i32, _c_i32, ctypes.c_uint64], ctypes.c_int),
    "pkv_scheduler_schedule": ([_c_p, _c_p, _c_p, _c_p], ctypes.c_int),
    "pkv_scheduler_plan": ([_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p], ctypes.c_int),
    "pkv_scheduler_update": ([_c_p, _c_p, _c_i32, _c_p], ctypes.c_int),
    "pkv_scheduler_finished": ([_c_p, _c_p], ctypes.c_int),
    "pkv_scheduler_remove_request": ([_c_p, _c_i64], ctypes.c_int),
    "pkv_scheduler_counts": ([_c_p, _c_p, _c_p], ctypes.c_int),
    "pkv_scheduler_request": ([_c_p, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32], ctypes.c_int),
    "pkv_seq_record_tokens": ([_c_p, _c_i64, _c_p, _c_i32], ctypes.c_int),
    "pkv_block_hash": ([_c_p, _c_i32, _c_p, _c_p], ctypes.c_int),
    "pkv_prefix_cache_stats": ([_c_p, _c_p, _c_p, _c_p], ctypes.c_int),
    "pkv_hash_block_tokens": ([_c_p, _c_p, ctypes.c_uint64, _c_p], ctypes.c_int),
    "pkv_sha256": ([_c_p, ctypes.c_size_t, _c_p], ctypes.c_int),
    "pkv_fill_block_table": ([_c_p, _c_p, _c_i32, _c_p, _c_i32, _c_p], ctypes.c_int),
    "pkv_block_refcount": ([_c_p, _c_i32, _c_p], ctypes.c_int),
    "pkv_num_free_blocks": ([_c_p, _c_p], ctypes.c_int),
    "pkv_allocator_stats": ([_c_p, ctypes.POINTER(Stats)], ctypes.c_int),
    "pkv_blocks_for_bytes": ([_c_i64, _c_i32, _c_i32, _c_i32, _c_p], ctypes.c_int),
    "pkv_reshape_and_cache": ([_c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i64, _c_i32, _c_i32,
                               _c_i32, _c_i32, _c_p], ctypes.c_int),
    "pkv_stage_copy": ([_c_p, _c_p, ctypes.c_size_t, _c_p], ctypes.c_int),
    "pkv_decode_shared_prefix_workspace_size": ([_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_p],
                                                ctypes.c_int),
    "pkv_paged_attention_decode_shared_prefix": ([_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32,
                                                 _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                 ctypes.c_float, _c_i32, _c_p, ctypes.c_size_t, _c_p],
                                                ctypes.c_int),
    "pkv_copy_blocks": ([_c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_p],
                        ctypes.c_int),
    "pkv_decode_workspace_size": ([_c_i32, _c_i32, _c_i32, _c_i32, ctypes.POINTER(_c_sz)],
                                  ctypes.c_int),
    "pkv_decode_set_waves_per_cu": ([_c_i32], ctypes.c_int),
    "pkv_paged_attention_decode": ([_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                    _c_i32, _c_i32, _c_i32, _c_f, _c_i32, _c_p, _c_sz, _c_p],
                                   ctypes.c_int),
    "pkv_paged_attention_decode_append": ([_c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_p, _c_p,
                                           _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f,
                                           _c_i32, _c_p, _c_sz, _c_p], ctypes.c_int),
    "pkv_paged_attention_decode_append_split": ([_c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_p,
                                                 _c_p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                 _c_i32, _c_f, _c_i32, _c_p, _c_sz, _c_p],
                                                ctypes.c_int),
    "pkv_paged_attention_decode_noalloc": ([_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32,
                                            _c_i32, _c_i32, _c_i32, _c_i32, _c_f, _c_i32, _c_p],
                                           ctypes.c_int),
    "pkv_paged_attention_decode_split": ([_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32,
                                          _c_i32, _c_i32, _c_i32, _c_i32, _c_f, _c_i32, _c_p,
                                          _c_sz, _c_p], ctypes.c_int),
    "pkv_paged_attention_decode_merge": ([_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32,
                                          _c_i32, _c_i32, _c_i32, _c_i32, _c_f, _c_i32, _c_p,
                                          _c_sz, _c_p], ctypes.c_int),
    "pkv_prefill_workspace_size": ([_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                    ctypes.POINTER(_c_sz)], ctypes.c_int),
    "pkv_paged_attention_prefill_chunk": ([_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32,
                                           _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                           _c_i32, _c_f, _c_i32, _c_p, _c_sz, _c_p], ctypes.c_int),
}


def library() -> ctypes.CDLL:
    """The loaded libpkv.so (built in place first if it is missing)."""
    global _lib
    with _lock:
        if _lib is None:
            host_only = os.environ.get("PKV_HOST_SANITIZED") == "1"
            path = HOST_SANITIZED_LIB_PATH if host_only else LIB_PATH
            # another build of the same library (same entry points), e.g. an
            # instrumented one
            path = os.environ.get("PKV_LIBRARY", path)
            if not os.path.exists(path):
                from . import build as _build
                if host_only:
                    _build.build_host_sanitized()
                else:
                    _build.build()
            lib = ctypes.CDLL(path)
            for name, (args, res) in _SIGNATURES.items():
                fn = getattr(lib, name, None) if host_only else getattr(lib, name)
                if fn is None:
                    continue
                fn.argtypes = args
                fn.restype = res
            _lib = lib
        return _lib


class Error(RuntimeError):
    """A negative status from libpkv; ``code`` is the PKV_ERR_* value."""

    def __init__(self, code: int, message: str):
        super().__init__("%s (%d): %s" % (library().pkv_strerror(code).decode(), code, message))
        self.code = code
        self.message = message


ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_OUT_OF_BLOCKS = -3
ERR_NO_SUCH_SEQ = -4
ERR_SEQ_EXISTS = -5
ERR_WORKSPACE = -6
ERR_HIP = -7


def _check(code: int) -> None:
    if code != 0:
        raise Error(code, library().pkv_last_error().decode())


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ctypes objects passed through as they are (values, pointers, byref())
_CTYPES_ARGS = (ctypes._SimpleCData, ctypes._Pointer, type(ctypes.byref(ctypes.c_int32())))


class Prepared:
    """A call whose arguments were checked and marshalled once: calling it
    makes the same library call again (same buffers, same stream) at the
    cost of one foreign call. It keeps alive the objects its pointers point
    into. Kernel entry points return one when given ``prepare=True``; the
    allocator's ``*_into`` methods too."""

    __slots__ = ("_fn", "_args", "_keep", "_out")

    def __init__(self, fn, args, keep=(), out=None):
        self._fn = fn
        # plain Python values are converted to their ctypes argument types
        # now, so that a call converts nothing
        self._args = tuple(a if a is None or isinstance(a, _CTYPES_ARGS) else t(a)
                           for t, a in zip(fn.argtypes, args))
        self._keep = keep
        self._out = out

    def __call__(self):
        code = self._fn(*self._args)
        if code:
            _check(code)
        return None if self._out is None else self._out.value


def _run(fn, args, keep, prepare, out=None):
    if prepare:
        return Prepared(fn, args, keep, out)
    _check(fn(*args))
    return None if out is None else out.value


# --------------------------------------------------------------- allocator
def sha256(data: bytes) -> bytes:
    """SHA-256 of a byte string (the library's own implementation)."""
    buf = ctypes.create_string_buffer(bytes(data), max(1, len(data)))
    out = ctypes.create_string_buffer(32)
    _check(library().pkv_sha256(buf, len(data), out))
    return out.raw


def hash_block_tokens(parent: Optional[bytes], tokens, extra_key: int = 0) -> bytes:
    """Chained content hash of one full block of 16 token ids."""
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    if t.size != BLOCK_SIZE:
        raise Error(ERR_INVALID_ARG, "a block holds %d token ids" % BLOCK_SIZE)
    par = None if parent is None else ctypes.create_string_buffer(bytes(parent), 32)
    out = ctypes.create_string_buffer(32)
    _check(library().pkv_hash_block_tokens(par, _ptr(t), int(extra_key), out))
    return out.raw


class Allocator:
    """Host block allocator (C++): null block 0, LIFO reuse, tail-first
    release, refcounted sharing with copy-on-write, optional prefix caching
    (content-hashed blocks, FIFO for cached free blocks, lazy eviction)."""

    def __init__(self, num_blocks: int):
        self._lib = library()
        h = _c_p()
        _check(self._lib.pkv_allocator_create(int(num_blocks), ctypes.byref(h)))
        self._h = h
        self.num_blocks = int(num_blocks)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.pkv_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_free_order(self, order) -> None:
        o = np.ascontiguousarray(order, dtype=np.int32)
        _check(self._lib.pkv_allocator_set_free_order(self._h, _ptr(o), int(o.size)))

    def shuffle_free_list(self, seed: int) -> None:
        """Seeded random physical placement (see pkv_allocator_shuffle_free_list)."""
        _check(self._lib.pkv_allocator_shuffle_free_list(self._h, int(seed) & (2 ** 64 - 1)))

    def add(self, sid: int) -> None:
        _check(self._lib.pkv_seq_add(self._h, int(sid)))

    # ------------------------------------------------------- prefix caching
    def enable_prefix_caching(self, enabled: bool = True) -> None:
        _check(self._lib.pkv_allocator_enable_prefix_caching(self._h, 1 if enabled else 0))

    def add_cached(self, sid: int, tokens, extra_key: int = 0, max_cached: int = -1) -> int:
        """New sequence for a prompt; attaches its longest cached prefix of
        full blocks and returns the number of tokens attached."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        got = _c_i32(0)
        _check(self._lib.pkv_seq_add_cached(self._h, int(sid), _ptr(t) if t.size else None,
                                            int(t.size), int(extra_key), int(max_cached),
                                            ctypes.byref(got)))
        return int(got.value)

    def lookup_cached(self, tokens, extra_key: int = 0, max_cached: int = -1):
        """(tokens add_cached would attach, blocks it would take back out of
        the free queue); changes nothing."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        got, rev = _c_i32(0), _c_i32(0)
        _check(self._lib.pkv_prefix_lookup(self._h, _ptr(t) if t.size else None, int(t.size),
                                           int(extra_key), int(max_cached), ctypes.byref(got),
                                           ctypes.byref(rev)))
        return int(got.value), int(rev.value)

    def record_tokens(self, sid: int, tokens) -> None:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(self._lib.pkv_seq_record_tokens(self._h, int(sid), _ptr(t) if t.size else None,
                                               int(t.size)))

    def block_hash(self, block: int) -> Optional[bytes]:
        out = ctypes.create_string_buffer(32)
        has = _c_i32(0)
        _check(self._lib.pkv_block_hash(self._h, int(block), out, ctypes.byref(has)))
        return out.raw if has.value else None

    def prefix_cache_stats(self) -> dict:
        c, l, h = _c_i32(0), _c_i64(0), _c_i64(0)
        _check(self._lib.pkv_prefix_cache_stats(self._h, ctypes.byref(c), ctypes.byref(l),
                                                ctypes.byref(h)))
        return {"cached_blocks": c.value, "lookups": l.value, "hit_blocks": h.value}

    def append(self, sid: int, n: int, max_pairs: int = 1) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        return self.batch_append([sid], [n], max_pairs)

    def batch_append(self, sids: Sequence[int], ns: Sequence[int], max_pairs: Optional[int] = None
                     ) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        """Append ns[i] tokens to sids[i]; returns (int64 slots, copy pairs)."""
        s = np.ascontiguousarray(sids, dtype=np.int64)
        n = np.ascontiguousarray(ns, dtype=np.int32)
        slots = np.empty(int(n.sum()), dtype=np.int64)
        mp = len(s) if max_pairs is None else int(max_pairs)
        pairs = np.empty(max(1, 2 * mp), dtype=np.int64)
        npairs = _c_i32(0)
        _check(self._lib.pkv_batch_append(self._h, _ptr(s), _ptr(n), int(s.size), _ptr(slots),
                                          _ptr(pairs), mp, ctypes.byref(npairs)))
        k = npairs.value
        return slots, [(int(pairs[2 * i]), int(pairs[2 * i + 1])) for i in range(k)]

    def batch_append_into(self, sids: np.ndarray, ns: np.ndarray, slots_ptr: int,
                          pairs: np.ndarray, prepare: bool = False):
        """Like batch_append, writing slots to raw host memory at slots_ptr
        (e.g. a pinned tensor) and copy pairs to ``pairs`` (int64 [2*k]);
        returns the number of pairs. With prepare=True, returns a Prepared
        call (same arrays each time; it returns the number of pairs)."""
        npairs = _c_i32(0)
        return _run(self._lib.pkv_batch_append,
                    (self._h, _ptr(sids), _ptr(ns), int(sids.size), slots_ptr, _ptr(pairs),
                     int(pairs.size // 2), ctypes.byref(npairs)),
                    (self, sids, ns, pairs), prepare, npairs)

    def fork(self, parent: int, child: int) -> None:
        _check(self._lib.pkv_seq_fork(self._h, int(parent), int(child)))

    def free(self, sid: int) -> None:
        _check(self._lib.pkv_seq_free(self._h, int(sid)))

    def seq_len(self, sid: int) -> int:
        out = _c_i64(0)
        _check(self._lib.pkv_seq_len(self._h, int(sid), ctypes.byref(out)))
        return out.value

    def block_table(self, sids: Sequence[int], max_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
        s = np.ascontiguousarray(sids, dtype=np.int64)
        table = np.empty((s.size, int(max_blocks)), dtype=np.int32)
        lens = np.empty(s.size, dtype=np.int32)
        _check(self._lib.pkv_fill_block_table(self._h, _ptr(s), int(s.size), _ptr(table),
                                              int(max_blocks), _ptr(lens)))
        return table, lens

    def fill_block_table_into(self, sids: np.ndarray, table_ptr: int, max_blocks: int,
                              lens_ptr: int, prepare: bool = False):
        """Write the table and lengths to raw host memory (e.g. pinned
        tensors); prepare=True returns a Prepared call instead."""
        return _run(self._lib.pkv_fill_block_table,
                    (self._h, _ptr(sids), int(sids.size), table_ptr, int(max_blocks), lens_ptr),
                    (self, sids), prepare)

    def refcount(self, block: int) -> int:
        out = _c_i32(0)
        _check(self._lib.pkv_block_refcount(self._h, int(block), ctypes.byref(out)))
        return out.value

    def num_free(self) -> int:
        out = _c_i32(0)
        _check(self._lib.pkv_num_free_blocks(self._h, ctypes.byref(out)))
        return out.value

    def stats(self) -> Dict[str, float]:
        st = Stats()
        _check(self._lib.pkv_allocator_stats(self._h, ctypes.byref(st)))
        return {name: getattr(st, name) for name, _ in Stats._fields_}


class StepPlan(NamedTuple):
    """One planned step: per scheduled request (plan order) its id, first
    position computed, number of positions and whether a token is sampled;
    the slots of all planned positions in plan order; the ids preempted."""
    req_ids: np.ndarray
    start: np.ndarray
    num_new: np.ndarray
    samples: np.ndarray
    slots: np.ndarray
    preempted: np.ndarray


class Scheduler:
    """Step scheduler (C++) over an Allocator: one token budget per step,
    running requests first, chunked prefill, preemption by recompute, prefix
    cache lookups at admission when the allocator has caching on."""

    WAITING, RUNNING, FINISHED = 0, 1, 2

    def __init__(self, alloc: Allocator, token_budget: int, long_prefill_threshold: int = 0,
                 chunked_prefill: bool = True, max_num_seqs: int = 0):
        self._lib = library()
        self.alloc = alloc                  # kept alive as long as the scheduler
        h = _c_p()
        _check(self._lib.pkv_scheduler_create(alloc._h, int(token_budget), int(long_prefill_threshold),
                                              int(bool(chunked_prefill)), int(max_num_seqs),
                                              ctypes.byref(h)))
        self._h = h

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.pkv_scheduler_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_request(self, req_id: int, prompt, max_new_tokens: int, extra_key: int = 0) -> None:
        t = np.ascontiguousarray(prompt, dtype=np.int32)
        _check(self._lib.pkv_scheduler_add_request(self._h, int(req_id), _ptr(t) if t.size else None,
                                                   int(t.size), int(max_new_tokens), int(extra_key)))

    def schedule(self) -> StepPlan:
        ns, nt, npre = _c_i32(0), _c_i64(0), _c_i32(0)
        _check(self._lib.pkv_scheduler_schedule(self._h, ctypes.byref(ns), ctypes.byref(nt),
                                                ctypes.byref(npre)))
        n = ns.value
        ids = np.empty(n, dtype=np.int64)
        start = np.empty(n, dtype=np.int32)
        num = np.empty(n, dtype=np.int32)
        smp = np.empty(n, dtype=np.int32)
        slots = np.empty(nt.value, dtype=np.int64)
        pre = np.empty(npre.value, dtype=np.int64)
        _check(self._lib.pkv_scheduler_plan(self._h, _ptr(ids), _ptr(start), _ptr(num), _ptr(smp),
                                            _ptr(slots), _ptr(pre)))
        return StepPlan(ids, start, num, smp.astype(bool), slots, pre)

    def update(self, sampled) -> np.ndarray:
        """The step ran; sampled holds one token per sampling request in plan
        order. Returns the ids of the requests that finished."""
        t = np.ascontiguousarray(sampled, dtype=np.int32)
        nf = _c_i32(0)
        _check(self._lib.pkv_scheduler_update(self._h, _ptr(t) if t.size else None, int(t.size),
                                              ctypes.byref(nf)))
        out = np.empty(nf.value, dtype=np.int64)
        _check(self._lib.pkv_scheduler_finished(self._h, _ptr(out)))
        return out

    def remove_request(self, req_id: int) -> None:
        """Drop a request: dequeue it, abort it (blocks freed) or release a
        finished one's record."""
        _check(self._lib.pkv_scheduler_remove_request(self._h, int(req_id)))

    def counts(self) -> Tuple[int, int]:
        w, r = _c_i32(0), _c_i32(0)
        _check(self._lib.pkv_scheduler_counts(self._h, ctypes.byref(w), ctypes.byref(r)))
        return w.value, r.value

    def request(self, req_id: int) -> dict:
        st, nt, comp, pre = _c_i32(0), _c_i32(0), _c_i32(0), _c_i32(0)
        _check(self._lib.pkv_scheduler_request(self._h, int(req_id), ctypes.byref(st), ctypes.byref(nt),
                                               ctypes.byref(comp), ctypes.byref(pre), None, 0))
        toks = np.empty(nt.value, dtype=np.int32)
        _check(self._lib.pkv_scheduler_request(self._h, int(req_id), None, None, None, None,
                                               _ptr(toks), int(toks.size)))
        return {"state": st.value, "num_tokens": nt.value, "computed": comp.value,
                "preemptions": pre.value, "tokens": toks}


def blocks_for_bytes(nbytes: int, num_kv_heads: int, head_dim: int, dtype: int) -> int:
    out = _c_i32(0)
    _check(library().pkv_blocks_for_bytes(int(nbytes), int(num_kv_heads), int(head_dim), int(dtype),
                                          ctypes.byref(out)))
    return out.value


# ------------------------------------------------------------------ kernels
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise Error(ERR_UNSUPPORTED, "tensor dtype %s not supported" % t.dtype)


def _dev(t, name: str, dtype=None):
    if not t.is_cuda:
        raise Error(ERR_INVALID_ARG, "%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise Error(ERR_INVALID_ARG, "%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise Error(ERR_INVALID_ARG, "%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _idx(t, name: str, dtype):
    """An index argument (slot mapping, block table, lengths, cu_q_lens):
    a device tensor, or a pinned host tensor that the kernels read in place
    (pinned host memory is mapped into the device's address space)."""
    if not t.is_cuda and not t.is_pinned():
        raise Error(ERR_INVALID_ARG, "%s must be a device tensor or pinned host memory" % name)
    if not t.is_contiguous():
        raise Error(ERR_INVALID_ARG, "%s must be contiguous" % name)
    if t.dtype != dtype:
        raise Error(ERR_INVALID_ARG, "%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _stream(stream) -> int:
    """A HIP stream handle from None (torch's current stream), a torch
    stream, or a raw handle (int)."""
    if isinstance(stream, int):
        return stream
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _pool_shape(k_cache):
    if k_cache.dim() != 4 or k_cache.shape[2] != BLOCK_SIZE:
        raise Error(ERR_INVALID_ARG, "pool must be [num_blocks, num_kv_heads, 16, head_dim]")
    nb, hkv, _, d = k_cache.shape
    return int(nb), int(hkv), int(d)


def reshape_and_cache(k_cache, v_cache, k_new, v_new, slot_mapping, stream=None, prepare=False):
    """Scatter k_new/v_new [T, Hkv, D] into the pools at slot_mapping (int64 [T])."""
    torch = _torch()
    nb, hkv, d = _pool_shape(k_cache)
    if tuple(v_cache.shape) != tuple(k_cache.shape) or v_cache.dtype != k_cache.dtype:
        raise Error(ERR_INVALID_ARG, "k_cache and v_cache differ")
    if k_new.dim() != 3 or tuple(k_new.shape[1:]) != (hkv, d) or tuple(v_new.shape) != tuple(k_new.shape):
        raise Error(ERR_INVALID_ARG, "k_new/v_new must be [T, %d, %d]" % (hkv, d))
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise Error(ERR_INVALID_ARG, "dtype mismatch")
    t = int(k_new.shape[0])
    if slot_mapping.numel() != t:
        raise Error(ERR_INVALID_ARG, "slot_mapping must hold %d entries" % t)
    return _run(library().pkv_reshape_and_cache, (
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(k_new, "k_new"),
        _dev(v_new, "v_new"), hkv * d, _idx(slot_mapping, "slot_mapping", torch.int64), t, nb, hkv, d,
        _dtype_code(k_cache), _stream(stream)), (k_cache, v_cache, k_new, v_new, slot_mapping), prepare)


def set_debug_checks(enabled: bool) -> None:
    """Switch the library's debug checks (see pkv_set_debug_checks)."""
    _check(library().pkv_set_debug_checks(1 if enabled else 0))


def check_slot_mapping(slots, num_blocks: int) -> None:
    """Host check of a slot mapping (numpy int64): raises Error for a repeated
    non-negative slot, a slot in the null block or one outside the pool."""
    s = np.ascontiguousarray(slots, dtype=np.int64)
    _check(library().pkv_check_slot_mapping(_ptr(s) if s.size else None, int(s.size), int(num_blocks)))


def stage_copy(dst, src, stream=None, prepare=False):
    """Copy src (pinned host or device tensor) into the device tensor dst
    (same number of bytes) with a kernel on the stream."""
    if not dst.is_cuda or not dst.is_contiguous():
        raise Error(ERR_INVALID_ARG, "dst must be a contiguous device tensor")
    if not (src.is_cuda or src.is_pinned()) or not src.is_contiguous():
        raise Error(ERR_INVALID_ARG, "src must be a contiguous device or pinned host tensor")
    nbytes = dst.numel() * dst.element_size()
    if src.numel() * src.element_size() != nbytes:
        raise Error(ERR_INVALID_ARG, "dst and src sizes differ")
    return _run(library().pkv_stage_copy, (dst.data_ptr(), src.data_ptr(), nbytes, _stream(stream)),
                (dst, src), prepare)


def stream_read(src, out, workgroups: int, stream=None, prepare=False):
    """Plain streaming read of the device tensor src (a measurement aid):
    `workgroups` workgroups each read one contiguous slice and write one
    folded word to out (uint32 device tensor of at least `workgroups`
    words)."""
    if not src.is_cuda or not src.is_contiguous() or not out.is_cuda:
        raise Error(ERR_INVALID_ARG, "src and out must be contiguous device tensors")
    if out.numel() * out.element_size() < 4 * int(workgroups):
        raise Error(ERR_INVALID_ARG, "out holds fewer than %d words" % int(workgroups))
    nbytes = src.numel() * src.element_size()
    return _run(library().pkv_stream_read, (src.data_ptr(), nbytes, out.data_ptr(), int(workgroups),
                                            _stream(stream)), (src, out), prepare)


def copy_blocks(k_cache, v_cache, pairs, stream=None, prepare=False):
    """For each row (src, dst) of pairs (int64 [n, 2]), copy block src to dst."""
    torch = _torch()
    nb, hkv, d = _pool_shape(k_cache)
    n = int(pairs.numel() // 2)
    return _run(library().pkv_copy_blocks, (
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(pairs, "pairs", torch.int64), n, nb,
        hkv, d, _dtype_code(k_cache), _stream(stream)), (k_cache, v_cache, pairs), prepare)


def decode_set_waves_per_cu(per_cu: int) -> None:
    """Single-wave workgroups per CU of the split-KV decode (0 = default);
    size decode workspaces after changing it."""
    _check(library().pkv_decode_set_waves_per_cu(int(per_cu)))


def decode_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int) -> int:
    out = _c_sz(0)
    _check(library().pkv_decode_workspace_size(int(num_seqs), int(num_q_heads), int(num_kv_heads),
                                               int(head_dim), ctypes.byref(out)))
    return out.value


def decode_workspace(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                     device="cuda"):
    """A decode workspace (uint8 device tensor) of the size the library asks for."""
    torch = _torch()
    return torch.empty(decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim),
                       dtype=torch.uint8, device=device)


def decode(out, q, k_cache, v_cache, block_table, context_lens, scale: float, workspace,
           stream=None, phase: str = "both", prepare=False):
    """Paged decode attention; q/out [S, Hq, D], block_table int32 [S, maxB],
    context_lens int32 [S], workspace a uint8 device tensor of at least
    decode_workspace_size(...) bytes (``decode_workspace`` allocates one).
    ``phase`` "split" or "merge" launches one of the two kernels only (call
    both, in that order, for the full result)."""
    torch = _torch()
    nb, hkv, d = _pool_shape(k_cache)
    if q.dim() != 3 or q.shape[2] != d or tuple(out.shape) != tuple(q.shape):
        raise Error(ERR_INVALID_ARG, "q/out must be [S, Hq, %d]" % d)
    if q.dtype != k_cache.dtype or out.dtype != k_cache.dtype:
        raise Error(ERR_INVALID_ARG, "dtype mismatch")
    s, hq = int(q.shape[0]), int(q.shape[1])
    if block_table.dim() != 2 or block_table.shape[0] != s or context_lens.numel() != s:
        raise Error(ERR_INVALID_ARG, "block_table must be [S, maxB] and context_lens [S]")
    fn = {"both": library().pkv_paged_attention_decode,
          "split": library().pkv_paged_attention_decode_split,
          "merge": library().pkv_paged_attention_decode_merge}[phase]
    return _run(fn, (
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _idx(block_table, "block_table", torch.int32), _idx(context_lens, "context_lens", torch.int32),
        s, nb, int(block_table.shape[1]), hq, hkv, d, float(scale), _dtype_code(q),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)),
        (out, q, k_cache, v_cache, block_table, context_lens, workspace), prepare)


def decode_append(out, q, k_new, v_new, k_cache, v_cache, block_table, context_lens, scale: float,
                  workspace, stream=None, phase: str = "both", prepare=False):
    """A decode step with the current token's cache write folded in: k_new/v_new
    [S, Hkv, D] are written to position context_lens[s] - 1 of each sequence
    (through its block table), then the decode runs on the updated pools.
    ``phase`` "split" launches the split-KV kernel (with the write) only,
    "merge" the merge kernel only (call both, in that order)."""
    torch = _torch()
    nb, hkv, d = _pool_shape(k_cache)
    if tuple(v_cache.shape) != tuple(k_cache.shape) or v_cache.dtype != k_cache.dtype:
        raise Error(ERR_INVALID_ARG, "k_cache and v_cache differ")
    if q.dim() != 3 or q.shape[2] != d or tuple(out.shape) != tuple(q.shape):
        raise Error(ERR_INVALID_ARG, "q/out must be [S, Hq, %d]" % d)
    s, hq = int(q.shape[0]), int(q.shape[1])
    if tuple(k_new.shape) != (s, hkv, d) or tuple(v_new.shape) != (s, hkv, d):
        raise Error(ERR_INVALID_ARG, "k_new/v_new must be [%d, %d, %d]" % (s, hkv, d))
    if any(x.dtype != k_cache.dtype for x in (q, out, k_new, v_new)):
        raise Error(ERR_INVALID_ARG, "dtype mismatch")
    if block_table.dim() != 2 or block_table.shape[0] != s or context_lens.numel() != s:
        raise Error(ERR_INVALID_ARG, "block_table must be [S, maxB] and context_lens [S]")
    idx = (_idx(block_table, "block_table", torch.int32), _idx(context_lens, "context_lens", torch.int32))
    ws = (_dev(workspace, "workspace"), workspace.numel() * workspace.element_size())
    if phase == "merge":
        return _run(library().pkv_paged_attention_decode_merge, (
            _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
            *idx, s, nb, int(block_table.shape[1]), hq, hkv, d, float(scale), _dtype_code(q), *ws,
            _stream(stream)), (out, q, k_cache, v_cache, block_table, context_lens, workspace), prepare)
    fn = {"both": library().pkv_paged_attention_decode_append,
          "split": library().pkv_paged_attention_decode_append_split}[phase]
    return _run(fn, (
        _dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"), hkv * d,
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), *idx, s, nb, int(block_table.shape[1]),
        hq, hkv, d, float(scale), _dtype_code(q), *ws, _stream(stream)),
        (out, q, k_new, v_new, k_cache, v_cache, block_table, context_lens, workspace), prepare)


def decode_noalloc(out, q, k_cache, v_cache, block_table, context_lens, scale: float,
                   stream=None, prepare=False):
    """Paged decode attention without a workspace: the library's per-GPU
    scratch array (PKV_DECODE_SCRATCH_BYTES) holds the partial states. Calls
    that overlap on one GPU race."""
    torch = _torch()
    nb, hkv, d = _pool_shape(k_cache)
    if q.dim() != 3 or q.shape[2] != d or tuple(out.shape) != tuple(q.shape):
        raise Error(ERR_INVALID_ARG, "q/out must be [S, Hq, %d]" % d)
    if q.dtype != k_cache.dtype or out.dtype != k_cache.dtype:
        raise Error(ERR_INVALID_ARG, "dtype mismatch")
    s, hq = int(q.shape[0]), int(q.shape[1])
    if block_table.dim() != 2 or block_table.shape[0] != s or context_lens.numel() != s:
        raise Error(ERR_INVALID_ARG, "block_table must be [S, maxB] and context_lens [S]")
    return _run(library().pkv_paged_attention_decode_noalloc, (
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _idx(block_table, "block_table", torch.int32), _idx(context_lens, "context_lens", torch.int32),
        s, nb, int(block_table.shape[1]), hq, hkv, d, float(scale), _dtype_code(q), _stream(stream)),
        (out, q, k_cache, v_cache, block_table, context_lens), prepare)


def decode_shared_prefix_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                        head_dim: int, prefix_blocks: int) -> int:
    out = _c_sz(0)
    _check(library().pkv_decode_shared_prefix_workspace_size(
        int(num_seqs), int(num_q_heads), int(num_kv_heads), int(head_dim), int(prefix_blocks),
        ctypes.byref(out)))
    return out.value


def decode_shared_prefix(out, q, k_cache, v_cache, block_table, context_lens, prefix_blocks: int,
                         scale: float, workspace=None, stream=None) -> None:
    """Decode for a batch sharing its first prefix_blocks blocks (row 0 of
    block_table holds them): the prefix is attended once for all sequences,
    then each sequence's own blocks. workspace: uint8 device tensor of at
    least decode_shared_prefix_workspace_size(...) bytes (allocated here if
    None)."""
    torch = _torch()
    nb, hkv, d = _pool_shape(k_cache)
    if q.dim() != 3 or q.shape[2] != d or tuple(out.shape) != tuple(q.shape):
        raise Error(ERR_INVALID_ARG, "q/out must be [S, Hq, %d]" % d)
    if q.dtype != k_cache.dtype or out.dtype != k_cache.dtype:
        raise Error(ERR_INVALID_ARG, "dtype mismatch")
    s, hq = int(q.shape[0]), int(q.shape[1])
    if block_table.dim() != 2 or block_table.shape[0] != s or context_lens.numel() != s:
        raise Error(ERR_INVALID_ARG, "block_table must be [S, maxB] and context_lens [S]")
    if workspace is None:
        workspace = torch.empty(max(1, decode_shared_prefix_workspace_size(s, hq, hkv, d, prefix_blocks)),
                                dtype=torch.uint8, device=q.device)
    _check(library().pkv_paged_attention_decode_shared_prefix(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _idx(block_table, "block_table", torch.int32), _idx(context_lens, "context_lens", torch.int32),
        s, nb, int(block_table.shape[1]), int(prefix_blocks), hq, hkv, d, float(scale),
        _dtype_code(q), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def prefill_workspace_size(num_chunks: int, total_q: int, num_q_heads: int, num_kv_heads: int,
                           head_dim: int, max_q_len: int, max_context_len: int) -> int:
    out = _c_sz(0)
    _check(library().pkv_prefill_workspace_size(int(num_chunks), int(total_q), int(num_q_heads),
                                                int(num_kv_heads), int(head_dim), int(max_q_len),
                                                int(max_context_len), ctypes.byref(out)))
    return out.value


def prefill_workspace(num_chunks: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                      max_q_len: int, device="cuda"):
    """A prefill workspace (uint8 device tensor) of the size the library asks
    for, or None when these sizes use none."""
    torch = _torch()
    n = prefill_workspace_size(num_chunks, 0, num_q_heads, num_kv_heads, head_dim, max_q_len, 0)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def prefill_chunk(out, q, cu_q_lens, context_lens, block_table, k_cache, v_cache, max_q_len: int,
                  scale: float, workspace=None, stream=None) -> None:
    """Causal chunked-prefill attention; q/out [Tq, Hq, D], cu_q_lens int32
    [C+1], context_lens int32 [C] (including the chunk), block_table int32
    [C, maxB]. ``workspace`` (``prefill_workspace``): with it, a bf16 call
    with fewer row blocks than CUs splits their positions over more
    workgroups."""
    torch = _torch()
    nb, hkv, d = _pool_shape(k_cache)
    if q.dim() != 3 or q.shape[2] != d or tuple(out.shape) != tuple(q.shape):
        raise Error(ERR_INVALID_ARG, "q/out must be [Tq, Hq, %d]" % d)
    if q.dtype != k_cache.dtype or out.dtype != k_cache.dtype:
        raise Error(ERR_INVALID_ARG, "dtype mismatch")
    c = int(context_lens.numel())
    if cu_q_lens.numel() != c + 1 or block_table.dim() != 2 or block_table.shape[0] != c:
        raise Error(ERR_INVALID_ARG, "cu_q_lens [C+1], context_lens [C], block_table [C, maxB]")
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size())
    _check(library().pkv_paged_attention_prefill_chunk(
        _dev(out, "out"), _dev(q, "q"), _idx(cu_q_lens, "cu_q_lens", torch.int32),
        _idx(context_lens, "context_lens", torch.int32), _idx(block_table, "block_table", torch.int32),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), c, int(q.shape[0]), nb,
        int(block_table.shape[1]), int(max_q_len), int(q.shape[1]), hkv, d, float(scale),
        _dtype_code(q), ws_ptr, ws_bytes, _stream(stream)))
