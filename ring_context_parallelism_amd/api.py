"""Python binding of libcpattn.so with the C ABI's names.

Only argument marshalling happens here: torch tensors are checked for shape,
dtype, device and contiguity and passed as raw pointers with torch's current
HIP stream; every step of the computation runs in the library's kernels.
"""

import ctypes

import torch

from . import _native as N

_DTYPES = {torch.bfloat16: N.BF16, torch.float32: N.FP32}
_LAYOUTS = {"zigzag": N.ZIGZAG, "contiguous": N.CONTIGUOUS}


def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


class Plan:
    """``cp_attn_plan(seq_len, cp_size, heads, head_dim, causal, layout)`` and its calls."""

    def __init__(self, seq_len, cp_size, heads, head_dim, causal=True, layout="zigzag", dtype=torch.bfloat16):
        self._h = ctypes.c_void_p()
        self.lib = N.lib()
        N.check(self.lib.cp_attn_plan(int(seq_len), int(cp_size), int(heads), int(head_dim), int(bool(causal)),
                                      _LAYOUTS[layout], ctypes.byref(self._h)), "cp_attn_plan")
        self.seq_len, self.cp_size, self.heads, self.head_dim = int(seq_len), int(cp_size), int(heads), int(head_dim)
        self.causal, self.layout = bool(causal), layout
        self.dtype = dtype
        self._workspace = None
        self.documents = None
        N.check(self.lib.cp_attn_set_dtype(self._h, _DTYPES[dtype]), "cp_attn_set_dtype")

    # -- lifetime -------------------------------------------------------
    def close(self):
        if self._h is not None and self._h.value:
            N.check(self.lib.cp_attn_plan_destroy(self._h), "cp_attn_plan_destroy")
        self._h = None
        self._workspace = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -- options --------------------------------------------------------
    def set_option(self, option, value):
        N.check(self.lib.cp_attn_set_option(self._h, int(option), int(value)), "cp_attn_set_option")

    def set_merge(self, separate):
        self.set_option(N.OPT_MERGE, 1 if separate else 0)

    def set_serialize(self, on):
        self.set_option(N.OPT_SERIALIZE, int(bool(on)))

    def set_recv(self, mode):
        self.set_option(N.OPT_RECV, {"kernel": 0, "memcpy": 1, "fused": 2, "hybrid": 3}[mode])

    def set_recv_blocks(self, n):
        self.set_option(N.OPT_RECV_BLOCKS, int(n))

    def set_graph(self, on):
        self.set_option(N.OPT_GRAPH, int(bool(on)))

    def set_key_split(self, on):
        self.set_option(N.OPT_KSPLIT, int(bool(on)))

    def set_backward_key_kernel(self, kind):
        """dK/dV kernel of the bf16, head_dim-128 backward: "eight" (default,
        two waves per 32-key column) or "four" (one wave per column)."""
        self.set_option(N.OPT_BWD_KEYS, {"eight": 0, "four": 1}[kind])

    def set_lockstep(self, on):
        """full_forward: every rank's ring step in one launch (on) or the ranks
        one after another (off, the default)."""
        self.set_option(N.OPT_LOCKSTEP, int(bool(on)))

    def set_fused_ring(self, mode):
        """Every ring step of a rank in one launch where served: True / 1 (the
        default), False / 0 (one launch per step), "timeout_test" (2: every
        receive wait gives up at once; results not valid) or "staged" (3: the
        launch waits for every receive first; for tools that run one kernel
        at a time)."""
        value = {"timeout_test": 2, "staged": 3}.get(mode) if isinstance(mode, str) else int(bool(mode))
        if value is None:
            raise ValueError(f"fused ring mode must be a bool, 'timeout_test' or 'staged', not {mode!r}")
        self.set_option(N.OPT_FUSED_RING, value)

    def set_backward_fused(self, mode):
        """Backward schedule: 0 dK/dV and dQ per ring step; 1 (default) dQ of
        every step in one launch; 2 dK/dV in one launch too (the all-gather
        form).  Served for bf16 head_dim 128 without documents or padding;
        elsewhere mode 0."""
        self.set_option(N.OPT_BWD_FUSED, int(mode))

    def fused_ring_active(self):
        """1 if the last forward call ran each rank as one fused launch, 2 if
        the last rank it computed also split its row tiles' keys in that
        launch, 0 otherwise."""
        t = ctypes.c_int32()
        N.check(self.lib.cp_attn_fused_ring_active(self._h, ctypes.byref(t)), "cp_attn_fused_ring_active")
        return int(t.value)

    def ring_wait_timeouts(self):
        """True if a fused-ring receive wait ran out since the last query
        (cleared); query after synchronizing the stream of the calls."""
        t = ctypes.c_int32()
        N.check(self.lib.cp_attn_ring_wait_timeouts(self._h, ctypes.byref(t)), "cp_attn_ring_wait_timeouts")
        return bool(t.value)

    def set_poison(self, on):
        self.set_option(N.OPT_POISON, int(bool(on)))

    def set_step_timing(self, on):
        self.set_option(N.OPT_STEP_TIMING, int(bool(on)))

    def workspace_bytes(self):
        n = ctypes.c_int64()
        N.check(self.lib.cp_attn_workspace_bytes(self._h, ctypes.byref(n)), "cp_attn_workspace_bytes")
        return n.value

    def set_workspace(self, tensor):
        """Caller-owned workspace (a uint8 CUDA tensor of >= workspace_bytes()); None to release."""
        if tensor is None:
            N.check(self.lib.cp_attn_set_workspace(self._h, None, 0), "cp_attn_set_workspace")
        else:
            N.check(self.lib.cp_attn_set_workspace(self._h, _ptr(tensor), tensor.numel() * tensor.element_size()),
                    "cp_attn_set_workspace")
        self._workspace = tensor

    def set_streams(self, copy_stream, merge_stream):
        c = ctypes.c_void_p(copy_stream.cuda_stream) if copy_stream is not None else None
        m = ctypes.c_void_p(merge_stream.cuda_stream) if merge_stream is not None else None
        N.check(self.lib.cp_attn_set_streams(self._h, c, m), "cp_attn_set_streams")
        self._streams = (copy_stream, merge_stream)

    def set_documents(self, starts):
        """Document masks: document d holds positions [starts[d], starts[d+1]) (the
        last runs to seq_len); starts increases strictly from 0.  None or [] clears."""
        starts = [] if starts is None else [int(x) for x in starts]
        arr = (ctypes.c_int64 * max(1, len(starts)))(*starts)
        N.check(self.lib.cp_attn_set_documents(self._h, arr, len(starts)), "cp_attn_set_documents")
        self.documents = tuple(starts) if starts else None

    # -- forward --------------------------------------------------------
    def _check_io(self, q, k, v, out, lse):
        shape = (self.seq_len, self.heads, self.head_dim)
        for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
            if tuple(t.shape) != shape or t.dtype != self.dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {self.dtype} CUDA tensor of shape {shape}")
        if tuple(lse.shape) != (self.heads, self.seq_len) or lse.dtype != torch.float32 or not lse.is_cuda \
                or not lse.is_contiguous():
            raise ValueError(f"lse must be a contiguous float32 CUDA tensor of shape {(self.heads, self.seq_len)}")

    def rank_forward(self, q, k, v, out, lse, rank, stream=None):
        self._check_io(q, k, v, out, lse)
        N.check(self.lib.cp_attn_rank_forward(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(rank),
                                              _stream_ptr(stream)), "cp_attn_rank_forward")

    def rank_forward_noalloc(self, q, k, v, out, lse, rank, stream=None):
        """rank_forward on the library's static device scratch: no allocation,
        every kernel on ``stream`` (graph-capturable).  Calls on one GPU share
        the scratch, so calls in flight at the same time race."""
        self._check_io(q, k, v, out, lse)
        N.check(self.lib.cp_attn_rank_forward_noalloc(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                                      int(rank), _stream_ptr(stream)), "cp_attn_rank_forward_noalloc")

    def allgather_forward(self, q, k, v, out, lse, rank, stream=None):
        self._check_io(q, k, v, out, lse)
        N.check(self.lib.cp_attn_allgather_forward(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), int(rank),
                                                   _stream_ptr(stream)), "cp_attn_allgather_forward")

    def full_forward(self, q, k, v, out, lse, stream=None):
        self._check_io(q, k, v, out, lse)
        N.check(self.lib.cp_attn_full_forward(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                              _stream_ptr(stream)), "cp_attn_full_forward")

    # -- Ulysses ----------------------------------------------------------
    def heads_per_rank(self):
        return self.heads // self.cp_size

    def ulysses_a2a(self, src, dst, to_heads, stream=None):
        """sequence layout ``[cp * local_rows, H, D]`` <-> head layout ``[cp, S, H/cp, D]``."""
        seq_n = self.cp_size * self.local_rows() * self.heads * self.head_dim
        head_n = self.seq_len * self.heads * self.head_dim
        want = {"src": head_n if not to_heads else seq_n, "dst": head_n if to_heads else seq_n}
        for name, t in (("src", src), ("dst", dst)):
            if t.numel() != want[name] or t.dtype != self.dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {self.dtype} CUDA tensor with {want[name]} elements")
        N.check(self.lib.cp_attn_ulysses_a2a(self._h, _ptr(src), _ptr(dst), int(bool(to_heads)), _stream_ptr(stream)),
                "cp_attn_ulysses_a2a")

    def ulysses_forward(self, q, k, v, out, lse, stream=None):
        """One rank's head slice: q, k, v, out ``[S, H/cp, D]``, lse ``[H/cp, S]``."""
        g = self.heads // self.cp_size
        shape = (self.seq_len, g, self.head_dim)
        for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
            if tuple(t.shape) != shape or t.dtype != self.dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {self.dtype} CUDA tensor of shape {shape}")
        if tuple(lse.shape) != (g, self.seq_len) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError(f"lse must be a contiguous float32 CUDA tensor of shape {(g, self.seq_len)}")
        N.check(self.lib.cp_attn_ulysses_forward(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                                 _stream_ptr(stream)), "cp_attn_ulysses_forward")

    # -- backward -------------------------------------------------------
    def _check_bwd(self, dout, dq, dk, dv):
        shape = (self.seq_len, self.heads, self.head_dim)
        if tuple(dout.shape) != shape or dout.dtype != self.dtype or not dout.is_cuda or not dout.is_contiguous():
            raise ValueError(f"dout must be a contiguous {self.dtype} CUDA tensor of shape {shape}")
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            if tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of shape {shape}")

    def rank_backward(self, q, k, v, out, lse, dout, dq, dk, dv, rank, stream=None):
        """dq at the rank's rows; the rank's terms ADDED to dk, dv."""
        self._check_io(q, k, v, out, lse)
        self._check_bwd(dout, dq, dk, dv)
        N.check(self.lib.cp_attn_rank_backward(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                                               _ptr(dq), _ptr(dk), _ptr(dv), int(rank), _stream_ptr(stream)),
                "cp_attn_rank_backward")

    def full_backward(self, q, k, v, out, lse, dout, dq, dk, dv, stream=None):
        self._check_io(q, k, v, out, lse)
        self._check_bwd(dout, dq, dk, dv)
        N.check(self.lib.cp_attn_full_backward(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                                               _ptr(dq), _ptr(dk), _ptr(dv), _stream_ptr(stream)),
                "cp_attn_full_backward")

    # -- host-only introspection -----------------------------------------
    def local_rows(self):
        n = ctypes.c_int64()
        N.check(self.lib.cp_attn_local_rows(self._h, ctypes.byref(n)), "cp_attn_local_rows")
        return n.value

    def rank_valid_rows(self, rank):
        n = ctypes.c_int64()
        N.check(self.lib.cp_attn_rank_valid_rows(self._h, int(rank), ctypes.byref(n)), "cp_attn_rank_valid_rows")
        return n.value

    def rank_chunks(self, rank):
        ch = (ctypes.c_int32 * 2)()
        cnt = ctypes.c_int32()
        N.check(self.lib.cp_attn_rank_chunks(self._h, int(rank), ch, ctypes.byref(cnt)), "cp_attn_rank_chunks")
        return tuple(ch[i] for i in range(cnt.value))

    def step_source(self, rank, step):
        j = ctypes.c_int32()
        N.check(self.lib.cp_attn_step_source(self._h, int(rank), int(step), ctypes.byref(j)), "cp_attn_step_source")
        return j.value

    def step_segments(self, rank, step):
        buf = (ctypes.c_int64 * 14)()
        cnt = ctypes.c_int32()
        N.check(self.lib.cp_attn_step_segments(self._h, int(rank), int(step), buf, ctypes.byref(cnt)),
                "cp_attn_step_segments")
        keys = ("q_start", "q_len", "kv_full", "diag", "first", "last", "q_global")
        return [dict(zip(keys, (buf[7 * i + j] for j in range(7)))) for i in range(cnt.value)]

    def valid_work(self, rank, step, bm, bn):
        t = ctypes.c_int64()
        p = ctypes.c_int64()
        N.check(self.lib.cp_attn_valid_work(self._h, int(rank), int(step), int(bm), int(bn), ctypes.byref(t),
                                            ctypes.byref(p)), "cp_attn_valid_work")
        return t.value, p.value

    # -- layout -----------------------------------------------------------
    def layout_gather(self, src, dst, stream=None):
        """natural order ``[S, H, D]`` -> local order ``[cp * local_rows, H, D]`` (pad rows zero)."""
        self._check_layout(natural=src, local=dst)
        N.check(self.lib.cp_attn_layout_gather(self._h, _ptr(src), _ptr(dst), _stream_ptr(stream)),
                "cp_attn_layout_gather")

    def layout_scatter(self, src, dst, stream=None):
        """local order ``[cp * local_rows, H, D]`` -> natural order ``[S, H, D]``."""
        self._check_layout(natural=dst, local=src)
        N.check(self.lib.cp_attn_layout_scatter(self._h, _ptr(src), _ptr(dst), _stream_ptr(stream)),
                "cp_attn_layout_scatter")

    def _check_layout(self, natural, local):
        row = self.heads * self.head_dim
        for name, t, rows in (("natural", natural, self.seq_len), ("local", local, self.cp_size * self.local_rows())):
            n = rows * row
            if t.numel() != n or t.dtype != self.dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name}-order tensor must be a contiguous {self.dtype} CUDA tensor with {n} elements")

    def last_step_times(self):
        n = self.cp_size * self.cp_size
        buf = (ctypes.c_float * n)()
        N.check(self.lib.cp_attn_last_step_times(self._h, buf, n), "cp_attn_last_step_times")
        return [[buf[r * self.cp_size + s] for s in range(self.cp_size)] for r in range(self.cp_size)]

    def set_counters(self, on):
        self.set_option(N.OPT_COUNTERS, int(bool(on)))

    def last_tile_counts(self):
        """([cp][cp] key tiles computed per (rank, step) by the last call, -1 where not run),
        (tile rows, tile keys))."""
        n = self.cp_size * self.cp_size
        buf = (ctypes.c_int64 * n)()
        tr, tk = ctypes.c_int32(), ctypes.c_int32()
        N.check(self.lib.cp_attn_last_tile_counts(self._h, buf, n, ctypes.byref(tr), ctypes.byref(tk)),
                "cp_attn_last_tile_counts")
        return [[buf[r * self.cp_size + s] for s in range(self.cp_size)] for r in range(self.cp_size)], (tr.value, tk.value)


def lse_merge(o_acc, lse_acc, o_s, lse_s, stream=None):
    """In-place exact LSE merge: o_* ``[rows, H, D]`` fp32, lse_* ``[H, rows]`` fp32."""
    rows, heads, dim = o_acc.shape
    for name, t, shp in (("o_acc", o_acc, (rows, heads, dim)), ("o_s", o_s, (rows, heads, dim)),
                         ("lse_acc", lse_acc, (heads, rows)), ("lse_s", lse_s, (heads, rows))):
        if tuple(t.shape) != shp or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of shape {shp}")
    lib = N.lib()
    N.check(lib.cp_attn_lse_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_s), _ptr(lse_s), int(rows), int(heads),
                                  int(dim), _stream_ptr(stream)), "cp_attn_lse_merge")
