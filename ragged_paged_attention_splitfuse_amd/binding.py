"""ctypes binding of libfg.so (include/fg.h), same entry-point names.

Argument marshalling only: every step of a pass runs in the library's HIP
kernels.  Tensors are torch tensors (device memory and streams come from
PyTorch) or raw integer device addresses.  Shapes, dtypes, devices and
contiguity of torch arguments are checked here against the plan before any
launch, because the C ABI receives bare pointers and cannot check sizes.

There is no fallback: if libfg.so is missing or cannot be loaded, every call
raises ``FgError``.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FG_LIBRARY", os.path.join(_HERE, "libfg.so"))

FG_OK = 0
FG_E_INVALID, FG_E_RANGE, FG_E_ALIAS, FG_E_UNSUPPORTED = -1, -2, -3, -4
FG_E_WORKSPACE, FG_E_HIP, FG_E_NOMEM = -5, -6, -7
FG_DTYPE_F32, FG_DTYPE_BF16 = 0, 1
FG_SPLIT_BALANCED, FG_SPLIT_ENGINE, FG_SPLIT_PER_1K = 0, 1, 2
FG_KERNEL_APPEND, FG_KERNEL_ATTENTION, FG_KERNEL_MERGE, FG_KERNEL_COUNT = 0, 1, 2, 3

_I32P = ctypes.POINTER(ctypes.c_int32)


class FgError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status) if _lib else status} ({status})")


class fg_pass_desc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("scale", ctypes.c_float),
        # const int32_t* in the header; set from array addresses (plain ints)
        ("q_lens", ctypes.c_void_p), ("ctx_lens", ctypes.c_void_p), ("block_tables", ctypes.c_void_p),
        ("target_cus", ctypes.c_int32), ("min_split_tokens", ctypes.c_int32),
        ("max_splits", ctypes.c_int32), ("force_splits", ctypes.c_int32),
        ("split_policy", ctypes.c_int32),
    ]


class fg_plan_info_t(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int64), ("metadata_bytes", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64), ("num_items", ctypes.c_int32),
        ("num_valu_items", ctypes.c_int32), ("num_mfma_items", ctypes.c_int32),
        ("num_merge_groups", ctypes.c_int32), ("num_partial_rows", ctypes.c_int32),
        ("max_splits_used", ctypes.c_int32), ("num_append_runs", ctypes.c_int32),
        ("target_cus", ctypes.c_int32), ("num_inlaunch_merge_groups", ctypes.c_int32),
    ]


class fg_plan_layout_t(ctypes.Structure):
    _fields_ = [
        ("seqs", ctypes.c_int64), ("block_ids", ctypes.c_int64), ("runs", ctypes.c_int64),
        ("items", ctypes.c_int64), ("merges", ctypes.c_int64), ("counters", ctypes.c_int64),
        ("num_seqs", ctypes.c_int32), ("num_block_ids", ctypes.c_int32),
        ("num_runs", ctypes.c_int32), ("num_items", ctypes.c_int32),
        ("num_merges", ctypes.c_int32), ("num_counters", ctypes.c_int32),
    ]


_lib = None

# name -> (restype, argtypes); the list mirrors include/fg.h
SIGNATURES = {
    "fg_plan_pass": (ctypes.c_int32, [ctypes.POINTER(fg_pass_desc), ctypes.POINTER(ctypes.c_void_p)]),
    "fg_plan_info": (ctypes.c_int32, [ctypes.c_void_p, ctypes.POINTER(fg_plan_info_t)]),
    "fg_plan_upload": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "fg_kv_append": (ctypes.c_int32, [ctypes.c_void_p] * 7),
    "fg_upload_append": (ctypes.c_int32, [ctypes.c_void_p] * 7),
    "fg_attention_ragged": (ctypes.c_int32, [ctypes.c_void_p] * 6 + [ctypes.c_int32, ctypes.c_void_p,
                                                                     ctypes.c_void_p, ctypes.c_size_t,
                                                                     ctypes.c_void_p]),
    "fg_attention_ragged_direct": (ctypes.c_int32, [ctypes.c_void_p] * 8 + [ctypes.c_int32, ctypes.c_void_p,
                                                                            ctypes.c_void_p, ctypes.c_size_t,
                                                                            ctypes.c_void_p]),
    "fg_pass": (ctypes.c_int32, [ctypes.c_void_p] * 8 + [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                                         ctypes.c_size_t, ctypes.c_void_p]),
    "fg_attention_ragged_noalloc": (ctypes.c_int32, [ctypes.c_void_p] * 6 + [ctypes.c_int32, ctypes.c_void_p,
                                                                             ctypes.c_void_p]),
    "fg_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "fg_plan_destroy": (None, [ctypes.c_void_p]),
    "fg_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "fg_abi_version": (ctypes.c_int32, []),
    "fg_plan_metadata": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.POINTER(fg_plan_layout_t)]),
    "fg_plan_resident_slots": (ctypes.c_int32, [ctypes.c_void_p, _I32P, _I32P]),
    "fg_profile_enable": (ctypes.c_int32, [ctypes.c_int32]),
    "fg_profile_read": (ctypes.c_int32, [ctypes.POINTER(ctypes.c_double), _I32P, ctypes.c_int32]),
    "fg_kernel_name": (ctypes.c_char_p, [ctypes.c_int32]),
    "fg_probe_read_stream": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                              ctypes.c_size_t, ctypes.c_void_p]),
    "fg_probe_mfma_loop": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
}


def lib():
    """Load libfg.so once; raise if it is missing (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FgError(FG_E_UNSUPPORTED, f"libfg.so not built (expected at {LIB_PATH}); "
                          "run __graft_entry__.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status):
    return lib().fg_status_string(int(status)).decode()


def fg_abi_version():
    return int(lib().fg_abi_version())


def _check(status, what):
    if status != FG_OK:
        raise FgError(status, what)


def _ptr(x):
    """Device address of a torch tensor (or an int address / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


class Plan:
    """Owner of one fg_plan; see fg_plan_pass in include/fg.h."""

    def __init__(self, q_lens, ctx_lens, block_tables, num_q_heads, num_kv_heads, head_dim,
                 block_size, num_blocks, scale=0.0, target_cus=0, min_split_tokens=0,
                 max_splits=0, force_splits=0, split_policy=0):
        self._h = None
        q = np.ascontiguousarray(q_lens, dtype=np.int32)
        c = np.ascontiguousarray(ctx_lens, dtype=np.int32)
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        if bt.ndim == 1:
            bt = bt.reshape(len(q), -1) if len(q) else bt.reshape(0, 0)
        if len(q) != len(c) or bt.shape[0] != len(q):
            raise ValueError("q_lens, ctx_lens and block_tables disagree on the sequence count")
        self.q_lens, self.ctx_lens, self.block_tables = q, c, bt
        d = fg_pass_desc()
        d.num_seqs = len(q)
        d.num_q_heads, d.num_kv_heads, d.head_dim = num_q_heads, num_kv_heads, head_dim
        d.block_size, d.num_blocks = block_size, num_blocks
        d.max_blocks_per_seq = bt.shape[1] if bt.ndim == 2 else 0
        d.scale = float(scale)
        d.q_lens = q.__array_interface__["data"][0]
        d.ctx_lens = c.__array_interface__["data"][0]
        d.block_tables = bt.__array_interface__["data"][0]
        d.target_cus, d.min_split_tokens = target_cus, min_split_tokens
        d.max_splits, d.force_splits = max_splits, force_splits
        d.split_policy = split_policy
        h = ctypes.c_void_p()
        _check(lib().fg_plan_pass(ctypes.byref(d), ctypes.byref(h)), "fg_plan_pass")
        self._h = h
        self.num_q_heads, self.num_kv_heads = num_q_heads, num_kv_heads
        self.head_dim, self.block_size, self.num_blocks = head_dim, block_size, num_blocks
        self.info = self._info()
        self.num_tokens = self.info["num_tokens"]
        self.meta = None

    @classmethod
    def from_spec(cls, spec, **knobs):
        return cls(spec.q_lens, spec.ctx_lens, spec.block_tables, spec.num_q_heads,
                   spec.num_kv_heads, spec.head_dim, spec.block_size, spec.num_blocks,
                   scale=spec.scale, **knobs)

    def _info(self):
        o = fg_plan_info_t()
        _check(lib().fg_plan_info(self._h, ctypes.byref(o)), "fg_plan_info")
        return {name: int(getattr(o, name)) for name, _ in o._fields_}

    @property
    def handle(self):
        if self._h is None:
            raise FgError(FG_E_INVALID, "plan already destroyed")
        return self._h

    def metadata(self):
        """Host copy of the packed metadata, parsed into int32 record arrays."""
        nbytes = self.info["metadata_bytes"]
        buf = np.zeros(max(16, nbytes), dtype=np.uint8)
        lay = fg_plan_layout_t()
        _check(lib().fg_plan_metadata(self.handle, buf.ctypes.data, buf.nbytes, ctypes.byref(lay)),
               "fg_plan_metadata")
        words = buf.view(np.int32)

        def section(off, count, width):
            start = off // 4
            return words[start:start + count * width].reshape(count, width).copy()

        return {
            "seqs": section(lay.seqs, lay.num_seqs, 8),
            "block_ids": words[lay.block_ids // 4: lay.block_ids // 4 + lay.num_block_ids].copy(),
            "runs": section(lay.runs, lay.num_runs, 4),
            "items": section(lay.items, lay.num_items, 12),
            "merges": section(lay.merges, lay.num_merges, 8),
            "counters": words[lay.counters // 4: lay.counters // 4 + lay.num_counters].copy(),
            "raw": buf[:nbytes].copy(),
        }

    def resident_slots(self):
        """(planned, device): work-groups per CU the planner assumed, and what the
        occupancy calculator gives for this plan's attention kernels (-1 without a GPU)."""
        planned, device = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().fg_plan_resident_slots(self.handle, ctypes.byref(planned), ctypes.byref(device)),
               "fg_plan_resident_slots")
        return planned.value, device.value

    def upload(self, d_meta=None, stream=None, device="cuda"):
        """fg_plan_upload into d_meta (allocated here as a torch uint8 tensor if None)."""
        if d_meta is None:
            import torch
            d_meta = torch.empty(max(16, self.info["metadata_bytes"]), dtype=torch.uint8, device=device)
        elif hasattr(d_meta, "numel") and d_meta.numel() * d_meta.element_size() < self.info["metadata_bytes"]:
            raise ValueError("metadata buffer too small")
        _check(lib().fg_plan_upload(self.handle, _ptr(d_meta), _stream(stream)), "fg_plan_upload")
        self.meta = d_meta
        return d_meta

    def close(self):
        if self._h is not None and _lib is not None:
            _lib.fg_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def plan_pass(*args, **kwargs):
    return Plan(*args, **kwargs)


def _check_tensor(t, shape, dtype_name, what):
    if t is None or isinstance(t, int):
        return
    import torch
    want = {"bf16": (torch.bfloat16, torch.int16, torch.uint16), "f32": (torch.float32,)}[dtype_name]
    if t.dtype not in want:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype_name}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous() or t.device.type != "cuda":
        raise ValueError(f"{what}: must be a contiguous device tensor")


def pool_shapes(num_blocks, num_kv_heads, block_size, head_dim):
    """(K pool shape, V pool shape) of the layouts in include/fg.h: V blocks
    are stored transposed in sub-blocks of min(block_size, 32) slots."""
    sub = min(block_size, 32)
    return ((num_blocks, num_kv_heads, block_size, head_dim),
            (num_blocks, num_kv_heads, block_size // sub, head_dim, sub))


def fg_kv_append(plan, d_meta, k_new, v_new, k_pool, v_pool, stream=None):
    t, hkv, d = plan.num_tokens, plan.num_kv_heads, plan.head_dim
    kshape, vshape = pool_shapes(plan.num_blocks, hkv, plan.block_size, d)
    _check_tensor(k_new, (t, hkv, d), "bf16", "k_new")
    _check_tensor(v_new, (t, hkv, d), "bf16", "v_new")
    _check_tensor(k_pool, kshape, "bf16", "k_pool")
    _check_tensor(v_pool, vshape, "bf16", "v_pool")
    _check(lib().fg_kv_append(plan.handle, _ptr(d_meta if d_meta is not None else plan.meta),
                              _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                              _stream(stream)), "fg_kv_append")


def fg_upload_append(plan, d_meta, k_new, v_new, k_pool, v_pool, stream=None, device="cuda"):
    """fg_upload_append: plan upload and KV append in one launch.  d_meta is
    allocated here (torch uint8) when None; returns it."""
    t, hkv, d = plan.num_tokens, plan.num_kv_heads, plan.head_dim
    kshape, vshape = pool_shapes(plan.num_blocks, hkv, plan.block_size, d)
    if d_meta is None:
        import torch
        d_meta = torch.empty(max(16, plan.info["metadata_bytes"]), dtype=torch.uint8, device=device)
    elif hasattr(d_meta, "numel") and d_meta.numel() * d_meta.element_size() < plan.info["metadata_bytes"]:
        raise ValueError("metadata buffer too small")
    _check_tensor(k_new, (t, hkv, d), "bf16", "k_new")
    _check_tensor(v_new, (t, hkv, d), "bf16", "v_new")
    _check_tensor(k_pool, kshape, "bf16", "k_pool")
    _check_tensor(v_pool, vshape, "bf16", "v_pool")
    _check(lib().fg_upload_append(plan.handle, _ptr(d_meta), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                                  _ptr(v_pool), _stream(stream)), "fg_upload_append")
    plan.meta = d_meta
    return d_meta


def fg_attention_ragged(plan, d_meta, q, k_pool, v_pool, out, lse=None, workspace=None,
                        stream=None, out_dtype=None):
    t, hq, hkv, d = plan.num_tokens, plan.num_q_heads, plan.num_kv_heads, plan.head_dim
    kshape, vshape = pool_shapes(plan.num_blocks, hkv, plan.block_size, d)
    if out_dtype is None:
        import torch
        out_dtype = FG_DTYPE_BF16 if (hasattr(out, "dtype") and out.dtype == torch.bfloat16) else FG_DTYPE_F32
    _check_tensor(q, (t, hq, d), "bf16", "q")
    _check_tensor(k_pool, kshape, "bf16", "k_pool")
    _check_tensor(v_pool, vshape, "bf16", "v_pool")
    _check_tensor(out, (t, hq, d), "bf16" if out_dtype == FG_DTYPE_BF16 else "f32", "out")
    _check_tensor(lse, (t, hq), "f32", "lse")
    ws_bytes = plan.info["workspace_bytes"]
    if workspace is None and ws_bytes > 0:
        import torch
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    have = 0
    if workspace is not None:
        have = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else ws_bytes
    _check(lib().fg_attention_ragged(plan.handle, _ptr(d_meta if d_meta is not None else plan.meta),
                                     _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), int(out_dtype),
                                     _ptr(lse), _ptr(workspace), int(have), _stream(stream)),
           "fg_attention_ragged")
    return workspace


def _check_pass_tensors(plan, q, k_new, v_new, k_pool, v_pool, out, lse, out_dtype):
    t, hq, hkv, d = plan.num_tokens, plan.num_q_heads, plan.num_kv_heads, plan.head_dim
    kshape, vshape = pool_shapes(plan.num_blocks, hkv, plan.block_size, d)
    _check_tensor(q, (t, hq, d), "bf16", "q")
    _check_tensor(k_new, (t, hkv, d), "bf16", "k_new")
    _check_tensor(v_new, (t, hkv, d), "bf16", "v_new")
    _check_tensor(k_pool, kshape, "bf16", "k_pool")
    _check_tensor(v_pool, vshape, "bf16", "v_pool")
    _check_tensor(out, (t, hq, d), "bf16" if out_dtype == FG_DTYPE_BF16 else "f32", "out")
    _check_tensor(lse, (t, hq), "f32", "lse")


def _out_dtype(out, out_dtype):
    if out_dtype is None:
        import torch
        out_dtype = FG_DTYPE_BF16 if (hasattr(out, "dtype") and out.dtype == torch.bfloat16) else FG_DTYPE_F32
    return out_dtype


def _workspace(plan, workspace, device="cuda"):
    ws_bytes = plan.info["workspace_bytes"]
    if workspace is None and ws_bytes > 0:
        import torch
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
    have = 0
    if workspace is not None:
        have = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else ws_bytes
    return workspace, have


def fg_attention_ragged_direct(plan, d_meta, q, k_new, v_new, k_pool, v_pool, out, lse=None,
                               workspace=None, stream=None, out_dtype=None):
    """Attention with this pass's own K/V read from k_new / v_new (no append)."""
    out_dtype = _out_dtype(out, out_dtype)
    _check_pass_tensors(plan, q, k_new, v_new, k_pool, v_pool, out, lse, out_dtype)
    workspace, have = _workspace(plan, workspace)
    _check(lib().fg_attention_ragged_direct(plan.handle, _ptr(d_meta if d_meta is not None else plan.meta),
                                            _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                                            _ptr(out), int(out_dtype), _ptr(lse), _ptr(workspace), int(have),
                                            _stream(stream)), "fg_attention_ragged_direct")
    return workspace


def fg_pass(plan, d_meta, q, k_new, v_new, k_pool, v_pool, out, lse=None, workspace=None, stream=None,
            out_dtype=None, device="cuda"):
    """One whole pass (upload, append, attention); d_meta is allocated here
    (torch uint8) when None.  Returns (d_meta, workspace)."""
    if d_meta is None:
        import torch
        d_meta = torch.empty(max(16, plan.info["metadata_bytes"]), dtype=torch.uint8, device=device)
    elif hasattr(d_meta, "numel") and d_meta.numel() * d_meta.element_size() < plan.info["metadata_bytes"]:
        raise ValueError("metadata buffer too small")
    out_dtype = _out_dtype(out, out_dtype)
    _check_pass_tensors(plan, q, k_new, v_new, k_pool, v_pool, out, lse, out_dtype)
    workspace, have = _workspace(plan, workspace, device)
    _check(lib().fg_pass(plan.handle, _ptr(d_meta), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                         _ptr(v_pool), _ptr(out), int(out_dtype), _ptr(lse), _ptr(workspace), int(have),
                         _stream(stream)), "fg_pass")
    plan.meta = d_meta
    return d_meta, workspace


def fg_attention_ragged_noalloc(plan, d_meta, q, k_pool, v_pool, out, lse=None, stream=None,
                                out_dtype=None):
    """fg_attention_ragged with the library's scratch array as its workspace
    (nothing is allocated, here or in the library)."""
    t, hq, hkv, d = plan.num_tokens, plan.num_q_heads, plan.num_kv_heads, plan.head_dim
    kshape, vshape = pool_shapes(plan.num_blocks, hkv, plan.block_size, d)
    if out_dtype is None:
        import torch
        out_dtype = FG_DTYPE_BF16 if (hasattr(out, "dtype") and out.dtype == torch.bfloat16) else FG_DTYPE_F32
    _check_tensor(q, (t, hq, d), "bf16", "q")
    _check_tensor(k_pool, kshape, "bf16", "k_pool")
    _check_tensor(v_pool, vshape, "bf16", "v_pool")
    _check_tensor(out, (t, hq, d), "bf16" if out_dtype == FG_DTYPE_BF16 else "f32", "out")
    _check_tensor(lse, (t, hq), "f32", "lse")
    _check(lib().fg_attention_ragged_noalloc(plan.handle, _ptr(d_meta if d_meta is not None else plan.meta),
                                             _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), int(out_dtype),
                                             _ptr(lse), _stream(stream)),
           "fg_attention_ragged_noalloc")


def fg_noalloc_scratch_bytes():
    return int(lib().fg_noalloc_scratch_bytes())


def fg_profile_enable(on=True, kernels=None):
    """Bracket launches with HIP events: every kernel, or only the FG_KERNEL_*
    ids in `kernels`; on=False turns it off."""
    mask = 0
    if on:
        mask = -1 if kernels is None else sum(1 << int(k) for k in kernels)
    _check(lib().fg_profile_enable(int(mask)), "fg_profile_enable")


def fg_profile_read():
    """{kernel name: (total ms, launches)} since the last read."""
    n = FG_KERNEL_COUNT
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(lib().fg_profile_read(ms, cnt, n), "fg_profile_read")
    return {lib().fg_kernel_name(i).decode(): (ms[i], cnt[i]) for i in range(n)}


def fg_probe_read_stream(buf, sink, stream=None):
    """One read-stream launch over the whole uint8 device tensor `buf`
    (measurement only); `sink` is a device tensor of >= 1024 bytes per CU."""
    _check(lib().fg_probe_read_stream(_ptr(buf), int(buf.numel() * buf.element_size()), _ptr(sink),
                                      int(sink.numel() * sink.element_size()), _stream(stream)),
           "fg_probe_read_stream")


def fg_probe_mfma_loop(iters, sink, clocks, stream=None):
    """One matrix-core loop launch (measurement only); `sink` holds >= 2 KiB and
    `clocks` (int64) >= 32 bytes per CU."""
    _check(lib().fg_probe_mfma_loop(int(iters), _ptr(sink), int(sink.numel() * sink.element_size()),
                                    _ptr(clocks), int(clocks.numel() * clocks.element_size()),
                                    _stream(stream)), "fg_probe_mfma_loop")


# short aliases used by tests and bench
kv_append = fg_kv_append
upload_append = fg_upload_append
attention_ragged = fg_attention_ragged
attention_ragged_noalloc = fg_attention_ragged_noalloc
attention_ragged_direct = fg_attention_ragged_direct
run_pass = fg_pass
