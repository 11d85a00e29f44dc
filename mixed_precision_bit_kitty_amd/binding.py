"""ctypes binding of libkitty.so (the C ABI in include/kitty.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the stream.
The functions keep the C names (``kitty_quantize_pages`` ...) and accept
torch CUDA tensors; ``KittyCache`` owns the caller-side buffers of one paged
cache (page pool, block table, fp16 tail, sequence lengths).

There is no fallback: if the library is missing or no GPU is present the
calls fail loudly.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkitty.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "kitty.h")

KITTY_OK = 0
KITTY_ERR_INVALID_ARG = -1
KITTY_ERR_UNSUPPORTED = -2
KITTY_ERR_WORKSPACE = -3
KITTY_ERR_HIP = -4
KITTY_ERR_NO_PAGES = -5
KITTY_RANK_PAGE = 0
KITTY_RANK_RUNNING = 1
KITTY_KEY_STATS_BYTES = 8192

HEAD_DIM = 128
PAGE_TOKENS = 32
MAX_SEQ_LEN = 4096 * 32 + 31  # the largest max_seq_len decode accepts (4096 pages and a tail)


class KittyError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"kitty error {code}: {msg}")
        self.code = code


class kitty_config_t(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("n_hi", ctypes.c_int32), ("lo_bit", ctypes.c_int32),
                ("rank_mode", ctypes.c_int32)]


class kitty_kv_view_t(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("n_pages", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("tail_k", ctypes.c_void_p),
                ("tail_v", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p), ("key_stats", ctypes.c_void_p)]


class kitty_pool_t(ctypes.Structure):
    _fields_ = [("free_list", ctypes.c_void_p), ("n_pages", ctypes.c_int64), ("n_free", ctypes.c_int64)]


_lib = None


BENCH_HEADER = os.path.join(os.path.dirname(PKG), "include", "kitty_bench.h")


def declared_symbols(header=None):
    """Names of the functions include/kitty.h (and kitty_bench.h) declare,
    or those of one given header."""
    out = set()
    for h in ([HEADER, BENCH_HEADER] if header is None else [header]):
        with open(h) as f:
            text = f.read()
        out |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(kitty_\w+)\s*\(", text, re.M))
    return sorted(out)


def load(path=None):
    """Load libkitty.so once and declare the C signatures.  KITTY_LIB (env)
    selects another build of the same library, e.g. for A/B comparisons."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("KITTY_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise KittyError(KITTY_ERR_HIP, f"{path} is missing; run __graft_entry__.build() first")
    try:  # torch first: its HIP runtime is then the one libkitty binds to (one runtime per process)
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp, viewp = P(kitty_config_t), P(kitty_kv_view_t)
    sig = {
        "kitty_abi_version": ([], ctypes.c_int),
        "kitty_last_error": ([], ctypes.c_char_p),
        "kitty_record_bytes": ([cfgp, P(sz)], ctypes.c_int),
        "kitty_page_bytes": ([cfgp, P(sz)], ctypes.c_int),
        "kitty_quantize_pages": ([cfgp, viewp, vp, vp, i32, vp, vp], ctypes.c_int),
        "kitty_append_token": ([cfgp, viewp, vp, vp, vp], ctypes.c_int),
        "kitty_decode_workspace_bytes": ([cfgp, i32, i32, i32, P(sz)], ctypes.c_int),
        "kitty_decode_plan": ([cfgp, i32, i32, i32, i32, P(i32)], ctypes.c_int),
        "kitty_decode_attention": ([cfgp, viewp, vp, i32, i32, vp, vp, sz, vp], ctypes.c_int),
        "kitty_decode_step": ([cfgp, viewp, vp, vp, vp, i32, i32, vp, vp, sz, vp], ctypes.c_int),
        "kitty_decode_step_noalloc": ([cfgp, viewp, vp, vp, vp, i32, i32, vp, vp], ctypes.c_int),
        "kitty_pool_init": ([P(kitty_pool_t), vp, ctypes.c_int64], ctypes.c_int),
        "kitty_pool_reserve": ([P(kitty_pool_t), vp, i32, i32], ctypes.c_int),
        "kitty_pool_release": ([P(kitty_pool_t), vp, i32], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def load_bench():
    """The library with the measurement entry points of include/kitty_bench.h
    declared (kitty_read_ceiling, kitty_stream_ceiling)."""
    lib = load()
    f = lib.kitty_read_ceiling
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    f.restype = ctypes.c_int
    f = lib.kitty_stream_ceiling
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    f.restype = ctypes.c_int
    return lib


def _check(rc):
    if rc != KITTY_OK:
        raise KittyError(rc, load().kitty_last_error().decode())


def config(n_kv_heads, n_hi, head_dim=HEAD_DIM, page_tokens=PAGE_TOKENS, lo_bit=2, rank_mode=0):
    """lo_bit 2: (hi_bit 4, lo_bit 2); lo_bit 4: (hi_bit 8, lo_bit 4).
    rank_mode: KITTY_RANK_PAGE (0) or KITTY_RANK_RUNNING (1)."""
    return kitty_config_t(head_dim, page_tokens, n_kv_heads, n_hi, lo_bit, rank_mode)


def kitty_abi_version():
    return load().kitty_abi_version()


def kitty_record_bytes(cfg):
    out = ctypes.c_size_t()
    _check(load().kitty_record_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def kitty_page_bytes(cfg):
    out = ctypes.c_size_t()
    _check(load().kitty_page_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def kitty_decode_workspace_bytes(cfg, batch, n_q_heads, max_seq_len):
    out = ctypes.c_size_t()
    _check(load().kitty_decode_workspace_bytes(ctypes.byref(cfg), batch, n_q_heads, max_seq_len,
                                               ctypes.byref(out)))
    return out.value


def kitty_decode_plan(cfg, batch, n_q_heads, max_seq_len, n_cus=0):
    """(workgroups per unit, waves per workgroup, largest workgroup) of the
    decode split plan on a device with n_cus compute units (0: the current
    device)."""
    out = (ctypes.c_int32 * 3)()
    _check(load().kitty_decode_plan(ctypes.byref(cfg), batch, n_q_heads, max_seq_len, n_cus, out))
    return tuple(out)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, shape=None, name="tensor"):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise KittyError(KITTY_ERR_INVALID_ARG, f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise KittyError(KITTY_ERR_INVALID_ARG, f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise KittyError(KITTY_ERR_INVALID_ARG, f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise KittyError(KITTY_ERR_INVALID_ARG, f"{name} shape {tuple(t.shape)} != {tuple(shape)}")


def kitty_quantize_pages(cfg, view, k, v, S, lens=None, stream=None):
    _check(load().kitty_quantize_pages(ctypes.byref(cfg), ctypes.byref(view), _ptr(k), _ptr(v), S,
                                       _ptr(lens), _stream(stream)))


def kitty_append_token(cfg, view, k_new, v_new, stream=None):
    _check(load().kitty_append_token(ctypes.byref(cfg), ctypes.byref(view), _ptr(k_new), _ptr(v_new),
                                     _stream(stream)))


def kitty_decode_attention(cfg, view, q, n_q_heads, max_seq_len, out, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().kitty_decode_attention(ctypes.byref(cfg), ctypes.byref(view), _ptr(q), n_q_heads,
                                         max_seq_len, _ptr(out), _ptr(workspace), nbytes, _stream(stream)))


def kitty_decode_step(cfg, view, k_new, v_new, q, n_q_heads, max_seq_len, out, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().kitty_decode_step(ctypes.byref(cfg), ctypes.byref(view), _ptr(k_new), _ptr(v_new), _ptr(q),
                                    n_q_heads, max_seq_len, _ptr(out), _ptr(workspace), nbytes,
                                    _stream(stream)))


def kitty_decode_step_noalloc(cfg, view, k_new, v_new, q, n_q_heads, max_seq_len, out, stream=None):
    _check(load().kitty_decode_step_noalloc(ctypes.byref(cfg), ctypes.byref(view), _ptr(k_new), _ptr(v_new),
                                            _ptr(q), n_q_heads, max_seq_len, _ptr(out), _stream(stream)))


class PagePool:
    """Host-side page pool (kitty_pool_*): a free list of physical page ids
    and the reservation / release of block-table rows (host numpy int32
    arrays, -1 = unmapped)."""

    def __init__(self, n_pages):
        import numpy as np
        self.free_list = np.empty(n_pages, dtype=np.int32)
        self.pool = kitty_pool_t()
        _check(load().kitty_pool_init(ctypes.byref(self.pool), self.free_list.ctypes.data, n_pages))

    @property
    def n_free(self):
        return int(self.pool.n_free)

    @staticmethod
    def _row(row):
        import numpy as np
        if not (isinstance(row, np.ndarray) and row.dtype == np.int32 and row.flags.c_contiguous and row.ndim == 1):
            raise KittyError(KITTY_ERR_INVALID_ARG, "row must be a contiguous 1-d numpy int32 array")
        return row

    def reserve(self, row, n_tokens):
        row = self._row(row)
        _check(load().kitty_pool_reserve(ctypes.byref(self.pool), row.ctypes.data, row.shape[0], n_tokens))

    def release(self, row):
        row = self._row(row)
        _check(load().kitty_pool_release(ctypes.byref(self.pool), row.ctypes.data, row.shape[0]))


class KittyCache:
    """Caller-side buffers of one paged cache on a CUDA device.

    pool        uint8 [n_pages, page_bytes]
    block_table int32 [batch, max_pages] (identity-like mapping by default:
                sequence b's page j -> physical page b * max_pages + j)
    tail_k/v    fp16  [batch, Hkv, 32, 128]
    seq_lens    int32 [batch]
    key_stats   uint8 [batch, Hkv, 8192] running sums (rank_mode KITTY_RANK_RUNNING only, else None)
    """

    def __init__(self, batch, n_kv_heads, n_hi, max_tokens, device="cuda", block_table=None, n_pages=None,
                 lo_bit=2, rank_mode=KITTY_RANK_PAGE):
        import torch
        self.cfg = config(n_kv_heads, n_hi, lo_bit=lo_bit, rank_mode=rank_mode)
        self.batch, self.n_kv_heads, self.n_hi, self.lo_bit = batch, n_kv_heads, n_hi, lo_bit
        self.rank_mode = rank_mode
        self.max_pages = max(1, -(-max_tokens // PAGE_TOKENS))
        self.page_bytes = kitty_page_bytes(self.cfg)
        self.record_bytes = kitty_record_bytes(self.cfg)
        if block_table is None:
            bt = torch.arange(batch * self.max_pages, dtype=torch.int32).reshape(batch, self.max_pages)
            n_pages = batch * self.max_pages if n_pages is None else n_pages
        else:
            bt = torch.as_tensor(block_table, dtype=torch.int32)
            if bt.dim() != 2 or bt.shape[0] != batch:
                raise KittyError(KITTY_ERR_INVALID_ARG, "block_table must be [batch, max_pages]")
            self.max_pages = int(bt.shape[1])
            if n_pages is None:
                raise KittyError(KITTY_ERR_INVALID_ARG, "n_pages is required with a block table")
        self.n_pages = int(n_pages)
        self.block_table = bt.to(device).contiguous()
        self.pool = torch.zeros((self.n_pages, self.page_bytes), dtype=torch.uint8, device=device)
        self.tail_k = torch.zeros((batch, n_kv_heads, PAGE_TOKENS, HEAD_DIM), dtype=torch.float16, device=device)
        self.tail_v = torch.zeros_like(self.tail_k)
        self.seq_lens = torch.zeros(batch, dtype=torch.int32, device=device)
        self.key_stats = None
        if rank_mode == KITTY_RANK_RUNNING:
            self.key_stats = torch.zeros((batch, n_kv_heads, KITTY_KEY_STATS_BYTES), dtype=torch.uint8, device=device)
        self.view = kitty_kv_view_t(self.pool.data_ptr(), self.n_pages, self.block_table.data_ptr(), batch,
                                    self.max_pages, self.tail_k.data_ptr(), self.tail_v.data_ptr(),
                                    self.seq_lens.data_ptr(),
                                    None if self.key_stats is None else self.key_stats.data_ptr())
        self._ws = None

    @classmethod
    def with_pool(cls, batch, n_kv_heads, n_hi, max_tokens, n_pages, device="cuda", lo_bit=2, rank_mode=KITTY_RANK_PAGE):
        """A serving cache: every slot starts inactive (seq_lens -1, no page
        mapped) and pages come from a shared PagePool of n_pages pages."""
        import numpy as np
        max_pages = max(1, -(-max_tokens // PAGE_TOKENS))
        c = cls(batch, n_kv_heads, n_hi, max_tokens, device=device,
                block_table=np.full((batch, max_pages), -1, np.int32), n_pages=n_pages, lo_bit=lo_bit,
                rank_mode=rank_mode)
        c.bt_host = np.full((batch, c.max_pages), -1, np.int32)
        c.page_pool = PagePool(n_pages)
        c.seq_lens.fill_(-1)
        return c

    def reserve(self, b, n_tokens):
        """Map the pages slot b needs to hold n_tokens tokens (before the
        prefill or decode step that reaches that length)."""
        import torch
        before = self.bt_host[b].copy()
        self.page_pool.reserve(self.bt_host[b], n_tokens)
        if not (before == self.bt_host[b]).all():
            self.block_table[b].copy_(torch.from_numpy(self.bt_host[b]))

    def release(self, b):
        """Return slot b's pages to the pool and mark the slot inactive."""
        import torch
        self.page_pool.release(self.bt_host[b])
        self.block_table[b].copy_(torch.from_numpy(self.bt_host[b]))
        self.seq_lens[b] = -1

    # -- hot path ---------------------------------------------------------
    def quantize_pages(self, k, v, lens=None, stream=None):
        import torch
        B, H, S, D = k.shape
        _need(k, torch.float16, (self.batch, self.n_kv_heads, S, HEAD_DIM), "k")
        _need(v, torch.float16, (self.batch, self.n_kv_heads, S, HEAD_DIM), "v")
        if lens is not None:
            _need(lens, torch.int32, (self.batch,), "lens")
        kitty_quantize_pages(self.cfg, self.view, k, v, S, lens, stream)

    def append_token(self, k_new, v_new, stream=None):
        import torch
        _need(k_new, torch.float16, (self.batch, self.n_kv_heads, HEAD_DIM), "k_new")
        _need(v_new, torch.float16, (self.batch, self.n_kv_heads, HEAD_DIM), "v_new")
        kitty_append_token(self.cfg, self.view, k_new, v_new, stream)

    def default_max_seq_len(self):
        """The bound decode calls use by default: the block table's capacity
        (a full tail page past its pages), at most MAX_SEQ_LEN."""
        return min(self.max_pages * PAGE_TOKENS + PAGE_TOKENS - 1, MAX_SEQ_LEN)

    def workspace(self, n_q_heads, max_seq_len):
        import torch
        nb = kitty_decode_workspace_bytes(self.cfg, self.batch, n_q_heads, max_seq_len)
        if self._ws is None or self._ws.numel() < max(nb, 256):
            self._ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=self.pool.device)
        return self._ws

    def decode_attention(self, q, max_seq_len=None, out=None, workspace=None, stream=None):
        import torch
        B, Hq, D = q.shape
        _need(q, torch.float16, (self.batch, Hq, HEAD_DIM), "q")
        msl = self.default_max_seq_len() if max_seq_len is None else max_seq_len
        if out is None:
            out = torch.empty((self.batch, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
        _need(out, torch.float32, (self.batch, Hq, HEAD_DIM), "out")
        ws = self.workspace(Hq, msl) if workspace is None else workspace
        kitty_decode_attention(self.cfg, self.view, q, Hq, msl, out, ws, stream)
        return out

    def decode_step(self, k_new, v_new, q, max_seq_len=None, out=None, workspace=None, stream=None):
        """append_token(k_new, v_new) then decode_attention(q), in one launch."""
        import torch
        B, Hq, D = q.shape
        _need(k_new, torch.float16, (self.batch, self.n_kv_heads, HEAD_DIM), "k_new")
        _need(v_new, torch.float16, (self.batch, self.n_kv_heads, HEAD_DIM), "v_new")
        _need(q, torch.float16, (self.batch, Hq, HEAD_DIM), "q")
        msl = self.default_max_seq_len() if max_seq_len is None else max_seq_len
        if out is None:
            out = torch.empty((self.batch, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
        _need(out, torch.float32, (self.batch, Hq, HEAD_DIM), "out")
        ws = self.workspace(Hq, msl) if workspace is None else workspace
        kitty_decode_step(self.cfg, self.view, k_new, v_new, q, Hq, msl, out, ws, stream)
        return out

    # -- inspection -------------------------------------------------------
    def record(self, b, j, h):
        """Bytes (torch uint8, on device) of sequence b's page j, head h."""
        phys = int(self.block_table[b, j])
        return self.pool[phys, h * self.record_bytes:(h + 1) * self.record_bytes]
