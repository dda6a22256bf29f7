"""ResidualKV hot path for MI355X (gfx950): Python binding of librkv.

Thin wrappers with the names of the C entry points in include/rkv.h.  They
only marshal arguments: tensors become device pointers, the current torch
stream becomes the HIP stream, and buffers of the right size come from
torch's allocator.  Every step of the path runs in librkv's HIP kernels; if
librkv.so is missing, every call raises.
"""

import ctypes as C

import torch

from . import _lib as L

__all__ = [
    "RkvError", "Cache", "rkv_num_refs", "rkv_ref_position", "rkv_encode",
    "rkv_select_refs", "rkv_quantize", "rkv_reconstruct", "rkv_decode_attn",
    "rkv_encode_workspace", "rkv_decode_workspace", "library_path",
]

_DT = {"f32": (L.RKV_F32, torch.float32), "bf16": (L.RKV_BF16, torch.bfloat16)}


class RkvError(RuntimeError):
    def __init__(self, msg, status):
        super().__init__(msg)
        self.status = status


def library_path() -> str:
    return L.LIB_PATH


def _load():
    return L.load()


def _check(status: int, what: str):
    if status != L.RKV_OK:
        lib = _load()
        msg = lib.rkv_status_string(status).decode()
        if status == L.RKV_ERR_HIP:
            msg += f" (hipError_t {lib.rkv_last_hip_error()})"
        raise RkvError(f"{what}: {msg}", status)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


def _stride(base, double_after):
    return L.RkvStride(int(base), int(double_after))


def rkv_num_refs(seq_len: int, base: int, double_after: int = 0) -> int:
    return int(_load().rkv_num_refs(int(seq_len), _stride(base, double_after)))


def rkv_ref_position(slot: int, base: int, double_after: int = 0) -> int:
    return int(_load().rkv_ref_position(int(slot), _stride(base, double_after)))


class Cache:
    """A compressed cache: the rkv_cache shape plus torch-owned device
    buffers (ref_idx, codes_k, codes_v, scales, ref_kv) as raw bytes."""

    BUFFERS = ("ref_idx", "codes_k", "codes_v", "scales", "ref_kv", "ref_scales")

    def __init__(self, n_inst, n_kv_heads, seq_len, dtype, stride_base, k, bits, group,
                 double_after=0, head_dim=128, device="cuda", allocate=True, ref_bits=0,
                 latent=0, latent_seed=0):
        self.dtype = dtype
        self.torch_dtype = _DT[dtype][1]
        s = L.RkvCache()
        s.dtype = _DT[dtype][0]
        s.n_inst = int(n_inst)
        s.n_kv_heads = int(n_kv_heads)
        s.seq_len = int(seq_len)
        s.head_dim = int(head_dim)
        s.stride = _stride(stride_base, double_after)
        s.k = int(k)
        s.bits = int(bits)
        s.group = int(group)
        s.ref_bits = int(ref_bits)
        s.latent = int(latent)
        s.latent_seed = int(latent_seed) & ((1 << 64) - 1)
        _check(_load().rkv_cache_init(C.byref(s)), "rkv_cache_init")
        self.c = s
        sizes = (C.c_size_t * 6)()
        _check(_load().rkv_cache_sizes(C.byref(s), sizes), "rkv_cache_sizes")
        self.sizes = dict(zip(self.BUFFERS, [int(x) for x in sizes]))
        self.buffers = {}
        if allocate:
            for name in self.BUFFERS:
                # cleared once: positions a streaming cache has not reached
                # (and the V-tile bits past seq_len) read as zero
                t = torch.zeros(max(1, self.sizes[name]), dtype=torch.uint8, device=device)
                self.buffers[name] = t
                setattr(s, name, t.data_ptr() if self.sizes[name] else None)

    @property
    def n_refs(self) -> int:
        return int(self.c.n_refs)

    def slice(self, i0: int, n: int) -> "Cache":
        """A view of instances [i0, i0+n): same shape, buffer pointers offset."""
        c = self.c
        if not (0 <= i0 and n >= 1 and i0 + n <= c.n_inst):
            raise ValueError("instance range out of bounds")
        v = Cache.__new__(Cache)
        v.dtype, v.torch_dtype = self.dtype, self.torch_dtype
        s = L.RkvCache()
        C.pointer(s)[0] = c
        s.n_inst = n
        v.c = s
        v.sizes = {k: sz // c.n_inst * n for k, sz in self.sizes.items()}
        v.buffers = {}
        for name in self.BUFFERS:
            per = self.sizes[name] // c.n_inst
            full = self.buffers[name]
            v.buffers[name] = full[i0 * per:(i0 + n) * per] if per else full[:1]
            setattr(s, name, v.buffers[name].data_ptr() if per else None)
        return v

    def nbytes(self) -> int:
        return sum(self.sizes.values())

    def __getattr__(self, name):
        b = self.__dict__.get("buffers", {})
        if name in b:
            return b[name]
        raise AttributeError(name)


def _ws(nbytes, device, ws):
    if ws is None:
        ws = torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)
    return ws


def rkv_encode_workspace(cache: Cache) -> int:
    n = C.c_size_t()
    _check(_load().rkv_encode_workspace(C.byref(cache.c), C.byref(n)), "rkv_encode_workspace")
    return int(n.value)


def rkv_decode_workspace(cache: Cache, n_q_heads: int, n_split: int) -> int:
    n = C.c_size_t()
    _check(_load().rkv_decode_workspace(C.byref(cache.c), int(n_q_heads), int(n_split),
                                       C.byref(n)), "rkv_decode_workspace")
    return int(n.value)


def _check_kv(K, V, cache):
    c = cache.c
    want = (c.n_inst, c.n_kv_heads, c.seq_len, c.head_dim)
    for name, t in (("K", K), ("V", V)):
        if t.dtype != cache.torch_dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {cache.torch_dtype} device tensor")
        if t.numel() != want[0] * want[1] * want[2] * want[3]:
            raise ValueError(f"{name} must hold {want} elements")


def rkv_encode(K, V, cache: Cache, ws=None, stream=None):
    _check_kv(K, V, cache)
    nb = rkv_encode_workspace(cache)
    ws = _ws(nb, K.device, ws)
    _check(_load().rkv_encode(_ptr(K), _ptr(V), C.byref(cache.c), _ptr(ws), ws.numel(),
                             _stream(stream)), "rkv_encode")
    return ws


def rkv_append(K_new, V_new, cache: Cache, pos0: int, ws, stream=None):
    """Encode positions pos0 .. pos0 + n_new - 1 from K_new/V_new
    [n_inst, n_kv_heads, n_new, head_dim]; `ws` is the encode workspace that
    earlier rkv_encode/rkv_append calls on this cache used (it carries the
    reference keys)."""
    c = cache.c
    for name, t in (("K_new", K_new), ("V_new", V_new)):
        if t.dtype != cache.torch_dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {cache.torch_dtype} device tensor")
        if t.dim() != 4 or tuple(t.shape[:2]) != (c.n_inst, c.n_kv_heads) or t.shape[3] != c.head_dim:
            raise ValueError(f"{name} must be [n_inst, n_kv_heads, n_new, head_dim]")
    if K_new.shape != V_new.shape:
        raise ValueError("K_new and V_new differ in shape")
    if ws is None or ws.numel() < rkv_encode_workspace(cache):
        raise ValueError("rkv_append needs the encode workspace of the earlier calls")
    _check(_load().rkv_append(_ptr(K_new), _ptr(V_new), int(K_new.shape[2]), C.byref(c),
                             int(pos0), _ptr(ws), ws.numel(), _stream(stream)), "rkv_append")


def rkv_select_refs(K, V, cache: Cache, ws=None, stream=None):
    _check_kv(K, V, cache)
    nb = rkv_encode_workspace(cache)
    ws = _ws(nb, K.device, ws)
    _check(_load().rkv_select_refs(_ptr(K), _ptr(V), C.byref(cache.c), _ptr(ws), ws.numel(),
                                  _stream(stream)), "rkv_select_refs")
    return ws


def rkv_quantize(K, V, cache: Cache, stream=None):
    _check_kv(K, V, cache)
    _check(_load().rkv_quantize(_ptr(K), _ptr(V), C.byref(cache.c), C.c_void_p(0), 0,
                               _stream(stream)), "rkv_quantize")


def rkv_reconstruct(cache: Cache, K_hat=None, V_hat=None, stream=None):
    c = cache.c
    shape = (c.n_inst, c.n_kv_heads, c.seq_len, c.head_dim)
    dev = cache.buffers["ref_kv"].device
    if K_hat is None:
        K_hat = torch.empty(shape, dtype=torch.float32, device=dev)
        V_hat = torch.empty(shape, dtype=torch.float32, device=dev)
    for t in (K_hat, V_hat):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != K_hat.numel():
            raise ValueError("K_hat/V_hat must be contiguous float32 of the cache shape")
    _check(_load().rkv_reconstruct(C.byref(c), _ptr(K_hat), _ptr(V_hat), _stream(stream)),
           "rkv_reconstruct")
    return K_hat, V_hat


def rkv_decode_split_hint(cache: Cache, n_q_heads: int) -> int:
    n = C.c_int32()
    _check(_load().rkv_decode_split_hint(C.byref(cache.c), int(n_q_heads), C.byref(n)),
           "rkv_decode_split_hint")
    return int(n.value)


def rkv_decode_attn(q, n_q_heads: int, cache: Cache, softmax_scale: float, out=None,
                    n_split: int = 1, ws=None, stream=None):
    c = cache.c
    if q.dtype != cache.torch_dtype or not q.is_cuda or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous {cache.torch_dtype} device tensor")
    if q.numel() != c.n_inst * n_q_heads * c.head_dim:
        raise ValueError("q must hold n_inst * n_q_heads * head_dim elements")
    if out is None:
        out = torch.empty((c.n_inst, n_q_heads, c.head_dim), dtype=torch.float32,
                          device=q.device)
    nb = rkv_decode_workspace(cache, n_q_heads, n_split)
    ws = _ws(nb, q.device, ws)
    _check(_load().rkv_decode_attn(_ptr(q), int(n_q_heads), C.byref(c), float(softmax_scale),
                                  _ptr(out), int(n_split), _ptr(ws), ws.numel(),
                                  _stream(stream)), "rkv_decode_attn")
    return out


def rkv_decode_attn_len(q, n_q_heads: int, cache: Cache, length: int, softmax_scale: float,
                        out=None, n_split: int = 1, ws=None, stream=None):
    """Decode attention over positions 0 .. length - 1."""
    c = cache.c
    if q.dtype != cache.torch_dtype or not q.is_cuda or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous {cache.torch_dtype} device tensor")
    if q.numel() != c.n_inst * n_q_heads * c.head_dim:
        raise ValueError("q must hold n_inst * n_q_heads * head_dim elements")
    if out is None:
        out = torch.empty((c.n_inst, n_q_heads, c.head_dim), dtype=torch.float32,
                          device=q.device)
    nb = rkv_decode_workspace(cache, n_q_heads, n_split)
    ws = _ws(nb, q.device, ws)
    _check(_load().rkv_decode_attn_len(_ptr(q), int(n_q_heads), C.byref(c), int(length),
                                      float(softmax_scale), _ptr(out), int(n_split), _ptr(ws),
                                      ws.numel(), _stream(stream)), "rkv_decode_attn_len")
    return out


def rkv_decode_attn_tiles(q, n_q_heads: int, cache: Cache, softmax_scale: float, tiles,
                          out=None, n_split: int = 1, ws=None, stream=None):
    """Decode attention over the selected 32-position tiles only; `tiles` is an
    int32 device tensor [n_inst, n_kv_heads, n_tiles]."""
    c = cache.c
    if q.dtype != cache.torch_dtype or not q.is_cuda or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous {cache.torch_dtype} device tensor")
    if q.numel() != c.n_inst * n_q_heads * c.head_dim:
        raise ValueError("q must hold n_inst * n_q_heads * head_dim elements")
    if (tiles.dtype != torch.int32 or not tiles.is_cuda or not tiles.is_contiguous()
            or tiles.dim() != 3 or tiles.shape[0] != c.n_inst or tiles.shape[1] != c.n_kv_heads):
        raise ValueError("tiles must be a contiguous int32 device tensor [n_inst, n_kv_heads, n]")
    if out is None:
        out = torch.empty((c.n_inst, n_q_heads, c.head_dim), dtype=torch.float32,
                          device=q.device)
    nb = rkv_decode_workspace(cache, n_q_heads, n_split)
    ws = _ws(nb, q.device, ws)
    _check(_load().rkv_decode_attn_tiles(_ptr(q), int(n_q_heads), C.byref(c),
                                        float(softmax_scale), _ptr(tiles), int(tiles.shape[2]),
                                        _ptr(out), int(n_split), _ptr(ws), ws.numel(),
                                        _stream(stream)), "rkv_decode_attn_tiles")
    return out


def rkv_decode_attn_noalloc(q, n_q_heads: int, cache: Cache, softmax_scale: float, out,
                            n_split: int = 1, stream=None):
    """rkv_decode_attn with the library's fixed device scratch as workspace
    (no workspace argument; `out` is the caller's [n_inst, n_q_heads,
    head_dim] float32 tensor)."""
    c = cache.c
    if q.dtype != cache.torch_dtype or not q.is_cuda or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous {cache.torch_dtype} device tensor")
    if q.numel() != c.n_inst * n_q_heads * c.head_dim:
        raise ValueError("q must hold n_inst * n_q_heads * head_dim elements")
    if (out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous()
            or out.numel() != c.n_inst * n_q_heads * c.head_dim):
        raise ValueError("out must be a contiguous float32 device tensor of the output shape")
    _check(_load().rkv_decode_attn_noalloc(_ptr(q), int(n_q_heads), C.byref(c),
                                          float(softmax_scale), _ptr(out), int(n_split),
                                          _stream(stream)), "rkv_decode_attn_noalloc")
    return out
