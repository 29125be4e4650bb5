"""Helpers for the GPU tests: device pools filled from the seeded generator,
pinned packed buffers, and host copies for the oracle. Plumbing only: the
operations under test run through the C ABI (paged_kv_offload_amd), and
every expected value comes from oracle/."""
import numpy as np

import oracle
import synth
from paged_kv_offload_amd import kvx as K

PATHS = {"staged": K.KVX_PATH_STAGED, "zerocopy": K.KVX_PATH_ZEROCOPY,
         "device": K.KVX_PATH_DEVICE}


def torch():
    import torch as t
    return t


def oracle_layout(w) -> oracle.Layout:
    ax = {"page": oracle.PAGE, "layer": oracle.LAYER, "kv": oracle.KV}
    return oracle.Layout(outer=tuple(ax[a] for a in w.outer),
                         inner=oracle.NHD if w.inner == "NHD" else oracle.HND,
                         num_pages=w.num_pages, num_layers=w.num_layers, num_kv=w.num_kv,
                         page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
                         dtype_bytes=w.dtype_bytes, byte_offset=w.byte_offset)


def kvx_layout(w):
    return K.make_layout(w.outer, w.inner, w.num_pages, w.num_layers, w.num_kv, w.page_size,
                         w.num_heads, w.head_dim)


class DevicePool:
    """A pool allocation on cuda:0 filled from stream `seed` (pool) and
    seed+1 (padding), registered through the binding's register_tensor."""

    def __init__(self, w, seed=None, generation=1, stream=None):
        t = torch()
        self.w = w
        self.seed = w.seed if seed is None else seed
        self.alloc = t.empty(w.alloc_bytes, dtype=t.uint8, device="cuda")
        assert self.alloc.data_ptr() % 16 == 0
        synth.fill_alloc_gpu(self.alloc.data_ptr(), w, self.seed,
                             stream=0 if stream is None else stream.cuda_stream)
        t.cuda.synchronize()
        dt = {1: t.uint8, 2: t.bfloat16, 4: t.float32}.get(w.dtype_bytes)
        if dt is not None:
            view = self.alloc[w.byte_offset:w.byte_offset + w.pool_bytes].view(dt)
            self.tensor = view.view(*w.tensor_shape())
            self.handle = K.register_tensor(self.tensor, kvx_layout(w), generation)
        else:
            # an element size torch has no dtype for: the C ABI takes the
            # allocation base, the byte offset and element shape and strides
            self.tensor = None
            shape = w.tensor_shape()
            stride = [int(np.prod(shape[i + 1:])) for i in range(len(shape))]
            base, _ = K.kvx_alloc_range(self.alloc.data_ptr())
            self.handle = K.kvx_register_pool(kvx_layout(w), base,
                                              self.alloc.data_ptr() + w.byte_offset - base,
                                              w.dtype_bytes, shape, stride, generation)

    def host_image(self) -> np.ndarray:
        torch().cuda.synchronize()
        return self.alloc.cpu().numpy()

    def close(self):
        if self.handle:
            K.kvx_unregister_pool(self.handle)
            self.handle = 0


class Packed:
    """A packed buffer for n pages: pinned host (staged / zerocopy) or device."""

    def __init__(self, w, n, path, fill_seed=None):
        self.nbytes = w.host_bytes(n)
        self.path = path
        if path == "device":
            t = torch()
            self.dev = t.empty(self.nbytes, dtype=t.uint8, device="cuda")
            self.ptr = self.dev.data_ptr()
            self.host = None
        else:
            self.host = K.HostBuffer(self.nbytes)
            self.ptr = self.host.ptr
            self.dev = None
        if fill_seed is not None:
            self.fill(fill_seed)

    def fill(self, seed):
        synth.fill_gpu(self.ptr, self.nbytes, seed, 0)
        torch().cuda.synchronize()

    def numpy(self) -> np.ndarray:
        torch().cuda.synchronize()
        if self.host is not None:
            return self.host.numpy().copy()
        return self.dev.cpu().numpy()

    def close(self):
        if self.host is not None:
            self.host.free()
