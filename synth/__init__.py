"""Seeded synthetic inputs for paged-KV backup/restore.

This module holds only input generation: page-ID permutations, the shapes of
the synthetic workloads, and a counter-based byte stream (SplitMix64,
Steele, Lea and Flood, OOPSLA 2014) used to fill pools and host buffers, in
numpy here and as a GPU fill kernel in ``fill.hip``. It contains none of the
backup/restore arithmetic, so both the oracle's tests and the HIP path's
tests may draw from it.

Stream definition: word j of stream `seed` is the (j+1)-th output of
SplitMix64 started at state `seed`; byte a of the stream is byte (a mod 8),
little-endian, of word floor(a / 8).
"""
import numpy as np

from .workloads import WORKLOADS, Workload  # noqa: F401

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def gen_words(seed: int, j0: int, count: int) -> np.ndarray:
    """Words j0 .. j0+count-1 of stream `seed` as uint64."""
    with np.errstate(over="ignore"):
        j = np.arange(j0, j0 + count, dtype=np.uint64)
        z = np.uint64(seed) + (j + np.uint64(1)) * GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def gen_bytes(seed: int, addr: int, nbytes: int) -> np.ndarray:
    """Bytes addr .. addr+nbytes-1 of stream `seed` as uint8."""
    if nbytes == 0:
        return np.zeros(0, dtype=np.uint8)
    j0 = addr // 8
    j1 = (addr + nbytes + 7) // 8
    w = gen_words(seed, j0, j1 - j0).astype("<u8")
    b = w.view(np.uint8)
    s = addr - 8 * j0
    return np.array(b[s:s + nbytes], copy=True)


def page_perm(seed: int, num_pages: int) -> np.ndarray:
    """A seeded random permutation of the page IDs [0, num_pages), as int32."""
    return np.random.default_rng(seed).permutation(num_pages).astype(np.int32)


def pool_alloc_image(w: "Workload", seed: int) -> np.ndarray:
    """Host image of a whole pool allocation: stream seed+1 everywhere, then
    stream `seed` over the pool region, both by allocation-relative address."""
    img = gen_bytes(seed + 1, 0, w.alloc_bytes)
    img[w.byte_offset:w.byte_offset + w.pool_bytes] = gen_bytes(seed, w.byte_offset, w.pool_bytes)
    return img


# ---------------------------------------------------------------------------
# GPU fill / compare (synth/libkvxsynth.so)
# ---------------------------------------------------------------------------
_gpu = None


def _gpu_lib():
    global _gpu
    if _gpu is None:
        import ctypes
        import os
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvxsynth.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built")
        L = ctypes.CDLL(path)
        vp, u64 = ctypes.c_void_p, ctypes.c_uint64
        L.synth_fill.argtypes = [vp, u64, u64, u64, vp]
        L.synth_fill.restype = ctypes.c_int
        L.synth_diff_blocks.argtypes = [vp, u64, u64, u64, u64, vp, vp]
        L.synth_diff_blocks.restype = ctypes.c_int
        _gpu = L
    return _gpu


def fill_gpu(ptr: int, nbytes: int, seed: int, addr0: int, stream: int = 0) -> None:
    """Writes stream bytes addr0 .. addr0+nbytes-1 of `seed` to the
    device-visible memory at ptr (device memory or mapped pinned host)."""
    rc = _gpu_lib().synth_fill(ptr, nbytes, seed, addr0, stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill failed ({rc})")


def diff_blocks_gpu(ptr: int, nbytes: int, seed: int, addr0: int, block_bytes: int,
                    flags_ptr: int, stream: int = 0) -> None:
    """Sets the uint32 flag of every block_bytes block of [ptr, ptr+nbytes)
    that differs from the stream (flags must be zeroed beforehand)."""
    rc = _gpu_lib().synth_diff_blocks(ptr, nbytes, seed, addr0, block_bytes, flags_ptr, stream)
    if rc != 0:
        raise RuntimeError(f"synth_diff_blocks failed ({rc})")


def fill_alloc_gpu(ptr: int, w: "Workload", seed: int, stream: int = 0) -> None:
    """GPU version of pool_alloc_image: stream seed+1 over the allocation,
    then stream `seed` over the pool region."""
    fill_gpu(ptr, w.alloc_bytes, seed + 1, 0, stream)
    fill_gpu(ptr + w.byte_offset, w.pool_bytes, seed, w.byte_offset, stream)
