"""The five synthetic pool workloads (shapes, seeds and page-ID schedules),
and one more: the Llama-shaped pool at one token per page.

Shapes follow the pools the source pages describe: a Llama-3-8B-shaped bf16
pool, an MLA/latent fp8 pool with page size 256 as in the PP-ticket PR's
benchmark setup (DeepSeek-V4-Flash, fp8_e4m3 KV cache, page size 256,
16,384-token inputs), and TRT-LLM's [NB, NL, 2, NH*BS*HS] head-major pool
from the LMCache RawCudaIPCWrapper article's integration section. Values
are random bits; nothing is interpreted as a number.

This module holds shapes and page-ID choices only; it computes no addresses.
"""
from dataclasses import dataclass
from typing import Dict, List, Tuple

import numpy as np

KIB = 1024
GIB = 1024 ** 3


@dataclass(frozen=True)
class Workload:
    name: str
    outer: Tuple[str, str, str]   # physical order of the outer axes, outermost first
    inner: str                    # "NHD" ([T][H][D]) or "HND" ([H][T][D])
    num_pages: int
    num_layers: int
    num_kv: int
    page_size: int
    num_heads: int
    head_dim: int
    dtype_bytes: int
    pages_per_request: int
    seed: int
    byte_offset: int = 0          # pool start inside its allocation
    alloc_tail: int = 0           # allocation bytes after the pool end
    merged_inner: bool = False    # tensor view merges the piece dims into one axis
    description: str = ""

    # ---- sizes -----------------------------------------------------------
    @property
    def row_bytes(self) -> int:
        return self.head_dim * self.dtype_bytes

    @property
    def piece_bytes(self) -> int:
        return self.page_size * self.num_heads * self.row_bytes

    @property
    def pool_bytes(self) -> int:
        return self.num_pages * self.num_layers * self.num_kv * self.piece_bytes

    @property
    def alloc_bytes(self) -> int:
        return self.byte_offset + self.pool_bytes + self.alloc_tail

    def payload_bytes(self, n: int = None) -> int:
        """KV bytes one backup or restore of n pages over all layers moves."""
        n = self.pages_per_request if n is None else n
        return self.num_layers * self.num_kv * n * self.piece_bytes

    def host_bytes(self, n: int = None) -> int:
        return self.payload_bytes(n)

    # ---- the caller's tensor view of the pool (elements) -------------------
    def tensor_shape(self) -> List[int]:
        dims = {"page": self.num_pages, "layer": self.num_layers, "kv": self.num_kv}
        outer = [dims[a] for a in self.outer]
        if self.merged_inner:
            return outer + [self.page_size * self.num_heads * self.head_dim]
        if self.inner == "NHD":
            return outer + [self.page_size, self.num_heads, self.head_dim]
        return outer + [self.num_heads, self.page_size, self.head_dim]

    def scaled(self, **changes) -> "Workload":
        d = dict(self.__dict__)
        d.update(changes)
        return Workload(**d)


def _wl(**kw) -> Workload:
    return Workload(**kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny": _wl(name="tiny", outer=("layer", "kv", "page"), inner="NHD", num_pages=64,
                num_layers=2, num_kv=2, page_size=16, num_heads=2, head_dim=64,
                dtype_bytes=2, pages_per_request=8, seed=101,
                description="tiny bf16 NHD pool [2L][2][64 pages][16 tok][2 heads][64]"),
    "llama8b": _wl(name="llama8b", outer=("layer", "kv", "page"), inner="NHD", num_pages=2048,
                   num_layers=32, num_kv=2, page_size=64, num_heads=8, head_dim=128,
                   dtype_bytes=2, pages_per_request=256, seed=102,
                   description="Llama-3-8B-shaped bf16 NHD pool [32L][2][2048 pages][64 tok]"
                               "[8 heads][128]; one 16384-token request = 256 fragmented pages"),
    "mla_fp8": _wl(name="mla_fp8", outer=("layer", "kv", "page"), inner="NHD", num_pages=1024,
                   num_layers=61, num_kv=1, page_size=256, num_heads=1, head_dim=576,
                   dtype_bytes=1, pages_per_request=64, seed=103,
                   description="MLA latent fp8 pool [61L][1][1024 pages][256 tok][1][576]; "
                               "16384-token requests = 64 pages, layer-wise restore"),
    "trtllm_hnd": _wl(name="trtllm_hnd", outer=("page", "layer", "kv"), inner="HND",
                      num_pages=4096, num_layers=32, num_kv=2, page_size=32, num_heads=8,
                      head_dim=128, dtype_bytes=2, pages_per_request=512, seed=104,
                      byte_offset=3 * 4 * KIB, alloc_tail=32 * KIB - 3 * 4 * KIB,
                      merged_inner=True,
                      description="TRT-LLM-style bf16 pool [4096, 32, 2, 8*32*128] head-major "
                                  "at byte offset 12288 of an allocation 32 KiB larger; 512 pages"),
    "mixed": _wl(name="mixed", outer=("layer", "kv", "page"), inner="NHD", num_pages=8192,
                 num_layers=32, num_kv=2, page_size=64, num_heads=8, head_dim=128,
                 dtype_bytes=2, pages_per_request=256, seed=105,
                 description="bf16 NHD pool [32L][2][8192 pages][64 tok][8 heads][128]; 128 "
                             "alternating backup/restore requests of 256 pages, 4 in flight"),
    # not one of the five: the Llama-shaped pool at one token per page, whose
    # 16,384-token request names 16,384 pages of 2 KiB pieces
    "token_pages": _wl(name="token_pages", outer=("layer", "kv", "page"), inner="NHD",
                       num_pages=131072, num_layers=32, num_kv=2, page_size=1, num_heads=8,
                       head_dim=128, dtype_bytes=2, pages_per_request=16384, seed=106,
                       description="Llama-3-8B-shaped bf16 NHD pool at one token per page "
                                   "[32L][2][131072 pages][1 tok][8 heads][128]; one 16384-token "
                                   "request = 16384 fragmented pages"),
}


def request_pair(w: Workload, r: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """(source pages, destination pages) of request r: disjoint, random and
    fragmented, drawn from one seeded permutation of the pool's pages."""
    from . import page_perm
    perm = page_perm(w.seed, w.num_pages)
    n = w.pages_per_request
    if w.name == "mla_fp8":
        # four requests: sources from the first 256 permuted pages, destinations
        # from the next 256
        return perm[n * r:n * (r + 1)].copy(), perm[256 + n * r:256 + n * (r + 1)].copy()
    return perm[:n].copy(), perm[n:2 * n].copy()


def mixed_schedule(w: Workload, num_requests: int = 128):
    """The alternating miss/hit schedule: request k even backs up 256 pages
    chosen from the resident half of the pool; k odd restores a primed host
    slot into one of 16 disjoint 256-page destination sets."""
    from . import page_perm
    perm = page_perm(w.seed, w.num_pages)
    half = w.num_pages // 2
    resident = perm[:half]
    dst_sets = perm[half:].reshape(-1, w.pages_per_request)
    rng = np.random.default_rng(w.seed + 7)
    sched = []
    for k in range(num_requests):
        if k % 2 == 0:
            sched.append(("backup", rng.choice(resident, w.pages_per_request,
                                               replace=False).astype(np.int32)))
        else:
            sched.append(("restore", dst_sets[((k - 1) // 2) % len(dst_sets)].astype(np.int32)))
    return sched
