"""CPU checks of the seeded input module (shapes, sizes and page choices)."""
import numpy as np

import synth
from synth.workloads import WORKLOADS, mixed_schedule, request_pair


def test_payload_sizes():
    # per-request payload = layers * kv * pages * piece bytes
    assert WORKLOADS["tiny"].payload_bytes(8) == 131_072
    assert WORKLOADS["llama8b"].payload_bytes() == 2_147_483_648
    assert WORKLOADS["mla_fp8"].payload_bytes() == 575_668_224
    assert WORKLOADS["trtllm_hnd"].payload_bytes() == 2_147_483_648
    assert WORKLOADS["mixed"].payload_bytes() == 2_147_483_648
    assert WORKLOADS["llama8b"].pool_bytes == 16 * 2**30
    assert WORKLOADS["mixed"].pool_bytes == 64 * 2**30
    assert WORKLOADS["trtllm_hnd"].alloc_bytes == WORKLOADS["trtllm_hnd"].pool_bytes + 32 * 1024
    assert WORKLOADS["trtllm_hnd"].byte_offset == 12_288


def test_piece_sizes():
    assert WORKLOADS["tiny"].piece_bytes == 4096
    assert WORKLOADS["llama8b"].piece_bytes == 131_072
    assert WORKLOADS["mla_fp8"].piece_bytes == 147_456
    assert WORKLOADS["trtllm_hnd"].piece_bytes == 65_536
    assert WORKLOADS["trtllm_hnd"].tensor_shape() == [4096, 32, 2, 8 * 32 * 128]


def test_page_perm_is_permutation():
    p = synth.page_perm(102, 2048)
    assert p.dtype == np.int32
    assert np.array_equal(np.sort(p), np.arange(2048))
    assert np.array_equal(p, synth.page_perm(102, 2048))


def test_request_pairs_disjoint():
    for name, w in WORKLOADS.items():
        if name == "mixed":
            continue
        reqs = range(4) if name == "mla_fp8" else range(1)
        for r in reqs:
            s, d = request_pair(w, r)
            assert len(s) == len(d) == w.pages_per_request
            assert len(set(s.tolist()) | set(d.tolist())) == 2 * w.pages_per_request


def test_mixed_schedule_shape():
    w = WORKLOADS["mixed"]
    sched = mixed_schedule(w, 128)
    assert len(sched) == 128
    resident = set(synth.page_perm(w.seed, w.num_pages)[:4096].tolist())
    dst_pages = set()
    for k, (kind, ids) in enumerate(sched):
        assert kind == ("backup" if k % 2 == 0 else "restore")
        assert len(set(ids.tolist())) == 256
        if kind == "backup":
            assert set(ids.tolist()) <= resident
        else:
            dst_pages |= set(ids.tolist())
    assert not (dst_pages & resident)


def test_gen_bytes_unaligned_window():
    whole = synth.gen_bytes(5, 0, 64)
    assert np.array_equal(synth.gen_bytes(5, 3, 50), whole[3:53])
