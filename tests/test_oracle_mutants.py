"""The oracle's pins have teeth (CPU only).

Copies of oracle/kvx_oracle.c with one planted mistake each - a transposed
index, a dropped term, a swapped axis, a wrong bound, an off-by-one step, a
wrong comparison - are compiled next to an unchanged copy, and the pin
tests (tests/test_oracle_pins.py) are run against each through
KVX_ORACLE_LIB. The unchanged copy passes them; every mutant fails at least
one. Every planted mistake keeps the oracle's memory accesses inside its
buffers, so a mutant fails by a pin's assertion, never by a crash.

The same for the host tier's model (oracle/tier_model.py): each mutant
replaces the model for a run of the hand-worked tier scenarios of
tests/test_tier_cpu.py (their model variants), and fails one of them."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvx_oracle.c")

# (name, function the change is confined to or None, text, replacement)
MUTANTS = [
    ("nhd_rows_head_major", "kvxo_row_in_piece",
     "return t * L->num_heads + h;", "return h * L->page_size + t;"),
    ("hnd_rows_token_major", "kvxo_row_in_piece",
     "return h * L->page_size + t;", "return t * L->num_heads + h;"),
    ("byte_offset_dropped", "kvxo_piece_start",
     "return L->byte_offset + kvxo_piece_index", "return kvxo_piece_index"),
    ("outer_order_ignored", "kvxo_piece_index", "int ax = L->outer[k];", "int ax = k;"),
    ("outer_order_reversed", "kvxo_piece_index", "int ax = L->outer[k];",
     "int ax = L->outer[2 - k];"),
    ("row_bytes_without_dtype", "kvxo_row_bytes", "return L->head_dim * L->dtype_bytes;",
     "return L->head_dim;"),
    ("host_layer_kv_swapped", "kvxo_host_row", "(((l * L->num_kv + c) * n + i)",
     "(((c * L->num_layers + l) * n + i)"),
    ("host_token_head_swapped", "kvxo_host_row",
     "* L->page_size + t) * L->num_heads + h;", "* L->num_heads + h) * L->page_size + t;"),
    ("host_slots_reversed", "kvxo_host_row", "* n + i) * L->page_size",
     "* n + (n - 1 - i)) * L->page_size"),
    ("backup_kv_always_k", "kvxo_backup", "kvxo_piece_start(L, ids[i], l, c)",
     "kvxo_piece_start(L, ids[i], l, 0)"),
    ("restore_from_layer_0", "kvxo_restore", "for (int64_t l = l0; l < l1; l++)",
     "for (int64_t l = 0; l < l1; l++)"),
    ("restore_last_layer_dropped", "kvxo_restore", "for (int64_t l = l0; l < l1; l++)",
     "for (int64_t l = l0; l + 1 < l1; l++)"),
    ("backup_slots_ignored", "kvxo_backup_slots", "slots[i], t, h)", "i, t, h)"),
    ("restore_slots_all_slot_0", "kvxo_restore_slots", "slots[i], t, h)", "slots[0], t, h)"),
    ("nhd_to_hnd_is_a_copy", "kvxo_nhd_to_hnd", "out[(h * T + t) * row_bytes + b]",
     "out[(t * H + h) * row_bytes + b]"),
    ("hnd_to_nhd_is_a_copy", "kvxo_hnd_to_nhd", "in[(h * T + t) * row_bytes + b]",
     "in[(t * H + h) * row_bytes + b]"),
    ("ready_prefix_is_max", "kvxo_ready_prefix", "(int64_t)counts[s] < m",
     "(int64_t)counts[s] > m"),
    ("ready_prefix_skips_last", "kvxo_ready_prefix", "s < num_slots", "s + 1 < num_slots"),
    ("ready_publish_overwrites", "kvxo_ready_publish", "counts[s] = counts[s] + n;", "counts[s] = n;"),
    ("ready_publish_ignores_l0", "kvxo_ready_publish", "for (int64_t l = l0; l < l1; l++)",
     "for (int64_t l = 0; l < l1; l++)"),
    ("ready_publish_ignores_slot_base", "kvxo_ready_publish", "int64_t s = slot_base + l;",
     "int64_t s = l;"),
    ("splitmix_shift_28", "kvxo_splitmix64_next", "(z >> 27)", "(z >> 28)"),
    ("generator_word_off_by_one", "kvxo_gen_word", "seed + j * 0x9e3779b97f4a7c15ULL",
     "seed + (j + 1) * 0x9e3779b97f4a7c15ULL"),
    ("generator_big_endian", "gen_byte", "(8 * (a & 7))", "(8 * (7 - (a & 7)))"),
    ("check_backup_layer_kv_swapped", "kvxo_check_backup_gen",
     "int64_t c = lc % L->num_kv, l = lc / L->num_kv;",
     "int64_t l = lc % L->num_layers, c = lc / L->num_layers;"),
    ("check_roundtrip_ignores_l0", "kvxo_check_alloc_roundtrip",
     "coord[1] >= l0 && coord[1] < l1", "coord[1] < l1"),
    ("check_roundtrip_outer_reversed", "kvxo_check_alloc_roundtrip", "int ax = L->outer[k];",
     "int ax = L->outer[2 - k];"),
]


def function_span(src: str, name: str):
    """[start, end) of the definition of function `name` in src."""
    for head in (f" {name}(", f"*{name}("):
        k = src.find(head)
        while k >= 0:
            line_end = src.find("\n", k)
            body = src.find("\n{\n", k)
            semi = src.find(";", k)
            brace_same_line = src.find("{", k, line_end) if line_end >= 0 else -1
            if brace_same_line >= 0 or (body >= 0 and (semi < 0 or body < semi)):
                start = src.rfind("\n", 0, k) + 1
                end = src.find("\n}\n", k)
                if brace_same_line >= 0 and (end < 0 or src.find("}\n", k) < end):
                    end = src.find("}\n", k)
                return start, end + 2
            k = src.find(head, k + 1)
    raise AssertionError(f"no definition of {name}")


def mutate(src: str, func, old: str, new: str) -> str:
    a, b = function_span(src, func) if func else (0, len(src))
    seg = src[a:b]
    assert seg.count(old) == 1, f"{old!r} is not unique in {func}"
    return src[:a] + seg.replace(old, new) + src[b:]


def build(text: str, out_dir: str, name: str) -> str:
    c = os.path.join(out_dir, f"{name}.c")
    so = os.path.join(out_dir, f"lib{name}.so")
    with open(c, "w") as f:
        f.write(text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-o", so, c], check=True)
    return so


def run_pins(lib_path: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, KVX_ORACLE_LIB=lib_path)
    return subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests",
                                                                          "test_oracle_pins.py"),
                           "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


def test_mutants_are_distinct_and_apply(source):
    names = [m[0] for m in MUTANTS]
    assert len(set(names)) == len(names)
    for name, func, old, new in MUTANTS:
        assert mutate(source, func, old, new) != source, name


def test_unchanged_copy_passes_the_pins(source, tmp_path):
    r = run_pins(build(source, str(tmp_path), "control"))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,func,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_the_planted_mistake(source, tmp_path, name, func, old, new):
    r = run_pins(build(mutate(source, func, old, new), str(tmp_path), name))
    # 1: a pin's assertion failed (a crash would give a negative code)
    assert r.returncode == 1, f"{name}: pins returned {r.returncode}\n" + r.stdout[-1500:]
    assert " failed" in r.stdout


# ---------------------------------------------------------------------------
# the host tier's model
# ---------------------------------------------------------------------------
MODEL = os.path.join(ROOT, "oracle", "tier_model.py")

# (name, text, replacement) in oracle/tier_model.py
MODEL_MUTANTS = [
    ("evicts_most_recent", "s = min(cands, key=lambda t: self.slots[t].last)",
     "s = max(cands, key=lambda t: self.slots[t].last)"),
    ("evicts_pinned", "return x.state == RESIDENT and x.pins == 0 and not x.doomed",
     "return x.state == RESIDENT and not x.doomed"),
    ("highest_free_slot_first", "s = free[0]", "s = free[-1]"),
    ("lookup_leaves_recency", "self.slots[s].pins += 1\n            self.slots[s].last = self.tick()",
     "self.slots[s].pins += 1"),
    ("commit_leaves_recency", "self.slots[s].state = RESIDENT\n                self.slots[s].last = self.tick()",
     "self.slots[s].state = RESIDENT"),
    ("writing_entries_hit", "if s is None or self.slots[s].state != RESIDENT:", "if s is None:"),
    ("invalidate_ignores_pins", "if x.state == RESIDENT and x.pins == 0:", "if x.state == RESIDENT:"),
    ("named_keys_can_be_victims",
     "cands = [t for t in range(self.num_slots) if self.evictable(t) and t not in present]",
     "cands = [t for t in range(self.num_slots) if self.evictable(t)]"),
    ("doomed_slot_kept_after_release",
     "if self.slots[s].pins == 0 and self.slots[s].doomed:\n                self.slots[s] = Slot()",
     "if self.slots[s].pins == 0 and self.slots[s].doomed:\n                pass"),
    ("doomed_backup_committed", "if self.slots[s].doomed:\n                self.slots[s] = Slot()\n            else:",
     "if False:\n                self.slots[s] = Slot()\n            else:"),
    ("release_unchecked", "self.slots[s].pins < named.count(s)", "self.slots[s].pins < 0"),
]

RUN_MODEL = """
import importlib.util, sys
spec = importlib.util.spec_from_file_location("oracle.tier_model", sys.argv[1])
m = importlib.util.module_from_spec(spec)
sys.modules["oracle.tier_model"] = m
spec.loader.exec_module(m)
import pytest
sys.exit(pytest.main([sys.argv[2], "-q", "-x", "-p", "no:cacheprovider", "-k", "model and not runtime"]))
"""


def run_model_scenarios(model_path: str) -> subprocess.CompletedProcess:
    return subprocess.run([sys.executable, "-c", RUN_MODEL, model_path,
                           os.path.join(ROOT, "tests", "test_tier_cpu.py")],
                          cwd=ROOT, capture_output=True, text=True, timeout=300)


@pytest.fixture(scope="module")
def model_source():
    with open(MODEL) as f:
        return f.read()


def write_model(text: str, out_dir: str) -> str:
    path = os.path.join(out_dir, "tier_model.py")
    with open(path, "w") as f:
        f.write(text)
    return path


def test_unchanged_model_passes_the_scenarios(model_source, tmp_path):
    r = run_model_scenarios(write_model(model_source, str(tmp_path)))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert " passed" in r.stdout and "deselected" in r.stdout


@pytest.mark.parametrize("name,old,new", MODEL_MUTANTS, ids=[m[0] for m in MODEL_MUTANTS])
def test_scenarios_catch_the_planted_model_mistake(model_source, tmp_path, name, old, new):
    assert model_source.count(old) == 1, f"{name}: {old!r} is not unique"
    r = run_model_scenarios(write_model(model_source.replace(old, new), str(tmp_path)))
    assert r.returncode == 1, f"{name}: scenarios returned {r.returncode}\n" + r.stdout[-1500:]
