"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle source (a wrong shift or
constant, wrong digest bits, a reversed tie-break, an inverted comparison, a
dropped write, an off-by-one), builds the copy with the host compiler and runs
the pin suite (tests/test_oracle.py) against it in a subprocess; the suite
must fail. Nothing here touches a GPU.
"""

import os
import pathlib
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = pathlib.Path(__file__).resolve().parent.parent
SOURCE = (ROOT / "oracle" / "hkv_oracle.cpp").read_text()

MUTANTS = {
    "fmix64_shift": ("  k ^= k >> 33;\n  k *= 0xff51afd7ed558ccdull;", "  k ^= k >> 31;\n  k *= 0xff51afd7ed558ccdull;"),
    "fmix64_constant": ("0xc4ceb9fe1a85ec53ull", "0xc4ceb9fe1a85ec55ull"),
    "digest_bits_31_24": ("return static_cast<uint8_t>((h >> 32) & 0xFF);", "return static_cast<uint8_t>((h >> 24) & 0xFF);"),
    "bucket_from_high_bits": ("r.b1 = h1 % t.buckets;", "r.b1 = (h1 >> 32) % t.buckets;"),
    "second_hash_equals_first": ("fmix64(k ^ kSecondHashSalt) % t.buckets", "fmix64(k) % t.buckets"),
    "tie_break_larger_key": ("return s1 < s2 || (s1 == s2 && k1 < k2);", "return s1 < s2 || (s1 == s2 && k1 > k2);"),
    "admission_inverted": ("if (!rank_below(t.score[p], t.key[p], sc, k)) {",
                           "if (rank_below(t.score[p], t.key[p], sc, k)) {"),
    "admission_by_score_only": ("if (!rank_below(t.score[p], t.key[p], sc, k)) {",
                                "if (sc < t.score[p]) {"),
    "victim_highest": ("if (rank_below(t.score[p], t.key[p], t.score[q], t.key[q])) m = s;",
                       "if (rank_below(t.score[q], t.key[q], t.score[p], t.key[p])) m = s;"),
    "d1_more_occupied": ("b = (o1 <= o2) ? r.b1 : r.b2;", "b = (o1 >= o2) ? r.b1 : r.b2;"),
    "d2_higher_minimum": ("if (rank_below(t.score[p2], t.key[p2], t.score[p1], t.key[p1])) {",
                          "if (rank_below(t.score[p1], t.key[p1], t.score[p2], t.key[p2])) {"),
    "first_empty_is_last": ("for (int s = 0; s < kSlots; ++s)\n    if (t.key[pos_of(b, s)] == kEmptyKey) return s;",
                            "for (int s = kSlots - 1; s >= 0; --s)\n    if (t.key[pos_of(b, s)] == kEmptyKey) return s;"),
    "update_drops_score": ("    const uint64_t p = pos_of(b, s);\n    t.score[p] = sc;\n    write_payload(t, p, v, tag);\n    return kUpdated;",
                           "    const uint64_t p = pos_of(b, s);\n    write_payload(t, p, v, tag);\n    return kUpdated;"),
    "find_skips_second_bucket": ("  if (t.dual && r.b2 != r.b1) {\n    if (count) ++t.probes;",
                                 "  if (false) {\n    if (count) ++t.probes;"),
    "assign_inserts_scores_of_absent": ("if (is_reserved(k) || !locate(t, k, route(t, k), &b, &s, false)) continue;\n    const uint64_t p = pos_of(b, s);\n    if (scores) t.score[p] = scores[i];",
                                        "if (is_reserved(k)) continue;\n    if (!locate(t, k, route(t, k), &b, &s, false)) { b = route(t, k).b1; s = 0; }\n    const uint64_t p = pos_of(b, s);\n    if (scores) t.score[p] = scores[i];"),
    "export_off_by_one": ("for (uint64_t p = offset; p < end; ++p) {", "for (uint64_t p = offset; p + 1 < end; ++p) {"),
    "find_pos_next_slot": ("if (pos_out) pos_out[i] = hit ? pos_of(b, s) : ~0ull;",
                           "if (pos_out) pos_out[i] = hit ? pos_of(b, s) + 1 : ~0ull;"),
    "evict_output_drops_rejected": ("    if (gone) record_offered(t, k, v, tag, sc, gone);\n    return kRejected;",
                                    "    return kRejected;"),
    "evict_output_reports_newcomer": ("  if (gone) record_resident(t, p, gone);", "  if (gone) record_offered(t, k, v, tag, sc, gone);"),
    # one pass in input order: a resident key can be evicted before its own
    # update, then comes back as a fresh insert
    "evict_in_input_order": ("    if (!res[i]) continue;\n    const float* v = t.tag_mode ? nullptr : values + i * t.dim;\n"
                             "    upsert_one(t, keys[i], v, t.tag_mode ? tags[i] : 0, scores[i]);\n  }\n  uint64_t m = 0;\n"
                             "  for (uint64_t i = 0; i < n; ++i) {\n    if (res[i] || is_reserved(keys[i])) continue;",
                             "    continue;\n  }\n  uint64_t m = 0;\n"
                             "  for (uint64_t i = 0; i < n; ++i) {\n    if (is_reserved(keys[i])) continue;"),
    # victim picked by score alone: the first minimum-score slot, whatever its key
    "victim_by_score_only": ("if (rank_below(t.score[p], t.key[p], t.score[q], t.key[q])) m = s;",
                             "if (t.score[p] < t.score[q]) m = s;"),
    # bucket index by mask: equal to the modulo only when B is a power of two
    "bucket_by_mask": ("r.b1 = h1 % t.buckets;", "r.b1 = h1 & (t.buckets - 1);"),
    "assign_drops_rows": ("    } else if (values) {\n      for (uint32_t c = 0; c < t.dim; ++c) t.value[p * t.dim + c] = values[i * t.dim + c];",
                          "    } else if (false) {\n      for (uint32_t c = 0; c < t.dim; ++c) t.value[p * t.dim + c] = values[i * t.dim + c];"),
    "first_empty_skips_slot0": ("for (int s = 0; s < kSlots; ++s)\n    if (t.key[pos_of(b, s)] == kEmptyKey) return s;",
                                "for (int s = 1; s < kSlots; ++s)\n    if (t.key[pos_of(b, s)] == kEmptyKey) return s;"),
    "find_or_insert_keeps_score": ("    t.score[p] = scores[i];\n    if (t.tag_mode) {\n      tags_inout[i] = t.tag[p];",
                                   "    if (t.tag_mode) {\n      tags_inout[i] = t.tag[p];"),
}


def build_mutant(name, old, new, workdir):
    assert SOURCE.count(old) >= 1, f"mutation anchor of {name} not found"
    src = pathlib.Path(workdir) / f"{name}.cpp"
    src.write_text(SOURCE.replace(old, new, 1))
    lib = pathlib.Path(workdir) / f"{name}.so"
    subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-o", str(lib), str(src)], check=True,
                   capture_output=True)
    return lib


def run_pins(lib):
    env = dict(os.environ, HKV_ORACLE_LIB=str(lib), OMP_NUM_THREADS="1")
    return subprocess.run([sys.executable, "-m", "pytest", str(ROOT / "tests" / "test_oracle.py"), "-x", "-q",
                           "-p", "no:cacheprovider", "-m", "not gpu"], env=env, cwd=str(ROOT),
                          capture_output=True, text=True, timeout=900)


def test_pin_suite_catches_every_planted_mistake(tmp_path):
    libs = {name: build_mutant(name, old, new, tmp_path) for name, (old, new) in MUTANTS.items()}
    libs["control"] = build_mutant("control", "int first_empty(", "int first_empty(", tmp_path)
    workers = max(1, min(8, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = dict(zip(libs, ex.map(run_pins, libs.values())))
    control = results.pop("control")
    assert control.returncode == 0, "unmutated copy fails its pins:\n" + control.stdout[-3000:]
    survivors = [name for name, r in results.items() if r.returncode == 0]
    caught_by = {name: next((l.split("::")[1].split(" ")[0] for l in r.stdout.splitlines()
                             if l.startswith("FAILED")), f"the suite ending with status {r.returncode}")
                 for name, r in results.items()}
    print("\n".join(f"{name:34s} caught by {caught_by[name]}" for name in sorted(results)))
    assert not survivors, f"mistakes no pin catches: {survivors}"
