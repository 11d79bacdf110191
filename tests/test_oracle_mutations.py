"""The pins catch plausible mistakes in the oracle.

Each case plants one mistake (one or more consistent edits) in a copy of oracle/hkvref.c (on the CPU), builds
it, points the oracle wrapper at it, and runs the pins of
test_oracle_pins.py until one fails.  A mutant that passes every pin would
mean the pins do not fix that part of the oracle.
"""
import ctypes
import os
import subprocess
import sys

import pytest

import oracle
from tests import golden_io
from tests import test_codec as codec
from tests import test_keys as keys
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "hkvref.c")

# name -> (original text, planted mistake)
MUTANTS = {
    "slab_base_ignores_num_blocks": (
        "lay->pool_offset[l] = (int64_t)lay->index_in_group[l] * lay->num_blocks * p;",
        "lay->pool_offset[l] = (int64_t)lay->index_in_group[l] * p;"),
    "path_b_offset_not_a_prefix_sum": (
        "                lay->pool_offset[l] = byte_offset;\n"
        "                byte_offset += lay->page[l];",
        "                byte_offset += lay->page[l];\n"
        "                lay->pool_offset[l] = byte_offset - lay->page[0];"),
    "object_block_offset_uses_stride": (
        "uint8_t* dst = obj + lay->obj_offset[l] + j * lay->obj_page[l];",
        "uint8_t* dst = obj + lay->obj_offset[l] + j * lay->stride[l] % 64;"),
    "block_table_index_transposed": (
        "return ids[((int64_t)c * lay->n_kv_groups + g) * lay->k + j];",
        "return ids[((int64_t)c * lay->k + j) * lay->n_kv_groups + g];"),
    "smaller_kda_groups_first": (
        "if (filled == base + (g < rem ? 1 : 0)) {",
        "if (filled == base + (g >= m - rem ? 1 : 0)) {"),
    "cover_rule_strict": (
        "while (n * tok_bytes < kda_page)",
        "while (n * tok_bytes <= kda_page)"),
    "retrieve_writes_padding": (
        "                       (size_t)valid_bytes(lay, l, j, t));",
        "                       (size_t)valid_bytes(lay, l, j, t));\n"
        "                memset(pool + lay->pool_offset[l] + id * lay->stride[l] + lay->page[l], 0,"
        " (size_t)(lay->reserved[l] - lay->page[l]));"),
    "retrieve_ignores_partial_rows": (
        "                       (size_t)valid_bytes(lay, l, j, t));",
        "                       (size_t)lay->page[l]);"),
    "null_page_not_zeroed_on_store": (
        "                    memset(dst, 0, (size_t)lay->obj_page[l]);\n                    continue;",
        "                    continue;"),
    "partial_rows_counted_from_block_start": (
        "    rows = t - j * lay->n;",
        "    rows = t;"),
    "object_groups_swapped": (
        "lay->obj_group[l] = lay->is_mla[l] ? 1 : 0;",
        "lay->obj_group[l] = lay->is_mla[l] ? 0 : 1;"),
    "chunk_rounds_down": (
        "    while (c < chunk_min)\n        c += n;",
        "    while (c + n <= chunk_min)\n        c += n;"),
    "stride_sums_groups": (
        "            if (byte_offset > stride)\n                stride = byte_offset;",
        "            stride += byte_offset;"),
    "one_slab_too_few": (
        "if (lay->index_in_group[l] + 1 > slabs)",
        "if (lay->index_in_group[l] > slabs)"),
    "last_block_of_chunk_skipped": (
        "            for (j = 0; j < lay->k; j++) {\n"
        "                int64_t id = block_id(lay, block_ids, c, lay->kv_group[l], j);\n"
        "                uint8_t* dst",
        "            for (j = 0; j < lay->k - (lay->k > 1); j++) {\n"
        "                int64_t id = block_id(lay, block_ids, c, lay->kv_group[l], j);\n"
        "                uint8_t* dst"),
    "chain_drops_the_parent_hash": (
        "H[i] = ref_mix64((H[i - 1] ^ content) + HKVREF_GAMMA);",
        "H[i] = ref_mix64(content + HKVREF_GAMMA);"),
    "chunk_hash_one_fine_block_early": (
        "uint64_t prefix = H[(c + 1) * lay->c / h];",
        "uint64_t prefix = H[(c + 1) * lay->c / h - 1];"),
    "block_content_ignores_token_order": (
        "content = ref_mix64(content ^ (t | ((uint64_t)j << 32)));",
        "content += ref_mix64(t);"),
    "fingerprint_without_block_size": (
        "    words[n++] = (uint64_t)lay->n;\n",
        ""),
    "key_ignores_object_group": (
        "ref_mix64(base ^ (prefix + (uint64_t)(o + 1) * HKVREF_GAMMA));",
        "ref_mix64(base ^ (prefix + HKVREF_GAMMA));"),
    "key_ignores_parallel_config": (
        "base = ref_mix64(hkvref_fingerprint(lay) ^ rank_tag);",
        "base = ref_mix64(hkvref_fingerprint(lay));"),
    "conv_state_keeps_kernel_columns": (
        "int64_t conv = (int64_t)conv_dim * (conv_kernel - 1) * conv_bytes;",
        "int64_t conv = (int64_t)conv_dim * conv_kernel * conv_bytes;"),
    # the INT8 codec of KDA recurrent states
    "codec_scale_over_128": (
        "    s = amax / 127.0f;",
        "    s = amax / 128.0f;"),
    "codec_truncates": (
        "        v = rintf(x[i] / s);",
        "        v = truncf(x[i] / s);"),
    "codec_rounds_half_away": (
        "        v = rintf(x[i] / s);",
        "        v = roundf(x[i] / s);"),
    "codec_absmax_sees_non_finite": (
        "        if (isfinite(x[i]) && fabsf(x[i]) > amax)",
        "        if (fabsf(x[i]) > amax && !isnan(x[i]))"),
    "codec_encodes_non_finite": (
        "        if (s == 0.0f || !isfinite(x[i])) {",
        "        if (s == 0.0f) {"),
    "codec_absmax_signed": (
        "        if (isfinite(x[i]) && fabsf(x[i]) > amax)\n            amax = fabsf(x[i]);",
        "        if (isfinite(x[i]) && x[i] > amax)\n            amax = x[i];"),
    "codec_scales_before_codes": [
        ("    uint8_t* codes = out + lay->conv_part;\n    uint8_t* scales = codes + rows * d;",
         "    uint8_t* scales = out + lay->conv_part;\n    uint8_t* codes = scales + rows * 4;"),
        ("    const uint8_t* codes = in + lay->conv_part;\n"
         "    const uint8_t* scales = codes + rows * d;",
         "    const uint8_t* scales = in + lay->conv_part;\n"
         "    const uint8_t* codes = scales + rows * 4;")],
    "codec_state_before_conv": [
        ("memcpy(x, page + lay->conv_part + r * d * 4, (size_t)d * 4);",
         "memcpy(x, page + r * d * 4, (size_t)d * 4);"),
        ("memcpy(page + lay->conv_part + r * d * 4, x, (size_t)d * 4);",
         "memcpy(page + r * d * 4, x, (size_t)d * 4);"),
        ("    memcpy(out, page, (size_t)lay->conv_part);",
         "    memcpy(out, page + rows * d * 4, (size_t)lay->conv_part);"),
        ("    memcpy(page, in, (size_t)lay->conv_part);",
         "    memcpy(page + rows * d * 4, in, (size_t)lay->conv_part);")],
    "codec_decode_keeps_nan_payloads": (
        "        if (isnan(x[i]))\n            memcpy(&x[i], &qnan, 4);",
        ""),
    "codec_decode_clamps_codes": (
        "        x[i] = (float)q[i] * scale;",
        "        x[i] = (float)(q[i] < -127 ? -127 : q[i]) * scale;"),
    "codec_drops_conv_part": (
        "    memcpy(out, page, (size_t)lay->conv_part);",
        "    memset(out, 0, (size_t)lay->conv_part);"),
    "codec_one_scale_per_page": (
        "        memcpy(&sc, scales + r * 4, 4);",
        "        memcpy(&sc, scales, 4);"),
    "codec_rows_per_head_only": (
        "            lay->obj_page[l] = lay->conv_part + rows * head_dim + rows * 4;",
        "            lay->obj_page[l] = lay->conv_part + heads * head_dim + heads * 4;"),
    "codec_accepts_any_head_dim": (
        "        (state_bytes != 4 || (head_dim != 16 && head_dim != 32 && head_dim != 64 &&\n"
        "                              head_dim != 128 && head_dim != 256) ||",
        "        (state_bytes != 4 ||"),
}


def pin_checks():
    """The pins, cheapest first (the property test last)."""
    out = []
    for row in golden_io.rows("block_sizes.txt"):
        out.append(lambda r=row: pins.test_unified_block_size_matches_pages(r))
    out += [pins.test_block_size_cover_is_inclusive, pins.test_tiny_block_size_and_tp_scaling,
            pins.test_state_dtype_reading_is_the_only_one_matching_both_pages]
    for row in golden_io.rows("chunk_negotiation.txt"):
        out.append(lambda r=row: pins.test_chunk_negotiation(r))
    out.append(pins.test_chunk_is_smallest_multiple)
    for row in golden_io.rows("batch_budget.txt"):
        out.append(lambda r=row: pins.test_batch_budget(r))
    out += [pins.test_k3_groups_and_slabs_match_flat_kv,
            pins.test_groups_hold_one_layer_type_and_are_contiguous,
            pins.test_config_closed_forms]
    for name in ("tiny", "kl_tp2", "kl_tp1", "k3_tp8", "long_ctx"):
        out.append(lambda n=name: pins.test_config_layouts_structure(n))
    out.append(pins.test_mla_object_is_chunk_tokens_by_latent_array)
    for case in pins.BRUTE:
        out.append(lambda c=case: pins.test_brute_force_every_injective_assignment(c))
    out += [pins.test_id_range_and_alias_errors, pins.test_whole_chunks_and_no_nulls_reduce_to_plain_copies,
            pins.test_random_layouts_store_retrieve_properties, pins.test_null_ids_and_partial_chunks]
    out += [codec.test_object_page_is_conv_then_codes_then_scales,
            codec.test_ties_round_half_to_even, codec.test_zero_and_non_finite_rows,
            codec.test_power_of_two_lattice_round_trips_exactly, codec.test_denormal_rows,
            codec.test_null_pages_and_mla_pages_under_the_codec,
            codec.test_codec_changes_the_fingerprint_and_rejects_unsupported_shapes,
            codec.test_decode_of_objects_the_encoder_did_not_write,
            codec.test_round_off_bound_and_extremal_code]
    out += [keys.test_fine_hash_covers_exactly_its_prefix,
            keys.test_chunk_hash_is_its_last_fine_block_hash,
            keys.test_chain_continues_from_a_parent, keys.test_hash_depends_on_token_order_within_a_block,
            keys.test_shared_prefix_shares_keys, keys.test_keys_separate_groups_ranks_and_roots,
            keys.test_fingerprint_tracks_object_format_only, keys.test_bad_arguments]
    return out


def run_pins_against(lib_path: str) -> int:
    """Runs the pins against the oracle build at lib_path; returns 1 if one
    fails, 0 if all pass (used in a child process)."""
    oracle._lib = oracle.bind(ctypes.CDLL(lib_path))
    for check in pin_checks():
        try:
            check()
        except (AssertionError, oracle.OracleError, pytest.fail.Exception):
            return 1
    return 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    edits = MUTANTS[name]
    src = open(SRC).read()
    for original, planted in (edits if isinstance(edits, list) else [edits]):
        assert src.count(original) == 1, "the mutation site moved; update the test"
        src = src.replace(original, planted)
    mutant = tmp_path / "hkvref.c"
    mutant.write_text(src)
    (tmp_path / "hkvref.h").write_text(open(SRC[:-1] + "h").read())
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-w", "-fPIC", "-shared", str(mutant), "-o", str(so), "-lm"],
                   check=True)
    # a child process: a mutant may also crash (e.g. divide by zero), which
    # counts as caught
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; from tests.test_oracle_mutations import run_pins_against; "
            f"sys.exit(10 + run_pins_against({str(so)!r}))")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 10, f"no pin fails with the planted mistake '{name}'"
    assert r.returncode == 11 or r.returncode < 0 or r.returncode > 11, r.stderr[-2000:]
