"""Planted mistakes in the CPU oracle must be caught by its pins.

Each case copies oracle/swa_oracle.c, applies one plausible mistake (a dropped
term, a wrong sign or index, a transposed operand, a wrong ring rule), builds
the copy with gcc into a temporary directory and runs every pin in
tests/oracle_pins.py against it.  The test passes when at least one pin fails
for every mutation; the real oracle is never modified.
"""
import pytest

import oracle
from tests import oracle_pins

MUTATIONS = {
    "drop_scale": ("s[t] = scale * dot;", "s[t] = dot;"),
    "band_right_exclusive": ("for (int64_t t = -wl; t <= wr; t++) {",
                             "for (int64_t t = -wl; t < wr; t++) {"),
    "band_left_inclusive_extra": ("for (int64_t t = -wl; t <= wr; t++) {",
                                  "for (int64_t t = -wl - 1; t <= wr; t++) {"),
    "dilation_sign": ("int64_t j = i + t * dil;", "int64_t j = i - t * dil;"),
    "dilation_ignored": ("int64_t j = i + t * dil;", "int64_t j = i + t;"),
    "kv_head_modulo": ("int64_t kh = h / group;\n            int64_t nk",
                       "int64_t kh = h % Hkv;\n            int64_t nk"),
    "globals_not_deduplicated": ("if (m == 0 || idx[t] != idx[m - 1]) idx[m++] = idx[t];",
                                 "idx[m++] = idx[t];"),
    "global_column_ignores_causal": ("if (!causal || G[t] <= i) idx[n++] = G[t];",
                                     "idx[n++] = G[t];"),
    "global_row_not_full": ("if (is_member(G, nG, i)) {", "if (0) {"),
    "global_row_ignores_causal": ("if (!causal || j <= i) idx[n++] = j;", "idx[n++] = j;"),
    "lse_without_max": ("*lse = M + log(L);", "*lse = log(L);"),
    "softmax_sign": ("double p = exp(s[t] - M);", "double p = exp(M - s[t]);"),
    "no_normalisation": ("for (int64_t c = 0; c < D; c++) out[c] /= L;", ""),
    "value_reads_key": ("out[c] += p * load_elem(v, dtype, vo + c);",
                        "out[c] += p * load_elem(k, dtype, vo + c);"),
    "query_layout_transposed": ("int64_t qoff = ((b * N + i) * Hq + h) * D;",
                                "int64_t qoff = ((b * Hq + h) * N + i) * D;"),
    "bf16_widening": ("(uint32_t)((const uint16_t*)base)[idx] << 16;",
                      "(uint32_t)((const uint16_t*)base)[idx] << 15;"),
    "ring_order_forward": ("keys[a] = ((ring_head[b] - 1 - a) % W + W) % W;",
                           "keys[a] = ((ring_head[b] + a) % W + W) % W;"),
    "ring_head_not_advanced": ("ring_head[b] = (slot + 1) % W;", "ring_head[b] = slot;"),
    "ring_writes_wrong_slot": ("int64_t slot = ring_head[b];",
                               "int64_t slot = (ring_head[b] + 1) % W;"),
    "cache_len_uncapped": ("cache_len[b] = cache_len[b] + 1 < W ? cache_len[b] + 1 : W;",
                           "cache_len[b] = cache_len[b] + 1;"),
    "decode_kv_head_modulo": ("int64_t b = bh / Hq, h = bh % Hq, kh = h / group;",
                              "int64_t b = bh / Hq, h = bh % Hq, kh = h % Hkv;"),
    "cached_age_limit_off_by_one": ("int64_t a_max = wl - 1 - t;", "int64_t a_max = wl - t;"),
    "cached_ring_slot_newest_missed": (
        "int64_t slot = ((ring_head[b] - 1 - a) % W + W) % W;\n                int64_t base",
        "int64_t slot = ((ring_head[b] - a) % W + W) % W;\n                int64_t base"),
    "cached_chunk_window_short": ("for (int64_t j = t - wl > 0 ? t - wl : 0; j <= t; j++)",
                                  "for (int64_t j = t - wl + 1 > 0 ? t - wl + 1 : 0; j <= t; j++)"),
    "cached_ring_ignores_len": ("if (a_max > cache_len[b] - 1) a_max = cache_len[b] - 1;",
                                "if (a_max > W - 1) a_max = W - 1;"),
    "cached_kv_head_modulo": ("b = row / (Hq * n), kh = h / group;",
                              "b = row / (Hq * n), kh = h % Hkv;"),
    "chunk_survivors_from_head": ("int64_t slot = (ring_head[b] + t) % W;",
                                  "int64_t slot = (ring_head[b] + t - first) % W;"),
    "chunk_head_advance_capped": ("ring_head[b] = (ring_head[b] + n) % W;",
                                  "ring_head[b] = (ring_head[b] + (n < W ? n : W)) % W;"),
    "chunk_len_uncapped": ("cache_len[b] = cache_len[b] + n < W ? cache_len[b] + n : W;",
                           "cache_len[b] = cache_len[b] + n;"),
    "sinks_skipped": ("for (int64_t t = 0; t < n_sink; t++) { /* the pinned entries */",
                      "for (int64_t t = 1; t < n_sink; t++) { /* the pinned entries */"),
    "sinks_kv_head_modulo": ("kh = (bh % Hq) / group;", "kh = (bh % Hq) % Hkv;"),
    "sinks_ring_oldest_dropped": ("for (int64_t a = 0; a < cache_len[b]; a++) { /* the valid",
                                  "for (int64_t a = 0; a + 1 < cache_len[b]; a++) { /* the valid"),
    "paged_write_slot": ("int64_t di = ((page * Hkv + h) * P + pos % P) * D + c;",
                         "int64_t di = ((page * Hkv + h) * P + (pos + 1) % P) * D + c;"),
    "paged_read_wrong_block": ("block_table[bb * nb + (pos / P) % nb];",
                               "block_table[bb * nb + (pos / P + 1) % nb];"),
    "paged_window_short": ("pos = seq_len[bb] > W ? seq_len[bb] - W : 0;",
                           "pos = seq_len[bb] > W ? seq_len[bb] - W + 1 : 0;"),
    "paged_count_not_advanced": ("        seq_len[b] += n;", "        seq_len[b] += n - (n > 1);"),
    "bwd_drop_row_term": ("const double ds = p[t] * (dp[t] - rowdot);",
                          "const double ds = p[t] * dp[t];"),
    "bwd_dq_no_scale": ("dq[qo + c] += scale * ds * load_elem(k, dtype, ko + c);",
                        "dq[qo + c] += ds * load_elem(k, dtype, ko + c);"),
    "bwd_dv_uses_ds": ("dv[ko + c] += p[t] * load_elem(dout, dtype, qo + c);",
                       "dv[ko + c] += ds * load_elem(dout, dtype, qo + c);"),
    "bwd_dk_uses_k": ("dk[ko + c] += scale * ds * load_elem(q, dtype, qo + c);",
                      "dk[ko + c] += scale * ds * load_elem(k, dtype, ko + c);"),
    "bwd_dp_uses_k": ("d += load_elem(dout, dtype, qo + c) * load_elem(v, dtype, vo + c);",
                      "d += load_elem(dout, dtype, qo + c) * load_elem(k, dtype, vo + c);"),
    "bwd_rows_drop_row_term": ("const double dsq = p[t] * (dp[t] - rowdot);",
                               "const double dsq = p[t] * dp[t];"),
    "bwd_keys_dv_uses_ds": ("dv_l[c] += p[t] * load_elem(dout, dtype, qo + c);",
                            "dv_l[c] += dsk * load_elem(dout, dtype, qo + c);"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle._SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, source, tmp_path):
    old, new = MUTATIONS[name]
    assert source.count(old) == 1, f"mutation anchor for {name} not unique or missing"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib = oracle.build(force=True, src=str(src), out=str(tmp_path / "libmutant.so"))
    orc = oracle.OracleLib(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"no pin catches mutation {name}"
