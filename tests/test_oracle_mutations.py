"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

A pin that passes for a broken oracle pins nothing; every mutation below must
make at least one of the pins in test_oracle.py fail.
"""
import numpy as np
import pytest

import oracle
import oracle.codec as codec
import oracle.paged_attention as pa
from tests import test_oracle as pins


def _attention_gqa_modulo(q, K, V, scale, visible):
    nq, hq, d = q.shape
    hkv = K.shape[1]
    out = np.zeros((nq, hq, d))
    for h in range(hq):
        kvh = h % hkv  # wrong grouping
        s = scale * (q[:, h, :] @ K[:, kvh, :].T)
        s = np.where(np.arange(len(K))[None, :] < np.asarray(visible)[:, None], s, -np.inf)
        w = np.exp(s - s.max(1, keepdims=True))
        out[:, h, :] = (w / w.sum(1, keepdims=True)) @ V[:, kvh, :]
    return out


def _attention_no_scale(q, K, V, scale, visible):
    return pa.__dict__["_orig_attention_rows"](q, K, V, 1.0, visible)


def _attention_transposed_v(q, K, V, scale, visible):
    out = pa.__dict__["_orig_attention_rows"](q, K, V, scale, visible)
    return out[:, ::-1, :].copy()  # heads' outputs permuted (operand mix-up)


def _slot_off_by_one(row, pos, block_size=16):
    return int(row[pos // block_size]) * block_size + (pos + 1) % block_size


def _decode_excluding_current(q, k_pool, v_pool, bt, ctx, scale, k_scale=None, v_scale=None, codec=None):
    ctx = [max(int(n) - 1, 1) for n in ctx]
    return pa.__dict__["_orig_decode"](q, k_pool, v_pool, bt, ctx, scale, k_scale, v_scale, codec)


def _prefill_causal_off_by_one(q, k_pool, v_pool, qsl, seq_lens, bt, scale, k_scale=None, v_scale=None, codec=None):
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros_like(q)
    for s in range(len(seq_lens)):
        a, b = int(qsl[s]), int(qsl[s + 1])
        n = int(seq_lens[s])
        K = pa.gather_sequence(k_pool, bt[s], n, k_scale, codec)
        V = pa.gather_sequence(v_pool, bt[s], n, v_scale, codec)
        visible = [max(n - (b - a) + i, 1) for i in range(b - a)]  # misses its own key
        out[a:b] = pa.attention_rows(q[a:b], K, V, scale, visible)
    return out


def _gather_ignores_scale(pool, row, n, scales=None, codec=None):
    return pa.__dict__["_orig_gather"](pool, row, n, None, codec)


def _gather_wrong_block_order(pool, row, n, scales=None, codec=None):
    nb = -(-n // 16)
    row = list(row[:nb])[::-1] + list(row[nb:])
    return pa.__dict__["_orig_gather"](pool, row, n, scales, codec)


_E4M3_WRONG_BIAS = np.array([
    (-1.0 if c & 0x80 else 1.0) * ((1 + (c & 7) / 8) * 2.0 ** (((c >> 3) & 15) - 8) if (c >> 3) & 15
                                   else (c & 7) / 8 * 2.0 ** -7)
    for c in range(256)])


MUTATIONS = {
    "gqa_modulo": ("attention_rows", _attention_gqa_modulo,
                   [lambda: pins.test_decode_matches_sdpa(4, 2, 64)]),
    "scale_dropped": ("attention_rows", _attention_no_scale,
                      [lambda: pins.test_decode_matches_sdpa(4, 2, 64)]),
    "head_mixup": ("attention_rows", _attention_transposed_v,
                   [lambda: pins.test_decode_matches_sdpa(8, 1, 32)]),
    "slot_off_by_one": ("slot_for_position", _slot_off_by_one,
                        [pins.test_token_by_token_decode_equals_recompute]),
    "ctx_excludes_new_token": ("decode", _decode_excluding_current,
                               [pins.test_token_by_token_decode_equals_recompute]),
    "causal_off_by_one": ("prefill_chunk", _prefill_causal_off_by_one,
                          [pins.test_prefill_matches_sdpa_causal,
                           pins.test_chunked_prefill_mixed_batch_equals_recompute]),
    "scale_not_applied": ("gather_sequence", _gather_ignores_scale,
                          [pins.test_quantized_single_token_is_decoded_code_times_scale]),
    "block_order": ("gather_sequence", _gather_wrong_block_order,
                    [pins.test_token_by_token_decode_equals_recompute]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn, checks = MUTATIONS[name]
    monkeypatch.setitem(pa.__dict__, "_orig_attention_rows", pa.attention_rows)
    monkeypatch.setitem(pa.__dict__, "_orig_decode", pa.decode)
    monkeypatch.setitem(pa.__dict__, "_orig_gather", pa.gather_sequence)
    monkeypatch.setattr(pa, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    for check in checks:
        with pytest.raises(AssertionError):
            check()


def test_fp8_wrong_bias_is_caught(monkeypatch):
    monkeypatch.setattr(codec, "_E4M3_TABLE", _E4M3_WRONG_BIAS)
    with pytest.raises(AssertionError):
        pins.test_e4m3fn_decode_all_codes_match_torch()


# ---- quantise-on-write: plausible mistakes, each must fail a pin in test_oracle_quant ----
from tests import test_oracle_quant as qpins  # noqa: E402


def _qcw_variant(no_reencode=False, scale_from_new_only=False, trunc_int8=False,
                 reencode_short=False):
    def f(codes, scales, x_new, slot_mapping, kind):
        codes = np.array(codes, copy=True)
        scales = np.array(scales, dtype=np.float32, copy=True)
        x_new = np.asarray(x_new, dtype=np.float32)
        qmax = np.float32(448.0 if kind == "fp8" else 127.0)
        if kind == "fp8":
            encode, values = codec.e4m3fn_encode, codec.e4m3fn_decode
        else:
            rnd = np.trunc if trunc_int8 else np.rint
            encode = lambda y: np.clip(rnd(np.asarray(y, np.float64)), -127, 127).astype(np.int8)
            values = codec.int8_decode
        runs = {}
        for t, slot in enumerate(np.asarray(slot_mapping)):
            if slot >= 0:
                runs.setdefault(int(slot) // 16, []).append((int(slot) % 16, t))
        for b, rows in runs.items():
            off0 = min(o for o, _ in rows)
            for h in range(codes.shape[1]):
                s_old = scales[b, h] if off0 > 0 else np.float32(0.0)
                amax = np.float32(np.max(np.abs(np.stack([x_new[t, h] for _, t in rows]))))
                s_new = np.float32(amax / qmax) if scale_from_new_only else np.maximum(s_old, np.float32(amax / qmax))
                n_old = max(off0 - 1, 0) if reencode_short else off0
                if s_new != s_old and off0 > 0 and not no_reencode:
                    ratio = np.float32(s_old / s_new)
                    old = values(codes[b, h, :n_old]).astype(np.float32)
                    codes[b, h, :n_old] = encode(np.clip((old * ratio).astype(np.float32), -qmax, qmax))
                for o, t in rows:
                    y = np.clip((x_new[t, h] / s_new).astype(np.float32), -qmax, qmax) if s_new > 0 else 0 * x_new[t, h]
                    codes[b, h, o] = encode(y)
                scales[b, h] = s_new
        return codes, scales
    return f


QUANT_MUTATIONS = {
    "no_reencode_on_growth": (_qcw_variant(no_reencode=True),
                              [lambda: qpins.test_dequantised_values_within_rounding_bound("fp8")]),
    "scale_from_new_rows_only": (_qcw_variant(scale_from_new_only=True),
                                 [lambda: qpins.test_scale_is_running_amax_over_valid_rows("i8")]),
    "int8_truncates": (_qcw_variant(trunc_int8=True),
                       [lambda: qpins.test_stored_codes_are_the_nearest_codes("i8")]),
    "reencode_misses_a_row": (_qcw_variant(reencode_short=True),
                              [lambda: qpins.test_dequantised_values_within_rounding_bound("i8")]),
}


@pytest.mark.parametrize("name", sorted(QUANT_MUTATIONS))
def test_quant_write_mutation_is_caught(name, monkeypatch):
    fn, checks = QUANT_MUTATIONS[name]
    monkeypatch.setattr(oracle, "quantised_cache_write", fn)
    for check in checks:
        with pytest.raises(AssertionError):
            check()


def test_quant_write_variant_without_mutation_passes(monkeypatch):
    # the variant machinery itself, unmutated, agrees with the oracle's pins
    monkeypatch.setattr(oracle, "quantised_cache_write", _qcw_variant())
    qpins.test_dequantised_values_within_rounding_bound("fp8")
    qpins.test_scale_is_running_amax_over_valid_rows("i8")
    qpins.test_stored_codes_are_the_nearest_codes("i8")


def _swap_kv_crossed(dst, src, pairs):
    out = pa.__dict__["_orig_swap_blocks"](dst, src, pairs)
    return (out[1], out[0], out[2], out[3])


def _swap_without_scales(dst, src, pairs):
    out = pa.__dict__["_orig_swap_blocks"](dst, src, pairs)
    return (out[0], out[1], dst[2], dst[3])


def _swap_reversed_pairs(dst, src, pairs):
    p = np.asarray(pairs).reshape(-1, 2)[:, ::-1]
    n = min(len(dst[0]), len(src[0]))
    p = np.where(p < n, p, 0)
    return pa.__dict__["_orig_swap_blocks"](dst, src, p)


def _swap_next_block(dst, src, pairs):
    p = np.asarray(pairs).reshape(-1, 2).copy()
    p[:, 0] = (p[:, 0] + 1) % len(src[0])
    return pa.__dict__["_orig_swap_blocks"](dst, src, p)


SWAP_MUTATIONS = {
    "k_v_crossed": _swap_kv_crossed,
    "scales_left_behind": _swap_without_scales,
    "pairs_reversed": _swap_reversed_pairs,
    "source_off_by_one": _swap_next_block,
}


@pytest.mark.parametrize("name", sorted(SWAP_MUTATIONS))
def test_swap_mutation_is_caught(name, monkeypatch):
    from tests import test_oracle_swap as swap_pins
    monkeypatch.setitem(pa.__dict__, "_orig_swap_blocks", pa.swap_blocks)
    monkeypatch.setattr(oracle, "swap_blocks", SWAP_MUTATIONS[name])
    caught = False
    for test in (swap_pins.test_request_reads_the_same_through_its_host_table,
                 swap_pins.test_out_and_back_in_is_the_identity_on_the_rows):
        for quant in (False, True):
            try:
                test(quant)
            except (AssertionError, IndexError, ValueError):
                caught = True
    assert caught, name
