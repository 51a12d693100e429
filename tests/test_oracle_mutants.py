"""Plant plausible mistakes in the oracle (on the CPU) and require that at
least one pin in ``oracle_pins.ALL_CHECKS`` catches each of them."""
import numpy as np
import pytest

import oracle.paged_attention as pa
from tests.oracle_pins import ALL_CHECKS


def _attention_variant(group_of=None, use_scale=True, shift=True, normalize=True, v_head=None):
    def attention(q, K, V, scale):
        Hq, D = q.shape
        L, Hkv = K.shape[0], K.shape[1]
        group = Hq // Hkv
        out = np.zeros((Hq, D))
        if L == 0:
            return out
        for h in range(Hq):
            g = group_of(h, group, Hkv) if group_of else h // group
            s = (scale if use_scale else 1.0) * (K[:, g, :] @ q[h])
            p = np.exp(s - s.max()) if shift else np.exp(s)
            if normalize:
                p = p / p.sum()
            out[h] = p @ V[:, g if v_head is None else v_head, :]
        return out
    return attention


def _gather_variant(v_layout_wrong=False, drop_last=False, reverse_k=False):
    def gather_sequence(k_cache, v_cache, table_row, context_len, page_size):
        L = int(context_len)
        n = (L + page_size - 1) // page_size
        pages = np.asarray(table_row[:n], dtype=np.int64)
        K = np.asarray(k_cache)[pages]
        V = np.asarray(v_cache)[pages]
        Hkv, D = K.shape[1], K.shape[3]
        if reverse_k:
            K = K[:, :, ::-1, :]
        K = K.transpose(0, 2, 1, 3).reshape(n * page_size, Hkv, D)
        if v_layout_wrong:
            V = V.reshape(n, Hkv, page_size, D).transpose(0, 2, 1, 3).reshape(n * page_size, Hkv, D)
        else:
            V = V.transpose(0, 3, 1, 2).reshape(n * page_size, Hkv, D)
        stop = L - 1 if drop_last else L
        return K[:stop], V[:stop]
    return gather_sequence


def _cache_write_variant(keep_negative=False, reverse_slot=False):
    def cache_write(k_cache, v_cache, key, value, slot_mapping, page_size):
        kc = np.array(k_cache, copy=True)
        vc = np.array(v_cache, copy=True)
        for t, s in enumerate(np.asarray(slot_mapping).tolist()):
            if s < 0 and not keep_negative:
                continue
            page, off = s // page_size, s % page_size
            if reverse_slot:
                off = page_size - 1 - off
            kc[page, :, off, :] = key[t]
            vc[page, :, :, off] = value[t]
        return kc, vc
    return cache_write


def _combine_variant(no_exp=False, flip_sign=False):
    def combine_partitions(m, lsum, o):
        Hq, n, D = o.shape
        if n == 0:
            return np.zeros((Hq, D))
        M = m.max(axis=1, keepdims=True)
        if no_exp:
            w = lsum
        else:
            w = lsum * np.exp((M - m) if flip_sign else (m - M))
        return (w[:, :, None] * o).sum(axis=1) / w.sum(axis=1, keepdims=True)
    return combine_partitions


def _partition_shifted(q, K, V, scale, partition_size):
    Hq, D = q.shape
    L, Hkv = K.shape[0], K.shape[1]
    group = Hq // Hkv
    n = (L + partition_size - 1) // partition_size
    m, lsum, o = np.zeros((Hq, n)), np.zeros((Hq, n)), np.zeros((Hq, n, D))
    for h in range(Hq):
        g = h // group
        for k in range(n):
            lo, hi = k * partition_size, min((k + 1) * partition_size + 1, L)  # overlaps
            s = scale * (K[lo:hi, g, :] @ q[h])
            m[h, k] = s.max()
            e = np.exp(s - m[h, k])
            lsum[h, k] = e.sum()
            o[h, k] = (e @ V[lo:hi, g, :]) / lsum[h, k]
    return m, lsum, o


def _bf16_shift15(bits):
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return wide.view(np.float32).astype(np.float64)


def _decode_wrong_row(query, k_cache, v_cache, block_tables, context_lens, scale, page_size, dtype):
    q64 = pa.to_float64(query, dtype)
    B, Hq, D = q64.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        row = block_tables[(b + 1) % B] if B > 1 and context_lens[(b + 1) % B] >= context_lens[b] \
            else block_tables[b]
        K, V = pa.gather_sequence(k_cache, v_cache, row, context_lens[b], page_size)
        out[b] = pa.attention(q64[b], pa.to_float64(K, dtype), pa.to_float64(V, dtype), scale)
    return out


def _causal_variant(limit):
    def causal_attention(q, K, V, scale, positions):
        T, Hq, D = q.shape
        out = np.zeros((T, Hq, D))
        for i in range(T):
            stop = limit(int(positions[i]), K.shape[0])
            out[i] = pa.attention(q[i], K[:stop], V[:stop], scale)
        return out
    return causal_attention


def _chunk_positions_from_zero(query, k_cache, v_cache, block_tables, context_lens, query_start,
                               scale, page_size, dtype):
    q64 = pa.to_float64(query, dtype)
    out = np.zeros(q64.shape)
    qs = np.asarray(query_start)
    for b in range(len(qs) - 1):
        lo, hi = int(qs[b]), int(qs[b + 1])
        if hi == lo:
            continue
        K, V = pa.gather_sequence(k_cache, v_cache, block_tables[b], context_lens[b], page_size)
        out[lo:hi] = pa.causal_attention(q64[lo:hi], pa.to_float64(K, dtype),
                                         pa.to_float64(V, dtype), scale, np.arange(hi - lo))
    return out


def _export_variant(swap=False, reverse=False, v_as_k=False):
    def export_pages(k_cache, v_cache, page_ids, buffer=None):
        kc, vc = np.asarray(k_cache), np.asarray(v_cache)
        ids = np.asarray(page_ids, dtype=np.int64)
        n, block = ids.shape[0], int(np.prod(kc.shape[1:]))
        out = (np.zeros((2, n, block), dtype=kc.dtype) if buffer is None
               else np.array(buffer, copy=True).reshape(2, n, block))
        order = range(n - 1, -1, -1) if reverse else range(n)
        for slot, i in enumerate(order):
            p = int(ids[i])
            if 0 <= p < kc.shape[0]:
                kb = kc[p].reshape(-1)
                vb = vc[p].transpose(0, 2, 1).reshape(-1) if v_as_k else vc[p].reshape(-1)
                out[0, slot], out[1, slot] = (vb, kb) if swap else (kb, vb)
        return out
    return export_pages


def _import_wraps_negative(k_cache, v_cache, buffer, page_ids):
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    ids = np.asarray(page_ids, dtype=np.int64)
    buf = np.asarray(buffer).reshape(2, ids.shape[0], -1)
    for i in range(ids.shape[0]):
        p = int(ids[i])
        if p < kc.shape[0]:
            kc[p] = buf[0, i].reshape(kc.shape[1:])
            vc[p] = buf[1, i].reshape(vc.shape[1:])
    return kc, vc


def _round_variant(mode):
    """Plausible mistakes in the rounding onto bf16."""
    import math

    def round_to_bf16_bits(x):
        a = np.asarray(x, dtype=np.float64).reshape(-1)
        out = np.zeros(a.shape, dtype=np.uint16)
        for i, v in enumerate(a.tolist()):
            if v != v:
                out[i] = 0x7FC0
                continue
            if mode == "via_float32":          # two roundings: float64 -> f32 -> bf16
                v = float(np.float32(v))
            sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
            m = abs(v)
            if m and m != math.inf:
                e = math.frexp(m)[1] - 1
                if mode != "no_subnormal_floor":
                    e = max(e, -126)
                q = math.ldexp(1.0, e - 7)
                r = m / q
                if mode == "truncate":
                    r = math.floor(r)
                elif mode == "ties_away":
                    r = math.floor(r + 0.5)
                else:
                    r = round(r)
                m = r * q
            if m >= math.ldexp(1.0, 128):
                out[i] = sign | 0x7F80
                continue
            out[i] = sign | (int(np.array([m], dtype=np.float32).view(np.uint32)[0]) >> 16)
        return out.reshape(np.shape(x))
    return round_to_bf16_bits


def _ulp_without_sign(a, b):
    return np.abs(np.asarray(a, dtype=np.int64) - np.asarray(b, dtype=np.int64))


MUTANTS = {
    "bf16_round_truncates": ("round_to_bf16_bits", _round_variant("truncate")),
    "bf16_round_ties_away": ("round_to_bf16_bits", _round_variant("ties_away")),
    "bf16_round_twice_via_f32": ("round_to_bf16_bits", _round_variant("via_float32")),
    "bf16_round_no_subnormals": ("round_to_bf16_bits", _round_variant("no_subnormal_floor")),
    "ulp_distance_ignores_sign": ("bf16_ulp_distance", _ulp_without_sign),
    "gqa_head_modulo": ("attention", _attention_variant(group_of=lambda h, G, Hkv: h % Hkv)),
    "scale_dropped": ("attention", _attention_variant(use_scale=False)),
    "no_max_shift": ("attention", _attention_variant(shift=False)),
    "no_normalisation": ("attention", _attention_variant(normalize=False)),
    "v_from_head0": ("attention", _attention_variant(v_head=0)),
    "v_layout_as_k": ("gather_sequence", _gather_variant(v_layout_wrong=True)),
    "context_off_by_one": ("gather_sequence", _gather_variant(drop_last=True)),
    "k_slots_reversed_in_gather": ("gather_sequence", _gather_variant(reverse_k=True)),
    "negative_slot_written": ("cache_write", _cache_write_variant(keep_negative=True)),
    "slot_reversed_in_write": ("cache_write", _cache_write_variant(reverse_slot=True)),
    "lse_weight_without_exp": ("combine_partitions", _combine_variant(no_exp=True)),
    "lse_weight_sign_flipped": ("combine_partitions", _combine_variant(flip_sign=True)),
    "partition_ranges_overlap": ("partition_attention", _partition_shifted),
    "bf16_widened_by_15_bits": ("bf16_bits_to_float64", _bf16_shift15),
    "block_table_row_swapped": ("decode", _decode_wrong_row),
    "chunk_without_causal_mask": ("causal_attention", _causal_variant(lambda p, L: L)),
    "chunk_excludes_own_token": ("causal_attention", _causal_variant(lambda p, L: max(p, 1))),
    "chunk_sees_one_token_ahead": ("causal_attention", _causal_variant(lambda p, L: p + 2)),
    "chunk_positions_from_zero": ("chunk_attention", _chunk_positions_from_zero),
    "export_swaps_k_and_v": ("export_pages", _export_variant(swap=True)),
    "export_reverses_page_order": ("export_pages", _export_variant(reverse=True)),
    "export_v_in_k_layout": ("export_pages", _export_variant(v_as_k=True)),
    "import_wraps_negative_ids": ("import_pages", _import_wraps_negative),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(pa, attr, fn)
    caught = []
    for check in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(pa)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_via_module():
    for check in ALL_CHECKS:
        check(pa)
