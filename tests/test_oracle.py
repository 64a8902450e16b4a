"""The float64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle.attention as oa
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS + pins.PREFILL_PINS + pins.ROPE_PINS +
                         pins.COMPOSED_PINS + pins.PREFILL_ROPE_PINS + pins.MLA_PINS +
                         [pins.pin_bf16],
                         ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oa)


def test_sdpa_pin_with_default_scale():
    # sm_scale=None must mean 1/sqrt(head_dim)
    pins.pin_sdpa(oa, seeds=(14,), default_scale=True)


# ---- planted mistakes: each must be caught by at least one pin ----------
def _wrong_gqa(h, G):
    return h % 2  # interleaved heads instead of consecutive groups


def _drop_last_page_len(kv_indptr, kv_indices, last_page_len, page_size, b):
    start, end = int(kv_indptr[b]), int(kv_indptr[b + 1])
    return [(int(kv_indices[j]), s) for j in range(start, end) for s in range(page_size)]


def _attend_no_scale(q_rows, K, V, sm_scale):
    return _orig_attend(q_rows, K, V, 1.0)


def _attend_lse_no_max(q_rows, K, V, sm_scale):
    o, lse = _orig_attend(q_rows, K, V, sm_scale)
    s = sm_scale * (q_rows @ K.T) if K.shape[0] else None
    return o, (lse - s.max(axis=1)) if s is not None else lse


def _attend_k_for_v(q_rows, K, V, sm_scale):
    return _orig_attend(q_rows, K, K, sm_scale)


def _attend_log2(q_rows, K, V, sm_scale):
    o, lse = _orig_attend(q_rows, K, V, sm_scale)
    return o, lse / np.log(2.0)


def _merge_swapped(v_a, s_a, v_b, s_b):
    return _orig_merge(v_a, s_b, v_b, s_a)


def _merge_no_max(v_a, s_a, v_b, s_b):
    v, s = _orig_merge(v_a, s_a, v_b, s_b)
    return v, s - np.maximum(s_a, s_b)


def _decode_scale_1_over_d(q, k, v, ip, ix, lp, sm_scale=None):
    if sm_scale is None:
        sm_scale = 1.0 / q.shape[-1]
    return _orig_decode(q, k, v, ip, ix, lp, sm_scale)


_orig_attend = oa.attend
_orig_merge = oa.merge_states
_orig_decode = oa.decode_attention

MUTATIONS = {
    "gqa_interleaved": ("kv_head_of", _wrong_gqa),
    "ignore_last_page_len": ("request_tokens", _drop_last_page_len),
    "missing_sm_scale": ("attend", _attend_no_scale),
    "lse_without_max": ("attend", _attend_lse_no_max),
    "k_used_as_v": ("attend", _attend_k_for_v),
    "lse_base_2": ("attend", _attend_log2),
    "merge_weights_swapped": ("merge_states", _merge_swapped),
    "merge_lse_without_max": ("merge_states", _merge_no_max),
    "default_scale_1_over_d": ("decode_attention", _decode_scale_1_over_d),
}


def _visible_off_by_one(kv_len, qo_len, i, causal):
    return max(0, kv_len - qo_len + i) if causal else kv_len


def _visible_top_left(kv_len, qo_len, i, causal):
    return min(kv_len, i + 1) if causal else kv_len


def _visible_no_mask(kv_len, qo_len, i, causal):
    return kv_len


PREFILL_MUTATIONS = {
    "causal_excludes_own_token": ("visible_tokens", _visible_off_by_one),
    "causal_top_left_aligned": ("visible_tokens", _visible_top_left),
    "causal_mask_ignored": ("visible_tokens", _visible_no_mask),
    "gqa_interleaved": ("kv_head_of", _wrong_gqa),
    "k_used_as_v": ("attend", _attend_k_for_v),
}


@pytest.mark.parametrize("name", sorted(PREFILL_MUTATIONS))
def test_prefill_oracle_mutations_are_caught(name, monkeypatch):
    attr, fn = PREFILL_MUTATIONS[name]
    monkeypatch.setattr(oa, attr, fn)
    caught = []
    for pin in pins.PREFILL_PINS:
        try:
            pin(oa)
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every prefill pin"


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_oracle_mutations_are_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oa, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(oa)
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every pin"


def test_e4m3_decoder_matches_the_format_and_torch():
    """The oracle's FP8 E4M3 decoder against points the format fixes (zero,
    the smallest subnormal 2^-9, one, the largest finite 448, NaN) and
    against torch's float8_e4m3fn for all 256 codes (the cast the input
    generator uses)."""
    import torch
    d = oa.dequantize_e4m3
    assert d(0x00) == 0.0 and d(0x80) == 0.0 and np.signbit(d(0x80))
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9 and d(0x08) == 2.0 ** -6
    assert d(0x38) == 1.0 and d(0xB8) == -1.0 and d(0x3C) == 1.5
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = d(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert d(codes, 0.25)[0x38] == 0.25


_orig_apply_rope = oa.apply_rope
_orig_rope_angles = oa.rope_angles


def _rope_interleaved(x, positions, theta=1e4, scale=1.0):
    # pairs (2i, 2i+1) instead of (i, i + d/2)
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    inv = np.argsort(perm)
    return _orig_apply_rope(x[:, perm], positions, theta, scale)[:, inv]


def _rope_angles_no_two(head_dim, positions, theta=1e4, scale=1.0):
    i = np.arange(head_dim // 2, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    return (pos / scale) * (theta ** (-i / head_dim))[None, :]


def _rope_angles_times_scale(head_dim, positions, theta=1e4, scale=1.0):
    return _orig_rope_angles(head_dim, positions, theta, 1.0 / scale)


def _rope_backwards(x, positions, theta=1e4, scale=1.0):
    return _orig_apply_rope(x, -np.asarray(positions, dtype=np.float64), theta, scale)


ROPE_MUTATIONS = {
    "rope_pairs_interleaved": ("apply_rope", _rope_interleaved),
    "rope_frequency_exponent": ("rope_angles", _rope_angles_no_two),
    "rope_scale_multiplies": ("rope_angles", _rope_angles_times_scale),
    "rope_turns_backwards": ("apply_rope", _rope_backwards),
    "rope_query_at_L": ("rope_query_position", lambda L: L),
}


@pytest.mark.parametrize("name", sorted(ROPE_MUTATIONS))
def test_rope_oracle_mutations_are_caught(name, monkeypatch):
    attr, fn = ROPE_MUTATIONS[name]
    monkeypatch.setattr(oa, attr, fn)
    caught = []
    for pin in pins.ROPE_PINS:
        try:
            pin(oa)
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every rope pin"


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_per_request_slices_equal_the_whole_batch(causal):
    """The full-size GPU parity evaluates the oracle one request at a time
    (tests.parity.prefill_request); those slices must give exactly the
    whole-batch result, including requests with no queries, an unmasked
    request with no pages, and a causal request whose every token queries."""
    from block_sparse_kv_bsr_amd.workloads import random_prefill_workload
    from tests.parity import prefill_request
    lens = [40, 0, 77, 1, 120, 33] if not causal else [40, 5, 77, 1, 120, 33]
    qo_lens = [0, 6, 77, 1, 30, 0] if not causal else [0, 5, 77, 1, 30, 0]
    w = random_prefill_workload(31, len(lens), 120, 8, 2, 64, 16, causal=causal, lens=lens,
                                qo_lens=qo_lens)
    q, k, v = (t.double().numpy() for t in w.make_values("cpu"))
    O, LSE = oa.prefill_attention(q, k, v, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                  w.last_page_len, causal, w.sm_scale)
    seen = np.zeros(w.num_qo_tokens, dtype=bool)
    for b in range(w.batch):
        q0, q1, qo, ip, ix, lp = prefill_request(w, b)
        o, s = oa.prefill_attention(q[q0:q1], k, v, qo, ip, ix, lp, causal, w.sm_scale)
        assert np.array_equal(o, O[q0:q1]) and np.array_equal(s, LSE[q0:q1])
        seen[q0:q1] = True
    assert seen.all()
    if not causal:
        assert np.isneginf(LSE[0:6]).all()  # request 1: no pages, unmasked


# ---- planted mistakes in the composed oracle: each is a whole copy of
# decode_attention_composed with one error, which some composed pin catches
def _composed_variant(mistake):
    import math as _m

    def f(q, k_pool, v_pool, kv_indptr, kv_indices, last_page_len, k_prefix, v_prefix,
          prefix_indptr, prefix_indices, prefix_last_page_len, prefix_of, sm_scale=None):
        q = np.asarray(q, dtype=np.float64)
        B, Hq, d = q.shape
        Hkv, P, Pp = k_pool.shape[1], k_pool.shape[2], k_prefix.shape[2]
        G = Hq // Hkv
        sm_scale = 1.0 / _m.sqrt(d) if sm_scale is None else sm_scale
        O, LSE = np.zeros((B, Hq, d)), np.full((B, Hq), -np.inf)
        for b in range(B):
            own = oa.request_tokens(kv_indptr, kv_indices, last_page_len, P, b)
            g = int(prefix_of[b])
            if mistake == "prefix_of_next":
                g = (g + 1) % (len(prefix_indptr) - 1) if g >= 0 else g
            pre = []
            if g >= 0 and mistake != "prefix_dropped":
                lastp = prefix_last_page_len
                if mistake == "prefix_last_len_ignored":
                    lastp = np.full_like(prefix_last_page_len, Pp)
                if mistake == "prefix_read_at_own_page_size":
                    Pp_ = P
                else:
                    Pp_ = Pp
                pre = oa.request_tokens(prefix_indptr, prefix_indices, lastp, Pp_, g)
                pre = [(p_, s_) for p_, s_ in pre if s_ < Pp]
            for kvh in range(Hkv):
                heads = [h for h in range(Hq) if h // G == kvh]
                src = (k_pool, v_pool) if mistake == "prefix_from_main_cache" else (k_prefix, v_prefix)
                Kp, Vp = oa.gather_kv(*src, pre, kvh) if pre else (np.zeros((0, d)), np.zeros((0, d)))
                Ko, Vo = oa.gather_kv(k_pool, v_pool, own, kvh)
                o, lse = oa.attend(q[b, heads, :], np.concatenate([Kp, Ko]),
                                   np.concatenate([Vp, Vo]), sm_scale)
                O[b, heads, :], LSE[b, heads] = o, lse
        return O, LSE
    return f


COMPOSED_MUTATIONS = ["prefix_of_next", "prefix_dropped", "prefix_last_len_ignored",
                      "prefix_read_at_own_page_size", "prefix_from_main_cache"]


@pytest.mark.parametrize("name", COMPOSED_MUTATIONS)
def test_composed_oracle_mutations_are_caught(name, monkeypatch):
    monkeypatch.setattr(oa, "decode_attention_composed", _composed_variant(name))
    caught = []
    for pin in pins.COMPOSED_PINS:
        try:
            pin(oa)
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every composed pin"


def test_composed_variant_without_mistake_passes():
    """The mutation harness itself is faithful: its copy with no mistake
    passes every composed pin."""
    import pytest as _p
    mp = _p.MonkeyPatch()
    try:
        mp.setattr(oa, "decode_attention_composed", _composed_variant("none"))
        for pin in pins.COMPOSED_PINS:
            pin(oa)
    finally:
        mp.undo()


# ---- planted mistakes in the prefill rotary embedding
def _qpos_plus_one(kv_len, qo_len, i):
    return kv_len - qo_len + i + 1


def _qpos_top_left(kv_len, qo_len, i):
    return i


def _qpos_last(kv_len, qo_len, i):
    return kv_len - 1


def _qpos_zero(kv_len, qo_len, i):
    return 0  # the query left unrotated


PREFILL_ROPE_MUTATIONS = {
    "query_one_past_its_position": ("prefill_query_position", _qpos_plus_one),
    "query_at_its_index": ("prefill_query_position", _qpos_top_left),
    "every_query_at_the_last_position": ("prefill_query_position", _qpos_last),
    "query_not_rotated": ("prefill_query_position", _qpos_zero),
}


@pytest.mark.parametrize("name", sorted(PREFILL_ROPE_MUTATIONS))
def test_prefill_rope_oracle_mutations_are_caught(name, monkeypatch):
    attr, fn = PREFILL_ROPE_MUTATIONS[name]
    monkeypatch.setattr(oa, attr, fn)
    caught = []
    for pin in pins.PREFILL_ROPE_PINS:
        try:
            pin(oa)
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every prefill RoPE pin"


_orig_gather_latent = oa.gather_latent
_orig_mla = oa.mla_attention


def _latent_no_rotary(ckv_pool, kpe_pool, tokens):
    C, R = _orig_gather_latent(ckv_pool, kpe_pool, tokens)
    return C, np.zeros_like(R)


def _latent_rotary_shifted(ckv_pool, kpe_pool, tokens):
    C, R = _orig_gather_latent(ckv_pool, kpe_pool, tokens)
    return C, np.roll(R, 1, axis=0)


def _latent_reversed(ckv_pool, kpe_pool, tokens):
    C, R = _orig_gather_latent(ckv_pool, kpe_pool, tokens)
    return C[::-1], R[::-1]


def _mla_rotary_unscaled(q_nope, q_pe, ckv, kpe, qo, ip, ix, lp, sm_scale, causal=True):
    return _orig_mla(q_nope, np.asarray(q_pe) / sm_scale, ckv, kpe, qo, ip, ix, lp, sm_scale,
                     causal)


def _mla_first_head_query(q_nope, q_pe, ckv, kpe, qo, ip, ix, lp, sm_scale, causal=True):
    qn = np.broadcast_to(np.asarray(q_nope)[:, :1], np.shape(q_nope))
    return _orig_mla(qn, q_pe, ckv, kpe, qo, ip, ix, lp, sm_scale, causal)


MLA_MUTATIONS = {
    "mla_rotary_key_dropped": ("gather_latent", _latent_no_rotary),
    "mla_rotary_key_of_previous_token": ("gather_latent", _latent_rotary_shifted),
    "mla_history_reversed": ("gather_latent", _latent_reversed),
    "mla_scale_misses_rotary_part": ("mla_attention", _mla_rotary_unscaled),
    "mla_heads_share_one_query": ("mla_attention", _mla_first_head_query),
    "causal_excludes_own_token": ("visible_tokens", _visible_off_by_one),
    "missing_sm_scale": ("attend", _attend_no_scale),
    "lse_base_2": ("attend", _attend_log2),
}


@pytest.mark.parametrize("name", sorted(MLA_MUTATIONS))
def test_mla_oracle_mutations_are_caught(name, monkeypatch):
    attr, fn = MLA_MUTATIONS[name]
    monkeypatch.setattr(oa, attr, fn)
    caught = []
    for pin in pins.MLA_PINS:
        try:
            pin(oa)
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every MLA pin"
