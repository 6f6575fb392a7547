"""Pins of the CPU float64 oracle against what the pages and mathematics fix.

None of these compare the oracle with itself: each checks a closed form, a
theorem the "Supported models" page lists under "Facts proved about the
specs", a special case stated in prose on the nnterp qwen3 page, the printed
constants, or an independent library routine.  A plausible mistake in the
oracle (a dropped term, a wrong sign or index, a transposed operand, a wrong
normaliser) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import decode_attention as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng_seed = 1234


def _rng(k=0):
    return np.random.default_rng([rng_seed, k])


# ---------------------------------------------------------------- constants

def test_constants_match_printed_spec():
    with open(os.path.join(GOLDEN, "qwen3_0_6b_constants.json")) as f:
        c = json.load(f)
    assert O.NUM_HEADS == c["num_attention_heads"]["value"]
    assert O.NUM_KV_HEADS == c["num_key_value_heads"]["value"]
    assert O.HEAD_DIM == c["head_dim"]["value"]
    assert O.RMS_EPS == c["rms_norm_eps"]["value"]
    assert O.ROPE_THETA == c["rope_theta"]["value"]
    assert O.ROPE_HALF == c["rope_active_pairs"]["value"]
    assert O.PAGE_SIZE == c["page_size"]["value"]
    # the oracle's GQA mapping h -> h // 2 reproduces the printed head groups
    groups = [[h for h in range(O.NUM_HEADS) if h // 2 == j] for j in range(O.NUM_KV_HEADS)]
    assert groups == c["query_heads_of_kv_head"]["value"]


# ---------------------------------------------------------------- bfloat16

def test_bf16_bits_known_values():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x7F7F, 0x0080, 0x3FC0], dtype=np.uint16)
    got = O.bf16_bits_to_f64(bits)
    want = [1.0, -2.0, math.inf, -math.inf, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127,
            2.0 ** -126, 1.5]
    assert list(got) == want


def test_round_to_bf16_ties_and_edges():
    one = 1.0
    cases = [
        (one, one),
        (one + 2 ** -8, one),                      # tie, 1.0 has even mantissa
        (one + 3 * 2 ** -8, one + 2 ** -6),        # tie, rounds up to even
        (one + 2 ** -8 + 2 ** -30, one + 2 ** -7),  # just above the tie
        (one + 2 ** -8 - 2 ** -30, one),            # just below the tie
        (-(one + 3 * 2 ** -8), -(one + 2 ** -6)),
        (2.0 ** -134, 0.0),                         # half the smallest subnormal: tie to 0
        (3 * 2.0 ** -134, 2.0 ** -132),             # subnormal tie to even
        (2.0 ** 128, math.inf),
        ((2 - 2 ** -7) * 2.0 ** 127, (2 - 2 ** -7) * 2.0 ** 127),
        ((2 - 2 ** -9) * 2.0 ** 127, math.inf),     # rounds past the largest finite
        (-0.0, -0.0),
    ]
    xs = np.array([c[0] for c in cases])
    got = O.round_to_bf16(xs)
    for (x, want), g in zip(cases, got):
        assert g == want, (x, g, want)
    assert math.copysign(1.0, O.round_to_bf16(np.array([-0.0]))[0]) == -1.0
    assert np.isnan(O.round_to_bf16(np.array([np.nan]))[0])


def test_round_to_bf16_matches_library_cast_on_float32():
    torch = pytest.importorskip("torch")
    x32 = (_rng(1).standard_normal(200_000) * np.exp(_rng(2).uniform(-40, 40, 200_000))).astype(np.float32)
    lib = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    ours = O.round_to_bf16(x32.astype(np.float64))
    np.testing.assert_array_equal(ours, lib)


def test_round_to_bf16_is_nearest_by_brute_force():
    x = _rng(3).standard_normal(5000) * 10.0 ** _rng(4).uniform(-5, 5, 5000)
    r = O.round_to_bf16(x)
    rb = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.all(O.bf16_bits_to_f64(rb) == r), "result is a bfloat16 value"
    for delta in (-1, 1):
        nb = O.bf16_bits_to_f64((rb.astype(np.int32) + delta).astype(np.uint16))
        assert np.all(np.abs(x - r) <= np.abs(x - nb))


# ---------------------------------------------------------------- qk_norm

def test_qk_norm_zero_input_gives_zero():
    # nnterp qwen3 page, "The Notes": zeroing the attention input gives zero q/k/v
    w = 1 + 0.1 * _rng(5).standard_normal(128)
    y = O.qk_norm(np.zeros((3, 128)), w)
    assert np.all(y == 0.0)


def test_qk_norm_constant_and_one_hot_closed_forms():
    eps = 1e-6
    w = np.ones(128)
    # constant vector c: mean square c^2, so y = c / sqrt(c^2 + eps)
    for c in (1.0, -2.5, 1e-3):
        y = O.qk_norm(np.full((1, 128), c), w, eps)
        assert np.allclose(y, c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
    # one-hot a*e_5: mean square a^2/128, so y_5 = a / sqrt(a^2/128 + eps) ~ sqrt(128)
    a = 3.0
    x = np.zeros((1, 128)); x[0, 5] = a
    y = O.qk_norm(x, w, eps)
    assert abs(y[0, 5] - math.sqrt(128) * a / math.sqrt(a * a + 128 * eps)) < 1e-13
    assert abs(y[0, 5] - math.sqrt(128)) < 1e-4          # the normaliser is 128, not 1024
    assert np.all(np.delete(y[0], 5) == 0.0)


def test_qk_norm_rms_closed_form_and_gain():
    x = _rng(6).standard_normal((4, 7, 128)) * 3
    w = 1 + 0.1 * _rng(7).standard_normal(128)
    eps = 1e-6
    y = O.qk_norm(x, w, eps)
    xhat = y / w
    m = np.mean(x * x, axis=-1)
    rms = np.sqrt(np.mean(xhat * xhat, axis=-1))
    np.testing.assert_allclose(rms, np.sqrt(m / (m + eps)), rtol=1e-14)
    # direction is preserved per head
    cos = np.sum(xhat * x, -1) / np.linalg.norm(xhat, axis=-1) / np.linalg.norm(x, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-14)


def test_qk_norm_undoes_scale_and_is_per_head():
    # nnterp qwen3 page: an edit to one head's slice is renormalised, and it
    # reaches that head only
    x = _rng(8).standard_normal((2, 16, 128))
    w = 1 + 0.1 * _rng(9).standard_normal(128)
    y = O.qk_norm(x, w)
    x2 = x.copy(); x2[1, 3] *= 1000.0
    y2 = O.qk_norm(x2, w)
    mask = np.ones((2, 16), bool); mask[1, 3] = False
    assert np.array_equal(y[mask], y2[mask])
    np.testing.assert_allclose(y2[1, 3], y[1, 3], rtol=2e-6)


# ---------------------------------------------------------------- RoPE

def test_rope_identity_at_pos_zero():
    x = _rng(10).standard_normal((5, 16, 128))
    assert np.array_equal(O.rope(x, np.zeros(5)), x)


@pytest.mark.parametrize("i", [0, 16, 32, 48, 63])
def test_rope_unit_vector_closed_form(i):
    # pair i is rotated by pos * theta^(-2i/128) = pos * 10^(-6 i / 64)
    pos = 37.0
    ang = pos * 10.0 ** (-6.0 * i / 64.0)
    x = np.zeros((1, 128)); x[0, i] = 1.0
    y = O.rope(x, np.array(pos))
    want = np.zeros(128); want[i] = math.cos(ang); want[i + 64] = math.sin(ang)
    np.testing.assert_allclose(y[0], want, atol=1e-14)
    x = np.zeros((1, 128)); x[0, i + 64] = 1.0
    y = O.rope(x, np.array(pos))
    want = np.zeros(128); want[i] = -math.sin(ang); want[i + 64] = math.cos(ang)
    np.testing.assert_allclose(y[0], want, atol=1e-14)


def test_rope_first_pair_turns_by_pos_radians():
    # theta^0 = 1: the first pair turns by exactly pos radians
    for pos in (1.0, 2.0, 40959.0):
        x = np.zeros((1, 128)); x[0, 0] = 2.0; x[0, 64] = 1.0
        y = O.rope(x, np.array(pos))
        assert abs(y[0, 0] - (2 * math.cos(pos) - math.sin(pos))) < 1e-12
        assert abs(y[0, 64] - (2 * math.sin(pos) + math.cos(pos))) < 1e-12


def test_rope_pairwise_isometry():
    x = _rng(11).standard_normal((6, 8, 128))
    pos = np.array([0, 1, 7, 1000, 32767, 40959], dtype=float)
    y = O.rope(x, pos)
    n_in = x[..., :64] ** 2 + x[..., 64:] ** 2
    n_out = y[..., :64] ** 2 + y[..., 64:] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-14)


def test_rope_preserves_inner_products():
    # theorem rope_isometry ("Supported models" page, "Facts proved about the specs")
    x = _rng(12).standard_normal((1, 128)); z = _rng(13).standard_normal((1, 128))
    for p in (3.0, 517.0, 40000.0):
        rx, rz = O.rope(x, np.array(p)), O.rope(z, np.array(p))
        assert abs(np.dot(rx[0], rz[0]) - np.dot(x[0], z[0])) < 1e-12


def test_rope_relative_positions():
    # theorem rope_relative: <R_p q, R_p' k> = <R_(p-p') q, k>
    q = _rng(14).standard_normal((1, 128)); k = _rng(15).standard_normal((1, 128))
    for p, pp in [(10.0, 3.0), (4096.0, 17.0), (40959.0, 40000.0), (5.0, 9.0)]:
        lhs = np.dot(O.rope(q, np.array(p))[0], O.rope(k, np.array(pp))[0])
        rhs = np.dot(O.rope(q, np.array(p - pp))[0], k[0])
        assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(rhs))


def test_rope_composes():
    x = _rng(16).standard_normal((1, 128))
    a, b = 123.0, 4567.0
    np.testing.assert_allclose(O.rope(O.rope(x, np.array(a)), np.array(b)),
                               O.rope(x, np.array(a + b)), atol=1e-11)


# ---------------------------------------------------------------- decodeGQA

def _kv(S, seed):
    r = _rng(seed)
    return r.standard_normal((S, 8, 128)), r.standard_normal((S, 8, 128))


def test_decode_single_position_returns_v():
    # one cached position: softmax weight 1, o[b,h] = v[0, h // 2]
    q = _rng(20).standard_normal((16, 128)) * 5
    k, v = _kv(1, 21)
    o = O.decode_gqa_dense(q, k, v)
    for h in range(16):
        assert np.array_equal(o[h], v[0, h // 2])


def test_decode_identical_keys_gives_mean_of_v():
    q = _rng(22).standard_normal((16, 128))
    _, v = _kv(37, 23)
    k = np.broadcast_to(_rng(24).standard_normal((1, 8, 128)), (37, 8, 128))
    o = O.decode_gqa_dense(q, k, v)
    for h in range(16):
        np.testing.assert_allclose(o[h], v[:, h // 2].mean(axis=0), rtol=0, atol=1e-14)


def test_decode_zero_query_attends_uniformly():
    # nnterp qwen3 page: a zero query attends uniformly over the prefix
    k, v = _kv(29, 25)
    o = O.decode_gqa_dense(np.zeros((16, 128)), k, v)
    for h in range(16):
        np.testing.assert_allclose(o[h], v[:, h // 2].mean(axis=0), atol=1e-14)


def test_decode_two_positions_closed_form():
    # scores 0 and ln 3 -> weights 1/4, 3/4
    a = 2.0
    q = np.zeros((16, 128)); q[:, 0] = a
    k = np.zeros((2, 8, 128)); k[1, :, 0] = math.log(3.0) * math.sqrt(128) / a
    _, v = _kv(2, 26)
    o = O.decode_gqa_dense(q, k, v)
    for h in range(16):
        np.testing.assert_allclose(o[h], 0.25 * v[0, h // 2] + 0.75 * v[1, h // 2], atol=1e-14)


def test_decode_scale_is_inverse_sqrt_128():
    # scores <q,k>/sqrt(128): with <q,k_1> - <q,k_0> = sqrt(128) the weight
    # ratio is e exactly
    q = np.zeros((16, 128)); q[:, 3] = 1.0
    k = np.zeros((2, 8, 128)); k[1, :, 3] = math.sqrt(128)
    w = O.attention_weights(q, k)
    np.testing.assert_allclose(w[:, 1] / w[:, 0], math.e, rtol=1e-14)


def test_decode_weights_form_distribution_and_convex_hull():
    # theorem attnWeights_distribution
    q = _rng(27).standard_normal((16, 128)) * 4
    k, v = _kv(300, 28)
    w = O.attention_weights(q, k)
    assert np.all(w >= 0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-15)
    o = O.decode_gqa_dense(q, k, v)
    for h in range(16):
        assert np.all(o[h] <= v[:, h // 2].max(axis=0) + 1e-14)
        assert np.all(o[h] >= v[:, h // 2].min(axis=0) - 1e-14)


def test_softmax_shift_invariance():
    # theorem softmax_shift
    z = _rng(29).standard_normal((4, 50)) * 30
    for c in (-1e3, 7.25, 512.0):
        np.testing.assert_allclose(O.softmax(z + c), O.softmax(z), atol=1e-15)


def test_decode_invariant_to_common_key_offset():
    # adding one vector u to every key adds <q,u>/sqrt(128) to all of a head's
    # scores, which the softmax ignores
    q = _rng(30).standard_normal((16, 128))
    k, v = _kv(64, 31)
    u = _rng(32).standard_normal((1, 8, 128)) * 3
    np.testing.assert_allclose(O.decode_gqa_dense(q, k + u, v), O.decode_gqa_dense(q, k, v),
                               atol=1e-13)


def test_decode_head_mapping():
    # nnterp qwen3 page: an edit to KV head j reaches query heads 2j and 2j+1 only
    q = _rng(33).standard_normal((16, 128))
    k, v = _kv(40, 34)
    o = O.decode_gqa_dense(q, k, v)
    for j in range(8):
        v2 = v.copy(); v2[:, j] *= 3.0
        k2 = k.copy(); k2[:, j] *= 0.5
        o2 = O.decode_gqa_dense(q, k2, v2)
        changed = [h for h in range(16) if not np.array_equal(o2[h], o[h])]
        assert changed == [2 * j, 2 * j + 1]


def test_decode_causal_prefix_invariance():
    # theorems forward_causal / attnHead_local: positions >= seq_len are never
    # read, so poisoning them (with NaN) leaves o unchanged, bit for bit
    S, n = 40, 23
    q = _rng(35).standard_normal((16, 128))
    k, v = _kv(S, 36)
    pool_k = np.full((5, 8, 16, 128), np.nan, np.float32)
    pool_v = np.full((5, 8, 16, 128), np.nan, np.float32)
    table = np.array([[3, 0, 4]], np.int32)
    for s in range(n):
        pool_k[table[0, s // 16], :, s % 16] = k[s]
        pool_v[table[0, s // 16], :, s % 16] = v[s]
    o = O.paged_decode_gqa(q[None], pool_k, pool_v, table, np.array([n]), "f32")
    want = O.decode_gqa_dense(q, k[:n].astype(np.float32), v[:n].astype(np.float32))
    assert np.array_equal(o[0], want)
    assert np.all(np.isfinite(o))


def test_paged_gather_matches_dense_scatter():
    # build the pool from a dense cache with vectorised reshapes (no per-slot
    # loop) and check the oracle's paged read returns the dense tensor
    r = _rng(37)
    lens = np.array([5, 16, 17, 50])
    num_pages = 20
    mpp = 4
    perm = r.permutation(num_pages)
    table = np.zeros((4, mpp), np.int32)
    pool = r.standard_normal((num_pages, 8, 16, 128)).astype(np.float32)
    dense = []
    at = 0
    for b, n in enumerate(lens):
        np_ = -(-n // 16)
        table[b, :np_] = perm[at:at + np_]; at += np_
        d = r.standard_normal((np_ * 16, 8, 128)).astype(np.float32)
        pool[table[b, :np_]] = d.reshape(np_, 16, 8, 128).transpose(0, 2, 1, 3)
        dense.append(d[:n])
    for b, n in enumerate(lens):
        got = O.gather_sequence(pool, table[b], int(n), "f32")
        assert np.array_equal(got, dense[b].astype(np.float64))


# ---------------------------------------------------------------- full step

def test_step_single_position_outputs_stored_v():
    r = _rng(40)
    B = 3
    q = r.standard_normal((B, 16, 128)); kn = r.standard_normal((B, 8, 128))
    vn = r.standard_normal((B, 8, 128))
    wq = 1 + 0.1 * r.standard_normal(128); wk = 1 + 0.1 * r.standard_normal(128)
    pool = np.zeros((4, 8, 16, 128), np.uint16)
    table = np.array([[1], [2], [3]], np.int32)
    res = O.decode_step(q, kn, vn, wq, wk, pool, pool, table, np.array([1, 1, 1]), "bf16")
    for b in range(B):
        for h in range(16):
            assert np.array_equal(res["o"][b, h], O.round_to_bf16(vn[b, h // 2]))
    # pos 0: RoPE is the identity, so q_out is the normed q
    np.testing.assert_allclose(res["q_out"], O.qk_norm(q, wq), rtol=0, atol=0)


def test_step_appended_slot_is_normed_roped_k():
    r = _rng(41)
    q = r.standard_normal((1, 16, 128)); kn = r.standard_normal((1, 8, 128)) * 7
    vn = r.standard_normal((1, 8, 128))
    wq = 1 + 0.1 * r.standard_normal(128); wk = 1 + 0.1 * r.standard_normal(128)
    pool = r.standard_normal((3, 8, 16, 128)).astype(np.float32)
    table = np.array([[2, 0]], np.int32)
    res = O.decode_step(q, kn, vn, wq, wk, pool, pool, table, np.array([20]), "f32")
    # the slot keeps the pairwise norms of the normed k (RoPE is an isometry)
    kh = O.qk_norm(kn, wk)[0]
    ks = res["k_slot"][0]
    np.testing.assert_allclose(ks[:, :64] ** 2 + ks[:, 64:] ** 2, kh[:, :64] ** 2 + kh[:, 64:] ** 2,
                               rtol=1e-13)
    assert np.array_equal(res["v_slot"][0], vn[0])


def test_error_metrics():
    ref = np.array([1.0, -4.0, 2.0]); imp = np.array([1.0, -3.5, 2.0])
    assert O.max_abs_err(imp, ref) == 0.5
    assert O.rel_to_max_err(imp, ref) == 0.125


# ---------------------------------------------------------------- family sizes

def test_family_sizes_fixture():
    with open(os.path.join(GOLDEN, "qwen3_family_sizes.json")) as f:
        c = json.load(f)
    groups = sorted({(s["num_heads"], s["num_kv_heads"]) for s in c["sizes"]["value"]})
    assert groups == [(16, 8), (32, 8), (40, 8), (64, 8)]
    assert [O.group_size(h, kv) for h, kv in groups] == [2, 4, 5, 8]
    assert c["head_dim"]["value"] == O.HEAD_DIM


@pytest.mark.parametrize("H", [16, 32, 40, 64])
def test_decode_head_mapping_family(H):
    # KV head j serves query heads j*G .. j*G + G - 1 (G = H / 8): an edit to
    # KV head j reaches exactly those heads
    G = H // 8
    q = _rng(50 + H).standard_normal((H, 128))
    k, v = _kv(23, 51 + H)
    o = O.decode_gqa_dense(q, k, v)
    for j in (0, 3, 7):
        v2 = v.copy(); v2[:, j] *= 3.0
        o2 = O.decode_gqa_dense(q, k, v2)
        changed = [h for h in range(H) if not np.array_equal(o2[h], o[h])]
        assert changed == list(range(j * G, (j + 1) * G))


@pytest.mark.parametrize("H", [32, 40, 64])
def test_decode_family_single_position_and_uniform(H):
    q = _rng(60 + H).standard_normal((H, 128))
    k, v = _kv(1, 61 + H)
    o = O.decode_gqa_dense(q, k, v)
    for h in range(H):
        assert np.array_equal(o[h], v[0, h // (H // 8)])
    k, v = _kv(31, 62 + H)
    o = O.decode_gqa_dense(np.zeros((H, 128)), k, v)
    for h in range(H):
        np.testing.assert_allclose(o[h], v[:, h // (H // 8)].mean(axis=0), atol=1e-14)


def test_group_size_rejects_uneven_heads():
    with pytest.raises(ValueError):
        O.group_size(20, 8)
