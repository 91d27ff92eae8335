"""GPU parity of the deterministic top-k gating kernel (tk_topk_gate) against
the oracle: indices and weights bit-exact, including ties and signed zeros."""
import numpy as np
import pytest
import torch

import moe_activation_bit_amd as tk
import oracle
from moe_activation_bit_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def run(scores, k, ng, tg, normalise):
    T, E = scores.shape
    sd = torch.from_numpy(scores).to(DEV)
    idx = torch.full((T * k + 64,), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T * k + 64,), -7.0, dtype=torch.float32, device=DEV)
    rc = tk.tk_topk_gate(sd, T, E, k, ng, tg, normalise, idx.data_ptr() + 128, w.data_ptr() + 128)
    assert rc == tk.TkStatus.TK_OK, tk.tk_status_str(rc)
    torch.cuda.synchronize()
    i, ww = idx.cpu().numpy(), w.cpu().numpy()
    assert (i[:32] == -7).all() and (i[32 + T * k:] == -7).all(), "index canary"
    assert (ww[:32] == -7).all() and (ww[32 + T * k:] == -7).all(), "weight canary"
    return i[32:32 + T * k].reshape(T, k), ww[32:32 + T * k].reshape(T, k)


def layout_supported(E, k, ng):
    """The library's layout rule (include/tk.h, tk_topk_gate): 32 lanes per
    token when E <= 256 and k <= 32, else 64; some experts-per-lane count C
    from ceil(E / lanes) to 8 must divide E / ng with a power-of-two quotient."""
    per = E // ng

    def fits(lanes):
        for c in range(-(-E // lanes), 9):
            if ng == 1:
                return True
            q = per // c
            if per % c == 0 and q & (q - 1) == 0:
                return True
        return False

    return (E <= 256 and k <= 32 and fits(32)) or fits(64)


SHAPES = [  # (experts, k, n_group, topk_group)
    (256, 8, 8, 4), (256, 8, 1, 1), (256, 64, 1, 1), (256, 6, 16, 2), (128, 4, 4, 2), (64, 6, 1, 1), (64, 8, 32, 4),
    (8, 2, 1, 1), (100, 3, 1, 1), (160, 8, 5, 2), (200, 5, 1, 1),
    # 5 to 8 experts per lane
    (320, 6, 1, 1), (384, 8, 1, 1), (384, 8, 12, 4), (448, 8, 1, 1), (512, 8, 8, 4), (512, 16, 16, 4),
    (512, 64, 1, 1), (500, 7, 1, 1),
    # group counts the all-pairs group rank covers: 2 groups of 32 lanes, 3, 6 (not a power of two), all kept
    (256, 3, 2, 1), (96, 5, 3, 2), (48, 4, 6, 3), (256, 8, 8, 8),
    # two tokens per wave up to k = 32, one token per wave above; 7 experts in every lane of the
    # two-token layout, whose lanes cannot hold 32-expert groups whole (the one-token kernel serves it)
    (256, 32, 1, 1), (256, 33, 1, 1), (224, 8, 1, 1), (224, 8, 7, 3),
    # the normalising sum as a running sum within 16 lanes (k <= 16) and serially above
    (256, 16, 1, 1), (256, 17, 1, 1), (128, 16, 4, 2),
    # groups that only the two-token layout holds whole (160 / 8: 5 experts per lane, 4 lanes per group;
    # 96 / 4: 3 per lane, 8 lanes), groups that need more experts per lane than the minimum (120 / 6 and
    # 100 / 5: 5 per lane, 4 lanes), and a shape no layout holds (9 experts per group)
    (160, 6, 8, 3), (96, 4, 4, 2), (120, 6, 6, 2), (100, 5, 5, 2), (72, 4, 8, 2),
    # four tokens per wave (kept groups within 16 lanes of the two-token layout, at most 8 groups,
    # k <= 16): every row filled, part-filled rows, 8 / 4 / 2 groups, k = 1 and 16, 2 to 8 experts
    # per lane (experts a multiple of 32 from 64 to 256 in 2, 4 or 8 groups take the one-pass row
    # layout with 4 to 16 experts per lane, the others two passes); and its neighbours that stay two
    # to a wave (20 kept lanes, k = 17, 16 groups)
    (256, 16, 8, 4), (256, 8, 8, 3), (256, 1, 8, 1), (256, 8, 4, 2), (256, 4, 2, 1), (192, 8, 8, 4),
    (64, 6, 8, 4), (128, 8, 8, 4), (128, 4, 4, 2), (128, 3, 2, 1), (128, 16, 8, 1), (256, 8, 8, 5),
    (256, 17, 8, 4), (256, 8, 16, 8), (224, 7, 8, 3), (160, 16, 8, 4), (96, 8, 2, 1), (64, 16, 4, 2),
    # no groups, up to 128 experts and k <= 16: one token per 16-lane row, 1 to 8 experts per lane,
    # the last lanes part-filled or empty when experts is not a multiple of 16; k = 17 stays two to a wave
    (128, 8, 1, 1), (128, 16, 1, 1), (60, 4, 1, 1), (112, 9, 1, 1), (16, 16, 1, 1), (120, 5, 1, 1),
    (17, 3, 1, 1), (128, 17, 1, 1),
    # no groups, 129 to 256 experts and k <= 16: two lists of 5 to 8 experts per lane; 257 to 512:
    # three or four lists of 6 to 8
    (160, 8, 1, 1), (256, 16, 1, 1), (129, 3, 1, 1), (250, 10, 1, 1), (192, 1, 1, 1), (224, 6, 1, 1),
    (384, 8, 1, 1), (512, 10, 1, 1), (320, 7, 1, 1), (448, 16, 1, 1), (257, 3, 1, 1), (500, 9, 1, 1),
]


@pytest.mark.parametrize("normalise", [0, 1])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_topk_matches_oracle(shape, normalise):
    E, k, ng, tg = shape
    print("[gpu-case] topk", shape, normalise, flush=True)
    key = wl.stream_key("topk_test", E * 1000 + k, "scores")
    T = 777
    u = wl.uniform(key, 0, T * E).reshape(T, E)
    s = np.where(np.arange(T)[:, None] % 3 == 0, np.floor(u * 8) / 8, u).astype(np.float32)  # ties on 1/3 of rows
    s[5] = 0.5
    s[6, ::2] = -0.0
    s[6, 1::2] = 0.0
    s[7] = -u[7].astype(np.float32)
    if not layout_supported(E, k, ng):
        sd = torch.from_numpy(s).to(DEV)
        idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        assert tk.tk_topk_gate(sd, T, E, k, ng, tg, normalise, idx, w) == tk.TkStatus.TK_ERR_UNSUPPORTED
        return
    gi, gw = run(s, k, ng, tg, normalise)
    oi, ow = oracle.topk_gate(s, k, ng, tg, bool(normalise))
    bad = np.argwhere(gi != oi)
    assert bad.size == 0, f"indices differ at {bad[:4].tolist()}: {gi[bad[0][0]]} vs {oi[bad[0][0]]}"
    assert np.array_equal(gw.view(np.uint32), ow.view(np.uint32)), np.argwhere(gw.view(np.uint32) != ow.view(np.uint32))[:4]


@pytest.mark.parametrize("shape", [(256, 8, 8, 4), (128, 16, 4, 2), (160, 6, 8, 3), (64, 3, 8, 2), (100, 8, 1, 1)],
                         ids=str)
def test_topk_last_wave_partly_past_the_tokens(shape):
    """Token counts around the four-tokens-per-wave grid: a last wave with 1,
    2 or 3 real tokens repeats the last one in its other rows and stores
    nothing from them (the canaries past the outputs stay)."""
    E, k, ng, tg = shape
    for T in (1, 2, 3, 4, 5, 6, 7, 63, 65, 66, 67):
        print("[gpu-case] topk tail", shape, T, flush=True)
        u = wl.uniform(wl.stream_key("topk_test", E * 1000 + k * 10 + T, "tail"), 0, T * E).reshape(T, E)
        s = (np.floor(u * 16) / 16).astype(np.float32)  # many ties
        for normalise in (0, 1):
            gi, gw = run(s, k, ng, tg, normalise)
            oi, ow = oracle.topk_gate(s, k, ng, tg, bool(normalise))
            assert np.array_equal(gi, oi), (T, normalise, np.argwhere(gi != oi)[:4])
            assert np.array_equal(gw.view(np.uint32), ow.view(np.uint32)), (T, normalise)


@pytest.mark.parametrize("shape", [(256, 8, 8, 4), (128, 16, 4, 2), (160, 6, 8, 3), (256, 8, 8, 5), (512, 8, 8, 4),
                                   (128, 8, 1, 1), (60, 4, 1, 1)],
                         ids=str)
def test_topk_scores_only_4_byte_aligned(shape):
    """Scores at an address that is 4 bytes past a 16-byte boundary (the
    interface asks for 4-byte alignment only): every layout's loads still
    read the right scores."""
    E, k, ng, tg = shape
    T = 37
    print("[gpu-case] topk scores 4-byte aligned", shape, flush=True)
    u = wl.uniform(wl.stream_key("topk_test", E * 1000 + k, "align"), 0, T * E).reshape(T, E).astype(np.float32)
    flat = torch.zeros(T * E + 4, dtype=torch.float32, device=DEV)
    flat[1:1 + T * E] = torch.from_numpy(u.reshape(-1)).to(DEV)
    assert (flat.data_ptr() + 4) % 16 == 4
    idx = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), -7.0, dtype=torch.float32, device=DEV)
    for normalise in (0, 1):
        rc = tk.tk_topk_gate(flat.data_ptr() + 4, T, E, k, ng, tg, normalise, idx, w)
        assert rc == tk.TkStatus.TK_OK, tk.tk_status_str(rc)
        torch.cuda.synchronize()
        oi, ow = oracle.topk_gate(u, k, ng, tg, bool(normalise))
        assert np.array_equal(idx.cpu().numpy(), oi)
        assert np.array_equal(w.cpu().numpy().view(np.uint32), ow.view(np.uint32))


def test_topk_deepseek_shape_full_size():
    """16384 tokens x 256 experts, 8 groups keep 4, top-8, normalised."""
    T, E = 16384, 256
    print("[gpu-case] topk full size", T, E, flush=True)
    s = wl.uniform(wl.stream_key("topk_test", 0, "full"), 0, T * E).reshape(T, E).astype(np.float32)
    gi, gw = run(s, 8, 8, 4, 1)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(T - 64, T), np.arange(0, T, 97)]))
    oi, ow = oracle.topk_gate(s[rows], 8, 8, 4, True)
    assert np.array_equal(gi[rows], oi) and np.array_equal(gw[rows].view(np.uint32), ow.view(np.uint32))
    assert ((gi >= 0) & (gi < E)).all()
    assert np.allclose(gw.sum(axis=1), 1.0, atol=1e-5)


def test_topk_special_values_and_extremes():
    """-inf and huge negative scores, subnormals, an all-zero row under
    normalisation (weights stay zero), k equal to the candidate count, one
    expert, one token."""
    print("[gpu-case] topk special values", flush=True)
    E, T = 256, 64
    u = wl.uniform(wl.stream_key("topk_test", 1, "special"), 0, T * E).reshape(T, E)
    s = (u - 0.5).astype(np.float32)
    s[0] = -np.inf
    s[1, :128] = -np.inf
    s[2] = np.float32(1e-40) * np.arange(E, dtype=np.float32)  # subnormal scores
    s[3] = 0.0
    s[4] = -3.0e38
    s[5, ::7] = np.inf
    for ng, tg, k in ((1, 1, 8), (8, 4, 8), (8, 2, 64), (1, 1, 64)):
        for normalise in (0, 1):
            if normalise and ng == 1 and k == 64:
                continue  # sums over infinite scores are not finite; not a gating case
            gi, gw = run(s, k, ng, tg, normalise)
            oi, ow = oracle.topk_gate(s, k, ng, tg, bool(normalise))
            assert np.array_equal(gi, oi), (ng, tg, k, normalise, np.argwhere(gi != oi)[:4])
            same = (gw.view(np.uint32) == ow.view(np.uint32)) | (np.isnan(gw) & np.isnan(ow))
            assert same.all(), (ng, tg, k, normalise, np.argwhere(~same)[:4])
    one = np.array([[0.25]], dtype=np.float32)
    gi, gw = run(one, 1, 1, 1, 1)
    assert gi[0, 0] == 0 and gw[0, 0] == 1.0


# Values that stress the per-lane sort of the four-token kernels (eight
# scores per lane sorted as doubles: score bits high, tie-break low): equal
# negative scores (their tie-break runs backwards as doubles), signed zeros,
# subnormals of both signs, the largest finite values and infinities.
LANE_ALPHABET = np.array([-np.inf, -3.0e38, -1.5, -1.5, -1e-40, -1e-45, -0.0, 0.0, 1e-45, 1e-40, 1.5, 1.5, 3.0e38,
                          np.inf], dtype=np.float32)


@pytest.mark.parametrize("shape", [(256, 8, 8, 4), (256, 6, 8, 3), (128, 8, 1, 1), (256, 8, 1, 1), (256, 16, 1, 1),
                                   (512, 8, 1, 1)], ids=str)
@pytest.mark.parametrize("finite", [False, True], ids=["with-inf", "finite"])
def test_topk_lane_sort_ties_and_special_values(shape, finite):
    """Every lane's eight scores drawn from a small alphabet of special values,
    so that ties, signed zeros, subnormals and infinities meet inside one lane's
    sort; indices and weights against the oracle (normalised when finite)."""
    E, k, ng, tg = shape
    print("[gpu-case] topk lane sort", shape, finite, flush=True)
    T = 257
    alphabet = LANE_ALPHABET[2:-2] if finite else LANE_ALPHABET  # finite: sums stay finite too
    u = wl.uniform(wl.stream_key("topk_test", E * 100 + k, "lane_sort"), 0, T * E).reshape(T, E)
    s = alphabet[np.minimum((u * len(alphabet)).astype(np.int64), len(alphabet) - 1)]
    s[3] = -1.5  # a row of equal negative scores
    s[4, ::2] = -0.0
    s[4, 1::2] = 0.0
    normalise = 1 if finite else 0
    gi, gw = run(s, k, ng, tg, normalise)
    oi, ow = oracle.topk_gate(s, k, ng, tg, bool(normalise))
    bad = np.argwhere(gi != oi)
    assert bad.size == 0, f"indices differ at {bad[:4].tolist()}: {gi[bad[0][0]]} vs {oi[bad[0][0]]}"
    same = (gw.view(np.uint32) == ow.view(np.uint32)) | (np.isnan(gw) & np.isnan(ow))
    assert same.all(), np.argwhere(~same)[:4]


@pytest.mark.parametrize("ng,tg", [(8, 4), (8, 7), (4, 2), (16, 3), (6, 3)])
def test_topk_nan_group_sums(ng, tg):
    """A group whose two best scores are +inf and -inf sums to NaN and ranks
    as -inf; such a group at every position, tied with an all -inf group, and
    groups with two +inf."""
    E = 256 if ng != 6 else 48
    per = E // ng
    k = min(8, tg * per)
    T = 3 * ng + 6
    print("[gpu-case] topk NaN group sums", ng, tg, flush=True)
    u = wl.uniform(wl.stream_key("topk_test", ng * 10 + tg, "nan_groups"), 0, T * E).reshape(T, E)
    s = (2 * u - 1).astype(np.float32)
    for t in range(T):
        g = t % ng
        if t < 2 * ng:
            s[t, g * per:(g + 1) * per] = -np.inf
            s[t, g * per + (t % per)] = np.inf
        if ng <= t < 2 * ng:
            h = (g + 1) % ng
            s[t, h * per:(h + 1) * per] = -np.inf
        elif 2 * ng <= t < 3 * ng:
            s[t, g * per] = s[t, g * per + 1] = np.inf
    gi, gw = run(s, k, ng, tg, 0)
    oi, ow = oracle.topk_gate(s, k, ng, tg, False)
    assert np.array_equal(gi, oi), np.argwhere(gi != oi)[:4]
    assert np.array_equal(gw.view(np.uint32), ow.view(np.uint32))


def _random_shape(rng):
    """A valid gating shape: experts up to 512, a group count dividing them
    with at least 2 experts per group, topk_group groups kept, k at most the
    candidates and at most 64.  A sixth of the draws have no groups, up to
    512 experts and k <= 16; a third of the rest are the one-pass row
    layout's shapes: a multiple of 32 experts from 64 to 256 in 2, 4 or 8
    groups whose kept groups fit half a 16-lane row."""
    if rng.random() < 1 / 6:  # no groups, up to 512 experts, k <= 16: one token per 16-lane row
        E = int(rng.integers(1, 513))
        return E, int(rng.integers(1, min(16, E) + 1)), 1, 1
    if rng.random() < 1 / 3:
        E = int(rng.choice([64, 96, 128, 160, 192, 224, 256]))
        ng = int(rng.choice([2, 4, 8]))
        tg = int(rng.integers(1, ng // 2 + 1))
        k = int(rng.integers(1, min(16, tg * (E // ng)) + 1))
        return E, k, ng, tg
    while True:
        E = int(rng.choice([8, 16, 32, 48, 64, 96, 100, 128, 160, 192, 200, 224, 256, 320, 384, 448, 512]))
        divisors = [g for g in range(1, 33) if E % g == 0 and (g == 1 or E // g >= 2)]
        ng = int(rng.choice(divisors))
        tg = int(rng.integers(1, ng + 1))
        k = int(rng.integers(1, min(64, tg * (E // ng)) + 1))
        if layout_supported(E, k, ng):
            return E, k, ng, tg


@pytest.mark.parametrize("seed", range(48))
def test_topk_random_shapes(seed):
    """Seeded random shapes and token counts (every layout the library picks:
    one token per 16-lane row, four tokens in two passes, two tokens, one
    token per wave), scores with ties on a third of the rows."""
    rng = np.random.default_rng(1000 + seed)
    E, k, ng, tg = _random_shape(rng)
    T = int(rng.integers(1, 700))
    normalise = int(rng.integers(0, 2))
    print("[gpu-case] topk random", seed, (E, k, ng, tg), T, normalise, flush=True)
    u = wl.uniform(wl.stream_key("topk_random", seed, "scores"), 0, T * E).reshape(T, E)
    s = np.where(np.arange(T)[:, None] % 3 == 0, np.floor(u * 8) / 8, u - 0.5).astype(np.float32)
    gi, gw = run(s, k, ng, tg, normalise)
    oi, ow = oracle.topk_gate(s, k, ng, tg, bool(normalise))
    assert np.array_equal(gi, oi), np.argwhere(gi != oi)[:4]
    assert np.array_equal(gw.view(np.uint32), ow.view(np.uint32))
