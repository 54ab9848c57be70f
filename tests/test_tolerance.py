"""The score tolerance of the GPU parity tests (tests/helpers.py) is itself checked here, on the
host: the binades it reads off two E4M3 codes are those of their exact product, its per-group
count equals the same count done on float64 products, it never exceeds the coarse bound
2^-10 * sum |q_i k_i| it refines, and a hand-built group gives the count the truncation model
predicts."""
import numpy as np
import torch

import oracle
import helpers


def all_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]                         # the two NaN codes are never generated


def lowest_set_bit(x: float) -> int:
    mant, ex = np.frexp(x)
    i = int(np.ldexp(mant, 53))
    return int(ex) - 53 + ((i & -i).bit_length() - 1)


def test_binades_of_every_product_of_two_codes():
    codes = all_codes()
    v = np.abs(oracle.e4m3_to_f64(codes))
    T, L, a = [x.numpy().astype(np.int64) for x in helpers._e4m3_binades(codes)]
    P = v[:, None] * v[None, :]
    nz = P > 0
    top = T[:, None] + T[None, :] + (a[:, None] * a[None, :] >= 128)
    low = L[:, None] + L[None, :]
    assert np.array_equal(top[nz], np.frexp(P[nz])[1] - 1)
    assert np.array_equal(low[nz], np.array([lowest_set_bit(x) for x in P[nz]]))


def float64_count(q_codes, k_codes, aw):
    q = oracle.e4m3_to_f64(q_codes)
    k = oracle.e4m3_to_f64(k_codes)
    p = np.abs(k[:, None, :] * q[None, :, :]).reshape(k.shape[0], q.shape[0], -1, helpers.SCORE_GROUP)
    mx = p.max(-1, keepdims=True)
    _, e = np.frexp(np.where(mx > 0, mx, 1.0))
    grid = np.ldexp(1.0, e - 1 - helpers.SCORE_FP8_GRID)
    steps = p / grid
    return ((steps != np.floor(steps)) * grid * (mx > 0)).sum((-1, -2)) @ aw


def test_count_equals_float64_form_and_stays_below_the_coarse_bound():
    gen = torch.Generator().manual_seed(5)
    q = (torch.randn(64, 128, generator=gen) * 2).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    k = (torch.randn(300, 128, generator=gen) * 40).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    k[:3] = 0                                             # zero rows: no products, no bound
    aw = torch.rand(64, generator=gen).double().numpy()
    got = helpers._truncation_bound(q, k, aw)
    np.testing.assert_array_equal(got, float64_count(q, k, aw))
    assert np.all(got[:3] == 0)
    coarse = helpers.SCORE_REL_COARSE * ((np.abs(oracle.e4m3_to_f64(k)) @ np.abs(oracle.e4m3_to_f64(q)).T) @ aw)
    assert np.all(got <= coarse)
    assert np.median(got[3:]) < 0.1 * np.median(coarse[3:])


def code_of(x: float) -> int:
    return int(torch.tensor([x]).to(torch.float8_e4m3fn).view(torch.uint8).item())


def test_hand_built_group():
    # one head, one group of 8 dims with query 1.0: products equal the key entries. The largest
    # is 256 (binade 8), so the grid is 2^(8-13) = 2^-5: 2^-5 and 0.75 lie on it, 2^-6 and
    # 2^-7 lie below it (one grid step each), 3 * 2^-6 = 0.046875 is off it (one step)
    q = np.zeros((1, 128), dtype=np.uint8)
    q[0, :8] = code_of(1.0)
    k = np.zeros((1, 128), dtype=np.uint8)
    for i, x in enumerate([256.0, 2.0 ** -5, 0.75, 2.0 ** -6, 2.0 ** -7, 3 * 2.0 ** -6]):
        k[0, i] = code_of(x)
    got = helpers._truncation_bound(q, k, np.array([1.0]))
    assert got[0] == 3 * 2.0 ** -5
    # the same group with its largest entry removed: the grid drops to 2^(0 - 13) (largest 0.75)
    k[0, 0] = 0
    assert helpers._truncation_bound(q, k, np.array([1.0]))[0] == 0.0
