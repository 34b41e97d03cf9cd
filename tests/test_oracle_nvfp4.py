"""Pins of the oracle's NVFP4 emulation ("ThriftAttention", Method step 2:
the FP4 path in NVFP4 micro-scaling, e2m1 values in blocks of 16 with an
E4M3 scale): hand-worked blocks (tensor scale, E4M3 rounding of the block
scale, e2m1 rounding and saturation of the values), values already on the
grid kept exactly, the one-hot row through the two-level P, and the
all-selected prefill equal to the all-bf16 one."""
import numpy as np

import oracle as orc
from tests.helpers import tau_for


def _slice(rows):
    X = np.zeros((1, len(rows), 16), np.float32)
    for r, vals in enumerate(rows):
        X[0, r, :len(vals)] = vals
    return X


def test_hand_worked_blocks():
    # slice max 2688 -> tensor scale 1; block 0: scale e4m3(448) = 448 -> 2688 (6), 1344 (3), 1000 -> 2 * 448
    # block 1: amax 100 -> scale e4m3(16.67) = 16 -> 100 / 16 = 6.25 saturates to 6 (96), 50 -> 3.125 -> 3 (48),
    #          20 -> 1.25 -> 1 (ties of the 0.5 grid go to even: 1.25 lies between 1 and 1.5, nearer 1) (16)
    X = _slice([[2688.0, 1344.0, 1000.0], [100.0, 50.0, 20.0, -28.0]])
    Y = orc.nvfp4_fake(X, 0)
    assert list(Y[0, 0, :3]) == [2688.0, 1344.0, 896.0]
    # -28 / 16 = -1.75 -> tie between 1.5 and 2 -> even mantissa (2) -> -32
    assert list(Y[0, 1, :4]) == [96.0, 48.0, 16.0, -32.0]


def test_tensor_scale_is_the_power_of_two_above():
    # slice max 3000: 3000 / 2688 = 1.116 -> g = 2; block scale e4m3(3000 / 12 = 250) = 256;
    # 3000 / 512 = 5.86 -> 6 -> 3072; 700 / 512 = 1.367 -> 1.5 -> 768
    X = _slice([[3000.0, 700.0]])
    Y = orc.nvfp4_fake(X, 0)
    assert list(Y[0, 0, :2]) == [3072.0, 768.0]


def test_grid_values_are_kept_and_axis_one_blocks_tokens():
    rng = np.random.default_rng(1)
    e2m1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    X = rng.choice(e2m1, (2, 64, 32)) * rng.choice([-1.0, 1.0], (2, 64, 32)).astype(np.float32)
    X[:, ::16, :] = 6.0                      # every token block and every channel block reaches 6
    X[:, :, ::16] = 6.0
    # slice max 6: g = 2^-8 (6 / 2688 = 0.00223 -> 2^-8 = 0.0039); block scales 6 / (6 g) = 256, exact in e4m3
    for axis in (0, 1):
        np.testing.assert_array_equal(orc.nvfp4_fake(X, axis), X)
    # along tokens: a channel whose 16 tokens hold one large value shares its scale only with them
    Y = X.copy()
    Y[0, 0:16, 1] = 0.25                     # below the block's grid once the block max is 6
    Y[0, 0, 1] = 6.0
    Z = orc.nvfp4_fake(Y, 1)
    assert Z[0, 1, 1] == 0.0 or Z[0, 1, 1] == 0.5  # 0.25 on the 0.5 grid: a tie, to even (0)
    assert Z[0, 1, 1] == 0.0


def test_one_hot_row_and_all_selected():
    rng = np.random.default_rng(6)
    N, d = 256, 128
    tau = tau_for(d)
    Q = np.zeros((N, d), np.float32)
    K = np.zeros((N, d), np.float32)
    Q[:, 0] = 16.0
    K[:, 0] = -16.0
    K[7, 0] = 16.0                          # key 7 dominates every row that sees it (score gap ~48 after tau)
    K[:, 1] = 0.5
    V = rng.standard_normal((N, d)).astype(np.float32)
    Qn, Kn, Vn = (orc.nvfp4_fake(x[None], a)[0] for x, a in ((Q, 0), (K, 0), (V, 1)))
    none = -np.ones((2, 2), np.int32)
    O, _ = orc.thrift_fwd_nv(Qn=Qn, Kn=Kn, Vn=Vn, Qh=Q, Kh=K, Vh=V, sel_idx=none, sel_cnt=np.zeros(2, np.int32),
                             Nq=N, Nk=N, d=d, causal=False, tau=tau)
    # exp(-48) of the other keys is below e2m1's grid after the first level: P^ is one-hot
    np.testing.assert_allclose(O, np.repeat(Vn[7:8], N, axis=0), rtol=0, atol=1e-12)
    # two tying top keys in different blocks of 16: both P' are 448 * 6, exact
    K2 = K.copy()
    K2[100, 0] = 16.0
    Kn2 = orc.nvfp4_fake(K2[None], 0)[0]
    O2t, _ = orc.thrift_fwd_nv(Qn=Qn, Kn=Kn2, Vn=Vn, Qh=Q, Kh=K2, Vh=V, sel_idx=none,
                               sel_cnt=np.zeros(2, np.int32), Nq=N, Nk=N, d=d, causal=False, tau=tau)
    np.testing.assert_allclose(O2t, np.repeat((Vn[7:8] + Vn[100:101]) / 2, N, axis=0), rtol=0, atol=1e-12)
    allsel = np.array([[0, 1], [0, 1]], np.int32)
    O1, l1 = orc.thrift_fwd_nv(Qn=Qn, Kn=Kn, Vn=Vn, Qh=Q, Kh=K, Vh=V, sel_idx=allsel,
                               sel_cnt=np.array([2, 2], np.int32), Nq=N, Nk=N, d=d, causal=True, tau=tau)
    qc, qs = orc.quant_mx_rows(Q[None])
    kc, ks = orc.quant_mx_rows(K[None])
    vc, vs = orc.quant_mx_cols(V[None])
    O2, l2 = orc.thrift_fwd(qc=qc[0], qs=qs[0], kc=kc[0], ks=ks[0], vc_t=vc[0], vs_t=vs[0], Qh=Q, Kh=K, Vh=V,
                            sel_idx=allsel, sel_cnt=np.array([2, 2], np.int32), Nq=N, Nk=N, d=d, blk=128, hp_tile=64,
                            causal=True, tau=tau)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(l1, l2)
