"""GPU parity of the standalone product sgd_gemm, and of the product shapes the step profiler records.

sgd_gemm is the SGEMM of the SPRINT report's section 3.3 table (C = op(A)
op(B)); the timing model of that section (eq. 6) is fitted over its
launches.  The reference is the oracle's fc product in fp64 (z = a w^T, the
definition written as loops), with op(A) and op(B) transposed on the host.
The bound is the classical one for a dot product of k terms rounded in
fp32 in any order: |C - ref| <= gamma_k (|op(A)| |op(B)|), gamma_k =
k u / (1 - k u), u = 2^-24.  Shapes cover the direct-load kernels (aligned
rows), the staged kernels (ragged rows), stream-K schedules with many
k-slices, padded strides and tiny products; the padding columns of C must
be left untouched.
"""
import numpy as np
import pytest

import oracle as O
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sgd_cnns_amd as S  # noqa: E402
from sgd_cnns_amd import timing_model as TM  # noqa: E402

U = 2.0 ** -24
# (m, n, k, row padding of the stored operands in floats)
# (200, 1100) and (256, 2100) are more than 8 tiles wide, so their tiles run in bands of 8 tile columns (a
# ragged last band of 1 column in the first; stream-K tiles shared between blocks, completed by the fixup, in
# the second).  In the tn form, (64, 28) and (48, 60) take the 64x64 tile (a first conv layer's dedw shape;
# the first split over many stream-K blocks, the second with a ragged tile).  A few tile rows and many
# k-slices give the grouped stream-K form (block groups of all tile rows by up to 8 tile columns running
# the same k-ranges): 2 x 2 groups in (256, 192), 2 x 1 in (256, 2100), 4 x 8 with ragged edges in
# (500, 1000), and 8 x 1 in (1000, 600).  One block per tile over more tiles than resident blocks, with a
# ragged last tile row and column, puts the edge tiles last: (3900, 3950) has 961 tiles (no XCD runs),
# (4000, 4000) 1024 (or 3969 64 x 64 tiles in the tn form).  With at most 32 valid rows (columns) in a
# 64-row (64-column) tile the outer wavefronts only load: (300, 20) on 128 x 64, and (64, 28) on 64 x 64 in the
# tn form; in the nt and nn forms, products of at most 32 rows on 64 x 128 tiles take the 1 x 4 wavefront
# layout (every wavefront over the tile's rows, the empty second row block skipped): (32, 2048), a batch-16
# fc layer's (16, 400, 120) and (16, 120, 84), one row, 32 rows over a ragged 65 columns (the tt and tn forms
# keep the 2 x 2 layout with idle outer wavefronts), odd sizes with padded rows.  Small outputs
# over long reductions whose rows miss the direct-load alignment take, in the tn form, the staged-in-LDS
# split-K kernel: LeNet-5's first conv layer's (6, 28, 12544), and (10, 50, 6000) and (21, 40, 8000) with
# padded rows.
SHAPES = [(77, 130, 1000, 0), (256, 192, 4096, 0), (128, 128, 30000, 0), (1000, 36, 4, 0), (5, 3, 7, 0),
          (300, 516, 260, 12), (513, 257, 1031, 3), (4096, 64, 576, 0), (200, 1100, 300, 0), (256, 2100, 4096, 0),
          (64, 28, 100000, 0), (48, 60, 5000, 0), (500, 1000, 3000, 0), (1000, 600, 4000, 0), (3900, 3950, 200, 0),
          (4000, 4000, 64, 0), (32, 2048, 3000, 0), (300, 20, 4000, 0), (16, 400, 120, 0), (16, 120, 84, 0),
          (1, 1000, 128, 0), (32, 65, 128, 0), (7, 129, 33, 5), (6, 28, 12544, 0), (10, 50, 6000, 3),
          (21, 40, 8000, 1)]


def stored(seed, tid, rows, cols, pad):
    """A [rows][cols + pad] host array with U[-1, 1) values in the first cols columns."""
    a = np.zeros((rows, cols + pad), np.float32)
    a[:, :cols] = 2.0 * workloads.uniform01(seed, tid, (rows, cols)) - 1.0
    return a


def on_device(a, cols):
    t = torch.from_numpy(a).to("cuda")
    return t[:, :cols]


@pytest.mark.parametrize("form", ["nt", "tn", "nn", "tt"])
@pytest.mark.parametrize("m,n,k,pad", SHAPES)
def test_gemm_matches_oracle(form, m, n, k, pad):
    a_t, b_t = TM.FORMS[form]
    print(f"[gemm] form={form} m={m} n={n} k={k} pad={pad}", flush=True)
    seed = 40 + m % 7
    A = stored(seed, 0, k, m, pad) if a_t else stored(seed, 0, m, k, pad)
    B = stored(seed, 1, k, n, pad) if b_t else stored(seed, 1, n, k, pad)
    opA = (A[:, :m].T if a_t else A[:, :k]).astype(np.float64)     # m x k
    opBt = (B[:, :n].T if b_t else B[:, :k]).astype(np.float64)    # n x k
    ref = O.fc_fwd(opA, opBt, np.zeros(n), dtype=np.float64)
    bound = k * U / (1 - k * U) * O.fc_fwd(np.abs(opA), np.abs(opBt), np.zeros(n), dtype=np.float64)

    Ad = on_device(A, m if a_t else k)
    Bd = on_device(B, n if b_t else k)
    padc = 5
    Cfull = torch.full((m, n + padc), float("nan"), device="cuda")
    Cd = Cfull[:, :n]
    nbytes = S.gemm_workspace_bytes(m, n, k, a_t, b_t)
    ws = torch.empty(max(nbytes, 4) // 4, device="cuda")
    S.gemm(Ad, Bd, Cd, a_t, b_t, ws)
    torch.cuda.synchronize()
    got = Cfull.cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(got[:, n:])), "padding columns of C were written"
    err = np.abs(got[:, :n] - ref)
    assert np.all(np.isfinite(got[:, :n]))
    worst = float((err / np.maximum(bound, 1e-300)).max())
    assert np.all(err <= bound), f"max err / bound = {worst:.3f}"


# Short reductions (k <= 32) in the tn form, with n and C's row stride multiples of 4 and 16-byte aligned
# rows, take the streaming weight-gradient kernel: ragged m, odd k, k at the 16 / 32 boundaries, a single
# k, VGG-16's fc weight-gradient shapes at batch 32.  C's 4 padding columns (a 16-byte run) must stay
# untouched.
SHORT = [(1000, 36, 4, 0), (77, 132, 31, 4), (120, 400, 16, 0), (33, 8, 1, 0), (10, 4, 17, 4), (300, 516, 3, 0),
         (4096, 4096, 32, 0), (1000, 4096, 32, 0), (65, 25088, 32, 0)]


@pytest.mark.parametrize("m,n,k,pad", SHORT)
def test_gemm_short_reduction_matches_oracle(m, n, k, pad):
    print(f"[gemm short] m={m} n={n} k={k} pad={pad}", flush=True)
    seed = 60 + m % 5
    A = stored(seed, 0, k, m, pad)
    B = stored(seed, 1, k, n, pad)
    opA = A[:, :m].T.astype(np.float64)
    opBt = B[:, :n].T.astype(np.float64)
    ref = O.fc_fwd(opA, opBt, np.zeros(n), dtype=np.float64)
    bound = k * U / (1 - k * U) * O.fc_fwd(np.abs(opA), np.abs(opBt), np.zeros(n), dtype=np.float64)
    Cfull = torch.full((m, n + 4), float("nan"), device="cuda")
    nbytes = S.gemm_workspace_bytes(m, n, k, True, True)
    ws = torch.empty(max(nbytes, 4) // 4, device="cuda")
    S.gemm(on_device(A, m), on_device(B, n), Cfull[:, :n], True, True, ws)
    torch.cuda.synchronize()
    got = Cfull.cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(got[:, n:])), "padding columns of C were written"
    err = np.abs(got[:, :n] - ref)
    assert np.all(np.isfinite(got[:, :n]))
    worst = float((err / np.maximum(bound, 1e-300)).max())
    assert np.all(err <= bound), f"max err / bound = {worst:.3f}"


# A logits layer's products on the skinny kernels: the forward form (nt) with at most 16 outputs per row
# and a k that is a multiple of 4, and the input-gradient form (nn) with a reduction of at most 16, n a
# multiple of 4 and at most 2^20 outputs (the largest case here is exactly that); C's 4 padding columns must
# stay untouched.  Many rows over a short k, (12544, 6, 28), stay on the tile kernels.
SKINNY = [("nt", 512, 10, 5000), ("nt", 16, 10, 84), ("nt", 3, 16, 4), ("nt", 130, 1, 512), ("nt", 12544, 6, 28),
          ("nn", 128, 512, 10), ("nn", 16, 84, 10), ("nn", 7, 4, 1), ("nn", 130, 512, 16), ("nn", 1024, 1024, 3)]


@pytest.mark.parametrize("form,m,n,k", SKINNY)
def test_gemm_skinny_products_match_oracle(form, m, n, k):
    a_t, b_t = TM.FORMS[form]
    print(f"[gemm skinny] form={form} m={m} n={n} k={k}", flush=True)
    seed = 70 + m % 3
    A = stored(seed, 0, m, k, 0)
    B = stored(seed, 1, k, n, 0) if b_t else stored(seed, 1, n, k, 0)
    opA = A.astype(np.float64)
    opBt = (B.T if b_t else B).astype(np.float64)
    ref = O.fc_fwd(opA, opBt, np.zeros(n), dtype=np.float64)
    bound = k * U / (1 - k * U) * O.fc_fwd(np.abs(opA), np.abs(opBt), np.zeros(n), dtype=np.float64)
    Cfull = torch.full((m, n + 4), float("nan"), device="cuda")
    nbytes = S.gemm_workspace_bytes(m, n, k, a_t, b_t)
    ws = torch.empty(max(nbytes, 4) // 4, device="cuda")
    S.gemm(on_device(A, k), on_device(B, n if b_t else k), Cfull[:, :n], a_t, b_t, ws)
    torch.cuda.synchronize()
    got = Cfull.cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(got[:, n:])), "padding columns of C were written"
    err = np.abs(got[:, :n] - ref)
    assert np.all(np.isfinite(got[:, :n]))
    assert np.all(err <= bound), f"max err / bound = {float((err / np.maximum(bound, 1e-300)).max()):.3f}"


def test_gemm_rejects_bad_arguments():
    """Argument errors are caught on the host, before any launch."""
    m, n, k = 128, 128, 30000
    A = torch.zeros(m, k, device="cuda")
    B = torch.zeros(n, k, device="cuda")
    Cm = torch.zeros(m, n, device="cuda")
    need = S.gemm_workspace_bytes(m, n, k)
    assert need > 0, "a 1 x 1 tile grid with many k-slices is planned with stream-K partial tiles"
    ws = torch.empty(need // 4 + 64, device="cuda")
    with pytest.raises(S.SgdError):
        S.gemm(A, B, Cm, False, False, ws[: need // 8])       # workspace too small
    with pytest.raises(S.SgdError):
        S.gemm(A, B, Cm, False, False, ws[1:])                # workspace not 256-byte aligned
    with pytest.raises(ValueError):
        S.gemm(A, B, Cm[:0], False, False, ws)                # C's rows do not match op(A)
    with pytest.raises(S.SgdError):
        S.gemm(A[:0], B, Cm[:0], False, False, ws)            # m = 0
    with pytest.raises(ValueError):
        S.gemm(A[:, :k // 2], B, Cm, False, False, ws)        # k of op(A) and op(B) differ


def test_profile_records_carry_product_shapes():
    """A small MLP's gradient step: every product is recorded once with its
    (m, n, k) and form, dedw with its ones column (n + 1) for dedb."""
    batch, inp = 8, 64
    layers = [("fc", 32), ("relu",), ("fc", 10), ("softmax_ce",)]
    wl = workloads.WORKLOADS["mlp5000"]
    net = S.Net((batch, inp, 1, 1), layers)
    n = net.param_count()
    W = torch.from_numpy(workloads.normal(wl.seed, 2, n, 0.1)).cuda()
    X = torch.from_numpy(workloads.uniform01(wl.seed, 0, (batch, inp, 1, 1))).cuda()
    y = torch.from_numpy(workloads.labels(wl.seed, 1, batch, 10)).cuda()
    grad = torch.empty(n, device="cuda")
    loss = torch.empty(1, device="cuda")
    ws = net.workspace("cuda")
    net.set_overlap(False)
    net.profile(True)
    net.compute_gradient(W, X, y, grad, loss, ws)
    torch.cuda.synchronize()
    net.profile(False)
    recs = net.profile_read()
    prods, others = TM.products_of(recs)
    got = sorted((p["form"], p["m"], p["n"], p["k"]) for p in prods)
    want = sorted([("nt", batch, 32, inp), ("nt", batch, 10, 32),      # forward
                   ("tn", 10, 33, batch), ("nn", batch, 32, 10),      # layer 2 dedw(+dedb), dedx
                   ("tn", 32, inp + 1, batch)])                      # layer 1 dedw(+dedb)
    assert got == want
    # batch 8: both weight gradients are short reductions, on the streaming kernel; the logits layer's
    # forward and input-gradient products are on the skinny kernels
    assert all(kn.startswith("gemm_dw_short_") for p in prods if p["form"] == "tn" for kn in p["kernels"]), prods
    skinny = {(p["form"], p["n"]) for p in prods if p["kernels"][0].startswith(("gemm_skinny_", "gemm_smallk_"))}
    assert skinny == {("nt", 10), ("nn", 32)}, prods
    assert others, "the softmax and loss kernels are recorded outside the products"
    for (name, _l, _p, ms, _f, _b, shape) in recs:
        assert ms >= 0
        if shape[3] < 0:
            assert shape[:3] == (0, 0, 0), name
