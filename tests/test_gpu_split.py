"""GPU tests of the split-K streaming path (patch_gemm_with_workspace): a narrow W
with a long K, four workgroups per block of W rows each taking a quarter of K, fp32
partials in the caller's workspace summed in a fixed order into Y."""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as I

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_gemm_patch_amd import api
    api.load()
    return api


def dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def y_host(y):
    return y.float().cpu().numpy().astype(np.float64)


def packed(P, prob):
    return P.pack(dev_u16(prob.w), torch.from_numpy(prob.bits).cuda(), tile=(prob.tn, prob.tk))


def workspace(P, pw, m, fill=float("nan")):
    nbytes = pw.workspace_size(m)
    # stale contents must not matter: every partial is written before it is read
    return torch.full((max(nbytes, 4) // 4,), fill, dtype=torch.float32, device="cuda"), nbytes


CASES = [(2048, 8192, tn, tk) for tn, tk in [(128, 128), (128, 64), (64, 128), (64, 64)]] + \
        [(4096, 8192, 128, 128), (3072, 8192, 64, 64)]


@pytest.mark.parametrize("n,k,tn,tk", CASES)
@pytest.mark.parametrize("m", [1, 16, 40, 128])
def test_split_matches_oracle(P, n, k, tn, tk, m):
    """2 W blocks per workgroup (2048 and 3072 rows) or 4 (4096), decode and batched m, every
    tile size; fp32 Y against the oracle, bf16 Y = fp32 Y rounded to nearest even, run to run
    bitwise, stale workspace contents ignored."""
    prob = I.make_problem("split", m, n, k, tn, tk, frac=0.6, cfg=300 + m, matrix=n // 1024)
    pw = packed(P, prob)
    x = dev_u16(prob.x)
    ws, nbytes = workspace(P, pw, m)
    # decode sizes split only a W whose unsplit grid leaves CUs idle (under 4096 rows)
    assert nbytes == (0 if m <= 16 and n >= 4096 else 4 * m * n * 4)
    y32 = pw.gemm(x, out_dtype=torch.float32, workspace=ws)
    ws.fill_(float("inf"))
    y32b = pw.gemm(x, out_dtype=torch.float32, workspace=ws)
    y16 = pw.gemm(x, out_dtype=torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    ref = O.gemm_ref(prob.x, O.masked_weight(prob.w, prob.mask))
    assert O.rel_error(y_host(y32), ref) <= 1e-4
    assert O.rel_error(y_host(y16), ref) <= TOL
    assert torch.equal(y32, y32b)
    assert torch.equal(y16, y32.to(torch.bfloat16))


def test_split_strided_and_one_hot_exact(P):
    """Strided X and Y, nothing written past n; one-hot X rows give the kept weights exactly."""
    n, k, m = 2048, 8192, 24
    prob = I.make_problem("split1h", m, n, k, 128, 64, frac=0.7, cfg=310)
    pw = packed(P, prob)
    ks = (np.arange(m) * 331 + 17) % k
    x1 = np.zeros((m, k), np.uint16)
    x1[np.arange(m), ks] = 0x3F80
    xs = torch.zeros((m, k + 16), dtype=torch.bfloat16, device="cuda")
    xs[:, :k] = dev_u16(x1)
    ys = torch.full((m, n + 8), float("nan"), dtype=torch.float32, device="cuda")
    ws, _ = workspace(P, pw, m)
    pw.gemm(xs[:, :k], out=ys[:, :n], out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    wm = O.masked_weight(prob.w, prob.mask)
    want = np.frombuffer((wm[:, ks].T.astype(np.uint32) << 16).tobytes(), np.float32).reshape(m, n)
    assert np.array_equal(ys[:, :n].cpu().numpy(), want)
    assert torch.isnan(ys[:, n:]).all()


@pytest.mark.parametrize("n,k,m", [(4096, 4096, 16), (5120, 8192, 16), (2048, 8192, 129), (1024, 8192, 16),
                                   (2048, 4096, 64), (4096, 8192, 16)])
def test_no_split_runs_like_patch_gemm(P, n, k, m):
    """Short K, a wide W, m past the streaming kernel, a W under 2048 rows, or a decode-sized m
    on a W of 4096 rows: no workspace is asked for, and with one the product runs exactly as
    patch_gemm."""
    prob = I.make_problem("nosplit", m, n, k, 128, 128, frac=0.9, cfg=311)
    pw = packed(P, prob)
    assert pw.workspace_size(m) == 0
    x = dev_u16(prob.x)
    ws = torch.zeros(1 << 16, dtype=torch.float32, device="cuda")
    y = pw.gemm(x, out_dtype=torch.float32, workspace=ws)
    y0 = pw.gemm(x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)


def test_small_workspace_runs_unsplit(P):
    """A workspace one float short of the size asked for: the product runs as patch_gemm."""
    prob = I.make_problem("wsshort", 16, 2048, 8192, 128, 128, frac=0.5, cfg=312)
    pw = packed(P, prob)
    x = dev_u16(prob.x)
    nbytes = pw.workspace_size(16)
    ws = torch.zeros(nbytes // 4 - 1, dtype=torch.float32, device="cuda")
    y = pw.gemm(x, out_dtype=torch.float32, workspace=ws)
    y0 = pw.gemm(x, out_dtype=torch.float32)
    full = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    ys = pw.gemm(x, out_dtype=torch.float32, workspace=full)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    assert not torch.equal(ys, y0)  # the split sums K in another order: the check can tell them apart
    ref = O.gemm_ref(prob.x, O.masked_weight(prob.w, prob.mask))
    assert O.rel_error(y_host(ys), ref) <= 1e-4


def test_workspace_rejects_forced_kernel(P):
    prob = I.make_problem("wsk", 16, 2048, 8192, 128, 128, frac=0.5, cfg=313)
    pw = packed(P, prob)
    ws = torch.zeros(pw.workspace_size(16) // 4, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        pw.gemm(dev_u16(prob.x), kernel="stream", workspace=ws)
