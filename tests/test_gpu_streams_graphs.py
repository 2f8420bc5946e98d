"""GPU tests of the stream and graph behaviour patch.h promises: calls on one
handle may overlap on different streams; launches never allocate or
synchronise, so they can be captured in a HIP graph and replayed; replays
give, bit for bit, what eager launches give."""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_gemm_patch_amd import api
    api.load()
    return api


def dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def test_one_handle_on_two_streams(P):
    prob = I.make_problem("st", 300, 640, 1024, 128, 128, frac=0.7, cfg=90)
    pw = P.pack(dev_u16(prob.w), torch.from_numpy(prob.bits).cuda(), tile=(128, 128))
    xs = [dev_u16(I.gen_x(300, 1024, I.rng_for(90, j, I.ROLE_X))) for j in range(4)]
    want = [pw.gemm(x, out_dtype=torch.float32) for x in xs]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [torch.empty((300, 640), dtype=torch.float32, device="cuda") for _ in xs]
    torch.cuda.synchronize()
    for rep in range(3):
        for j, x in enumerate(xs):
            st = s1 if j % 2 == 0 else s2
            with torch.cuda.stream(st):
                pw.gemm(x, out=outs[j], out_dtype=torch.float32, stream=st)
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w)


def test_one_handle_from_two_host_threads(P):
    """Two host threads launch on one handle, each on its own stream (ctypes
    drops the interpreter lock during the call, so the library runs in both at
    once): every Y equals the single-threaded one bit for bit."""
    import threading
    prob = I.make_problem("th", 256, 512, 1024, 128, 128, frac=0.9, cfg=91)
    pw = P.pack(dev_u16(prob.w), torch.from_numpy(prob.bits).cuda(), tile=(128, 128))
    ms = (16, 256)  # the streaming and the tiled kernel
    xs = {m: dev_u16(I.gen_x(m, 1024, I.rng_for(91, m, I.ROLE_X))) for m in ms}
    want = {m: pw.gemm(xs[m]) for m in ms}
    torch.cuda.synchronize()
    outs = {(t, r): None for t in range(2) for r in range(20)}
    errors = []

    def worker(t):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for r in range(20):
                    outs[(t, r)] = pw.gemm(xs[ms[(t + r) % 2]])
            st.synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a launching thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for (t, r), y in outs.items():
        assert torch.equal(y, want[ms[(t + r) % 2]]), (t, r)


def test_grouped_layer_in_a_graph(P):
    """q+k+v and o stages of a shrunk 1B layer captured once, replayed on new inputs."""
    names = list(I.LLAMA32_1B)
    probs = [I.make_problem(lbl, 200, n // 4, k // 4, 128, 128, frac=0.9, cfg=91, matrix=i)
             for i, (lbl, (n, k)) in enumerate(I.LLAMA32_1B.items()) if lbl in ("q", "k", "v", "o")]
    pws = [P.pack(dev_u16(p.w), torch.from_numpy(p.bits).cuda(), tile=(128, 128)) for p in probs]
    xs = [torch.empty((200, p.k), dtype=torch.bfloat16, device="cuda") for p in probs]
    ys = [torch.empty((200, p.n), dtype=torch.bfloat16, device="cuda") for p in probs]
    # warm up (the first launch sets the kernels' LDS limits) before capturing
    P.gemm_grouped(list(zip(pws[:3], xs[:3])), outs=ys[:3])
    pws[3].gemm(xs[3], out=ys[3])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            P.gemm_grouped(list(zip(pws[:3], xs[:3])), outs=ys[:3], stream=s)
            pws[3].gemm(xs[3], out=ys[3], stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        inputs = [I.gen_x(200, p.k, I.rng_for(91, 10 * rep + j, I.ROLE_X)) for j, p in enumerate(probs)]
        for x, a in zip(xs, inputs):
            x.copy_(dev_u16(a))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [y.clone() for y in ys]
        eager = [pw.gemm(x) for pw, x in zip(pws, xs)]
        torch.cuda.synchronize()
        for j, (a, e) in enumerate(zip(got, eager)):
            assert torch.equal(a, e), (rep, j)
        ref = O.gemm_ref(inputs[0], O.masked_weight(probs[0].w, probs[0].mask))
        assert O.rel_error(got[0].float().cpu().numpy().astype(np.float64), ref) <= 1e-2
