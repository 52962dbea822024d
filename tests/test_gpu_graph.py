"""The library's calls captured into one HIP graph and replayed, as the
benchmark runs them: every replay must give the eager call's bits.

One graph holds a call of each kernel family (the band, pointwise, split-
precision fp32 and GEMM dense kernels; the per-wave, padded-row and row-per-
thread depthwise kernels). Between replays the program does its own eager
work and synchronises, and the outputs are cleared with a fill kernel (no
memset node is recorded in the graph).
"""
import pytest
import torch

import convolution_forward_amd as cf
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _calls():
    bf = torch.bfloat16
    X3 = wl.random_tensor((4, 20, 30, 64), 9500, dist="normal").to(bf).to(DEV)
    F3 = (wl.random_tensor((3, 3, 64, 64), 9501, dist="normal") * 0.05).to(bf).to(DEV)
    Y3 = torch.empty((4, 18, 28, 64), dtype=bf, device=DEV)
    X1 = wl.random_tensor((4, 10, 13, 256), 9502, dist="normal").to(bf).to(DEV)
    F1 = (wl.random_tensor((1, 1, 256, 256), 9503, dist="normal") * 0.06).to(bf).to(DEV)
    Y1 = torch.empty((4, 10, 13, 256), dtype=bf, device=DEV)
    Xf = wl.random_tensor((2, 9, 11, 64), 9504, dist="normal").to(DEV)
    Ff = (wl.random_tensor((1, 1, 64, 96), 9505, dist="normal") * 0.1).to(DEV)
    Yf = torch.empty((2, 9, 11, 96), device=DEV)
    Xs = wl.random_tensor((2, 30, 30, 64), 9506, dist="normal").to(bf).to(DEV)
    Fs = (wl.random_tensor((3, 3, 64, 128), 9507, dist="normal") * 0.05).to(bf).to(DEV)
    Ys = torch.empty((2, 15, 15, 128), dtype=bf, device=DEV)
    Xd = wl.random_tensor((4, 12, 56, 56), 9508).to(DEV)
    wd = wl.random_tensor((12, 5, 5), 9509).to(DEV)
    Yd = torch.empty((4, 12, 28, 28), device=DEV)
    Xe = wl.random_tensor((2, 6, 28, 28), 9510).to(DEV)
    we = wl.random_tensor((6, 5, 5), 9511).to(DEV)
    Ye = torch.empty((2, 6, 28, 28), device=DEV)
    Xr = wl.random_tensor((4, 40, 7, 7), 9512).to(DEV)
    wr = wl.random_tensor((40, 5, 5), 9513).to(DEV)
    Yr = torch.empty((4, 40, 7, 7), device=DEV)
    calls = [
        lambda: cf.conv2d_nhwc(X3, F3, out=Y3),
        lambda: cf.conv2d_nhwc(X1, F1, out=Y1),
        lambda: cf.conv2d_nhwc(Xf, Ff, out=Yf),
        lambda: cf.conv2d_nhwc(Xs, Fs, out=Ys, stride=2, padding=1),
        lambda: cf.conv_depthwise(Xd, wd, stride=2, padding=2, exact=True, out=Yd),
        lambda: cf.conv_depthwise(Xe, we, stride=1, padding=2, exact=False, out=Ye),
        lambda: cf.conv_depthwise(Xr, wr, stride=1, padding=2, exact=False, out=Yr),
    ]
    return calls, [Y3, Y1, Yf, Ys, Yd, Ye, Yr]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_gpu_graph_replay_matches_eager():
    calls, outs = _calls()
    for c in calls:
        c()
    torch.cuda.synchronize()
    eager = [_bits(y).clone() for y in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    torch.cuda.synchronize()
    for rep in range(4):
        for y in outs:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, e) in enumerate(zip(outs, eager)):
            assert torch.equal(_bits(y), e), f"replay {rep}, call {i}"
        # eager work of the program between replays
        calls[rep % len(calls)]()
        torch.cuda.synchronize()
