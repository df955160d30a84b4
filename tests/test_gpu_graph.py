"""The C-ABI calls captured in a HIP graph: every replay must reproduce the
eager results bit for bit.  The packer clears and accumulates its exponent
bins with kernels (no memset node), the products keep no state between
calls; the graph is replayed several times, with eager work and
synchronizations between the replays, and the outputs and the packer's
workspace are overwritten before each replay so that stale values cannot
pass for new ones."""
import numpy as np
import pytest
import torch

import datagen
import ternary_weight_absmean_amd as bl
from _gpu import bf16, f32, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected only where a GPU exists
    pytest.skip("no GPU visible", allow_module_level=True)


def test_graph_replays_match_eager():
    rng = np.random.default_rng(21)
    n, k, f = 2560, 8192, 1024
    w = f32((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    w_glu = f32((rng.standard_normal((2 * f, k)) * 0.02).astype(np.float32))
    cols = rng.choice(k, size=8, replace=False)
    x = {m: bf16(datagen.activations_bf16(int(rng.integers(1 << 40)), m, k, cols, 20.0)) for m in (1, 4, 16, 300)}
    dy = bf16(datagen.f32_to_bf16((rng.standard_normal((300, n)) * 0.01).astype(np.float32)))

    def run(outs):
        """Packer, the single-token / token-block / ring / GEMM products, the gated
        product (token-block and ring) and both gradients, writing into the
        tensors of `outs`."""
        bl.bl_ternarize_pack(w, packed=outs["packed"], gamma=outs["gamma"], workspace=outs["ws"])
        for m in (1, 4, 16, 300):
            bl.bl_bitlinear(outs["packed"], outs["gamma"], x[m], n, xq=outs[f"xq{m}"], alpha=outs[f"a{m}"],
                            acc=outs[f"acc{m}"], y=outs[f"y{m}"])
        bl.bl_ternarize_pack_glu(w_glu, packed=outs["pglu"], gamma=outs["gglu"], workspace=outs["ws"])
        bl.bl_bitlinear_glu(outs["pglu"], outs["gglu"], x[16], f, xq=outs["xqg"], alpha=outs["ag"], h=outs["h"])
        bl.bl_bitlinear_glu(outs["pglu"], outs["gglu"], x[4], f, xq=outs["xqg4"], alpha=outs["ag4"], h=outs["h4"])
        bl.bl_pack_transposed(outs["packed"], n, k, packed_t=outs["packed_t"])
        bl.bl_bitlinear_backward_x(outs["packed_t"], outs["gamma"], dy, k, dx=outs["dx"])
        bl.bl_bitlinear_backward_w(dy, outs["xq300"], outs["a300"], dw=outs["dw"], workspace=outs["wsw"])

    def buffers():
        d = torch.device("cuda", 0)
        o = {"packed": torch.empty(bl.bl_packed_bytes(n, k), dtype=torch.uint8, device=d),
             "gamma": torch.empty(1, dtype=torch.float32, device=d),
             "ws": torch.empty(bl.bl_ternarize_pack_workspace_bytes(2 * f, k), dtype=torch.uint8, device=d),
             "pglu": torch.empty(bl.bl_packed_bytes(2 * f, k), dtype=torch.uint8, device=d),
             "gglu": torch.empty(1, dtype=torch.float32, device=d),
             "xqg": torch.empty((16, k), dtype=torch.int8, device=d),
             "ag": torch.empty(16, dtype=torch.float32, device=d),
             "h": torch.empty((16, f), dtype=torch.bfloat16, device=d),
             "xqg4": torch.empty((4, k), dtype=torch.int8, device=d),
             "ag4": torch.empty(4, dtype=torch.float32, device=d),
             "h4": torch.empty((4, f), dtype=torch.bfloat16, device=d),
             "packed_t": torch.empty(bl.bl_packed_bytes(k, n), dtype=torch.uint8, device=d),
             "dx": torch.empty((300, k), dtype=torch.float32, device=d),
             "dw": torch.empty((n, k), dtype=torch.float32, device=d),
             "wsw": torch.empty(bl.bl_backward_w_workspace_bytes(300, n, k), dtype=torch.uint8, device=d)}
        for m in (1, 4, 16, 300):
            o[f"xq{m}"] = torch.empty((m, k), dtype=torch.int8, device=d)
            o[f"a{m}"] = torch.empty(m, dtype=torch.float32, device=d)
            o[f"acc{m}"] = torch.empty((m, n), dtype=torch.int32, device=d)
            o[f"y{m}"] = torch.empty((m, n), dtype=torch.bfloat16, device=d)
        return o

    say("graph: eager reference")
    eager = buffers()
    run(eager)
    torch.cuda.synchronize()

    say("graph: capture")
    static = buffers()
    run(static)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(static)
    torch.cuda.synchronize()

    for r in range(3):
        # eager work of the program between replays
        bl.bl_bitlinear(eager["packed"], eager["gamma"], x[16], n)
        junk = torch.randn(1 << 20, device="cuda").square().sum()
        for t in static.values():
            t.view(torch.uint8).fill_(0xA5 + r)  # stale bits in every output and workspace
        torch.cuda.synchronize()
        say(f"graph: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        for name in eager:
            if name in ("ws", "wsw"):
                continue  # scratch
            a, b = eager[name].view(torch.uint8), static[name].view(torch.uint8)
            assert torch.equal(a, b), f"replay {r}: {name} differs in {(a != b).sum().item()} bytes"
        assert float(junk) > 0


def test_two_streams_do_not_interfere():
    """The library keeps no state between calls (workspaces are the caller's):
    the packer and the products running on two streams at once give the
    results of running them one after the other."""
    rng = np.random.default_rng(22)
    n, k = 3840, 2560
    ws = [f32((rng.standard_normal((n, k)) * 0.02).astype(np.float32)) for _ in range(2)]
    xs = [bf16(datagen.activations_bf16(int(rng.integers(1 << 40)), m, k)) for m in (1, 16)]

    def chain(w, x1, x16):
        packed, gamma = bl.bl_ternarize_pack(w)
        out = [packed, gamma]
        for _ in range(3):
            acc1, y1, _, _ = bl.bl_bitlinear(packed, gamma, x1, n)
            acc16, y16, _, _ = bl.bl_bitlinear(packed, gamma, x16, n)
            out += [acc1, y1, acc16, y16]
        return out

    say("streams: one after the other")
    want = [chain(w, xs[0], xs[1]) for w in ws]
    torch.cuda.synchronize()
    say("streams: two at once")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None, None]
    for i in (0, 1):
        streams[i].wait_stream(torch.cuda.current_stream())
    for i in (0, 1):
        with torch.cuda.stream(streams[i]):
            got[i] = chain(ws[i], xs[0], xs[1])
    torch.cuda.synchronize()
    for i in (0, 1):
        for a, b in zip(want[i], got[i]):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
