"""The passes replayed from a HIP graph (torch.cuda.CUDAGraph capture of the
C-ABI calls, all inputs, outputs and workspaces allocated before the
capture) give the eager results bit for bit, on every replay.

The kernels are deterministic (fixed-order reductions, no atomics), so a
replay must equal the eager call exactly.  Between replays the program does
its own eager work -- outputs overwritten with NaN, an unrelated eager
convolution, a synchronisation -- and every replay is checked, so a graph
node that only works on its first replay, or an output the graph does not
write, fails."""
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

# float32 small layer (split reduction with a workspace, split-K
# backward-weight), bf16 16x16 (unsplit), bf16 8x8 with a split reduction
CASES = [("f32", (2, 64, 64, 32, 32)), ("f32", (3, 17, 33, 5, 13)),
         ("bf16", (2, 64, 128, 16, 16)), ("bf16", (32, 1024, 512, 8, 8))]


def _buffers(lib3, layer, dev):
    N, C, K, H, W = layer.shape
    inp = wl.make_inputs(layer)
    t = {k: inp[k].to(dev) for k in ("x", "w", "g", "b")}
    code = lib3.CONV3X3_F32 if layer.dtype == "f32" else lib3.CONV3X3_BF16
    ws = {p: torch.empty(max(lib3.conv3x3_workspace_size(p, N, C, K, H, W, code), 1),
                         dtype=torch.uint8, device=dev)
          for p in (lib3.PASS_FWD, lib3.PASS_BWD_DATA)}
    ws_w = torch.empty(max(lib3.conv3x3_bwd_weight_workspace_size(N, C, K, H, W, code), 1),
                       dtype=torch.uint8, device=dev)
    out = {"y": torch.empty((N, K, H, W), device=dev), "dx": torch.empty((N, C, H, W), device=dev),
           "dw": torch.empty((K, C, 3, 3), device=dev), "db": torch.empty((K,), device=dev)}

    def step():
        lib3.conv3x3_fwd(t["x"], t["w"], t["b"], out=out["y"], workspace=ws[lib3.PASS_FWD])
        lib3.conv3x3_bwd_data(t["g"], t["w"], out=out["dx"], workspace=ws[lib3.PASS_BWD_DATA])
        lib3.conv3x3_bwd_weight(t["x"], t["g"], dw=out["dw"], db=out["db"], workspace=ws_w)
    return t, out, step


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0] + "_" + "x".join(map(str, c[1])))
def test_graph_replays_equal_eager(case):
    import diffusion_unet_x3_amd as lib3
    dtype, shape = case
    dev = torch.device("cuda", 0)
    layer = wl.small_layer(*shape, dtype=dtype, seed=97)
    print(f"[graph] {dtype} {shape}", flush=True)
    t, out, step = _buffers(lib3, layer, dev)
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = wl.small_layer(2, 16, 16, 8, 8, dtype="f32", seed=98)
    ot, oout, ostep = _buffers(lib3, other, dev)
    for r in range(3):
        for v in out.values():
            v.fill_(float("nan"))
        ostep()  # the program's own eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v, ref[k]), (shape, r, k)
