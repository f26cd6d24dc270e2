"""GPU parity of the time path, text fusion and backbone entry points against the CPU oracle."""
import numpy as np
import pytest

import flow_matching_diffusion_amd as k2
from flow_matching_diffusion_amd import synth as S
from oracle import k2_oracle as O
from tests.k2_testutil import device, parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,dt", [(256, "f32"), (6144, "bf16")])
def test_time_path(H, dt):
    import torch
    dev = device()
    tw = S.time_weights(7, H, 256, dt)
    t = np.array([0.0, 0.7, 0.31, 1.0], np.float32)
    temb, e = k2.timestep_modulation_forward(H, 256, dt, k2.upload(tw, dt, dev), torch.from_numpy(t).to(dev))
    torch.cuda.synchronize()
    parity(f"time path temb H={H}", dt, temb.cpu().numpy(), lambda rnd: O.time_path(t, tw, rnd=rnd)[0])
    parity(f"time path e H={H}", dt, e.cpu().numpy(), lambda rnd: O.time_path(t, tw, rnd=rnd)[1])


TEXT_SMALL = S.TextDims(hidden=256, num_heads=2, num_kv_heads=2, head_dim=128, intermediate=200, num_layers=5,
                        num_layerwise_blocks=2, num_refiner_blocks=2)


@pytest.mark.parametrize("tdims,dt,B,T,valid", [
    (TEXT_SMALL, "f32", 2, 9, (7, 2)),
    (TEXT_SMALL, "bf16", 2, 9, (7, 2)),
    (S.TextDims(), "bf16", 2, 40, (33, 5)),
])
def test_text_fusion(tdims, dt, B, T, valid):
    import torch
    dev = device()
    seed = 200 + T
    tw = S.text_weights(seed, tdims, dt)
    enc = S.as_dtype(S.normal(seed, "enc", (B, T, tdims.num_layers, tdims.hidden)), dt)
    mask = S.text_mask(B, T, valid)
    cfg = k2.text_cfg(tdims, dt)
    td = torch.bfloat16 if dt == "bf16" else torch.float32
    out = k2.text_fusion_forward(cfg, k2.upload(tw, dt, dev), torch.from_numpy(enc).to(dev).to(td),
                                 torch.from_numpy(mask).to(dev))
    torch.cuda.synchronize()
    parity(f"text fusion D={tdims.hidden} {dt} T={T}", dt, out.cpu().numpy(),
           lambda rnd: O.text_fusion(enc, mask, tw, S.text_block_dims(tdims), rnd=rnd))


def _backbone_case(dims, tdims, dt, B, T, grid, valid, layers, seed, in_ch=64, temb_dim=256):
    import torch
    dev = device()
    wl = S.Workload("bb", seed, dt, B, T, grid, valid, dims=dims, text=tdims, num_layers=layers, in_channels=in_ch,
                    timestep_embed_dim=temb_dim)
    mw = S.model_weights(seed, wl)
    inp = S.backbone_inputs(wl)
    td = torch.bfloat16 if dt == "bf16" else torch.float32
    x = torch.from_numpy(S.as_dtype(inp["x"], dt)).to(dev).to(td)
    enc = torch.from_numpy(inp["enc"]).to(dev).to(td)
    cfg = k2.model_cfg(dims, tdims, layers, in_ch, temb_dim, dt)
    m = None if inp["mask"] is None else torch.from_numpy(inp["mask"]).to(dev)
    out = k2.backbone_forward(cfg, k2.upload(mw, dt, dev), x, enc, torch.from_numpy(inp["timestep"]).to(dev),
                              torch.from_numpy(inp["position_ids"]).to(dev), m)
    torch.cuda.synchronize()
    fn = lambda rnd: O.backbone_forward(S.as_dtype(inp["x"], dt), inp["enc"], inp["timestep"], inp["position_ids"],
                                        inp["mask"], mw, dims, S.text_block_dims(tdims), T, time_dim=temb_dim, rnd=rnd)
    return out.cpu().numpy(), fn, wl


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backbone_small(dt):
    dims = S.BlockDims(hidden=256, num_heads=4, num_kv_heads=1, head_dim=64, intermediate=384, axes_dims=(16, 24, 24))
    got, fn, wl = _backbone_case(dims, TEXT_SMALL, dt, 2, 12, (6, 5), (9, 3), 3, 301)
    assert got.shape == (2, 30, 64)
    parity(f"backbone small {dt}", dt, got, fn)


def test_backbone_quickstart_shape():
    # architecture article §七: B=1, 16 text tokens, 8x8 grid, in_channels 64 -> (1, 64, 64)
    dims = S.BlockDims(hidden=256, num_heads=4, num_kv_heads=1, head_dim=64, intermediate=256, axes_dims=(16, 24, 24))
    got, fn, _ = _backbone_case(dims, TEXT_SMALL, "f32", 1, 16, (8, 8), None, 2, 302)
    assert got.shape == (1, 64, 64)
    parity("backbone quick-start shape", "f32", got, fn)


def test_backbone_full_width_two_layers():
    # full-size block and text dims, two blocks, short sequences: every kernel at its real width
    got, fn, _ = _backbone_case(S.BlockDims(), S.TextDims(), "bf16", 2, 24, (8, 8), (20, 4), 2, 303)
    parity("backbone full width, 2 layers", "bf16", got, fn)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_text_embed_and_cached_backbone(dt):
    """k2_text_embed against the oracle's text rows, and k2_backbone_forward_cached on its output
    bit-identical to k2_backbone_forward (same kernels on the same values), also on a second call
    with other latents and timesteps (the cache does not depend on them)."""
    import torch
    dims = S.BlockDims(hidden=256, num_heads=4, num_kv_heads=1, head_dim=64, intermediate=384, axes_dims=(16, 24, 24))
    seed = 304
    wl = S.Workload("bbc", seed, dt, 2, 12, (6, 5), (9, 3), dims=dims, text=TEXT_SMALL, num_layers=2, in_channels=64,
                    timestep_embed_dim=256)
    dev = device()
    mw = S.model_weights(seed, wl)
    inp = S.backbone_inputs(wl)
    td = torch.bfloat16 if dt == "bf16" else torch.float32
    cfg = k2.model_cfg(dims, TEXT_SMALL, 2, 64, 256, dt)
    wdev = k2.upload(mw, dt, dev)
    enc = torch.from_numpy(inp["enc"]).to(dev).to(td)
    mask = torch.from_numpy(inp["mask"]).to(dev)
    pos = torch.from_numpy(inp["position_ids"]).to(dev)
    txt_h = k2.text_embed(cfg, wdev, enc, mask)
    torch.cuda.synchronize()
    assert txt_h.shape == (2, 12, 256)
    parity(f"text embed {dt}", dt, txt_h.cpu().numpy(),
           lambda rnd: O.text_embed(inp["enc"], inp["mask"], mw, S.text_block_dims(TEXT_SMALL), rnd=rnd))
    for i, t in enumerate(([0.7, 0.7], [0.25, 0.9])):
        x = torch.from_numpy(S.as_dtype(S.normal(seed + i, "x", (2, 30, 64)), dt)).to(dev).to(td)
        tt = torch.tensor(t, dtype=torch.float32, device=dev)
        v_full = k2.backbone_forward(cfg, wdev, x, enc, tt, pos, mask)
        v_cached = k2.backbone_forward_cached(cfg, wdev, x, txt_h, tt, pos, mask)
        torch.cuda.synchronize()
        assert torch.equal(v_full, v_cached), f"call {i}: max diff {(v_full - v_cached).abs().max().item()}"
    assert k2.backbone_cached_workspace_bytes(cfg, 2, 12, 30) < k2.backbone_workspace_bytes(cfg, 2, 12, 30)
