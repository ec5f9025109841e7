"""moe_pack_weight against the packed layout include/moe.h documents, built
here by concatenating the blocks in storage order (bit-exact: packing only
moves elements)."""
import numpy as np
import pytest
import torch

import routed_relu_expert_amd as M

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _blocks_out_in(w):
    """[out][in]: 256-row tiles in order, each as its 32-column steps in order,
    each step a row-major [rn][kw] block."""
    G, R, C = w.shape
    parts = []
    for g in range(G):
        for r0 in range(0, R, 256):
            for c0 in range(0, C, 32):
                parts.append(w[g, r0:r0 + 256, c0:c0 + 32].reshape(-1))
    return np.concatenate(parts) if parts else np.zeros(0, w.dtype)


def _blocks_neuron_major(w):
    """neuron-major: 256-column strips in order, each row-major [R][cn]."""
    G, R, C = w.shape
    parts = []
    for g in range(G):
        for c0 in range(0, C, 256):
            parts.append(w[g, :, c0:c0 + 256].reshape(-1))
    return np.concatenate(parts) if parts else np.zeros(0, w.dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", [(1, 256, 32), (2, 300, 264), (3, 33, 520), (1, 1856, 2688),
                                   (1, 8, 8)])
@pytest.mark.parametrize("kind", [M.MOE_PACK_OUT_IN, M.MOE_PACK_NEURON_MAJOR],
                         ids=["out_in", "neuron_major"])
def test_pack_matches_documented_layout(kind, shape, dtype):
    g = torch.Generator().manual_seed(hash((kind, shape)) & 0xffff)
    w = torch.randn(shape, generator=g).to(dtype)
    got = M.moe_pack_weight(w.to(DEV), kind)
    torch.cuda.synchronize()
    assert got.shape == w.shape
    ints = torch.int16 if dtype == torch.bfloat16 else torch.int32
    src = w.view(ints).numpy()
    want = _blocks_out_in(src) if kind == M.MOE_PACK_OUT_IN else _blocks_neuron_major(src)
    assert np.array_equal(got.view(ints).cpu().numpy().reshape(-1), want)


def test_pack_two_dims_is_one_group():
    w = torch.randn(300, 264).to(torch.bfloat16)
    a = M.moe_pack_weight(w.to(DEV), M.MOE_PACK_OUT_IN)
    b = M.moe_pack_weight(w[None].to(DEV), M.MOE_PACK_OUT_IN)
    assert torch.equal(a.reshape(-1), b.reshape(-1))


@pytest.mark.parametrize("shape", [(1, 256, 32), (2, 300, 272), (3, 33, 528), (1, 1856, 2688), (1, 8, 16)])
@pytest.mark.parametrize("kind", [M.MOE_PACK_OUT_IN, M.MOE_PACK_NEURON_MAJOR],
                         ids=["out_in", "neuron_major"])
def test_pack_fp8_codes_matches_documented_layout(kind, shape):
    """One-byte E4M3 codes: the same layout, element for element."""
    g = torch.Generator().manual_seed(hash((kind, shape, "fp8")) & 0xffff)
    w = torch.randint(0, 256, shape, generator=g, dtype=torch.uint8)
    got = M.moe_pack_weight(w.to(DEV), kind)
    torch.cuda.synchronize()
    src = w.numpy()
    want = _blocks_out_in(src) if kind == M.MOE_PACK_OUT_IN else _blocks_neuron_major(src)
    assert np.array_equal(got.cpu().numpy().reshape(-1), want)


def _nibbles(b):
    """[..., n] bytes -> [..., 2n] 4-bit codes (element 2i in the low nibble)."""
    b = np.asarray(b, dtype=np.uint8)
    return np.stack([b & 15, b >> 4], axis=-1).reshape(b.shape[:-1] + (2 * b.shape[-1],))


@pytest.mark.parametrize("shape", [(1, 256, 32), (2, 300, 288), (3, 33, 544), (1, 1856, 2688)])
@pytest.mark.parametrize("kind", [M.MOE_PACK_OUT_IN, M.MOE_PACK_NEURON_MAJOR],
                         ids=["out_in", "neuron_major"])
def test_pack_mxfp4_codes_matches_documented_layout(kind, shape):
    """Two codes per byte: the packed matrix is the documented element order,
    two elements per byte in that order."""
    g = torch.Generator().manual_seed(hash((kind, shape, "fp4")) & 0xffff)
    G, R, C = shape
    codes = torch.randint(0, 256, (G, R, C // 2), generator=g, dtype=torch.uint8)
    packed = M.moe_pack_weight(codes.to(DEV), kind, fp4=True)
    torch.cuda.synchronize()
    elems = _nibbles(codes.numpy())
    want = _blocks_out_in(elems) if kind == M.MOE_PACK_OUT_IN else _blocks_neuron_major(elems)
    assert np.array_equal(_nibbles(packed.cpu().numpy()).reshape(-1), want)


def test_fp4_transpose():
    g = torch.Generator().manual_seed(7)
    codes = torch.randint(0, 256, (3, 64, 48), generator=g, dtype=torch.uint8)
    t = M.fp4_transpose(codes.to(DEV)).cpu().numpy()
    want = np.swapaxes(_nibbles(codes.numpy()), -1, -2)
    assert t.shape == (3, 96, 32) and np.array_equal(_nibbles(t), want)
