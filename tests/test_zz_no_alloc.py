"""nvfp4_quantize_noalloc (no caller workspace: the amax partials live in
the library's static per-GPU scratch array) against nvfp4_quantize with a
caller workspace, through the C ABI: codes, scales and global scale bit for
bit, on consecutive calls whose sizes shrink and grow again (the scratch
keeps the previous call's contents), dynamic and static, bf16 and float32,
the one-launch small path and the two-launch path; plus the oracle; and
the call captured in a HIP graph and replayed."""
import numpy as np
import pytest
import torch

import bit_linear_layer_amd as nv
from tests.gpu_util import DEV, assert_quant_exact, host_q, say

pytestmark = pytest.mark.gpu


def x_of(rows, cols, seed, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-2, 2)
    x[:, rng.integers(0, cols)] *= 60
    return torch.from_numpy(x.astype(np.float32)).to(dtype).to(DEV)


def both(x, flags=nv.SCALE_DYNAMIC, g=None):
    q_ref = nv.empty_nvfp4(x.shape[0], x.shape[1], DEV)
    q_new = nv.empty_nvfp4(x.shape[0], x.shape[1], DEV)
    q_new.codes.fill_(0xAB)
    q_new.scales.fill_(0xCD)
    if g is not None:
        q_ref.global_scale.fill_(g)
        q_new.global_scale.fill_(g)
    ws = None if flags == nv.SCALE_STATIC else nv.workspace_for(x.shape[0], x.shape[1], DEV)
    nv.nvfp4_quantize(x, q_ref, flags, ws)
    nv.nvfp4_quantize_noalloc(x, q_new, flags)
    a, b = host_q(q_ref), host_q(q_new)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert a[2].view(np.uint32) == b[2].view(np.uint32)
    return q_new


# (rows, cols): two-launch path, smaller two-launch, one-launch (<= 1024
# blocks), larger two-launch again, the largest one-launch shape
SEQ = [(700, 5120), (96, 2048), (40, 256), (2048, 1024), (64, 256)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_entry_on_a_sequence(dtype):
    for i, (r, c) in enumerate(SEQ):
        say(f"quantize_noalloc dynamic {r}x{c} {dtype}")
        x = x_of(r, c, 100 + i, dtype)
        q = both(x)
        if r * c <= 700 * 5120:
            assert_quant_exact(x, q)


def test_noalloc_static_scale():
    for i, (r, c) in enumerate(SEQ[:3]):
        say(f"quantize_noalloc static {r}x{c}")
        x = x_of(r, c, 200 + i, torch.bfloat16)
        q = both(x, nv.SCALE_STATIC, g=0.0123)
        assert_quant_exact(x, q, g=np.float32(0.0123))


def test_noalloc_rejects_precomputed_amax():
    x = x_of(4, 32, 1, torch.bfloat16)
    q = nv.empty_nvfp4(4, 32, DEV)
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_quantize_noalloc(x, q, nv.AMAX_PRECOMPUTED)


def test_noalloc_replayed_from_a_hip_graph():
    """What the entry point is for: a call captured in a HIP graph (nothing
    allocates inside the capture), replayed four times on new inputs with
    eager calls of the same entry point in between (they share the scratch
    array, in stream order); every replay bit for bit nvfp4_quantize's
    result with a workspace."""
    r, c = 700, 5120
    x = x_of(r, c, 300, torch.bfloat16)
    q = nv.empty_nvfp4(r, c, DEV)
    nv.nvfp4_quantize_noalloc(x, q)  # outside the capture: the scratch address lookup
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.nvfp4_quantize_noalloc(x, q)
    ws = nv.workspace_for(r, c, DEV)
    for i in range(4):
        say(f"quantize_noalloc graph replay {i}")
        x.copy_(x_of(r, c, 301 + i, torch.bfloat16))
        both(x_of(64, 256, 400 + i, torch.bfloat16))  # eager use of the same scratch in between
        q.codes.fill_(0xAB)
        graph.replay()
        q_ref = nv.empty_nvfp4(r, c, DEV)
        nv.nvfp4_quantize(x, q_ref, nv.SCALE_DYNAMIC, ws)
        a, b = host_q(q_ref), host_q(q)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert a[2].view(np.uint32) == b[2].view(np.uint32)
