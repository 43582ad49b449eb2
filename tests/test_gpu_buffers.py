"""GPU tests of the handles' device buffers: one block per handle from a
per-device cache, released behind events on every stream the handle ran on
(dsp_destroy does not wait for the device) and reused by later prepares."""
import numpy as np
import pytest

from synthetic import bf_pixels, data_stack_numpy, workload

torch = pytest.importorskip("torch")
dsp = pytest.importorskip("stem_direct_ptychography_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(f"[gpu-buffers] {msg}", flush=True)


def _c2():
    w = workload("c2")
    pix, k = bf_pixels(w)
    G = torch.as_tensor(data_stack_numpy(w, pix), device=DEV)
    return w, k, G


def _prep(w, k, G, optics, stream=None, method="phase"):
    return dsp.prepare(G, k, optics, step=w.step, upsampling=w.upsampling, method=method, smoothness=w.smoothness,
                       stream=stream)


def test_block_reuse_across_streams():
    """A handle prepared on one stream is solved on a second and destroyed at
    once; a prepare of other optics on a third stream then takes its block.
    The solves queued before the destroy must read the first handle's
    systems: every one equals a reference solve."""
    w, k, G = _c2()
    other = w.optics.replace(aberrations=[(1, 0, -120.0, 0.0), (3, 0, 1e4, 0.0)])
    strengths = list(np.logspace(-4, 0, 48))
    ref = _prep(w, k, G, w.optics)
    x_ref = ref.solve(strengths)
    aug_ref, _ = ref.export_system()
    torch.cuda.synchronize()
    del ref
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    xs, augs, others = [], [], []
    for it in range(4):
        _say(f"round {it}: prepare on s1, solve on s2, destroy, prepare other optics on s3")
        a = _prep(w, k, G, w.optics, stream=s1)
        s2.wait_stream(s1)
        with torch.cuda.stream(s2):
            xs.append(a.solve(strengths, stream=s2))
            augs.append(a.export_system(stream=s2)[0])
        del a   # no wait: the block goes back behind an event on s1 and one on s2
        b = _prep(w, k, G, other, stream=s3)
        with torch.cuda.stream(s3):
            others.append(b.solve(strengths, stream=s3))
        del b
    torch.cuda.synchronize()
    for x, aug in zip(xs, augs):
        assert torch.equal(x, x_ref)
        assert torch.equal(aug, aug_ref)
    # the other optics give other solutions (the blocks really were shared)
    assert not torch.equal(others[0], x_ref)
    for x in others[1:]:
        assert torch.equal(x, others[0])


@pytest.mark.parametrize("method", ["phase", "complex"])
def test_repeated_prepares_allocate_nothing(method):
    """After the first prepare of a workload, prepare / destroy cycles take
    the cached block: the device's free memory does not move, and the systems
    are bitwise the same every time."""
    w, k, G = _c2()
    first = _prep(w, k, G, w.optics, method=method)
    aug0, _ = first.export_system()
    del first
    free = []
    for _ in range(6):
        p = _prep(w, k, G, w.optics, method=method)
        aug, _ = p.export_system()
        del p
        assert torch.equal(aug, aug0)
        del aug
        torch.cuda.synchronize()
        free.append(torch.cuda.mem_get_info()[0])
    free0, free1 = free[0], free[-1]   # the first round also warms torch's own cache
    _say(f"{method}: device free memory {free0} -> {free1} bytes over five prepares")
    assert free1 == free0
