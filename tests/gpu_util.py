"""Helpers shared by the GPU parity tests: moving seeded inputs to the device
and comparing the library's outputs with the oracle's."""
import sys

import numpy as np
import torch

import fp4_microscaling_quantization_quant2d_amd as fq


def note(msg):
    """Name the case on stdout before a GPU step (survives a crashed run)."""
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits -> bfloat16 cuda tensor; float32 -> float32 cuda tensor."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    raise TypeError(x.dtype)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def planes(q: fq.QTensor):
    torch.cuda.synchronize()
    ct = host(q.codes_t) if q.codes_t is not None else None
    return host(q.codes), ct, host(q.scales)


def assert_planes_equal(q: fq.QTensor, ref, what=""):
    c, ct, s = planes(q)
    rc, rct, rs = ref
    assert np.array_equal(s, rs), "%s scales differ at %s" % (what, np.argwhere(s != rs)[:5])
    bad = np.argwhere(c != rc)
    assert bad.size == 0, "%s row plane differs at %s (gpu %s, oracle %s)" % (
        what, bad[:5].tolist(), c[tuple(bad[0])], rc[tuple(bad[0])])
    if rct is not None and ct is not None:
        bad = np.argwhere(ct != rct)
        assert bad.size == 0, "%s transposed plane differs at %s" % (what, bad[:5].tolist())


def check_gemm_tol(got: np.ndarray, ref: np.ndarray, bound: np.ndarray, what=""):
    """The GEMM tolerance: |err| <= 1e-5 * sum_k |a||b| per element."""
    err = np.abs(got.astype(np.float64) - ref)
    tol = 1e-5 * bound
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d elements out of tolerance, first at %s: gpu %r oracle %r "
                             "bound %r" % (what, int(bad.sum()), i.tolist(), got[tuple(i)],
                                           ref[tuple(i)], bound[tuple(i)]))
    return float((err / np.maximum(bound, 1e-300)).max())
