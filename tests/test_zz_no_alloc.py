"""The no-allocation sparse decode (fixed library-owned device scratch, for callers that
cannot allocate) against twilight_sparse_decode with a caller's workspace, through the C ABI:
the same kernels, so the outputs must be identical, on two calls in a row, the second with a
smaller input (the fixed buffer then holds the first call's partials). Both are also checked
against the oracle's attention over the same kept sets."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import adaptive_top_sparse_amd as twl  # noqa: E402
from adaptive_top_sparse_amd import workloads  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def _kept_lists(w, p):
    """A decode step's inputs on the GPU: kept lists from the library's own pipeline."""
    from adaptive_top_sparse_amd import pipeline
    c = pipeline.upload(w)
    c.build_caches()
    buf = pipeline.alloc_step(c)
    pipeline.run_step(c, buf, p)
    torch.cuda.synchronize()
    return c, buf


def _both(c, buf):
    lay = c.layout()
    stride = c.cand_stride_pages * twl.PAGE_SIZE
    sm = parity.sm_scale_for(c.d)
    ref = torch.full_like(buf.out, -1.0)
    got = torch.full_like(buf.out, -2.0)
    twl.twilight_sparse_decode(lay, c.q, c.k_cache, c.v_cache, buf.kept, buf.kept_count, stride,
                               sm, ref, buf.workspace)
    twl.twilight_sparse_decode_noalloc(lay, c.q, c.k_cache, c.v_cache, buf.kept, buf.kept_count,
                                       stride, sm, got)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def _check_against_oracle(w, buf, out):
    s = w.spec
    G = s.G
    sm = parity.sm_scale_for(s.d)
    kept = buf.kept.cpu().numpy()
    kc = buf.kept_count.cpu().numpy()
    for b in range(s.B):
        for g in range(s.Hkv):
            k = kept[b, g, :kc[b, g]]
            ref = oracle.sparse_attention(w.q[b, g * G:(g + 1) * G], w.k[b][g], w.v[b][g],
                                                 k, sm)
            err = np.abs(out[b, g * G:(g + 1) * G].astype(np.float64) - ref).max()
            assert err <= parity.OUT_ATOL, (b, g, err)


def test_noalloc_decode_equals_the_workspace_decode_on_two_calls():
    p = 0.9
    # first call: a 128k-token GQA layer (the largest partials of the two)
    print("\n[noalloc] call 1: llama31-8b-gqa n=131072", flush=True)
    w1 = workloads.make_workload(3)
    c1, b1 = _kept_lists(w1, p)
    ref1, got1 = _both(c1, b1)
    assert np.array_equal(ref1.view(np.uint16), got1.view(np.uint16))
    G = w1.spec.G
    sm = parity.sm_scale_for(w1.spec.d)
    kept = b1.kept.cpu().numpy()
    kc = b1.kept_count.cpu().numpy()
    for b, g in [(0, 0), (0, 5)]:  # a unit with planted keys and a plain one
        k = kept[b, g, :kc[b, g]]
        ref = oracle.sparse_attention(w1.q[b, g * G:(g + 1) * G], w1.k[b][g], w1.v[b][g],
                                             k, sm)
        assert np.abs(got1[b, g * G:(g + 1) * G].astype(np.float64) - ref).max() <= parity.OUT_ATOL
    del c1, b1
    torch.cuda.empty_cache()
    # second call: a smaller ragged MHA batch, on the same fixed buffer
    print("[noalloc] call 2: ragged MHA B=4", flush=True)
    w2 = workloads.make_workload(4, B=4, n_range=(40, 3000), budget=32)
    c2, b2 = _kept_lists(w2, 0.85)
    ref2, got2 = _both(c2, b2)
    assert np.array_equal(ref2.view(np.uint16), got2.view(np.uint16))
    _check_against_oracle(w2, b2, got2)
    print("[noalloc] both calls identical to the workspace decode", flush=True)
