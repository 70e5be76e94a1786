"""The allocation-free MUL merge (intlora_merge_mul_noalloc) against the workspace MUL
merge (intlora_merge_mul), through the C ABI: every output bit for bit, on consecutive
calls that share the library's per-device scratch -- a layer merged in several row
chunks, then a smaller one-chunk layer, then a chunked layer of the general path with a
caller-supplied row range.  Sorted last so that a failure here hides no other test."""
import numpy as np
import pytest
import torch

from integer_rank_adaptation_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from integer_rank_adaptation_amd import ops as _ops

    _ops.B.lib()
    return _ops


def _state(seed, d, n, r, w_bits):
    wr = synth.random_codes(seed, (d, n), w_bits)
    z = synth.random_ints(seed + 1, d, 0, (1 << w_bits) - 1)
    s = synth.random_positive(seed + 2, d, 1e-3, 5e-2)
    c = synth.random_positive(seed + 3, d, 1e-4, 1e-2)
    A = synth.random_matrix(seed + 4, (d, r), 0.5)
    Bm = synth.random_matrix(seed + 5, (r, n), 0.0316)
    if w_bits == 4:
        wr = (wr[:, 0::2] & 15) | ((wr[:, 1::2] & 15) << 4)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return dict(wround=t(wr), z=t(z), s=t(s), c=t(c)), t(A), t(Bm)


# (d, n, r, w_bits, u_bits): several 64 MiB row chunks with a short last one; then one
# chunk; then the general path (n odd, rank 5) in chunks, with saturating 8-bit codes
CASES = [(3072, 12288, 32, 4, 4), (320, 320, 4, 8, 8), (700, 50001, 5, 8, 8)]


def test_noalloc_merge_equals_workspace_merge(ops):
    for k, (d, n, r, w_bits, u_bits) in enumerate(CASES):
        print(f"noalloc case {k}: d={d} n={n} r={r} w_bits={w_bits} u_bits={u_bits}", flush=True)
        st, A, Bm = _state(500 + k, d, n, r, w_bits)
        rng = None
        if k == 2:
            umin, umax = ops.u_minmax(st, A, Bm, w_bits, 9, 3 + k)
            rng = ((umin * 0.75).contiguous(), (umax * 0.75).contiguous())
        ref = ops.merge_mul(st, A, Bm, w_bits, u_bits, 9, 3 + k, dbg=True, u_range=rng)
        got = ops.merge_mul_noalloc(st, A, Bm, w_bits, u_bits, 9, 3 + k, dbg=True, u_range=rng)
        torch.cuda.synchronize()
        for key in ("m", "uround", "sbar", "zbar", "split"):
            assert torch.equal(ref[key], got[key]), (k, key)
        assert int(ref["sat"][0]) == int(got["sat"][0]), k
        if k == 2:
            assert int(got["sat"][0]) > 0  # the chunks' saturation counts add up
        del st, A, Bm, ref, got
