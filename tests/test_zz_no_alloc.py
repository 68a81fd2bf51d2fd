"""infini_decode_noalloc against infini_decode: same outputs, cache writes and
state, bit for bit, on two calls in a row (the second smaller), each checked
against a call of the workspace entry point on copies of the same buffers.

The second call runs after the first has left its own values in the static
scratch, so a read of anything the call did not write first would show."""
import numpy as np
import pytest

from compressive_linear_memory_amd import inputs as I
from gpu_util import dev, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressive_linear_memory_amd import binding
    binding.lib()


def _inputs(Bn, Hq, Hkv, T, d, L, pos, dtype, seed):
    g = np.random.default_rng(seed)
    draw = lambda *shp: I.storage(g.standard_normal(shp).astype(np.float32) / np.float32(np.sqrt(d)), dtype)
    q, k, v = draw(Bn, Hq, T, d), draw(Bn, Hkv, T, d), draw(Bn, Hkv, T, d)
    kc, vc = draw(Bn, Hkv, L, d), draw(Bn, Hkv, L, d)           # rows >= pos are overwritten or unread
    Kp, Vp = draw(Bn, Hkv, 40, d), draw(Bn, Hkv, 40, d)
    # a consistent carried state: sums over 40 earlier tokens of sigma(K)^T V, sigma(K)
    sk = np.where(Kp > 0, Kp + 1.0, np.exp(np.minimum(Kp, 0.0)))
    M = np.einsum("bhta,bhtc->bhac", sk, Vp).astype(np.float32)
    z = sk.sum(axis=2).astype(np.float32)
    beta = g.standard_normal(Hq).astype(np.float32)
    return q, k, v, kc, vc, M, z, beta


CALLS = [
    # B, Hq, Hkv, T, d, L, pos, dtype: the first completes its segment (key
    # splits and the memory update use the scratch), the second is smaller
    (2, 8, 2, 112, 128, 512, 400, "bf16"),
    (1, 4, 4, 2, 64, 300, 150, "bf16"),
]


def test_decode_noalloc_equals_decode_two_calls():
    from compressive_linear_memory_amd import binding as Bi
    for n, (Bn, Hq, Hkv, T, d, L, pos, dtype) in enumerate(CALLS):
        log(f"noalloc call {n}: B{Bn} Hq{Hq} Hkv{Hkv} T{T} d{d} L{L} pos{pos} {dtype}")
        q, k, v, kc, vc, M, z, beta = _inputs(Bn, Hq, Hkv, T, d, L, pos, dtype, 40 + n)
        tq, tk, tv, tb, tM, tz = dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(beta), dev(M), dev(z)
        closes = pos + T == L
        res = []
        for noalloc in (False, True):
            kcache, vcache = dev(kc, dtype), dev(vc, dtype)
            out = torch.empty_like(tq)
            state = (torch.empty_like(tM), torch.empty_like(tz)) if closes else None
            if noalloc:
                r = Bi.decode_noalloc(tq, tk, tv, tb, L, pos, kcache, vcache, tM, tz, out=out, state_out=state)
            else:
                r = Bi.decode(tq, tk, tv, tb, L, pos, kcache, vcache, tM, tz, out=out, state_out=state)
            torch.cuda.synchronize()
            res.append((out, kcache, vcache) + (state if closes else ()))
        for a, b in zip(*res):
            assert torch.equal(a, b)
        assert bool(torch.isfinite(res[1][0].float()).all())
        log(f"   equal to infini_decode ({len(res[0])} tensors)")
