"""K and V in one launch (rq_encode_kv, rq_encode_append_kv,
rq_encode_append_paged_kv): each must equal the two single-tensor calls bit
for bit. Those calls are checked against the oracle in their own files; the
oracle pins the codes here too, on the one-launch encode."""
import numpy as np
import pytest
import torch

import looped_transformer_kv_rq_amd as rq
import oracle
import workloads
from rq_parity import compare_codes, to_dev, to_host_u16, to_host_words

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _states(rng, shape, n, sigma=0.2):
    ref = workloads.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    xs = [workloads.f32_to_bf16_bits((workloads.bf16_bits_to_f32(ref) + sigma * (l + 1) *
                                      rng.standard_normal(shape)).astype(np.float32)) for l in range(n)]
    return xs, ref


def _outputs(rows, d, bits, fill=0):
    codes = [torch.full(rows + (d * b // 32,), fill, dtype=torch.int32, device=DEV) for b in bits]
    scales = [torch.full(rows + (d // 32,), fill, dtype=torch.int16, device=DEV).view(torch.float16) for _ in bits]
    return codes, scales


def _same(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.float16 else x,
                           y.view(torch.int16) if y.dtype == torch.float16 else y)


@pytest.mark.parametrize("d,s,bits", [(128, 131, (2, 2, 2)), (64, 77, (8, 4, 3, 2)), (128, 64, (4, 3))])
def test_encode_kv_equals_two_encodes(d, s, bits):
    rng = np.random.default_rng(d + s)
    kx, kref = _states(rng, (2, 3, s, d), len(bits))
    vx, vref = _states(rng, (2, 3, s, d), len(bits))
    kd, vd = [to_dev(x) for x in kx], [to_dev(x) for x in vx]
    kr, vr = to_dev(kref), to_dev(vref)
    rows = (2, 3, s)
    kc, ks = _outputs(rows, d, bits, fill=-1)
    vc, vs = _outputs(rows, d, bits, fill=-1)
    rq.encode_kv_into(kd, vd, kr, vr, bits, kc, ks, vc, vs)
    kc1, ks1 = rq.encode(kd, kr, bits)
    vc1, vs1 = rq.encode(vd, vr, bits)
    torch.cuda.synchronize()
    _same(kc + ks + vc + vs, kc1 + ks1 + vc1 + vs1)
    for l, b in enumerate(bits):  # and the oracle's codes, away from thresholds
        ow, os_ = oracle.encode(vx[l], vref, b)
        compare_codes(to_host_words(vc[l]), to_host_u16(vs[l]), ow, os_, vx[l], vref, b)


@pytest.mark.parametrize("t_new", [1, 3])
def test_append_kv_equals_two_appends(t_new):
    """Dense cache of capacity 40; one sequence's positions run past the capacity
    (those write nothing)."""
    rng = np.random.default_rng(t_new)
    d, bits, s_cap = 128, (2, 4), 40
    kx, kref = _states(rng, (3, 2, t_new, d), 2)
    vx, vref = _states(rng, (3, 2, t_new, d), 2)
    pos = torch.tensor([0, 17, s_cap - 2], dtype=torch.int32, device=DEV)
    rows = (3, 2, s_cap)

    def caches():
        kcache = torch.zeros((3, 2, s_cap, d), dtype=torch.bfloat16, device=DEV)
        vcache = torch.zeros_like(kcache)
        return (kcache, vcache) + _outputs(rows, d, bits, fill=7) + _outputs(rows, d, bits, fill=7)

    a = caches()
    rq.encode_append_kv([to_dev(x) for x in kx], [to_dev(x) for x in vx], to_dev(kref), to_dev(vref), bits, pos,
                        a[0], a[1], a[2], a[3], a[4], a[5])
    b = caches()
    rq.encode_append([to_dev(x) for x in kx], to_dev(kref), bits, pos, b[0], b[2], b[3])
    rq.encode_append([to_dev(x) for x in vx], to_dev(vref), bits, pos, b[1], b[4], b[5])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    _same(a[2] + a[3] + a[4] + a[5], b[2] + b[3] + b[4] + b[5])


def test_append_paged_kv_equals_two_paged_appends():
    """Shuffled blocks of 64 positions, one sequence with an unmapped block."""
    rng = np.random.default_rng(9)
    d, bits, P, t_new = 64, (8, 3), 64, 2
    kx, kref = _states(rng, (3, 2, t_new, d), 2)
    vx, vref = _states(rng, (3, 2, t_new, d), 2)
    table = torch.tensor([[3, 0, 5, -1], [1, 7, 4, 6], [8, 2, -1, -1]], dtype=torch.int32, device=DEV)
    pos = torch.tensor([190, 63, 130], dtype=torch.int32, device=DEV)  # sequence 2: an unmapped block
    n_blocks = 9
    rows = (n_blocks, 2, P)

    def caches():
        kp = torch.zeros((n_blocks, 2, P, d), dtype=torch.bfloat16, device=DEV)
        vp = torch.zeros_like(kp)
        return (kp, vp) + _outputs(rows, d, bits, fill=3) + _outputs(rows, d, bits, fill=3)

    a = caches()
    rq.encode_append_paged_kv([to_dev(x) for x in kx], [to_dev(x) for x in vx], to_dev(kref), to_dev(vref), bits,
                              pos, table, a[0], a[1], a[2], a[3], a[4], a[5])
    b = caches()
    rq.encode_append_paged([to_dev(x) for x in kx], to_dev(kref), bits, pos, table, b[0], b[2], b[3])
    rq.encode_append_paged([to_dev(x) for x in vx], to_dev(vref), bits, pos, table, b[1], b[4], b[5])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    _same(a[2] + a[3] + a[4] + a[5], b[2] + b[3] + b[4] + b[5])
