"""GPU tests of the packing helpers (df_pack_padded / df_unpack_packed,
through the C ABI binding) against the packing oracle: packed rows,
cu_seqlens and max_seqlen must match bit for bit, and unpacking must give
the oracle's padded tensor bit for bit (zeros at invalid positions).

Masks: right-padded with lengths from 0 to L (the pages' case), fully valid,
and masks with holes (valid tokens are packed in order); rows of several
sizes; the L=512 bf16 workload's shape (32 sequences of 512 tokens, hidden
768)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def _mask(kind, B, L, rng):
    if kind == "right":
        lens = rng.integers(0, L + 1, size=B)
        lens[0], lens[-1] = 0, L
        return (np.arange(L)[None, :] < lens[:, None]).astype(np.uint8)
    if kind == "full":
        return np.ones((B, L), dtype=np.uint8)
    return (rng.random((B, L)) < 0.6).astype(np.uint8)


@pytest.mark.parametrize("kind,B,L,row", [
    ("right", 5, 300, (768,)), ("right", 1, 7, (8,)), ("full", 3, 257, (2, 64)),
    ("holes", 4, 600, (16,)), ("right", 32, 512, (768,)),
])
def test_pack_unpack_bit_exact(kind, B, L, row):
    import deberta_disentangled_attention_rel_amd as df
    print(f"pack {kind} B={B} L={L} row={row}", flush=True)
    rng = np.random.default_rng(B * 1000 + L)
    m = _mask(kind, B, L, rng)
    x = torch.from_numpy(rng.standard_normal((B, L) + row)).to(torch.bfloat16)
    ref_p, ref_cu, ref_mx = oracle.pack_padded(x.view(torch.int16).numpy(), m)
    xd, md = x.cuda(), torch.from_numpy(m).cuda()
    packed, cu, mx = df.pack_padded(xd, md)
    torch.cuda.synchronize()
    assert mx == ref_mx
    np.testing.assert_array_equal(cu.cpu().numpy(), ref_cu)
    np.testing.assert_array_equal(packed.cpu().view(torch.int16).numpy(), ref_p)
    back = df.unpack_packed(packed, cu, md)
    torch.cuda.synchronize()
    ref_b = oracle.unpack_packed(ref_p, ref_cu, L, m)
    np.testing.assert_array_equal(back.cpu().view(torch.int16).numpy(), ref_b)


def test_packed_attention_through_helpers():
    """Pack q, k, v with the helpers, run the packed forward, unpack: equal,
    bit for bit, to the packed forward run on the oracle-packed inputs, and
    within the forward tolerance of the padded forward with the same mask."""
    import deberta_disentangled_attention_rel_amd as df
    rng = np.random.default_rng(5)
    B, L, H, D, span, buckets = 3, 200, 2, 64, 64, 32
    att, R = oracle.att_and_rows(span, buckets)
    m = _mask("right", B, L, rng)
    m[0, :L // 2] = 1
    q, k, v = (torch.from_numpy(rng.standard_normal((B, L, H, D)) / 8).to(torch.bfloat16).cuda() for _ in range(3))
    q_r, k_r = (torch.from_numpy(rng.standard_normal((H, R, D)) / 8).to(torch.bfloat16).cuda() for _ in range(2))
    md = torch.from_numpy(m).cuda()
    (qp, cu, mx), (kp, _, _), (vp, _, _) = (df.pack_padded(t, md) for t in (q, k, v))
    out_p, lse_p = df.fwd(qp, kp, vp, q_r, k_r, span, buckets, cu_seqlens=cu, max_seqlen=mx)
    # the same packed forward on inputs packed by the oracle's helper
    packed_ref = [oracle.pack_padded(t.cpu().view(torch.int16).numpy(), m) for t in (q, k, v)]
    ref_cu, ref_mx = packed_ref[0][1], packed_ref[0][2]
    qo, ko, vo = (torch.from_numpy(pr[0]).view(torch.bfloat16).cuda() for pr in packed_ref)
    out_o, lse_o = df.fwd(qo, ko, vo, q_r, k_r, span, buckets, cu_seqlens=torch.from_numpy(ref_cu).cuda(),
                          max_seqlen=ref_mx)
    torch.cuda.synchronize()
    assert torch.equal(out_p.view(torch.int16), out_o.view(torch.int16))
    assert torch.equal(lse_p, lse_o)
    out_u = df.unpack_packed(out_p, cu, md).float().cpu().numpy()
    out_pad, _ = df.fwd(q, k, v, q_r, k_r, span, buckets, key_mask=md.reshape(-1))
    ref = (out_pad.float().cpu().numpy() * m[:, :, None, None])
    err = np.linalg.norm(out_u - ref) / np.linalg.norm(ref)
    print(f"packed vs padded rel-L2 {err:.2e}", flush=True)
    assert err <= 1e-2
