"""One device's share of a sequence split across devices: each shard holds a
disjoint run of every sequence's pages (its own block table and key counts);
pkv_paged_decode_partials runs on every shard, the shards' partials are laid
side by side along the split axis (as an all-gather would), and pkv_combine
merges them.  The result must match the fp64 oracle on the whole problem, as
the one-call path does."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_split_amd as pkv
import workloads

pytestmark = pytest.mark.gpu

from gpu_util import check, dev_tensors, note, problem, run  # noqa: E402


def shard_outputs(w, bounds, splits_per_shard):
    """Partials of each page range [bounds[k], bounds[k+1]) of every
    sequence, merged by pkv_combine; returns (out_bf16 bits, out_f32)."""
    d = dev_tensors(w)
    dev = d["q"].device
    P = w.page_size
    rows = w.B * w.q_len * w.Hq
    o_parts, ml_parts = [], []
    for k in range(len(bounds) - 1):
        p0, p1 = bounds[k], bounds[k + 1]
        j0 = p0 * P
        bt = np.ascontiguousarray(w.block_table[:, p0:p1])
        kl = np.clip(w.kv_lens.astype(np.int64) - j0, 0, (p1 - p0) * P).astype(np.int32)
        S = splits_per_shard[k]
        msb, msq = w.mask_strides
        co = None
        if w.causal_offsets is not None:
            # key j of the shard is key j0 + j of the sequence; a sequence
            # without keys in the shard takes any offset
            c = np.where(kl > 0, w.causal_offsets.astype(np.int64) - j0, 0)
            assert (c >= 0).all()
            co = torch.from_numpy(c.astype(np.int32)).to(dev)
        p = pkv.make_problem(batch=w.B, q_len=w.q_len, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
                             page_size=P, num_pages=w.num_pages, max_pages_per_seq=p1 - p0,
                             max_kv_len=int(kl.max()), scale=w.scale, causal_offset=-1, num_splits=S,
                             mask_stride_b=msb, mask_stride_q=msq)
        ob, mb = pkv.partials_bytes(p, S)
        o_part = torch.empty(ob // 4, dtype=torch.float32, device=dev)
        ml_part = torch.empty(mb // 4, dtype=torch.float32, device=dev)
        mask = None if d["mask"] is None else d["mask"].view(-1)[j0:]   # column j0 onward
        pkv.paged_decode_partials(d["q"], d["k"], d["v"], torch.from_numpy(bt).to(dev), torch.from_numpy(kl).to(dev),
                                  o_part=o_part, ml_part=ml_part, problem=p, causal_offsets=co, mask=mask)
        o_parts.append(o_part.view(rows, S, w.D))
        ml_parts.append(ml_part.view(rows, S, 2))
    o_all = torch.cat(o_parts, dim=1).contiguous()
    ml_all = torch.cat(ml_parts, dim=1).contiguous()
    S_all = o_all.shape[1]
    out32 = torch.empty((rows, w.D), dtype=torch.float32, device=dev)
    out = pkv.combine(o_all, ml_all, rows=rows, splits=S_all, head_dim=w.D, out_f32=out32)
    torch.cuda.synchronize()
    shape = (w.B, w.q_len, w.Hq, w.D)
    return (out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(shape), out32.cpu().numpy().reshape(shape))


CASES = [
    # long sequences, one kv head per matrix-core tile row block; three shards of unequal size
    (lambda: workloads.build("shard_long", B=2, q_len=1, Hq=32, Hkv=8, D=128, page_size=64,
                             kv_lens=[9000, 5000], seed=6001, outlier_p=0.01), [0, 30, 100, 141], [4, 1, 2]),
    # a 2D mask sliced per shard, sequences shorter than some shards (empty shards)
    (lambda: workloads.build("shard_mask", B=3, q_len=1, Hq=8, Hkv=8, D=64, page_size=32,
                             kv_lens=[3000, 700, 40], seed=6002, mask="2d"), [0, 20, 50, 94], [2, 3, 1]),
    # several query tokens with causal offsets at the end of each sequence
    (lambda: workloads.build("shard_causal", B=2, q_len=4, Hq=16, Hkv=2, D=64, page_size=16,
                             kv_lens=[2100, 900], seed=6003, causal="last"), [0, 40, 57, 132], [3, 2, 5]),
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_key_shards_merged_by_combine(i):
    build, bounds, splits = CASES[i]
    w = build()
    assert bounds[-1] == w.max_pages_per_seq
    note(f"sharded {w.name}: page bounds {bounds}, splits {splits}")
    s16, s32 = shard_outputs(w, bounds, splits)
    ref = oracle.decode(w)
    check(s16, s32, ref, f"sharded {w.name}")
    # and it agrees with the one-call path well inside the fp32 bound
    o16, o32 = run(w)
    assert float(np.abs(o32.astype(np.float64) - s32).max()) <= 1e-4
