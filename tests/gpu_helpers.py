"""Shared helpers of the GPU tests: device upload, descriptors, tolerance checks."""
import numpy as np
import pytest
import torch

import decode_attention_sequence_amd as dcp
import workloads as W

# Tolerances. bf16 / fp8 caches with fp32 accumulation: relative L2 over the
# whole output <= 5e-3, max |O - O*| <= 1e-2, max |LSE - LSE*| <= 1e-3. The fp32
# path accumulates products of fp32 inputs in fp32; its error is a few ulp
# per term times sqrt(length), far below 1e-5 at the tested lengths.
TOL = {
    "bf16": dict(rel_l2=5e-3, max_abs=1e-2, lse_abs=1e-3),
    "fp8": dict(rel_l2=5e-3, max_abs=1e-2, lse_abs=1e-3),
    "f32": dict(rel_l2=1e-5, max_abs=1e-5, lse_abs=1e-5),
}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test started without a visible GPU")
    dcp.lib()  # raises LibraryMissing if libdcp.so is absent


def desc_for(w, dev, out_dtype=dcp.F32, num_shards=None):
    kind = dcp.KV_LATENT if w.spec.kind == "mla" else dcp.KV_SEPARATE
    return dcp.make_desc(kind, dev.q, dev.k_cache, dev.block_table,
                         num_shards=w.spec.num_shards if num_shards is None else num_shards,
                         v_dim=w.spec.v_dim, softmax_scale=w.spec.softmax_scale,
                         max_seq_len=int(max(1, w.seq_lens.max(initial=0))), out_dtype=out_dtype,
                         q_len=getattr(w.spec, "q_len", 1))


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(o, lse, o_ref, lse_ref, *, rel_l2, max_abs, lse_abs, rows=None, label=""):
    """Element-wise comparison with the oracle over the given batch rows.

    Rows whose reference LSE is -inf (no tokens) must be exactly O = 0 and
    LSE = -inf. Returns the measured errors.
    """
    o = to_np(o)
    lse = to_np(lse) if lse is not None else None
    if rows is not None:
        o, o_ref = o[rows], o_ref[rows]
        if lse is not None:
            lse = lse[rows]
        lse_ref = lse_ref[rows]
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    empty = ~np.isfinite(lse_ref)
    if empty.any():
        assert np.all(o[empty] == 0), f"{label}: empty rows must be zero"
        if lse is not None:
            assert np.all(lse[empty] == -np.inf), f"{label}: empty rows must have LSE = -inf"
    live = ~empty
    stats = {"rel_l2": 0.0, "max_abs": 0.0, "lse_abs": 0.0, "worst_seq_rel_l2": 0.0}
    if live.any():
        diff = o[live] - o_ref[live]
        stats["rel_l2"] = float(np.linalg.norm(diff) / max(np.linalg.norm(o_ref[live]), 1e-30))
        stats["max_abs"] = float(np.max(np.abs(diff)))
        if lse is not None:
            stats["lse_abs"] = float(np.max(np.abs(lse[live] - lse_ref[live])))
        per_seq = []
        for b in range(o.shape[0]):
            m = live[b]
            if m.any():
                d = o[b][m] - o_ref[b][m]
                per_seq.append(np.linalg.norm(d) / max(np.linalg.norm(o_ref[b][m]), 1e-30))
        stats["worst_seq_rel_l2"] = float(max(per_seq))
    assert stats["rel_l2"] <= rel_l2, f"{label}: rel L2 {stats['rel_l2']:.3e} > {rel_l2}"
    assert stats["max_abs"] <= max_abs, f"{label}: max abs {stats['max_abs']:.3e} > {max_abs}"
    assert stats["lse_abs"] <= lse_abs, f"{label}: LSE abs {stats['lse_abs']:.3e} > {lse_abs}"
    return stats


def run_all_shards(w, out_dtype=dcp.F32, num_shards=None):
    dev = W.to_torch(w)
    desc = desc_for(w, dev, out_dtype, num_shards)
    o, lse = dcp.decode_all_shards(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                   dev.block_table, dev.seq_lens)
    torch.cuda.synchronize()
    return o, lse, dev, desc


def run_per_shard(w, dev=None, num_shards=None, ownership="interleaved"):
    """remap -> decode_partial for every shard -> (O_r [D,B,H,Dv], LSE_r [D,B,H])."""
    dev = dev or W.to_torch(w)
    d = w.spec.num_shards if num_shards is None else num_shards
    desc = desc_for(w, dev, num_shards=d)
    lt, ll = dcp.block_remap(dev.block_table, dev.seq_lens, w.spec.block_size, d,
                             ownership=ownership)
    ws = dcp.alloc_workspace(desc, dev.q.device)
    outs, lses = [], []
    for r in range(d):
        o, l = dcp.decode_partial(desc, dev.q, dev.k_cache, dev.v_cache, dev.kv_scale,
                                  lt[r].contiguous(), ll[r].contiguous(), workspace=ws)
        outs.append(o.clone())
        lses.append(l.clone())
    torch.cuda.synchronize()
    return torch.stack(outs), torch.stack(lses), lt, ll
