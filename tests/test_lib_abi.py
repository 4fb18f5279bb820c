"""The C ABI on the host (no GPU needed): symbols, struct layout, argument checks.

Calls here either return before any HIP call (argument errors) or touch no
device at all (dcp_workspace_size). Pointers are fake but aligned; on an
argument error the library returns before using them.
"""
import ctypes
import re
import shutil
import subprocess
from pathlib import Path

import pytest

import decode_attention_sequence_amd as dcp

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "dcp.h"
FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced on the host


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dcp_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = dcp.lib()
    names = declared_functions()
    assert set(names) >= {"dcp_block_remap", "dcp_block_remap_ex", "dcp_workspace_size", "dcp_decode_partial",
                          "dcp_lse_merge", "dcp_decode_all_shards", "dcp_status_str",
                          "dcp_version"}
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_descriptor_layout_matches_c(tmp_path):
    fields = [f for f, _ in dcp.AttnDesc._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(dcp_attn_desc_t, {f}));' for f in fields)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "dcp.h"\n'
                   "int main(void) {\n" + body +
                   '\n  printf("sizeof %zu\\n", sizeof(dcp_attn_desc_t));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT / 'include'}", "-I/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    for f in fields:
        assert int(out[f]) == getattr(dcp.AttnDesc, f).offset, f
    assert int(out["sizeof"]) == ctypes.sizeof(dcp.AttnDesc)


def mla_desc(**kw):
    d = dcp.AttnDesc()
    d.struct_size = ctypes.sizeof(dcp.AttnDesc)
    d.batch, d.num_q_heads, d.num_kv_heads, d.qk_dim, d.v_dim = 64, 64, 1, 576, 512
    d.block_size, d.max_blocks_per_seq, d.num_shards = 64, 12024, 8
    d.max_seq_len, d.num_cache_blocks = 769505, 79176
    d.kv_kind, d.q_dtype, d.kv_dtype, d.out_dtype = dcp.KV_LATENT, dcp.BF16, dcp.BF16, dcp.F32
    d.softmax_scale = 1.0 / 24.0
    d.kv_block_stride, d.kv_token_stride, d.kv_head_stride = 64 * 576, 576, 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def gqa_desc(**kw):
    d = mla_desc(num_kv_heads=8, qk_dim=128, v_dim=128, block_size=16, kv_kind=dcp.KV_SEPARATE,
                 max_seq_len=12024 * 16,
                 kv_block_stride=16 * 8 * 128, kv_token_stride=8 * 128, kv_head_stride=128)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def call_all_shards(desc, ws_bytes=1 << 40, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, scale=FAKE, table=FAKE, lens=FAKE, out=FAKE, lse=FAKE, ws=FAKE)
    p.update(ptrs)
    return dcp.lib().dcp_decode_all_shards(ctypes.byref(desc), p["q"], p["k"], p["v"], p["scale"],
                                           p["table"], p["lens"], p["out"], p["lse"], p["ws"],
                                           ws_bytes, None)


def test_valid_descriptors_have_a_workspace():
    for d in (mla_desc(), mla_desc(kv_dtype=dcp.FP8_E4M3, kv_block_stride=64 * 576),
              gqa_desc(), gqa_desc(q_dtype=dcp.F32, kv_dtype=dcp.F32)):
        n = dcp.lib().dcp_workspace_size(ctypes.byref(d))
        # At least one partial slot (fp32 output and LSE) per sequence: the
        # 64-head latent kernel keeps one partial per work group and sequence,
        # the others one per work group and (sequence, shard).
        per = d.batch if d.kv_kind == dcp.KV_LATENT else d.batch * d.num_shards
        assert n >= per * d.num_q_heads * (d.v_dim + 1) * 4


INVALID = [
    ("struct_size", lambda: mla_desc(struct_size=8)),
    ("zero heads", lambda: mla_desc(num_q_heads=0)),
    ("zero shards", lambda: mla_desc(num_shards=0)),
    ("zero block size", lambda: mla_desc(block_size=0)),
    ("max_seq_len above table", lambda: mla_desc(max_seq_len=12024 * 64 + 1)),
    ("negative cache blocks", lambda: mla_desc(num_cache_blocks=-1)),
    ("latent with 2 kv heads", lambda: mla_desc(num_kv_heads=2)),
    ("heads not multiple of kv heads", lambda: gqa_desc(num_q_heads=60)),
    ("misaligned token stride", lambda: mla_desc(kv_token_stride=577)),
    ("nan scale", lambda: mla_desc(softmax_scale=float("nan"))),
    ("bad dtype", lambda: mla_desc(kv_dtype=7)),
    ("negative q_len", lambda: mla_desc(q_len=-1)),
    ("q_len above 64", lambda: gqa_desc(q_len=65)),
]
UNSUPPORTED = [
    ("latent width", lambda: mla_desc(qk_dim=512, v_dim=512, kv_token_stride=512,
                                      kv_block_stride=64 * 512)),
    ("latent heads 48", lambda: mla_desc(num_q_heads=48)),
    ("gqa group 32", lambda: gqa_desc(num_q_heads=256)),
    ("gqa head dim 96", lambda: gqa_desc(qk_dim=96, v_dim=96, kv_head_stride=96,
                                         kv_token_stride=8 * 96, kv_block_stride=16 * 8 * 96)),
    ("gqa mixed dtypes", lambda: gqa_desc(q_dtype=dcp.F32)),
    ("fp8 gqa", lambda: gqa_desc(q_dtype=dcp.BF16, kv_dtype=dcp.FP8_E4M3,
                                  kv_token_stride=8 * 128, kv_block_stride=16 * 8 * 128)),
    ("fp8 output", lambda: mla_desc(out_dtype=dcp.FP8_E4M3)),
    ("latent 5 x 64 query rows", lambda: mla_desc(q_len=5)),
    ("latent 2 x 8 heads", lambda: mla_desc(num_q_heads=8, q_len=2)),
]


@pytest.mark.parametrize("name,make", INVALID, ids=[n for n, _ in INVALID])
def test_invalid_descriptor_rejected(name, make):
    d = make()
    assert dcp.lib().dcp_workspace_size(ctypes.byref(d)) == 0
    assert call_all_shards(d) == dcp.DCP_ERR_INVALID_ARG


@pytest.mark.parametrize("name,make", UNSUPPORTED, ids=[n for n, _ in UNSUPPORTED])
def test_unsupported_descriptor_rejected(name, make):
    d = make()
    assert dcp.lib().dcp_workspace_size(ctypes.byref(d)) == 0
    assert call_all_shards(d) == dcp.DCP_ERR_UNSUPPORTED


def test_pointer_and_workspace_errors():
    d = mla_desc()
    assert call_all_shards(d, q=None) == dcp.DCP_ERR_INVALID_ARG
    assert call_all_shards(d, table=None) == dcp.DCP_ERR_INVALID_ARG
    assert call_all_shards(d, out=None) == dcp.DCP_ERR_INVALID_ARG
    assert call_all_shards(d, q=ctypes.c_void_p((1 << 20) + 2)) == dcp.DCP_ERR_INVALID_ARG
    assert call_all_shards(gqa_desc(), v=None) == dcp.DCP_ERR_INVALID_ARG
    f8 = mla_desc(kv_dtype=dcp.FP8_E4M3)
    assert call_all_shards(f8, scale=None) == dcp.DCP_ERR_INVALID_ARG
    need = dcp.lib().dcp_workspace_size(ctypes.byref(d))
    assert call_all_shards(d, ws_bytes=need - 1) == dcp.DCP_ERR_WORKSPACE
    assert call_all_shards(d, ws=None) == dcp.DCP_ERR_WORKSPACE
    assert call_all_shards(d, ws=ctypes.c_void_p((1 << 20) + 64)) == dcp.DCP_ERR_WORKSPACE


def test_remap_and_merge_argument_errors():
    L = dcp.lib()
    assert L.dcp_block_remap(None, FAKE, 1, 1, 1, 1, FAKE, FAKE, None) == dcp.DCP_ERR_INVALID_ARG
    assert L.dcp_block_remap(FAKE, FAKE, 1, 1, 1, 0, FAKE, FAKE, None) == dcp.DCP_ERR_INVALID_ARG
    assert L.dcp_block_remap(FAKE, FAKE, 0, 1, 1, 1, FAKE, FAKE, None) == dcp.DCP_ERR_INVALID_ARG
    for own in (-1, 2, 99):
        assert L.dcp_block_remap_ex(FAKE, FAKE, 1, 1, 1, 1, own, FAKE, FAKE, None) == \
            dcp.DCP_ERR_INVALID_ARG
    assert L.dcp_block_remap_ex(FAKE, FAKE, 1, 1, 1, 0, dcp.OWN_CONTIGUOUS, FAKE, FAKE, None) == \
        dcp.DCP_ERR_INVALID_ARG
    assert L.dcp_lse_merge(FAKE, FAKE, 0, 1, 1, 4, FAKE, dcp.F32, None, None) == \
        dcp.DCP_ERR_INVALID_ARG
    assert L.dcp_lse_merge(FAKE, FAKE, 2, 1, 1, 6, FAKE, dcp.F32, None, None) == \
        dcp.DCP_ERR_UNSUPPORTED
    assert L.dcp_lse_merge(FAKE, FAKE, 2, 1, 1, 8, FAKE, dcp.FP8_E4M3, None, None) == \
        dcp.DCP_ERR_INVALID_ARG
    assert L.dcp_lse_merge(None, FAKE, 2, 1, 1, 8, FAKE, dcp.F32, None, None) == \
        dcp.DCP_ERR_INVALID_ARG


def test_descriptor_without_q_len_reads_as_single_token():
    d = mla_desc()
    full = dcp.lib().dcp_workspace_size(ctypes.byref(d))
    assert full > 0
    d.struct_size = dcp.AttnDesc.q_len.offset  # a caller built before the q_len field
    d.q_len = 7  # past the caller's struct: never read
    assert dcp.lib().dcp_workspace_size(ctypes.byref(d)) == full
    d.struct_size = dcp.AttnDesc.q_len.offset - 8
    assert dcp.lib().dcp_workspace_size(ctypes.byref(d)) == 0
    d = mla_desc()
    d.q_len = 4  # 4 x 64 query rows per sequence: four times the partial rows
    assert dcp.lib().dcp_workspace_size(ctypes.byref(d)) > full
    d.q_len = 5  # 320 rows: more than the latent kernels take
    assert dcp.lib().dcp_workspace_size(ctypes.byref(d)) == 0


def test_append_update_and_mtp_argument_errors():
    """Argument errors of the per-step entry points return before any HIP call."""
    L = dcp.lib()
    d = mla_desc()

    def append(desc=d, n=1, shard=-1, new_dtype=dcp.BF16, k_new=FAKE, pos=FAKE, table=FAKE,
               k=FAKE, scale=FAKE):
        return L.dcp_kv_append(ctypes.byref(desc), n, None, pos, k_new, None, new_dtype, shard,
                               table, k, None, scale, None)

    assert append(n=-1) == dcp.DCP_ERR_INVALID_ARG
    assert append(shard=8) == dcp.DCP_ERR_INVALID_ARG
    assert append(shard=-2) == dcp.DCP_ERR_INVALID_ARG
    assert append(new_dtype=dcp.F32) == dcp.DCP_ERR_UNSUPPORTED  # bf16 cache takes bf16 rows
    assert append(new_dtype=9) == dcp.DCP_ERR_INVALID_ARG
    assert append(pos=None) == dcp.DCP_ERR_INVALID_ARG
    assert append(k_new=ctypes.c_void_p((1 << 20) + 8)) == dcp.DCP_ERR_INVALID_ARG
    assert append(desc=mla_desc(num_q_heads=0)) == dcp.DCP_ERR_INVALID_ARG
    f8 = mla_desc(kv_dtype=dcp.FP8_E4M3)
    assert append(desc=f8, scale=None) == dcp.DCP_ERR_INVALID_ARG
    assert append(desc=f8, new_dtype=dcp.FP8_E4M3) == dcp.DCP_ERR_UNSUPPORTED
    assert append(n=0, pos=None) == dcp.DCP_OK  # nothing to write, nothing enqueued
    g = gqa_desc()
    assert L.dcp_kv_append(ctypes.byref(g), 1, None, FAKE, FAKE, None, dcp.BF16, -1, FAKE, FAKE,
                           FAKE, None, None) == dcp.DCP_ERR_INVALID_ARG  # GQA needs v rows
    assert L.dcp_block_remap_update(FAKE, None, FAKE, 1, 1, 1, 1, FAKE, FAKE, None) == \
        dcp.DCP_ERR_INVALID_ARG
    assert L.dcp_block_remap_update(FAKE, FAKE, FAKE, 0, 1, 1, 1, FAKE, FAKE, None) == \
        dcp.DCP_ERR_INVALID_ARG
    assert L.dcp_block_remap_update(FAKE, FAKE, FAKE, 1, 1, 1, 0, FAKE, FAKE, None) == \
        dcp.DCP_ERR_INVALID_ARG

    def mtp(desc, shard=0, qpos=FAKE):
        return L.dcp_decode_partial_mtp(ctypes.byref(desc), shard, qpos, FAKE, FAKE, None, None,
                                        FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)

    m2 = mla_desc(q_len=2)
    assert mtp(m2, shard=8) == dcp.DCP_ERR_INVALID_ARG
    assert mtp(m2, shard=-1) == dcp.DCP_ERR_INVALID_ARG
    assert mtp(m2, qpos=None) == dcp.DCP_ERR_INVALID_ARG
    assert L.dcp_decode_partial(ctypes.byref(m2), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE,
                                FAKE, 1 << 40, None) == dcp.DCP_ERR_INVALID_ARG


def test_status_strings_and_version():
    assert dcp.status_str(0) == "ok"
    assert "workspace" in dcp.status_str(3)
    assert dcp.version() >= 100


def call_partial_token(desc, shard, ws_bytes=1 << 40):
    return dcp.lib().dcp_decode_partial_token(ctypes.byref(desc), shard, FAKE, FAKE, FAKE, FAKE,
                                              FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)


def test_token_partial_argument_errors():
    """Token-level interleave: blocks must split evenly over the shards, the shard
    index must be in range and the call is single-token; all rejected on the host
    before anything is enqueued."""
    assert call_partial_token(mla_desc(block_size=64, num_shards=3,
                                       max_blocks_per_seq=12024), 0) == dcp.DCP_ERR_UNSUPPORTED
    assert call_partial_token(gqa_desc(num_shards=3), 1) == dcp.DCP_ERR_UNSUPPORTED
    assert call_partial_token(mla_desc(), -1) == dcp.DCP_ERR_INVALID_ARG
    assert call_partial_token(mla_desc(), 8) == dcp.DCP_ERR_INVALID_ARG
    assert call_partial_token(mla_desc(q_len=2), 0) == dcp.DCP_ERR_INVALID_ARG
    assert call_partial_token(mla_desc(), 0, ws_bytes=16) == dcp.DCP_ERR_WORKSPACE


def test_plan_and_run_argument_errors():
    """Plan / run entry points: the unplanned calls' host checks, all rejected
    before anything is enqueued (every workspace here is too small to plan in)."""
    L = dcp.lib()

    def pplan(desc, lens=FAKE, n=16):
        return L.dcp_decode_partial_plan(ctypes.byref(desc), lens, FAKE, n, None)

    def prun(desc, q=FAKE, table=FAKE, o=FAKE, lse=FAKE, n=16):
        return L.dcp_decode_partial_run(ctypes.byref(desc), q, FAKE, FAKE, FAKE, table, o, lse,
                                        FAKE, n, None)

    def aplan(desc, lens=FAKE, n=16):
        return L.dcp_decode_all_shards_plan(ctypes.byref(desc), lens, FAKE, n, None)

    def arun(desc, q=FAKE, table=FAKE, out=FAKE, n=16):
        return L.dcp_decode_all_shards_run(ctypes.byref(desc), q, FAKE, FAKE, FAKE, table, out,
                                           FAKE, FAKE, n, None)

    d = mla_desc()
    for call in (pplan, prun, aplan, arun):
        assert call(d) == dcp.DCP_ERR_WORKSPACE
        assert call(mla_desc(num_q_heads=0)) == dcp.DCP_ERR_INVALID_ARG
        assert call(mla_desc(out_dtype=dcp.FP8_E4M3)) == dcp.DCP_ERR_UNSUPPORTED
    assert pplan(d, lens=None) == dcp.DCP_ERR_INVALID_ARG
    assert aplan(d, lens=None) == dcp.DCP_ERR_INVALID_ARG
    assert pplan(mla_desc(q_len=2)) == dcp.DCP_ERR_INVALID_ARG
    assert prun(mla_desc(q_len=2)) == dcp.DCP_ERR_INVALID_ARG
    assert prun(d, q=None) == dcp.DCP_ERR_INVALID_ARG
    assert prun(d, table=None) == dcp.DCP_ERR_INVALID_ARG
    assert prun(d, o=None) == dcp.DCP_ERR_INVALID_ARG
    assert prun(d, lse=None) == dcp.DCP_ERR_INVALID_ARG
    assert prun(d, o=ctypes.c_void_p((1 << 20) + 4)) == dcp.DCP_ERR_INVALID_ARG
    assert arun(d, q=None) == dcp.DCP_ERR_INVALID_ARG
    assert arun(d, table=None) == dcp.DCP_ERR_INVALID_ARG
    assert arun(d, out=None) == dcp.DCP_ERR_INVALID_ARG
    assert arun(gqa_desc(), n=16) == dcp.DCP_ERR_WORKSPACE
