"""Plant one plausible mistake at a time in a copy of the oracle; a pin must catch it.

Each mutant is a copy of the oracle package with one source substitution
(a dropped term, a wrong sign or index, a transposed operand, a wrong
constant). All of this runs on the CPU.
"""
import importlib.util
import shutil
import sys
from pathlib import Path

import pytest

from oracle_pins import ALL_CHECKS

ORACLE = Path(__file__).resolve().parent.parent / "oracle"

MUTANTS = [
    ("attention.py", "heads = slice(g * group, (g + 1) * group)", "heads = slice(g, hq, hkv)",
     "query head h reads KV head h % Hkv"),
    ("attention.py", "s = scale * (q[heads] @ k[:, g, :].T)", "s = (q[heads] @ k[:, g, :].T)",
     "softmax scale dropped"),
    ("attention.py", "lse_g = m[:, 0] + np.log(", "lse_g = np.log(", "max term dropped from LSE"),
    ("attention.py", "p = np.exp(s - lse_g[:, None])", "p = np.exp(s - m)",
     "partial output left unnormalised"),
    ("attention.py", "out[heads] = p @ v[:, g, :]", "out[heads] = p @ v[:, 0, :]",
     "value always from KV head 0"),
    ("attention.py", "s = scale * (q[heads] @ k[:, g, :].T)",
     "s = scale * (q[heads][:, ::-1] @ k[:, g, :].T)", "query reversed against key"),
    ("attention.py", "return k, k[:, :, : spec.v_dim]", "return k, k[:, :, -spec.v_dim:]",
     "MLA value taken from the last columns"),
    ("attention.py", "k = k * sigma.reshape((-1,) + (1,) * (k.ndim - 1))",
     "k = k / sigma.reshape((-1,) + (1,) * (k.ndim - 1))", "fp8 scale divided"),
    ("attention.py", "return _decode(w.q[b], w.spec.q_dtype)",
     "return _decode(w.q[0], w.spec.q_dtype)", "query of sequence 0 used for all"),
    ("attention.py", "weight = e / np.where(live, denom, 1.0)", "weight = e",
     "merge weights not normalised"),
    ("attention.py", "lse_out = np.where(live, shift + np.log(", "lse_out = np.where(live, np.log(",
     "merged LSE misses the shift"),
    ("attention.py", "e = np.exp(lse - shift)", "e = np.exp(shift - lse)", "merge weight sign"),
    ("attention.py", "merged = (o * factor[..., None]).sum(axis=0) / safe[..., None]",
     "merged = o.sum(axis=0) / safe[..., None]", "(m, l) merge drops the rescale"),
    ("attention.py", "total = (l * factor).sum(axis=0)", "total = l.sum(axis=0)",
     "(m, l) merge sums l without rescale"),
    ("attention.py", "if owner_of_block(j, num_shards, ownership, nb) == shard:",
     "if owner_of_block(j, num_shards, ownership, nb) == (shard + 1) % num_shards:",
     "shard tokens shifted"),
    ("attention.py", "seen = max(0, p + 1)", "seen = max(0, p)", "causal mask hides the query's own position"),
    ("attention.py", "keep = pos <= p", "keep = pos < p", "shard causal mask off by one"),
    ("attention.py", "return [int(w.seq_lens[b]) - n + t for t in range(n)]",
     "return [int(w.seq_lens[b]) - 1 - t for t in range(n)]", "query positions reversed"),
    ("attention.py", "rows = slice(t * hq, (t + 1) * hq)\n            seen",
     "rows = slice(t, n * hq, n)\n            seen", "queries read head-major"),
    ("paged.py", "return j // chunk_of(nb, num_shards)",
     "return min(num_shards - 1, j * num_shards // max(nb, 1))", "contiguous chunks balanced differently"),
    ("paged.py", "return j % num_shards", "return (j + 1) % num_shards", "owner off by one"),
    ("paged.py", "return t % num_shards", "return (t + 1) % num_shards", "token owner off by one"),
    ("paged.py", "return t // num_shards", "return t // num_shards + (t % num_shards > 0)",
     "token local index rounded up"),
    ("attention.py", "if owner_of_token(t, num_shards) == shard]",
     "if owner_of_token(t // block_size, num_shards) == shard]",
     "token ownership taken per block"),
    ("paged.py", "return j // num_shards", "return (j + 1) // num_shards", "local index off by one"),
    ("paged.py", "return cache[phys, pos % block_size]",
     "return cache[phys, (block_size - 1) - pos % block_size]", "slot reversed in block"),
    ("paged.py", "phys = np.asarray(table_row, dtype=np.int64)[pos // block_size]",
     "phys = np.asarray(table_row, dtype=np.int64)[pos // block_size * 0]",
     "block table ignored"),
    ("paged.py", "return max(0, min(block_size, seq_len - j * block_size))",
     "return max(0, min(block_size, seq_len - j * block_size + 1))", "last block over-counted"),
    ("paged.py", "local[r, b, i] = table[b, j]", "local[r, b, i] = table[b, i]",
     "remap reads the local index"),
    ("codecs.py", "(e - 7)", "(e - 8)", "e4m3 bias"),
    ("codecs.py", "np.ldexp(m / 8.0, -6)", "np.ldexp(m / 8.0, -7)", "e4m3 subnormal scale"),
    ("codecs.py", "(b << np.uint32(16))", "(b << np.uint32(15))", "bf16 shift"),
    ("codecs.py", "n = np.rint(np.ldexp(a, -(e - 3)))", "n = np.floor(0.5 + np.ldexp(a, -(e - 3)))",
     "e4m3 encode rounds ties away from even"),
    ("codecs.py", "e = np.maximum(k.astype(np.int64) - 1, -6)", "e = np.maximum(k.astype(np.int64) - 1, -7)",
     "e4m3 encode subnormal spacing"),
    ("codecs.py", "a = np.minimum(np.abs(y), E4M3_MAX)", "a = np.abs(y)", "e4m3 encode not saturated"),
    ("append.py", "sigma = amax / np.float32(E4M3_MAX)", "sigma = amax / np.float32(240.0)",
     "fp8 scale for the wrong format maximum"),
    ("append.py", "y = x32 * inv", "y = x32 * inv * np.float32(0.5)", "fp8 values not stretched to 448"),
    ("append.py", "j = j // num_shards", "j = j % num_shards", "append local index"),
    ("append.py", "return int(table_row[j]), position % block_size",
     "return int(table_row[j]), (position + 1) % block_size", "append slot off by one"),
    ("append.py", "if j % num_shards != shard:", "if j % num_shards == shard:",
     "append writes the tokens of the other shards"),
]


def _load_mutant(tmp_path, idx, fname, old, new):
    dst = tmp_path / f"oracle_mut{idx}"
    shutil.copytree(ORACLE, dst)
    path = dst / fname
    src = path.read_text()
    assert src.count(old) >= 1, f"mutation anchor missing in {fname}: {old!r}"
    path.write_text(src.replace(old, new, 1))
    name = f"oracle_mut{idx}"
    spec = importlib.util.spec_from_file_location(name, dst / "__init__.py",
                                                  submodule_search_locations=[str(dst)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("idx", range(len(MUTANTS)), ids=[m[3] for m in MUTANTS])
def test_pin_catches_mutant(tmp_path, idx):
    fname, old, new, _ = MUTANTS[idx]
    mod = _load_mutant(tmp_path, idx, fname, old, new)
    caught = []
    try:
        for check in ALL_CHECKS:
            try:
                check(mod)
            except Exception as e:  # noqa: BLE001 - any failure counts as caught
                caught.append((check.__name__, type(e).__name__))
                break
    finally:
        for key in [k for k in sys.modules if k.startswith(f"oracle_mut{idx}")]:
            del sys.modules[key]
    assert caught, f"no pin catches mutant: {MUTANTS[idx][3]}"
