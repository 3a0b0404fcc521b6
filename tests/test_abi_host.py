"""The C-ABI library on the CPU: it loads, exports what include/nexus.h declares,
its structs match the ctypes mirrors, and host-side validation rejects bad
arguments before anything reaches a GPU (no compute calls are made here)."""

import ctypes
import os
import re
import subprocess

import pytest

from streaming_weighted_sampling_amd import _lib
from streaming_weighted_sampling_amd._lib import NxDesc, NxUnit

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nexus.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nx_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libnexus.so not built")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (nx_[a-z_]+)$", nm, flags=re.M))
    assert set(names) <= exported
    assert set(_lib.SIGNATURES) == set(names)


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stddef.h>
#include <stdio.h>
#include "nexus.h"
#define F(s, m) printf(#s "." #m " %zu\n", offsetof(s, m))
int main(void) {
  printf("nx_desc %zu\nnx_unit %zu\n", sizeof(nx_desc), sizeof(nx_unit));
  F(nx_desc, max_out_rows); F(nx_desc, kv_head_stride); F(nx_desc, workspace);
  F(nx_desc, stream); F(nx_desc, n_avg); F(nx_unit, app_v); F(nx_unit, kv_head_stride); F(nx_unit, n_tokens);
  F(nx_unit, seq_id); F(nx_unit, head_cap); F(nx_unit, head_budget);
  F(nx_desc, head_alloc); F(nx_desc, head_floor); F(nx_desc, out_w); F(nx_unit, out_w);
  return 0;
}''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", f"-I{os.path.join(ROOT, 'include')}", str(src), "-o",
                    str(exe)], check=True)
    out = dict(line.rsplit(" ", 1) for line in subprocess.run(
        [str(exe)], capture_output=True, text=True, check=True).stdout.splitlines())
    assert int(out["nx_desc"]) == ctypes.sizeof(NxDesc)
    assert int(out["nx_unit"]) == ctypes.sizeof(NxUnit)
    assert int(out["nx_desc.max_out_rows"]) == NxDesc.max_out_rows.offset
    assert int(out["nx_desc.kv_head_stride"]) == NxDesc.kv_head_stride.offset
    assert int(out["nx_desc.workspace"]) == NxDesc.workspace.offset
    assert int(out["nx_desc.stream"]) == NxDesc.stream.offset
    assert int(out["nx_desc.n_avg"]) == NxDesc.n_avg.offset
    assert int(out["nx_unit.app_v"]) == NxUnit.app_v.offset
    assert int(out["nx_unit.kv_head_stride"]) == NxUnit.kv_head_stride.offset
    assert int(out["nx_unit.n_tokens"]) == NxUnit.n_tokens.offset
    assert int(out["nx_unit.seq_id"]) == NxUnit.seq_id.offset
    assert int(out["nx_unit.head_cap"]) == NxUnit.head_cap.offset
    assert int(out["nx_unit.head_budget"]) == NxUnit.head_budget.offset
    assert int(out["nx_desc.head_alloc"]) == NxDesc.head_alloc.offset
    assert int(out["nx_desc.head_floor"]) == NxDesc.head_floor.offset
    assert int(out["nx_desc.out_w"]) == NxDesc.out_w.offset
    assert int(out["nx_unit.out_w"]) == NxUnit.out_w.offset


def _desc(**kw):
    d = NxDesc()
    d.n_q_heads, d.n_kv_heads, d.head_dim, d.window = 32, 8, 128, 32
    d.dtype, d.lambda_, d.eps_tie = _lib.NX_BF16, 0.5, 1e-6
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.nx_status_str(code).decode().startswith("NX_")
    assert lib.nx_status_str(-99).decode() == "unknown nx_status"
    assert lib.nx_stage_name(0) == b"score_stats"
    assert lib.nx_stage_name(3) == b"walk_coef"
    assert lib.nx_stage_name(6) == b"kv_compact"
    assert lib.nx_stage_name(7) == b"sample_select"
    assert lib.nx_stage_name(8) == b"estimate_keys"
    assert lib.nx_stage_name(9) == b"head_budget"
    assert lib.nx_stage_name(10) == b"unknown"


def test_workspace_query(lib):
    d = _desc()
    small = lib.nx_evict_workspace_bytes(ctypes.byref(d), 4096, 1, 3)
    big = lib.nx_evict_workspace_bytes(ctypes.byref(d), 32768, 32, 3)
    assert 0 < small < big
    # At 32K tokens x 256 head units the intermediates (a, walk rows, keys) dominate.
    assert big >= 256 * 32768 * (4 + 3 * 4 + 8)
    assert lib.nx_evict_workspace_bytes(ctypes.byref(_desc(head_dim=96)), 4096, 1, 3) == 0
    assert lib.nx_evict_workspace_bytes(ctypes.byref(d), 4096, 1, 33) == 0     # H > W
    assert lib.nx_evict_workspace_bytes(ctypes.byref(d), 0, 1, 3) == 0
    assert lib.nx_evict_workspace_bytes(None, 4096, 1, 3) == 0


FAKE = 1 << 40   # never dereferenced: every call below fails validation first


def _step(lib, d, n=4096, b=819, h=3, q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32),
          keep=FAKE + (3 << 32), ok=FAKE + (4 << 32), ov=FAKE + (5 << 32)):
    return lib.nx_evict_step(ctypes.byref(d) if d is not None else None, q, k, v, n, b, h, 0,
                             keep, ok, ov)


def test_host_validation_codes(lib):
    assert _step(lib, None) == _lib.NX_EINVAL
    assert _step(lib, _desc(n_q_heads=30)) == _lib.NX_EINVAL            # H_q % H_kv
    assert _step(lib, _desc(window=0)) == _lib.NX_EINVAL
    assert _step(lib, _desc(), h=33) == _lib.NX_EINVAL                   # H > W
    assert _step(lib, _desc(), h=-1) == _lib.NX_EINVAL
    assert _step(lib, _desc(), b=0) == _lib.NX_EINVAL
    assert _step(lib, _desc(), n=0) == _lib.NX_EINVAL
    assert _step(lib, _desc(n_sink=500, n_recent=500)) == _lib.NX_EINVAL
    assert _step(lib, _desc(), q=None) == _lib.NX_EINVAL
    assert _step(lib, _desc(head_dim=96)) == _lib.NX_EUNSUPPORTED
    assert _step(lib, _desc(dtype=7)) == _lib.NX_EUNSUPPORTED
    assert _step(lib, _desc(window=80), h=65) == _lib.NX_EUNSUPPORTED    # walk depth > 64
    # deep walks (H > 8) need G <= 32: 64 query heads on one KV head is G = 64
    assert _step(lib, _desc(n_q_heads=64, n_kv_heads=1, window=12), h=9) == _lib.NX_EUNSUPPORTED
    assert _step(lib, _desc(), h=9) == _lib.NX_EWORKSPACE                 # deep walk: valid
    assert _step(lib, _desc(), h=32) == _lib.NX_EWORKSPACE                # H = W
    assert _step(lib, _desc(n_q_heads=64, n_kv_heads=2)) == _lib.NX_EUNSUPPORTED  # 1024 rows
    assert _step(lib, _desc(kv_head_stride=100)) == _lib.NX_EINVAL       # stride < N*D
    # outputs overlapping inputs
    assert _step(lib, _desc(), ok=FAKE + (1 << 32) + 64) == _lib.NX_EALIAS
    assert _step(lib, _desc(), ov=FAKE) == _lib.NX_EALIAS
    assert _step(lib, _desc(), keep=FAKE + (4 << 32)) == _lib.NX_EALIAS
    # the weight export overlapping the cache, the keep array or an output
    assert _step(lib, _desc(out_w=FAKE + (1 << 32) + 4096)) == _lib.NX_EALIAS
    assert _step(lib, _desc(out_w=FAKE + (3 << 32))) == _lib.NX_EALIAS
    assert _step(lib, _desc(out_w=FAKE + (5 << 32) + 256)) == _lib.NX_EALIAS
    # valid arguments but no workspace
    assert _step(lib, _desc()) == _lib.NX_EWORKSPACE
    d = _desc(workspace=FAKE + (6 << 32), workspace_bytes=1024)
    assert _step(lib, d) == _lib.NX_EWORKSPACE


def test_stage_entry_points_validate(lib):
    d = _desc()
    assert lib.nx_nexus_weights(ctypes.byref(d), None, FAKE, 4096, 3, FAKE) == _lib.NX_EINVAL
    assert lib.nx_nexus_weights(ctypes.byref(d), FAKE, FAKE, 4096, 3, FAKE) == _lib.NX_EWORKSPACE
    assert lib.nx_reservoir_select(ctypes.byref(d), FAKE, 4096, 0, 0, FAKE, None) == _lib.NX_EINVAL
    assert lib.nx_reservoir_select(ctypes.byref(d), FAKE, 4096, 10, 0, FAKE, None) == \
        _lib.NX_EWORKSPACE
    assert lib.nx_kv_compact(ctypes.byref(d), FAKE, FAKE + (1 << 32), FAKE + (2 << 32), 4096,
                             819, FAKE, FAKE + (4 << 32)) == _lib.NX_EALIAS
    assert lib.nx_kv_compact(ctypes.byref(d), FAKE, FAKE + (1 << 32), FAKE + (2 << 32), 4096,
                             819, FAKE + (3 << 32), FAKE + (4 << 32)) == _lib.NX_EWORKSPACE
    assert lib.nx_evict_batch(ctypes.byref(d), None, 32, 32768, 3, 0) == _lib.NX_EINVAL
    assert lib.nx_evict_batch(ctypes.byref(d), FAKE, 0, 32768, 3, 0) == _lib.NX_EINVAL
    assert lib.nx_evict_batch(ctypes.byref(d), FAKE, 32, 32768, 3, 0) == _lib.NX_EWORKSPACE
    assert lib.nx_evict_batch(ctypes.byref(d), FAKE, 9000, 4096, 3, 0) == _lib.NX_EUNSUPPORTED
    assert lib.nx_read_device_status(None) == _lib.NX_EINVAL
    # per-head budgets: batch calls and nx_head_budgets only
    for mode in (_lib.NX_HEADS_GIVEN, _lib.NX_HEADS_ALLOC):
        assert _step(lib, _desc(head_alloc=mode)) == _lib.NX_EINVAL
        assert lib.nx_reservoir_select(ctypes.byref(_desc(head_alloc=mode)), FAKE, 4096, 10, 0,
                                       FAKE, None) == _lib.NX_EINVAL
    assert _step(lib, _desc(head_alloc=3)) == _lib.NX_EINVAL
    assert _step(lib, _desc(head_floor=-1)) == _lib.NX_EINVAL
    alloc = _desc(head_alloc=_lib.NX_HEADS_ALLOC)
    assert lib.nx_head_budgets(ctypes.byref(_desc()), FAKE, 4096, 10, 0, FAKE) == _lib.NX_EINVAL
    assert lib.nx_head_budgets(ctypes.byref(alloc), None, 4096, 10, 0, FAKE) == _lib.NX_EINVAL
    assert lib.nx_head_budgets(ctypes.byref(alloc), FAKE, 4096, 0, 0, FAKE) == _lib.NX_EINVAL
    assert lib.nx_head_budgets(ctypes.byref(alloc), FAKE, 4096, 10, 0, FAKE) == _lib.NX_EWORKSPACE
    wide = _desc(head_alloc=_lib.NX_HEADS_ALLOC, n_q_heads=512, n_kv_heads=512)
    assert lib.nx_head_budgets(ctypes.byref(wide), FAKE, 4096, 10, 0, FAKE) == \
        _lib.NX_EUNSUPPORTED


def test_static_scratch_holds_the_stated_shape(lib):
    """The no-allocation entry point's scratch covers 8 KV heads x 32768 tokens at
    walk depth 8 (the header's example), and that call rejects larger shapes
    before any launch (no GPU is touched: validation fails first)."""
    d = _desc(window=32)
    assert lib.nx_evict_workspace_bytes(ctypes.byref(d), 32768, 1, 8) <= _lib.NX_SCRATCH_BYTES
    assert lib.nx_evict_workspace_bytes(ctypes.byref(d), 131072, 1, 3) > _lib.NX_SCRATCH_BYTES
    assert lib.nx_evict_step_noalloc(None, FAKE, FAKE, FAKE, 4096, 819, 3, 0, FAKE, FAKE,
                                     FAKE) == _lib.NX_EINVAL
