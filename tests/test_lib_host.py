"""Host-side checks of libks.so that need no GPU: the library loads, exports
every function include/ks.h declares, and rejects bad arguments before it
launches anything."""
import ctypes
import subprocess

import pytest

import kv_cache_compaction_amd as ks
from kv_cache_compaction_amd import _lib

FAKE = ctypes.c_void_p(4096)  # aligned non-null; never dereferenced on these paths


@pytest.fixture(scope="module")
def lib():
    return ks.load_library()


def test_exports_every_declared_symbol(lib):
    import glob
    import os
    names = sorted({n for h in glob.glob(os.path.join(os.path.dirname(ks._lib.HEADER), "*.h"))
                    for n in ks.header_functions(h)})
    assert {"ks_rope_logical", "ks_evict_attn_fwd", "ks_evict_attn_bwd",
            "ks_compact_block_table", "ks_paged_decode", "ks_last_error"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", ks.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(lib, n)
    assert lib.ks_version().startswith(b"libks")


def _status(lib, fn, *args):
    st = getattr(lib, fn)(*args)
    return st, lib.ks_last_error().decode()


def test_compaction_rejects_aliasing(lib):
    st, msg = _status(lib, "ks_compact_block_table", FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                      4, 32, None)
    assert st == 1 and "alias" in msg
    st, msg = _status(lib, "ks_compact_block_table", FAKE, FAKE, FAKE, ctypes.c_void_p(1 << 20),
                      FAKE, FAKE, None, 4, 32, None)
    assert st == 1 and "pos_in" in msg
    st, _ = _status(lib, "ks_compact_block_table", None, None, None, None, None, None, None, 0,
                    32, None)
    assert st == 0  # B == 0 is a no-op


def test_attention_argument_checks(lib):
    # Hq not a multiple of Hkv
    st, msg = _status(lib, "ks_evict_attn_fwd", FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 3, 2,
                      128, 1, 0.1, FAKE, 1 << 20, None)
    assert st == 1 and "Hq" in msg
    # unsupported head dim for bf16
    st, _ = _status(lib, "ks_evict_attn_fwd", FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 4, 2, 96,
                    1, 0.1, FAKE, 1 << 20, None)
    assert st == 2
    # workspace too small
    need = lib.ks_evict_attn_fwd_workspace(1, 4096, 8, 2, 128, 1)
    assert need > 0
    st, msg = _status(lib, "ks_evict_attn_fwd", FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4096, 8,
                      2, 128, 1, 0.1, FAKE, need - 1, None)
    assert st == 4 and "workspace" in msg
    # misaligned tensor
    st, msg = _status(lib, "ks_evict_attn_fwd", ctypes.c_void_p(4098), FAKE, FAKE, FAKE, FAKE,
                      FAKE, 1, 64, 4, 2, 128, 1, 0.1, FAKE, 1 << 20, None)
    assert st == 1 and "aligned" in msg
    # backward: fp32 is not provided
    st, _ = _status(lib, "ks_evict_attn_bwd", *([FAKE] * 10), 1, 64, 4, 2, 128, 0, 0.1, FAKE,
                    1 << 20, None)
    assert st == 2
    need_b = lib.ks_evict_attn_bwd_workspace(2, 1000, 8, 2, 128, 1)
    assert need_b >= 2 * 1000 * 8 * 4


def test_decode_and_rope_argument_checks(lib):
    st, _ = _status(lib, "ks_paged_decode", *([FAKE] * 7), 2, 32, 8, 64, 10, 100, 1, 0.1, FAKE,
                    1 << 20, None)
    assert st == 2  # D = 64 not provided for decode
    need = lib.ks_paged_decode_workspace(64, 32, 128, 4097)
    st, msg = _status(lib, "ks_paged_decode", *([FAKE] * 7), 64, 32, 8, 128, 4097, 10, 1, 0.1,
                      FAKE, need - 1, None)
    assert st == 4
    st, _ = _status(lib, "ks_rope_logical", FAKE, FAKE, FAKE, 1, 8, 4, 2, 100, 1, 10000.0, 0,
                    None)
    assert st == 1  # D must be a multiple of 16
    st, _ = _status(lib, "ks_rope_logical", FAKE, FAKE, FAKE, 1, 8, 4, 2, 64, 7, 10000.0, 0,
                    None)
    assert st == 1  # bad dtype


def test_python_binding_error_type():
    err = _lib.KSError("ks_x", 4, "workspace 1 < 2 bytes")
    assert "WORKSPACE_TOO_SMALL" in str(err) and err.status == 4


def test_append_argument_checks(lib):
    st, _ = _status(lib, "ks_append_kv", *([FAKE] * 7), 2, 8, 64, 10, 100, 1, 10000.0, None)
    assert st == 2  # D = 64 not provided
    st, _ = _status(lib, "ks_append_kv", *([FAKE] * 7), 2, 8, 128, 10, 100, 1, 0.5, None)
    assert st == 1  # base must exceed 1
    st, _ = _status(lib, "ks_append_kv", *([FAKE] * 7), 0, 8, 128, 10, 100, 1, 10000.0, None)
    assert st == 0  # nothing to do


def test_compaction_rounds_argument_checks(lib):
    st, msg = _status(lib, "ks_compact_block_table_rounds", FAKE, FAKE, FAKE, 65, FAKE,
                      ctypes.c_void_p(1 << 20), None, None, 4, 32, None)
    assert st == 1 and "rounds" in msg
    st, msg = _status(lib, "ks_compact_block_table_rounds", FAKE, FAKE, FAKE, 2, FAKE,
                      ctypes.c_void_p(1 << 20), None, None, 4, 65537, None)
    assert st == 1 and "max_blocks" in msg
    st, msg = _status(lib, "ks_compact_block_table_rounds", FAKE, FAKE, FAKE, 2, FAKE, FAKE,
                      None, None, 4, 32, None)
    assert st == 1 and "alias" in msg
    st, _ = _status(lib, "ks_compact_block_table_rounds", None, None, None, 3, None, None, None,
                    None, 0, 32, None)
    assert st == 0  # B == 0 is a no-op


def test_single_token_block_argument_checks(lib):
    st, _ = _status(lib, "ks_paged_decode_bs1", *([FAKE] * 7), 2, 32, 8, 64, 10, 100, 1, 0.1,
                    FAKE, 1 << 20, None)
    assert st == 2  # D = 64 not provided
    need = lib.ks_paged_decode_bs1_workspace(64, 32, 128, 65537)
    assert need == lib.ks_paged_decode_workspace(64, 32, 128, 4097)
    st, _ = _status(lib, "ks_paged_decode_bs1", *([FAKE] * 7), 64, 32, 8, 128, 65537, 10, 1,
                    0.1, FAKE, need - 1, None)
    assert st == 4
    st, msg = _status(lib, "ks_paged_decode_bs1", *([FAKE] * 7), 4, 32, 6, 128, 100, 10, 1, 0.1,
                      FAKE, 1 << 20, None)
    assert st == 1 and "Hq" in msg
    st, _ = _status(lib, "ks_append_kv_bs1", *([FAKE] * 7), 2, 8, 128, 10, 100, 1, 0.5, None)
    assert st == 1  # base must exceed 1
    st, _ = _status(lib, "ks_append_kv_bs1", *([FAKE] * 7), 0, 8, 128, 10, 100, 1, 10000.0,
                    None)
    assert st == 0


def test_input_check_argument_checks(lib):
    st, _ = _status(lib, "ks_check_block_table", FAKE, FAKE, 2, 10, 10, 8, FAKE, None)
    assert st == 1  # block size 8
    st, _ = _status(lib, "ks_check_eviction_record", None, 0, 10, None, None)
    assert st == 0  # nothing to check
    st, _ = _status(lib, "ks_check_eviction_record", FAKE, -1, 10, FAKE, None)
    assert st == 1


def test_fused_rope_decode_argument_checks(lib):
    st, msg = _status(lib, "ks_paged_decode_rope", *([FAKE] * 8), 2, 32, 8, 128, 10, 100, 8,
                      1, 0.1, 10000.0, FAKE, 1 << 20, None)
    assert st == 1 and "block_size" in msg
    st, msg = _status(lib, "ks_paged_decode_rope", *([FAKE] * 8), 2, 32, 8, 128, 10, 100, 16,
                      1, 0.1, 0.5, FAKE, 1 << 20, None)
    assert st == 1 and "base" in msg
    need = lib.ks_paged_decode_workspace(2, 32, 128, 10)
    st, msg = _status(lib, "ks_paged_decode_rope", *([FAKE] * 8), 2, 32, 8, 128, 10, 100, 16,
                      1, 0.1, 10000.0, FAKE, need - 1, None)
    assert st == 4 and "workspace" in msg


def test_binding_signatures_match_header():
    """Every function the binding describes has the header's parameter count
    (a wrong count would pass garbage through ctypes without an error)."""
    import glob
    import os
    import re
    decls = {}
    for h in glob.glob(os.path.join(os.path.dirname(ks._lib.HEADER), "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        decls.update(re.findall(r"\b(ks_[a-z0-9_]+)\s*\(([^;{]*)\)\s*;", text))
    for name, (args, _) in _lib._SIGS.items():
        assert name in decls, name
        params = decls[name].strip()
        n = 0 if params in ("", "void") else len(params.split(","))
        assert n == len(args), (name, n, len(args))



def test_decode_pool_must_have_blocks_when_entries_exist(lib):
    need = lib.ks_paged_decode_workspace(2, 32, 128, 10)
    st, msg = _status(lib, "ks_paged_decode", *([FAKE] * 7), 2, 32, 8, 128, 10, 0, 1, 0.1,
                      FAKE, need, None)
    assert st == 1 and "no blocks" in msg
    need1 = lib.ks_paged_decode_bs1_workspace(2, 32, 128, 10)
    st, msg = _status(lib, "ks_paged_decode_bs1", *([FAKE] * 7), 2, 32, 8, 128, 10, 0, 1, 0.1,
                      FAKE, need1, None)
    assert st == 1 and "no blocks" in msg
    # a null table or pool is refused while entries exist
    st, msg = _status(lib, "ks_paged_decode", FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 32, 8,
                      128, 10, 4, 1, 0.1, FAKE, need, None)
    assert st == 1 and "null" in msg


def test_decode_workspace_query_covers_empty_tables(lib):
    """A table with no entries still launches one split per (sequence, head):
    the size query must cover it, so a C caller that sizes the workspace by
    the query gets no KS_ERR_WORKSPACE on the empty-table case."""
    for fn in ("ks_paged_decode_workspace", "ks_paged_decode_bs1_workspace"):
        one = getattr(lib, fn)(4, 32, 128, 1)
        assert one > 0
        assert getattr(lib, fn)(4, 32, 128, 0) == one
        assert getattr(lib, fn)(4, 32, 128, -3) == one
        assert getattr(lib, fn)(0, 32, 128, 0) == 0


def test_fused_rope_attention_argument_checks(lib):
    """The RoPE-fused training entry points refuse bad arguments before any
    launch: fp32, D other than 128, base <= 1, outputs aliasing the inputs
    they are rotated from, short workspaces; empty sizes are no-ops."""
    B, N, H, D = 1, 64, 2, 128
    big = ctypes.c_void_p(1 << 30)      # distinct aligned addresses, never dereferenced
    q, k, qr, kr = (ctypes.c_void_p((i + 1) << 24) for i in range(4))
    need_f = lib.ks_evict_attn_fwd_rope_workspace(B, N, H, H, D, ks.KS_BF16)
    need_b = lib.ks_evict_attn_bwd_rope_workspace(B, N, H, H, D, ks.KS_BF16)
    assert need_f > lib.ks_evict_attn_fwd_workspace(B, N, H, H, D, ks.KS_BF16)
    assert need_b > lib.ks_evict_attn_bwd_workspace(B, N, H, H, D, ks.KS_BF16)
    fwd = lambda *a: _status(lib, "ks_evict_attn_fwd_rope", *a)
    st, _ = fwd(q, k, FAKE, FAKE, FAKE, qr, kr, FAKE, FAKE, B, N, H, H, D, ks.KS_F32, 0.1,
                10000.0, big, need_f, None)
    assert st == 2                                          # fp32: unsupported
    st, _ = fwd(q, k, FAKE, FAKE, FAKE, qr, kr, FAKE, FAKE, B, N, H, H, 64, ks.KS_BF16, 0.1,
                10000.0, big, need_f, None)
    assert st == 2                                          # D = 64: unsupported
    st, msg = fwd(q, k, FAKE, FAKE, FAKE, qr, kr, FAKE, FAKE, B, N, H, H, D, ks.KS_BF16, 0.1,
                  1.0, big, need_f, None)
    assert st == 1 and "base" in msg
    st, msg = fwd(q, k, FAKE, FAKE, FAKE, q, kr, FAKE, FAKE, B, N, H, H, D, ks.KS_BF16, 0.1,
                  10000.0, big, need_f, None)
    assert st == 1 and "alias" in msg                       # q_rot is q
    st, msg = fwd(q, k, FAKE, FAKE, FAKE, qr, k, FAKE, FAKE, B, N, H, H, D, ks.KS_BF16, 0.1,
                  10000.0, big, need_f, None)
    assert st == 1 and "alias" in msg                       # k_rot is k
    v, o = ctypes.c_void_p(5 << 24), ctypes.c_void_p(6 << 24)
    st, msg = fwd(q, k, v, FAKE, FAKE, qr, v, o, FAKE, B, N, H, H, D, ks.KS_BF16, 0.1,
                  10000.0, big, need_f, None)
    assert st == 1 and "overlap" in msg                     # k_rot is v
    st, msg = fwd(q, k, v, FAKE, FAKE, qr, kr, qr, FAKE, B, N, H, H, D, ks.KS_BF16, 0.1,
                  10000.0, big, need_f, None)
    assert st == 1 and "overlap" in msg                     # o is q_rot
    st, _ = fwd(q, k, v, FAKE, FAKE, qr, kr, o, FAKE, B, N, H, H, D, ks.KS_BF16, 0.1,
                10000.0, big, need_f - 1, None)
    assert st == 4                                          # workspace short of the table
    st, msg = fwd(q, k, FAKE, FAKE, FAKE, qr, kr, FAKE, None, B, N, H, H, D, ks.KS_BF16, 0.1,
                  10000.0, big, need_f, None)
    assert st == 1 and "null" in msg                        # lse is required
    st, _ = fwd(None, None, None, None, None, None, None, None, None, 0, N, H, H, D, ks.KS_BF16,
                0.1, 10000.0, None, 0, None)
    assert st == 0                                          # B == 0 is a no-op
    bwd = lambda *a: _status(lib, "ks_evict_attn_bwd_rope", *a)
    st, _ = bwd(qr, kr, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, N, H, H, D,
                ks.KS_BF16, 0.1, 10000.0, big, need_b - 1, None)
    assert st == 4                                          # workspace short of the table
    st, msg = bwd(qr, kr, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, N, H, H, D,
                  ks.KS_BF16, 0.1, 10000.0, big, need_b, None)
    assert st == 1 and "null" in msg                        # pos is required
    st, msg = bwd(qr, kr, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, N, 3, H, D,
                  ks.KS_BF16, 0.1, 10000.0, big, need_b, None)
    assert st == 1 and "Hq" in msg
    st, _ = bwd(None, None, None, None, None, None, None, None, None, None, None, B, 0, H, H, D,
                ks.KS_BF16, 0.1, 10000.0, None, 0, None)
    assert st == 0                                          # N == 0 is a no-op


def test_decode_split_length_follows_the_grid(lib):
    """The decode's split length is chosen from the sizes alone: 48-group
    splits, or 16-group splits when 48-group splits would give fewer than
    4096 waves (four query heads per wave).  The workspace query shows the
    choice: (D + 2) floats per (sequence, head, split), plus 256 bytes."""
    def slots(B, Hq, groups, sg):
        return B * Hq * ((groups + sg - 1) // sg)
    # 8 sequences, 64 heads, 1036-group rows: 8 * 16 * 22 = 2816 waves -> 16
    assert lib.ks_paged_decode_workspace(8, 64, 128, 1036) == slots(8, 64, 1036, 16) * 130 * 4 + 256
    # 64 sequences, 32 heads, 4097-group rows: 64 * 8 * 86 waves -> 48
    assert lib.ks_paged_decode_workspace(64, 32, 128, 4097) == slots(64, 32, 4097, 48) * 130 * 4 + 256
    # just below and at the threshold (one head per wave counted as 4 heads / 4)
    assert lib.ks_paged_decode_workspace(1, 4, 128, 48 * 4095) == slots(1, 4, 48 * 4095, 16) * 130 * 4 + 256
    assert lib.ks_paged_decode_workspace(1, 4, 128, 48 * 4096) == slots(1, 4, 48 * 4096, 48) * 130 * 4 + 256
    # token tables count 16 tokens per group
    assert lib.ks_paged_decode_bs1_workspace(8, 64, 128, 16 * 1036) == \
        lib.ks_paged_decode_workspace(8, 64, 128, 1036)
