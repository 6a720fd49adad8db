"""The C ABI: the library loads, exports every function include/*.h declares,
and its host-only paths (capacity, workspace size, status text, argument
validation that returns before any launch) behave as documented. No GPU."""
import ctypes
import glob
import os
import re

import pytest

from tests.conftest import ROOT


def _declared():
    names = set()
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def G():
    import __graft_entry__ as entry
    B = entry._build_module()   # by path: the package import needs a built library
    if not os.path.exists(B.LIB):
        B.build()
    import grouped_expert_ffn_amd as G
    return G


def test_every_declared_symbol_is_exported(G):
    names = _declared()
    assert names >= {"moe_route", "moe_permute", "moe_grouped_ffn", "moe_unpermute_combine",
                     "moe_layer_forward", "moe_topk_from_logits", "moe_workspace_size",
                     "moe_capacity_from_factor", "moe_status_str"}
    lib = ctypes.CDLL(G.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert set(G.EXPORTED) == names


def test_capacity_from_factor(G):
    assert G.capacity_from_factor(1.0, 4096, 2, 8) == 1024
    assert G.capacity_from_factor(1.25, 16384, 8, 128) == 1280
    assert G.capacity_from_factor(1.0, 10, 1, 3) == 3
    assert G.capacity_from_factor(None, 10, 1, 3) == -1


def test_workspace_size_grows_with_rows(G):
    a = G.workspace_size(G.make_desc(8192, 4096, 8, 2, 14336, "bf16", "softmax_topk_renorm", "swiglu"))
    b = G.workspace_size(G.make_desc(4096, 4096, 8, 2, 14336, "bf16", "softmax_topk_renorm", "swiglu"))
    assert a > b > 0 and a % 256 == 0
    # the activation buffer dominates: max_rows * d_ff bf16
    assert a >= 16384 * 14336 * 2


def test_status_strings(G):
    for s in range(9):
        assert G.status_str(s)
    assert G.status_str(0) == "ok"


def _call_route(G, desc, h=1024, ws=None, ws_bytes=0):
    lib = G._lib
    p = ctypes.c_void_p
    return lib.moe_route(ctypes.byref(desc) if desc is not None else None, p(h), p(1024), None,
                         p(2048), p(4096), p(8192), p(16384), p(ws), ws_bytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("k", 0, 2), ("k", 17, 2), ("k", 9, 2), ("E", 2000, 2), ("ep_size", 3, 2),
    ("ep_rank", 1, 2), ("dtype", 5, 4), ("gate", 9, 5), ("act", 7, 5), ("d", 100, 2),
    ("d_ff", 96, 2), ("max_rows", 1 << 31, 2), ("reserved", 1, 2),
])
def test_bad_descriptors_rejected_before_launch(G, field, value, status):
    desc = G.make_desc(64, 128, 8, 2, 128, "bf16", "softmax", "swiglu")
    setattr(desc, field, value)
    assert _call_route(G, desc) == status


def test_null_and_alignment_and_workspace_errors(G):
    desc = G.make_desc(64, 128, 8, 2, 128, "bf16", "softmax", "swiglu")
    assert _call_route(G, None) == 1
    assert _call_route(G, desc, h=0) == 1
    assert _call_route(G, desc, h=1032) == 3           # bf16 data needs 16-byte alignment
    assert _call_route(G, desc, ws=None) == 6           # workspace required
    need = G.workspace_size(desc)
    assert _call_route(G, desc, ws=256, ws_bytes=need - 1) == 6
    assert _call_route(G, desc, ws=300, ws_bytes=need) == 6   # not 256-aligned


def test_bf16_weights_beyond_32bit_tile_offsets_rejected(G):
    """The bf16 expert GEMMs address one expert's gate and up weight rows
    with 32-bit byte offsets from the tile's weight pointer."""
    ok = G.make_desc(64, 4096, 8, 2, 14336, "bf16", "softmax", "swiglu")
    assert G.workspace_size(ok) > 0
    too_wide = G.make_desc(64, 8192, 8, 2, 131072, "bf16", "softmax", "swiglu")
    assert _call_route(G, too_wide) == 2


def test_gather_rejects_token_rows_beyond_32bit_offsets(G):
    """The gathered first GEMM addresses bf16 token rows of h with 32-bit
    byte offsets: T*d*2 must stay below 4 GiB; nothing is launched."""
    lib = G._lib
    p = ctypes.c_void_p
    big = G.make_desc(1 << 19, 4096, 8, 2, 128, "bf16", "softmax", "swiglu")
    st = lib.moe_grouped_ffn_gather(ctypes.byref(big), p(1024), p(2048), p(4096), p(8192),
                                    p(16384), p(32768), None, p(65536), 1 << 40, None)
    assert st == 2
    assert lib.moe_grouped_ffn_gather(None, p(1024), p(2048), p(4096), p(8192), p(16384),
                                      p(32768), None, p(65536), 1 << 40, None) == 1


def test_grouped_ffn_flags_word_is_optional_but_checked(G):
    """moe_grouped_ffn's flags word may be NULL; a misaligned one is refused
    before anything is enqueued."""
    lib = G._lib
    p = ctypes.c_void_p
    desc = G.make_desc(64, 128, 8, 2, 128, "bf16", "softmax", "swiglu")
    args = [p(1024), p(2048), p(4096), p(8192), p(16384)]
    assert lib.moe_grouped_ffn(ctypes.byref(desc), *args, p(1026), p(1 << 20), 1 << 30, None) == 3
    # NULL flags passes the argument checks (then the missing workspace is reported)
    assert lib.moe_grouped_ffn(ctypes.byref(desc), *args, None, None, 0, None) == 6


def _layer_call(G, desc, bufs, ws=None, ws_bytes=0):
    p = ctypes.c_void_p
    return G._lib.moe_layer_forward(ctypes.byref(desc), p(1 << 12), p(1 << 13), None,
                                    p(1 << 14), p(1 << 15), p(1 << 16),
                                    None if bufs is None else ctypes.byref(bufs),
                                    p(ws), ws_bytes, None)


def test_layer_forward_optional_outputs(G):
    """Every buffer of the fused call but y_perm may be NULL (the workspace
    holds those intermediates); a NULL buffers struct or y_perm is refused,
    and a given optional buffer is still checked. All before any launch."""
    desc = G.make_desc(64, 128, 8, 2, 128, "bf16", "softmax", "swiglu")
    assert _layer_call(G, desc, None) == 1
    b = G.LayerBuffers()                       # every field NULL
    assert _layer_call(G, desc, b) == 1        # y_perm is required
    b.y_perm = 1 << 20
    assert _layer_call(G, desc, b) == 6        # only the workspace is missing now
    b.logits = 1 << 21 | 2                     # a given buffer must be aligned
    assert _layer_call(G, desc, b) == 3
    b.logits = None
    b.x_perm = 1 << 22 | 8                     # bf16 rows need 16-byte alignment
    assert _layer_call(G, desc, b) == 3


def test_workspace_holds_the_fused_calls_optional_outputs(G):
    """The workspace has room for every optional output of the fused call:
    logits [T,E] f32, ids, gates and dest [T,k], the inverse map [max_rows]
    twice, counts, offsets, splits and a flag word."""
    T, E, k = 32768, 256, 8
    desc = G.make_desc(T, 7168, E, k, 2048, "bf16", "sigmoid_topk_renorm", "swiglu",
                       ep_size=8)
    need = T * E * 4 + 3 * T * k * 4 + 2 * T * k * 4
    act = T * k * 2048 * 2
    assert G.workspace_size(desc) >= act + need


def test_fp32_allows_any_width(G):
    desc = G.make_desc(64, 30, 4, 2, 50, "f32", "softmax", "relu")
    assert G.workspace_size(desc) > 0


def test_missing_library_fails_loudly(G, monkeypatch):
    """Without the built library the binding raises; nothing falls back to a
    CPU path."""
    monkeypatch.setattr(G, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libmoe_dispatch.so"))
    with pytest.raises(ImportError, match="no CPU fallback"):
        G._load()


def test_product_code_never_reaches_the_oracle():
    """The package (binding, build script, HIP sources) neither imports nor
    names the oracle, so no call of the library can be answered by it."""
    pkg = os.path.join(ROOT, "grouped_expert_ffn_amd")
    files = [p for ext in ("py", "hip", "h", "cpp")
             for p in glob.glob(os.path.join(pkg, "**", f"*.{ext}"), recursive=True)]
    files += glob.glob(os.path.join(ROOT, "include", "*.h"))
    assert files
    for p in files:
        assert not re.search(r"\boracle\b|moe_oracle", open(p).read()), p


def test_permute_no_workspace_limit(G):
    """The no-workspace permute holds its plan histograms in a fixed 2^20-entry
    device array: ceil(T / 128) * E above that is refused with
    MOE_ERR_SCRATCH before anything is enqueued; other argument errors are
    the ones moe_permute reports."""
    p = ctypes.c_void_p
    args = [p(1 << 20)] * 11
    big = G.make_desc(131073, 64, 1024, 2, 64, "bf16", "softmax", "swiglu")   # 1025 tiles
    assert G._lib.moe_permute_no_workspace(ctypes.byref(big), *args, None) == 8
    assert "fixed device scratch" in G.status_str(8)
    assert G._lib.moe_permute_no_workspace(None, *args, None) == 1
    ok = G.make_desc(131072, 64, 1024, 2, 64, "bf16", "softmax", "swiglu")
    args[1] = p(2)            # misaligned topk_idx
    assert G._lib.moe_permute_no_workspace(ctypes.byref(ok), *args, None) == 3
