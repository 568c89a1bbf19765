"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

import expert_ffn_layer_gemm_amd as moe
from expert_ffn_layer_gemm_amd._binding import SIGNATURES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declarations_match_binding():
    assert _declared_functions() == sorted(SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = moe.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_shape_struct_matches_header():
    fields = re.search(r"typedef struct \{(.*?)\} moe_shape;", open(HEADER).read(), re.S).group(1)
    names = re.findall(r"int32_t (\w+);", fields)
    assert names == [f for f, _ in moe.MoeShape._fields_]
    assert ctypes.sizeof(moe.MoeShape) == 4 * len(names)


def test_workspace_alias():
    # moe_workspace_bytes is the layer-level name of moe_forward_workspace_bytes
    for sh in (moe.make_shape(64, 4096, 128, 8, 1536), moe.make_shape(4096, 7168, 256, 8, 2048, 1, "fp8"),
               moe.make_shape(64, 4096, 128, 8, 1536, 0, "mxfp8", 16, 16), moe.make_shape(64, 100, 8, 2, 128)):
        assert moe.moe_workspace_bytes(sh) == moe.moe_forward_workspace_bytes(sh)
    assert moe.moe_workspace_bytes(moe.make_shape(64, 100, 8, 2, 128)) == 0


def test_abi_version():
    assert moe.moe_abi_version() == 5


FAKE = 0x10000  # a non-NULL, aligned address; never dereferenced (validation fails first)


def _call(fn, *args):
    return getattr(moe.lib(), fn)(*args)


def test_workspace_sizes_and_bad_shapes():
    good = moe.make_shape(64, 4096, 128, 8, 1536)
    assert moe.moe_forward_workspace_bytes(good) > moe.moe_ffn_workspace_bytes(good) > 64 * 8 * 1536 * 2
    r = moe.moe_route_workspace_bytes(good)          # partial sums [KS][T][E] fp32, or none
    assert r >= 0 and r % (64 * 128 * 4) == 0
    fp8 = moe.make_shape(4096, 7168, 256, 8, 2048, 1, "fp8")
    assert moe.moe_ffn_workspace_bytes(fp8) >= 4096 * 9 * 2048
    for bad in (moe.make_shape(64, 100, 128, 8, 1536), moe.make_shape(64, 4096, 128, 8, 100),
                moe.make_shape(64, 4096, 4, 8, 1536), moe.make_shape(64, 4096, 2048, 8, 1536),
                moe.make_shape(64, 4096, 128, 17, 1536), moe.make_shape(64, 4096, 128, 8, 1536, 2),
                moe.make_shape(-1, 4096, 128, 8, 1536), moe.MoeShape(64, 4096, 128, 8, 1536, 0, 7)):
        assert moe.moe_forward_workspace_bytes(bad) == 0
        assert moe.moe_ffn_workspace_bytes(bad) == 0


def test_error_codes_before_launch():
    sh = moe.make_shape(64, 256, 8, 2, 512)
    P = ctypes.byref
    # NULL shape
    assert _call("moe_route", None, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    # NULL / misaligned pointers
    assert _call("moe_route", P(sh), None, FAKE, None, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert "x is NULL" in moe.moe_last_error()
    assert _call("moe_route", P(sh), FAKE + 2, FAKE, None, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert "aligned" in moe.moe_last_error()
    # router workspace missing when H is split (slices of at least 256 channels)
    assert moe.moe_route_workspace_bytes(sh) == 0
    sh_split = moe.make_shape(64, 1024, 8, 2, 512)
    assert moe.moe_route_workspace_bytes(sh_split) == 4 * 64 * 8 * 4
    assert _call("moe_route", P(sh_split), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_WORKSPACE
    # unsupported shapes
    bad = moe.make_shape(64, 256, 8, 9, 512)
    assert _call("moe_route", P(bad), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_UNSUPPORTED
    assert _call("moe_route_from_logits", P(bad), FAKE, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    bad_dt = moe.MoeShape(64, 256, 8, 2, 512, 0, 3)
    assert _call("moe_combine", P(bad_dt), FAKE, FAKE, FAKE, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    # the shared rows' start comes from offsets
    sh1 = moe.make_shape(64, 256, 8, 2, 512, 1)
    assert _call("moe_combine", P(sh1), FAKE, FAKE, FAKE, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert "offsets is NULL" in moe.moe_last_error()
    # workspace too small / missing
    need = moe.moe_forward_workspace_bytes(sh)
    args = [P(sh), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None, FAKE, None, None]
    assert _call("moe_forward", *args, FAKE, need - 1, None) == moe.MOE_ERR_WORKSPACE
    assert _call("moe_forward", *args, None, need, None) == moe.MOE_ERR_WORKSPACE
    assert _call("moe_forward", *args, FAKE + 16, need, None) == moe.MOE_ERR_INVALID_ARG
    ffn_need = moe.moe_ffn_workspace_bytes(sh)
    assert _call("moe_grouped_ffn", P(sh), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, None,
                 FAKE, FAKE, ffn_need - 256, None) == moe.MOE_ERR_WORKSPACE
    # fp8 needs every scale pointer
    s8 = moe.make_shape(64, 256, 8, 2, 512, 0, "fp8")
    assert _call("moe_grouped_ffn", P(s8), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                 FAKE, FAKE, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    assert "x_perm_scale" in moe.moe_last_error()
    assert _call("moe_permute", P(s8), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20,
                 None) == moe.MOE_ERR_INVALID_ARG
    # permute workspace missing / too small
    pneed = moe.moe_permute_workspace_bytes(s8)
    assert pneed == 8 * 4
    assert _call("moe_permute", P(s8), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                 None) == moe.MOE_ERR_WORKSPACE
    assert _call("moe_permute", P(s8), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                 pneed - 1, None) == moe.MOE_ERR_WORKSPACE


def test_expert_share_shapes():
    whole = moe.make_shape(64, 4096, 128, 8, 1536)
    share = moe.make_shape(64, 4096, 128, 8, 1536, 0, "bf16", 16, 16)     # experts 16..31
    assert 0 < moe.moe_permute_workspace_bytes(share) < moe.moe_permute_workspace_bytes(whole)
    # 16 experts leave the streaming GEMMs short of waves: the share's
    # workspace holds split-K partials (at least two K ranges of gate|up)
    assert moe.moe_ffn_workspace_bytes(share) >= 2 * (64 * 8) * 2 * 1536 * 4
    assert moe.moe_ffn_workspace_bytes(whole) < moe.moe_ffn_workspace_bytes(share)
    assert moe.moe_forward_workspace_bytes(share) > 0
    last = moe.make_shape(64, 4096, 128, 8, 1536, 1, "bf16", 112, 16)     # experts 112..127 + shared
    assert moe.moe_forward_workspace_bytes(last) > 0
    for ef, el in ((0, -1), (-1, 4), (120, 16), (3, 0), (0, 129)):
        bad = moe.make_shape(64, 4096, 128, 8, 1536, 0, "bf16", ef, el)
        assert moe.moe_forward_workspace_bytes(bad) == 0
        assert moe.moe_permute_workspace_bytes(bad) == 0
    bad = moe.make_shape(64, 256, 8, 2, 512, 0, "bf16", 6, 4)
    assert _call("moe_combine", ctypes.byref(bad), FAKE, FAKE, FAKE, None, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert "share" in moe.moe_last_error()


def test_zero_tokens_is_a_no_op():
    sh = moe.make_shape(0, 256, 8, 2, 512)
    P = ctypes.byref
    assert _call("moe_route", P(sh), None, None, None, None, None, None, None, 0, None) == moe.MOE_OK
    assert _call("moe_combine", P(sh), None, None, None, None, None, None) == moe.MOE_OK
    assert _call("moe_forward", P(sh), *([None] * 12), None, 0, None) == moe.MOE_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import expert_ffn_layer_gemm_amd._binding as b
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(b, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        b.lib()


def test_noalloc_rejects_shapes_beyond_its_scratch():
    # Checked on the host before any HIP call: the DeepSeek-like layer needs far
    # more intermediates than the fixed scratch holds; T = 0 is a no-op.
    P = ctypes.byref
    big = moe.make_shape(4096, 7168, 256, 8, 2048, 1, "fp8")
    assert moe.moe_forward_workspace_bytes(big) > moe.NOALLOC_SCRATCH_BYTES
    args = [FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None]
    assert _call("moe_forward_noalloc", P(big), *args) == moe.MOE_ERR_WORKSPACE
    assert "scratch" in moe.moe_last_error()
    decode = moe.make_shape(64, 4096, 128, 8, 1536)
    assert moe.moe_forward_workspace_bytes(decode) <= moe.NOALLOC_SCRATCH_BYTES
    assert _call("moe_forward_noalloc", P(decode), None, *args[1:]) == moe.MOE_ERR_INVALID_ARG
    assert _call("moe_forward_noalloc", P(moe.make_shape(0, 256, 8, 2, 512)), *([None] * 13)) == moe.MOE_OK

