"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments before any launch (no GPU needed: every call here fails validation
or touches no device)."""
import ctypes
import os
import re

import pytest

import ring_parallelism_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ring_attn.h")
FAKE = 0x10000  # 64 KiB-aligned fake device address; never dereferenced by a failing call


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:ra_status|const char\*|int32_t)\s+(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(ra.EXPORTS)
    lib = ra.lib()
    for n in names:
        assert hasattr(lib, n), n
    header = open(os.path.join(ROOT, "include", "ring_attn.h")).read()
    assert ra.abi_version() == int(re.search(r"#define RA_ABI_VERSION (\d+)", header).group(1))


def test_descriptor_layout_matches_c(tmp_path):
    """The ctypes mirror of ra_attn_desc has the C struct's size and offsets."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no host C compiler")
    fields = [f[0] for f in ra.AttnDesc._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "ring_attn.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(ra_attn_desc));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(ra_attn_desc, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(ra.AttnDesc)
    assert got[1:] == [getattr(ra.AttnDesc, f).offset for f in fields]


def good_desc(**kw):
    d = dict(seq_len=1024, n_shards=4, split=ra.SPLIT_ZIGZAG, batch=1, h_q=4, h_kv=1, head_dim=128,
             in_dtype=ra.BF16, out_dtype=ra.F32, causal=True, scale=128 ** -0.5)
    d.update(kw)
    return ra.AttnDesc(d["seq_len"], d["n_shards"], d["split"], d["batch"], d["h_q"], d["h_kv"],
                       d["head_dim"], d["in_dtype"], d["out_dtype"], int(d["causal"]), d["scale"],
                       d.get("flags", 0))


def expect(status, fn, *a, match=None, **kw):
    with pytest.raises(ra.RingAttnError) as ei:
        fn(*a, **kw)
    assert ei.value.status == status, str(ei.value)
    if match:
        assert re.search(match, str(ei.value)), str(ei.value)


def test_tile_shape():
    tq, tk = ra.ring_attn_tile_shape(good_desc())
    assert tq % 32 == 0 and tq >= 64 and tk in (32, 64)
    assert ra.ring_attn_tile_shape(good_desc(in_dtype=ra.F32, head_dim=64)) == (16, 32)
    assert ra.ring_attn_tile_shape(good_desc(in_dtype=ra.F32, head_dim=128)) == (16, 32)


@pytest.mark.parametrize("kw,status,match", [
    (dict(seq_len=0), ra.EINVAL, "seq_len"),
    (dict(n_shards=0), ra.EINVAL, "n_shards"),
    (dict(seq_len=1000, n_shards=8), ra.EINVAL, "zig-zag"),
    (dict(seq_len=1001, split=ra.SPLIT_CONTIGUOUS), ra.EINVAL, "divisible|%|n_shards"),
    (dict(split=7), ra.EINVAL, "split"),
    (dict(batch=0), ra.EINVAL, "batch"),
    (dict(h_q=6, h_kv=4), ra.EINVAL, "h_q"),
    (dict(h_kv=0), ra.EINVAL, "h_kv"),
    (dict(head_dim=96), ra.EUNSUPPORTED, "head_dim"),
    (dict(in_dtype=5), ra.EINVAL, "in_dtype"),
    (dict(out_dtype=9), ra.EINVAL, "out_dtype"),
    (dict(in_dtype=ra.F32, out_dtype=ra.BF16), ra.EUNSUPPORTED, "bf16 output"),
    (dict(causal=2), ra.EINVAL, "causal"),
    (dict(scale=0.0), ra.EINVAL, "scale"),
    (dict(scale=float("nan")), ra.EINVAL, "scale"),
    (dict(seq_len=1 << 31, n_shards=2), ra.EUNSUPPORTED, "2\\^31"),
    (dict(flags=8), ra.EINVAL, "flags"),
    (dict(flags=ra.FLAG_SYNC_LOADS, in_dtype=ra.F32), ra.EUNSUPPORTED, "bf16 inputs only"),
])
def test_descriptor_validation(kw, status, match):
    expect(status, ra.ring_attn_tile_shape, good_desc(**kw), match=match)
    kb = [FAKE] * 4
    expect(status, ra.ring_attn_shard_fwd, good_desc(**kw), 0, FAKE, kb, kb, FAKE, FAKE, match=match)


def test_shard_fwd_argument_validation():
    d = good_desc()
    kb = [FAKE] * 4
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 4, FAKE, kb, kb, FAKE, FAKE, match="rank")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, -1, FAKE, kb, kb, FAKE, FAKE, match="rank")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, FAKE, [], [], FAKE, FAKE, match="n_blocks")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, FAKE, [FAKE] * 5, [FAKE] * 5, FAKE, FAKE, match="n_blocks")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, None, kb, kb, FAKE, FAKE, match="q, out")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, FAKE, kb, kb, None, FAKE, match="q, out")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, FAKE, kb, kb, FAKE, None, match="q, out")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, FAKE + 8, kb, kb, FAKE, FAKE, match="aligned")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, FAKE, kb, kb, FAKE, FAKE + 2, match="lse")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, FAKE, kb, kb, FAKE, FAKE, stats=FAKE + 4, match="stats")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, FAKE, [FAKE, None, FAKE, FAKE], kb, FAKE, FAKE, match="NULL")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, FAKE, [FAKE, FAKE + 4, FAKE, FAKE], kb, FAKE, FAKE, match="aligned")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, FAKE, kb[:2], kb[:2], FAKE, FAKE, block_owner=[0, 4], match="block_owner")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, FAKE, kb[:2], kb[:2], FAKE, FAKE, block_owner=[1, 1], match="repeats")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd, d, 0, FAKE, kb[:2], kb[:2], FAKE, FAKE, block_owner=[-1, 0], match="block_owner")
    with pytest.raises(ValueError):
        ra.ring_attn_shard_fwd(d, 0, FAKE, kb, kb[:3], FAKE, FAKE)


def test_all_shards_validation():
    d = good_desc()
    kb = [FAKE] * 4
    expect(ra.EINVAL, ra.ring_attn_all_shards_fwd, d, None, kb, kb, FAKE, FAKE, match="q, out")
    expect(ra.EINVAL, ra.ring_attn_all_shards_fwd, d, FAKE, kb, kb, None, FAKE, match="q, out")
    expect(ra.EINVAL, ra.ring_attn_all_shards_fwd, d, FAKE, kb, kb, FAKE, None, match="q, out")
    expect(ra.EINVAL, ra.ring_attn_all_shards_fwd, d, FAKE + 8, kb, kb, FAKE, FAKE, match="aligned")
    expect(ra.EINVAL, ra.ring_attn_all_shards_fwd, d, FAKE, [FAKE, None, FAKE, FAKE], kb, FAKE, FAKE, match="NULL")
    expect(ra.EINVAL, ra.ring_attn_all_shards_fwd, d, FAKE, kb, kb, FAKE, FAKE, stats=FAKE + 4, match="stats")
    expect(ra.EINVAL, ra.ring_attn_all_shards_fwd, good_desc(seq_len=0), FAKE, kb, kb, FAKE, FAKE, match="seq_len")
    with pytest.raises(ValueError):
        ra.ring_attn_all_shards_fwd(d, FAKE, kb[:3], kb[:3], FAKE, FAKE)
    L = ra.lib()
    assert L.ring_attn_all_shards_fwd(ctypes.byref(d), FAKE, None, None, FAKE, FAKE, None, None) == ra.EINVAL
    big = good_desc(seq_len=256 * 200, n_shards=200, split=ra.SPLIT_CONTIGUOUS)
    kb200 = [FAKE] * 200
    expect(ra.EUNSUPPORTED, ra.ring_attn_all_shards_fwd, big, FAKE, kb200, kb200, FAKE, FAKE, match="RA_MAX_BLOCKS")


def test_too_many_blocks():
    d = good_desc(seq_len=256 * 200, n_shards=200, split=ra.SPLIT_CONTIGUOUS)
    kb = [FAKE] * 129
    expect(ra.EUNSUPPORTED, ra.ring_attn_shard_fwd, d, 0, FAKE, kb, kb, FAKE, FAKE, match="RA_MAX_BLOCKS")


def test_partition_validation():
    expect(ra.EINVAL, ra.zigzag_partition, 1000, 8, ra.SPLIT_ZIGZAG, FAKE, match="zig-zag")
    expect(ra.EINVAL, ra.zigzag_partition, 1000, 3, ra.SPLIT_CONTIGUOUS, FAKE)
    expect(ra.EINVAL, ra.zigzag_partition, 0, 1, ra.SPLIT_CONTIGUOUS, FAKE)
    expect(ra.EINVAL, ra.zigzag_partition, 64, 0, ra.SPLIT_CONTIGUOUS, FAKE)
    expect(ra.EINVAL, ra.zigzag_partition, 64, 2, 3, FAKE, match="split")
    expect(ra.EINVAL, ra.zigzag_partition, 64, 2, ra.SPLIT_ZIGZAG, None, match="nothing")
    expect(ra.EINVAL, ra.zigzag_partition, 64, 2, ra.SPLIT_ZIGZAG, FAKE + 4, match="aligned")
    expect(ra.EINVAL, ra.zigzag_partition, 64, 2, ra.SPLIT_ZIGZAG, None, FAKE, None, 1, 16, match="both")
    expect(ra.EINVAL, ra.zigzag_partition, 64, 2, ra.SPLIT_ZIGZAG, None, FAKE, FAKE * 4, 0, 16, match="outer")
    expect(ra.EINVAL, ra.zigzag_partition, 64, 2, ra.SPLIT_ZIGZAG, None, FAKE, FAKE + 64, 1, 16, match="overlap")
    expect(ra.EINVAL, ra.zigzag_unpartition, 64, 2, ra.SPLIT_ZIGZAG, None, FAKE, 1, 16, match="set")


def test_merge_validation():
    o, l = [FAKE, FAKE * 2], [FAKE * 3, FAKE * 4]
    expect(ra.EINVAL, ra.ring_attn_merge, 0, 1, 8, 128, o, ra.F32, l, FAKE * 5, ra.F32, FAKE * 6, match=">= 1")
    expect(ra.EINVAL, ra.ring_attn_merge, 1, 1, 8, 128, [], ra.F32, [], FAKE * 5, ra.F32, FAKE * 6, match="n_parts")
    expect(ra.EINVAL, ra.ring_attn_merge, 1, 1, 8, 128, [FAKE] * 65, ra.F32, [FAKE] * 65, FAKE * 5, ra.F32, FAKE * 6, match="n_parts")
    expect(ra.EUNSUPPORTED, ra.ring_attn_merge, 1, 1, 8, 96, o, ra.F32, l, FAKE * 5, ra.F32, FAKE * 6, match="head_dim")
    expect(ra.EINVAL, ra.ring_attn_merge, 1, 1, 8, 128, o, 3, l, FAKE * 5, ra.F32, FAKE * 6, match="dtype")
    expect(ra.EINVAL, ra.ring_attn_merge, 1, 1, 8, 128, [FAKE + 4, FAKE * 2], ra.F32, l, FAKE * 5, ra.F32, FAKE * 6, match="misaligned")
    expect(ra.EINVAL, ra.ring_attn_merge, 1, 1, 8, 128, o, ra.F32, l, FAKE * 2, ra.F32, FAKE * 6, match="alias")
    expect(ra.EINVAL, ra.ring_attn_merge, 1, 1, 8, 128, o, ra.BF16, l, FAKE, ra.F32, FAKE * 6, match="in-place")
    expect(ra.EINVAL, ra.ring_attn_merge, 1, 1, 8, 128, [FAKE, None], ra.F32, l, FAKE * 5, ra.F32, FAKE * 6, match="NULL")


def test_last_error_is_thread_local():
    import threading
    d = good_desc(batch=0)
    msgs = {}

    def worker():
        try:
            ra.ring_attn_tile_shape(good_desc(head_dim=96))
        except ra.RingAttnError:
            pass
        msgs["t"] = ra.lib().ring_attn_last_error().decode()

    try:
        ra.ring_attn_tile_shape(d)
    except ra.RingAttnError:
        pass
    th = threading.Thread(target=worker)
    th.start()
    th.join()
    assert "batch" in ra.lib().ring_attn_last_error().decode()
    assert "head_dim" in msgs["t"]


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(ra, "_lib", None)
    monkeypatch.setattr(ra, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        ra.lib()


def test_decode_validation():
    kb = [FAKE] * 4
    d = good_desc()
    expect(ra.EUNSUPPORTED, ra.ring_attn_decode, good_desc(in_dtype=ra.F32), FAKE, kb, kb, 1, FAKE, FAKE,
           match="bf16")
    expect(ra.EUNSUPPORTED, ra.ring_attn_decode, good_desc(out_dtype=ra.BF16), FAKE, kb, kb, 1, FAKE, FAKE,
           match="fp32")
    expect(ra.EINVAL, ra.ring_attn_decode, good_desc(flags=ra.FLAG_SYNC_LOADS), FAKE, kb, kb, 1, FAKE, FAKE,
           match="flags")
    expect(ra.EUNSUPPORTED, ra.ring_attn_decode, good_desc(h_q=64, h_kv=1), FAKE, kb, kb, 1, FAKE, FAKE,
           match="32")
    expect(ra.EINVAL, ra.ring_attn_decode, d, FAKE, [], [], 1, FAKE, FAKE, match="n_blocks")
    expect(ra.EINVAL, ra.ring_attn_decode, d, FAKE, [FAKE] * 5, [FAKE] * 5, 1, FAKE, FAKE, match="n_blocks")
    expect(ra.EINVAL, ra.ring_attn_decode, d, FAKE, kb, kb, 0, FAKE, FAKE, match="n_splits")
    expect(ra.EINVAL, ra.ring_attn_decode, d, FAKE, kb, kb, 257, FAKE, FAKE, match="n_splits")
    expect(ra.EINVAL, ra.ring_attn_decode, d, None, kb, kb, 1, FAKE, FAKE, match="must be set")
    expect(ra.EINVAL, ra.ring_attn_decode, d, FAKE + 8, kb, kb, 1, FAKE, FAKE, match="aligned")
    expect(ra.EINVAL, ra.ring_attn_decode, d, FAKE, [FAKE, None, FAKE, FAKE], kb, 1, FAKE, FAKE, match="NULL")


def test_merge_strided_validation():
    m = ra.ring_attn_merge_strided
    # batch, heads, rows, head_dim, outs, parts_dtype, lses, out, out_dtype, lse, n_parts, out_stride, lse_stride
    expect(ra.EINVAL, m, 1, 2, 3, 64, FAKE, ra.F32, FAKE, FAKE * 16, ra.F32, FAKE * 32, 0, 384, 6,
           match="n_parts")
    expect(ra.EINVAL, m, 1, 2, 3, 64, FAKE, ra.F32, FAKE, FAKE * 16, ra.F32, FAKE * 32, 2, 383, 6,
           match="strides")
    expect(ra.EINVAL, m, 1, 2, 3, 64, FAKE, ra.F32, FAKE, FAKE * 16, ra.F32, FAKE * 32, 2, 384, 5,
           match="strides")
    expect(ra.EUNSUPPORTED, m, 1, 2, 3, 96, FAKE, ra.F32, FAKE, FAKE * 16, ra.F32, FAKE * 32, 2, 576, 6,
           match="head_dim")
    expect(ra.EINVAL, m, 1, 2, 3, 64, FAKE + 4, ra.F32, FAKE, FAKE * 16, ra.F32, FAKE * 32, 2, 384, 6,
           match="misaligned")
    # out inside part 1 (not part 0 exactly)
    expect(ra.EINVAL, m, 1, 2, 3, 64, FAKE, ra.F32, FAKE * 16, FAKE + 384 * 4, ra.F32, FAKE * 32, 2, 384, 6,
           match="overlaps")
    expect(ra.EINVAL, m, 1, 2, 3, 64, FAKE, ra.F32, FAKE * 16, FAKE * 8, ra.F32, FAKE * 16 + 24, 2, 384, 6,
           match="lse overlaps")
    expect(ra.EINVAL, m, 1, 2, 3, 64, FAKE, ra.F32, FAKE * 16, FAKE, ra.BF16, FAKE * 32, 2, 384, 6,
           match="in-place")


def test_shard_fwd_split_validation():
    kb = [FAKE] * 4
    f = ra.ring_attn_shard_fwd_split
    W = FAKE * 64
    expect(ra.EUNSUPPORTED, f, good_desc(in_dtype=ra.F32, head_dim=64), 0, FAKE, kb, kb, 2, W, W, FAKE, FAKE,
           match="bf16")
    expect(ra.EUNSUPPORTED, f, good_desc(flags=ra.FLAG_NATURAL_QO), 0, FAKE, kb, kb, 2, W, W, FAKE, FAKE,
           match="NATURAL")
    expect(ra.EINVAL, f, good_desc(), 0, FAKE, kb, kb, 0, W, W, FAKE, FAKE, match="n_splits")
    expect(ra.EINVAL, f, good_desc(), 0, FAKE, kb, kb, 5, W, W, FAKE, FAKE, match="n_splits")
    expect(ra.EINVAL, f, good_desc(), 0, FAKE, kb, kb, 2, None, W, FAKE, FAKE, match="work")
    expect(ra.EINVAL, f, good_desc(), 0, FAKE, kb, kb, 2, W + 8, W, FAKE, FAKE, match="aligned")
    expect(ra.EINVAL, f, good_desc(), 0, FAKE, kb, kb, 2, W, W * 2, W + 16, FAKE, match="overlaps")
    expect(ra.EINVAL, f, good_desc(), 9, FAKE, kb, kb, 2, W, W, FAKE, FAKE, match="rank")


def test_noalloc_split_validation_before_any_device_call():
    """ring_attn_shard_fwd_split_noalloc rejects a call whose partials exceed
    its static scratch (2^24 floats of partial output) before touching the
    device, and reports the split pass's own argument errors."""
    assert ra.NOALLOC_MAX_PARTIAL_FLOATS == 1 << 24 and ra.NOALLOC_MAX_LSE_FLOATS == 1 << 17
    # 8 192 tokens, c = 8, 32 / 8 heads: 4 groups fill the scratch exactly, 8 do not fit.
    d = good_desc(seq_len=8192, n_shards=8, h_q=32, h_kv=8)
    kb = [FAKE] * 8
    expect(ra.EINVAL, ra.ring_attn_shard_fwd_split_noalloc, d, 0, FAKE, kb, kb, 8, FAKE, FAKE, match="static scratch")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd_split_noalloc, d, 0, FAKE, kb, kb, 0, FAKE, FAKE, match="n_splits")
    expect(ra.EINVAL, ra.ring_attn_shard_fwd_split_noalloc, good_desc(seq_len=0), 0, FAKE, kb[:4], kb[:4], 2,
           FAKE, FAKE, match="seq_len")


def test_binding_constants_match_the_header():
    """Every #define and enum value the binding mirrors equals the header's."""
    text = open(HEADER).read()
    def value(expr):  # "4u", "128", "1 << 24"
        parts = [int(x) for x in expr.replace("u", "").split("<<")]
        return parts[0] << parts[1] if len(parts) == 2 else parts[0]

    defs = {m.group(1): value(m.group(2))
            for m in re.finditer(r"#define (RA_\w+) \(?([0-9][0-9 <]*u?)\)?", text)}
    assert defs["RA_FLAG_SYNC_LOADS"] == ra.FLAG_SYNC_LOADS
    assert defs["RA_FLAG_NATURAL_QO"] == ra.FLAG_NATURAL_QO
    assert defs["RA_FLAG_EVENT_COUNTS"] == ra.FLAG_EVENT_COUNTS
    assert defs["RA_STATS_EVENTS_LEN"] == ra.STATS_EVENTS_LEN
    assert defs["RA_MAX_BLOCKS"] == ra.MAX_BLOCKS and defs["RA_MAX_PARTS"] == ra.MAX_PARTS
    assert defs["RA_NOALLOC_MAX_PARTIAL_FLOATS"] == ra.NOALLOC_MAX_PARTIAL_FLOATS
    assert defs["RA_NOALLOC_MAX_LSE_FLOATS"] == ra.NOALLOC_MAX_LSE_FLOATS
    enums = dict(re.findall(r"(RA_\w+) = (\d+)", text))
    assert (int(enums["RA_OK"]), int(enums["RA_EINVAL"]), int(enums["RA_EUNSUPPORTED"]), int(enums["RA_EHIP"])) == \
        (ra.OK, ra.EINVAL, ra.EUNSUPPORTED, ra.EHIP)
    assert (int(enums["RA_SPLIT_ZIGZAG"]), int(enums["RA_SPLIT_STRIPED"])) == (ra.SPLIT_ZIGZAG, ra.SPLIT_STRIPED)
    assert (int(enums["RA_F32"]), int(enums["RA_BF16"])) == (ra.F32, ra.BF16)


def test_noalloc_size_check_does_not_wrap():
    """Sizes whose product overflows 64 bits are still rejected by the size check."""
    d = good_desc(seq_len=(1 << 30), n_shards=2, batch=1 << 20, h_q=1 << 20, h_kv=1 << 20)
    kb = [FAKE] * 2
    expect(ra.EINVAL, ra.ring_attn_shard_fwd_split_noalloc, d, 0, FAKE, kb, kb, 2, FAKE, FAKE, match="static scratch")


def test_descriptor_size_bound_does_not_wrap():
    """batch * h_q * S/c beyond 2^40 is refused even where the product overflows 64 bits."""
    expect(ra.EUNSUPPORTED, ra.ring_attn_tile_shape, good_desc(seq_len=1 << 24, n_shards=2, batch=1 << 30,
                                                               h_q=1 << 30, h_kv=1 << 30), match="too large")


def test_merge_size_bound_does_not_wrap():
    """batch * heads * rows past 2^40 is refused even where the product overflows 64 bits."""
    o, l = [FAKE, FAKE * 2], [FAKE * 3, FAKE * 4]
    expect(ra.EINVAL, ra.ring_attn_merge, 1 << 30, 1 << 30, 1 << 40, 128, o, ra.F32, l, FAKE * 5, ra.F32, FAKE * 6,
           match="too large")
