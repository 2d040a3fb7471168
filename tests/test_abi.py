"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching a device (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muse_attn.h")


def _lib():
    from global_muse_rope_amd import _capi
    if not os.path.exists(_capi.LIB_PATH):
        from global_muse_rope_amd import build_lib
        build_lib.build()
    return _capi, _capi.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int32_t|size_t|const char\*)\s+(muse_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ["muse_rope_qknorm", "muse_attn_prefill", "muse_attn_decode",
                     "muse_attn_prefill_workspace_size", "muse_attn_decode_workspace_size",
                     "muse_layer_is_global", "muse_last_error", "muse_version"]:
        assert required in names


def test_library_exports_every_declared_symbol():
    capi, lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in capi.SIGNATURES, name


def test_struct_layouts_match_header(tmp_path):
    """Sizes and field offsets of the ctypes mirrors equal what a C compiler
    makes of the header."""
    import shutil
    import subprocess
    capi, _ = _lib()
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = {"muse_attn_params": capi.MuseAttnParams, "muse_kv_cache": capi.MuseKvCache,
              "muse_block_weights": capi.MuseBlockWeights}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "muse_attn.h"', "int main(void) {"]
    for cname, cls in fields.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            c, f, v = line.split()
            got[(c, f)] = int(v)
    for cname, cls in fields.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, (cname, fname)


def test_layer_schedule():
    _, lib = _lib()
    assert [i for i in range(52) if lib.muse_layer_is_global(i, 52) == 1] == list(range(3, 52, 4))
    assert [i for i in range(62) if lib.muse_layer_is_global(i, 62) == 1] == list(range(1, 62, 4))
    assert lib.muse_layer_is_global(-1, 52) == -1
    assert lib.muse_layer_is_global(52, 52) == -1
    assert lib.muse_version() >= 100


def params(capi, **kw):
    base = dict(num_q_heads=32, num_kv_heads=2, head_dim=128, sliding_window=2048, rope_theta=10000.0,
                qk_scale=3.87, qk_norm_eps=1e-5, out_norm=0, out_norm_eps=1e-6)
    base.update(kw)
    return capi.MuseAttnParams(**base)


FAKE = 0x1000  # 16-byte-aligned stand-in pointer; never dereferenced by a failing call


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), 2),
    (dict(num_q_heads=30), 2),
    (dict(num_q_heads=96, num_kv_heads=2), 2),
    (dict(num_kv_heads=0), 1),
    (dict(sliding_window=-1), 1),
    (dict(rope_theta=-5.0), 1),
    (dict(qk_scale=0.0), 1),
    (dict(qk_norm_eps=0.0), 1),
    (dict(out_norm=1, out_norm_eps=0.0), 1),
    (dict(out_norm=2), 1),
])
def test_prefill_rejects_bad_params(kw, code):
    capi, lib = _lib()
    p = params(capi, **kw)
    rc = lib.muse_attn_prefill(ctypes.byref(p), 1, 64, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE,
                               1 << 30, None)
    assert rc == code
    assert lib.muse_last_error()


def test_prefill_argument_checks():
    capi, lib = _lib()
    p = params(capi)
    assert lib.muse_attn_prefill(None, 1, 64, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 1 << 30, None) == 1
    # empty problem is a no-op
    assert lib.muse_attn_prefill(ctypes.byref(p), 0, 64, None, None, None, None, None, None, None, None, 0, None) == 0
    assert lib.muse_attn_prefill(ctypes.byref(p), 1, 0, None, None, None, None, None, None, None, None, 0, None) == 0
    # null tensor, misalignment
    assert lib.muse_attn_prefill(ctypes.byref(p), 1, 64, None, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.muse_attn_prefill(ctypes.byref(p), 1, 64, FAKE + 2, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 1 << 30, None) == 1
    # workspace too small
    need = lib.muse_attn_prefill_workspace_size(ctypes.byref(p), 1, 64)
    assert need > 0
    assert lib.muse_attn_prefill(ctypes.byref(p), 1, 64, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, need - 1, None) == 3
    assert lib.muse_attn_prefill(ctypes.byref(p), 1, 64, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, need, None) == 3
    # strides: not a multiple of 8, token stride below H * D
    bad = (ctypes.c_int64 * 10)(*([4096 * 64, 4100] + [256 * 64, 256] * 2 + [4096 * 64, 4096] * 2))
    assert lib.muse_attn_prefill(ctypes.byref(p), 1, 64, FAKE, FAKE, FAKE, FAKE, bad, None, FAKE, FAKE, need, None) == 1
    bad2 = (ctypes.c_int64 * 10)(*([4096 * 64, 2048] + [256 * 64, 256] * 2 + [4096 * 64, 4096] * 2))
    assert lib.muse_attn_prefill(ctypes.byref(p), 1, 64, FAKE, FAKE, FAKE, FAKE, bad2, None, FAKE, FAKE, need, None) == 1


def test_workspace_sizes():
    capi, lib = _lib()
    p = params(capi)
    a = lib.muse_attn_prefill_workspace_size(ctypes.byref(p), 1, 1000)
    b = lib.muse_attn_prefill_workspace_size(ctypes.byref(p), 1, 2000)
    assert 0 < a < b
    # k_hat fp16 + v bf16 over 64-key tiles: 2 * B * Hkv * ceil(T/64) * 64 * D * 2
    assert a >= 2 * 2 * 16 * 64 * 128 * 2
    bad = params(capi, head_dim=80)
    assert lib.muse_attn_prefill_workspace_size(ctypes.byref(bad), 1, 1000) == 0


def test_decode_workspace_follows_paged_chunk_choice():
    """Paged decode splits each (sequence, KV head) into chunks of 8192, 4096 or
    2048 positions: the largest that still gives 2048 workgroups for the batch,
    KV heads and max_kv_len (2048 when none does).  The workspace holds one fp32
    partial of G * (D + 2) values per chunk, so its size shows the choice."""
    capi, lib = _lib()
    p = params(capi, num_q_heads=128, num_kv_heads=16, head_dim=64, qk_scale=5.473, out_norm=1)
    paged = capi.MuseKvCache(capi.MUSE_KV_PAGED, 0, FAKE, FAKE, FAKE, 40000, 32, 1 << 22)

    def expect(B, max_len, chunk):
        a256 = lambda n: (n + 255) // 256 * 256
        chunks = (max_len + chunk - 1) // chunk + 1
        return a256(B * 128 * 64 * 4) + a256(B * 16 * 64 * 4) + a256(B * 16 * chunks * 8 * 66 * 4)

    def got(B, max_len):
        return lib.muse_attn_decode_workspace_size(ctypes.byref(p), B, max_len, ctypes.byref(paged))

    assert got(16, 1 << 20) == expect(16, 1 << 20, 8192)   # 256 * 129 workgroups
    assert got(16, 30000) == expect(16, 30000, 4096)       # 8192 would give 256 * 5
    assert got(16, 8000) == expect(16, 8000, 2048)         # none reaches 2048: the smallest
    assert got(1, 1 << 17) == expect(1, 1 << 17, 2048)
    assert got(1, 1 << 20) == expect(1, 1 << 20, 8192)     # 16 * 129 = 2064


def test_decode_argument_checks():
    capi, lib = _lib()
    p = params(capi, num_q_heads=128, num_kv_heads=16, head_dim=64, qk_scale=5.473, out_norm=1)
    ring = capi.MuseKvCache(capi.MUSE_KV_RING, 2048, FAKE, FAKE, None, 0, 0, 0)
    need = lib.muse_attn_decode_workspace_size(ctypes.byref(p), 16, 1 << 20, ctypes.byref(ring))
    assert need > 0

    def call(cache, max_len=1 << 20, ws=need, **kw):
        pp = params(capi, **{**dict(num_q_heads=128, num_kv_heads=16, head_dim=64, qk_scale=5.473, out_norm=1), **kw})
        return lib.muse_attn_decode(ctypes.byref(pp), 16, FAKE, FAKE, FAKE, FAKE, FAKE, max_len,
                                    ctypes.byref(cache) if cache is not None else None, FAKE, FAKE, ws, None)

    assert call(None) == 1
    assert call(ring, ws=need - 1) == 3
    assert call(ring, max_len=0) == 1
    # ring capacity must equal the window
    assert call(capi.MuseKvCache(capi.MUSE_KV_RING, 1024, FAKE, FAKE, None, 0, 0, 0)) == 1
    # ring on a global layer
    assert call(ring, sliding_window=0) == 1
    # paged: block-table capacity, page size
    paged = capi.MuseKvCache(capi.MUSE_KV_PAGED, 0, FAKE, FAKE, FAKE, 100, 32, 10000)
    assert call(paged, max_len=100 * 32 + 1, sliding_window=0) == 1
    assert call(capi.MuseKvCache(capi.MUSE_KV_PAGED, 0, FAKE, FAKE, FAKE, 100, 24, 10000), max_len=64,
                sliding_window=0) == 2
    assert call(capi.MuseKvCache(capi.MUSE_KV_PAGED, 0, FAKE, FAKE, None, 100, 32, 10000), max_len=64,
                sliding_window=0) == 1
    assert call(capi.MuseKvCache(7, 0, FAKE, FAKE, None, 0, 0, 0)) == 1


def test_decode_noalloc_rejects_beyond_its_scratch():
    """The allocation-free decode checks its scratch need against the fixed
    array before any launch (and before looking for a device)."""
    capi, lib = _lib()
    pp = params(capi, num_q_heads=128, num_kv_heads=16, head_dim=64, qk_scale=5.473, out_norm=1, sliding_window=0,
                rope_theta=0.0)
    paged = capi.MuseKvCache(capi.MUSE_KV_PAGED, 0, FAKE, FAKE, FAKE, 1 << 15, 32, 10000)
    need = lib.muse_attn_decode_workspace_size(ctypes.byref(pp), 64, 1 << 20, ctypes.byref(paged))
    assert need > (80 << 20)
    rc = lib.muse_attn_decode_noalloc(ctypes.byref(pp), 64, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                                      ctypes.byref(paged), FAKE, None)
    assert rc == 3 and b"scratch" in lib.muse_last_error()
    # the full decode workload (16 sequences up to 2^20 positions) fits
    assert lib.muse_attn_decode_workspace_size(ctypes.byref(pp), 16, 1 << 20, ctypes.byref(paged)) <= (80 << 20)
    assert lib.muse_attn_decode_noalloc(ctypes.byref(pp), 16, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None,
                                        FAKE, None) == 1


def test_rope_qknorm_argument_checks():
    capi, lib = _lib()
    p = params(capi)
    f = lib.muse_rope_qknorm
    assert f(ctypes.byref(p), 4, None, 0, None, 0, None, None, None, 0, None) == 1        # no q, no k
    assert f(ctypes.byref(p), 4, FAKE, 4096, None, 0, None, None, None, 0, None) == 1     # q without q_out
    assert f(ctypes.byref(p), 4, FAKE, 4096, None, 0, None, FAKE, None, 9, None) == 1     # bad dtype
    assert f(ctypes.byref(p), 4, FAKE, 100, None, 0, None, FAKE, None, 0, None) == 1      # stride < Hq * D
    assert f(ctypes.byref(p), 0, FAKE, 4096, None, 0, None, FAKE, None, 0, None) == 0     # empty: no-op
    assert f(ctypes.byref(p), -1, FAKE, 4096, None, 0, None, FAKE, None, 0, None) == 1


TILE_BYTES = {128: (64 * 16 + 128 * 8) * 16, 64: (64 * 8 + 64 * 8) * 16}  # one 64-key tile image (K rows, V^T rows)


def _align(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("name", ["muse_attn_prefill_chunk", "muse_attn_draft_block"])
def test_chunk_and_draft_argument_checks(name):
    capi, lib = _lib()
    p = params(capi)  # a Glimmer local layer: 32/2 heads x 128, window 2048
    f, wsf = getattr(lib, name), getattr(lib, name + "_workspace_size")
    ring = capi.MuseKvCache(capi.MUSE_KV_RING, 2048, FAKE, FAKE, None, 0, 0, 0)
    need = wsf(ctypes.byref(p), 2, 16, 4096)
    assert need > 0

    def call(B=2, T=16, max_start=4096, cache=ring, ws=need, start=FAKE, q=FAKE, pp=p):
        return f(ctypes.byref(pp), B, T, q, FAKE, FAKE, FAKE, None, start, max_start,
                 ctypes.byref(cache) if cache is not None else None, FAKE, FAKE, ws, None)

    assert call(T=-1) == 1
    assert call(max_start=-1) == 1
    assert call(max_start=0x7FFFFFFF) == 2          # positions past the 32-bit range
    assert call(cache=None) == 1
    assert call(start=None) == 1
    assert call(q=FAKE + 2) == 1                    # misaligned tensor
    assert call(ws=need - 1) == 3
    assert call(B=0) == 0 and call(T=0) == 0        # empty problems are no-ops
    assert call(cache=capi.MuseKvCache(capi.MUSE_KV_RING, 1024, FAKE, FAKE, None, 0, 0, 0)) == 1  # capacity != W
    # a paged cache of 4096 positions on a global layer: a chunk writes positions up to
    # max_start + T - 1 and needs them all; a drafter's block only reads below max_start
    pg = params(capi, sliding_window=0, rope_theta=0.0)
    paged = capi.MuseKvCache(capi.MUSE_KV_PAGED, 0, FAKE, FAKE, FAKE, 128, 32, 10000)
    need_g = wsf(ctypes.byref(pg), 2, 16, 4096)
    rc = call(cache=paged, pp=pg, ws=need_g - 1)
    assert rc == (1 if name == "muse_attn_prefill_chunk" else 3)


def test_chunk_workspace_covers_key_pieces():
    """A launch with fewer query blocks than CUs splits each block over key
    pieces and needs room for their fp32 partial sums; one with many blocks
    needs only the tile images, the RoPE table and one fp32 per tile (the
    tile's largest cached-key mean square)."""
    capi, lib = _lib()
    p = params(capi)  # G = 16: one query block covers 16 tokens
    B, hkv, d, hq = 16, 2, 128, 32
    tiles = lambda T, hist: B * hkv * ((hist + T + 63) // 64) * TILE_BYTES[d]
    rope = lambda T: B * T * (d // 2) * 8
    hist = 2047 + 63                                    # the window's history, rounded down to a tile
    for name in ("muse_attn_prefill_chunk_workspace_size", "muse_attn_draft_block_workspace_size"):
        wsf = getattr(lib, name)
        # 16 tokens: 32 query blocks, split
        small = wsf(ctypes.byref(p), B, 16, 131072)
        base = _align(tiles(16, hist)) + _align(rope(16))
        assert small >= base + 2 * B * 16 * hq * (d + 1) * 4
        # 4096 tokens: 512 query blocks, not split
        big = wsf(ctypes.byref(p), B, 4096, 131072)
        n_tiles = (hist + 4096 + 63) // 64
        assert big == _align(tiles(4096, hist)) + _align(rope(4096)) + _align(B * hkv * n_tiles * 4)


def test_draft_split_workspace():
    """Blocks of at most 64 tokens with at most 128 (token, head) columns per
    KV head take the few-token decode path.  Its workspace is one fp32
    partial row (O, max, sum, padded to D + 4) per (sequence, KV head, group
    of 64 columns, split workgroup, column).  Each workgroup covers a chunk
    of the context of a multiple of 64 positions; the last one also takes
    the block's own keys.  Wider blocks keep the tile-image size."""
    capi, lib = _lib()
    wsf = lib.muse_attn_draft_block_workspace_size
    p = params(capi, num_kv_heads=8)                 # Glimmer assistant: 32 / 8 heads x 128, window 2048
    B, T, hkv, d = 16, 16, 8, 128
    row = 64 * (d + 4) * 4                           # 64 columns of one (sequence, KV head, slot)
    got = wsf(ctypes.byref(p), B, T, 131072)
    assert got % (B * hkv * row) == 0
    slots = got // (B * hkv * row)
    # the context (at most W + 30 positions past the 32-aligned base) in chunks of at least 64
    assert 1 <= slots <= -(-(2048 + 30) // 64)
    # no context at all: one workgroup (the block's own keys)
    assert wsf(ctypes.byref(p), B, T, 0) == B * hkv * row
    # 128 columns per KV head: two groups
    p8 = params(capi, num_kv_heads=4)
    assert wsf(ctypes.byref(p8), B, 16, 0) == 2 * B * 4 * row
    # a global layer's context grows the partials, never a tile image
    pg = params(capi, num_kv_heads=8, sliding_window=0, rope_theta=0.0)
    assert wsf(ctypes.byref(pg), B, T, 1 << 20) > wsf(ctypes.byref(pg), B, T, 1 << 16) > B * hkv * row
    # 65 tokens, or 160 columns per KV head: the tile path
    assert wsf(ctypes.byref(p), B, 65, 131072) == lib.muse_attn_prefill_chunk_workspace_size(ctypes.byref(p), B, 65,
                                                                                               131072)
    assert wsf(ctypes.byref(p), B, 40, 131072) == lib.muse_attn_prefill_chunk_workspace_size(ctypes.byref(p), B, 40,
                                                                                               131072)


def test_draft_split_argument_checks():
    """The few-token path keeps the block call's checks."""
    capi, lib = _lib()
    p = params(capi, num_kv_heads=8)
    f, wsf = lib.muse_attn_draft_block, lib.muse_attn_draft_block_workspace_size
    ring = capi.MuseKvCache(capi.MUSE_KV_RING, 2048, FAKE, FAKE, None, 0, 0, 0)
    need = wsf(ctypes.byref(p), 2, 16, 4096)

    def call(B=2, T=16, max_start=4096, cache=ring, ws=need, start=FAKE, q=FAKE, pp=p):
        return f(ctypes.byref(pp), B, T, q, FAKE, FAKE, FAKE, None, start, max_start,
                 ctypes.byref(cache) if cache is not None else None, FAKE, FAKE, ws, None)

    assert call(T=-1) == 1
    assert call(max_start=-1) == 1
    assert call(max_start=0x7FFFFFFF) == 2
    assert call(cache=None) == 1
    assert call(start=None) == 1
    assert call(q=FAKE + 2) == 1
    assert call(ws=need - 1) == 3
    assert call(B=0) == 0 and call(T=0) == 0
    assert call(cache=capi.MuseKvCache(capi.MUSE_KV_RING, 1024, FAKE, FAKE, None, 0, 0, 0)) == 1
    pg = params(capi, num_kv_heads=8, sliding_window=0, rope_theta=0.0)
    small = capi.MuseKvCache(capi.MUSE_KV_PAGED, 0, FAKE, FAKE, FAKE, 128, 32, 10000)  # 4096 positions
    assert call(cache=small, pp=pg, max_start=4097, ws=wsf(ctypes.byref(pg), 2, 16, 4097)) == 1


def test_block_prefill_argument_checks():
    capi, lib = _lib()
    p = params(capi, num_q_heads=128, num_kv_heads=16, head_dim=64, qk_scale=5.473, out_norm=1)
    f, wsf = lib.muse_attn_block_prefill, lib.muse_attn_block_prefill_workspace_size

    def weights(hidden=8192, gate=FAKE, temp=0.3, post=None, w_o=FAKE):
        return capi.MuseBlockWeights(hidden, FAKE, FAKE, w_o, post, gate, temp)

    w = weights()
    need = wsf(ctypes.byref(p), ctypes.byref(w), 1, 256)
    assert need > 0

    def call(wt=w, B=1, T=256, ws=need, x=FAKE):
        return f(ctypes.byref(p), ctypes.byref(wt) if wt is not None else None, B, T, x, FAKE, FAKE, ws, None)

    assert call(wt=None) == 1
    assert call(B=-1) == 1
    assert call(wt=weights(hidden=8190)) == 2           # not a multiple of 8
    assert call(wt=weights(hidden=16384)) == 2          # wider than the row kernels take
    assert call(wt=weights(w_o=None)) == 1
    assert call(wt=weights(temp=0.0)) == 1              # residual gate needs a positive temperature
    assert call(wt=weights(gate=None)) == 1             # a plain add needs post_norm
    assert call(B=0) == 0 and call(T=0) == 0
    assert call(x=None) == 1
    assert call(ws=need - 1) == 3
    # the workspace holds the bf16 intermediates (h, the projection, o, a) at least
    n = (2 * 128 + 2 * 16) * 64
    assert need >= 256 * (8192 + n + 128 * 64 + 8192) * 2


def test_only_the_tuning_call_waits_for_the_device():
    """Calls are asynchronous: the only host waits in the library sit in the
    GEMM candidate timing, and only muse_attn_block_tune asks for it."""
    import re
    src = os.path.join(ROOT, "global_muse_rope_amd", "csrc")
    waits = re.compile(r"hip(Event|Device|Stream)Synchronize|hipMemcpy(?!Async)|hipFree\b|hipMalloc\b")
    for name in sorted(os.listdir(src)):
        text = open(os.path.join(src, name)).read()
        for m in waits.finditer(text):
            enclosing = text.rfind("int fastest_candidate(", 0, m.start())
            assert name == "block.hip" and enclosing >= 0 and text.find("\nint block_gemm(", enclosing) > m.start(), \
                f"{name}: {m.group(0)} outside the candidate timing"
    api = open(os.path.join(src, "api.hip")).read()
    tuned = [m.start() for m in re.finditer(r"block_gemm\([^;]*,\s*true\)", api, re.S)]
    assert tuned, "the tuning entry point asks for candidate timing"
    for pos in tuned:
        assert api.rfind("int32_t muse_attn_block_tune(", 0, pos) > api.rfind("int32_t muse_attn_block_decode(", 0, pos)
