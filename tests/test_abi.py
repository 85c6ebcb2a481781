"""CPU checks of the C ABI: exports, struct layout, host-side argument guards.

Nothing here launches a kernel; every call below returns from the host-side
guard before any device work (the container running these has no GPU).
"""

import ctypes
import os
import re
import subprocess

import pytest

import load_balanced_paged_amd as lbp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lbp.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lbp.LIB_PATH):
        pytest.fail("liblbp.so is not built (run __graft_entry__.build())")
    return lbp.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lbp_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names, "no declarations parsed"
    assert set(names) == set(lbp.EXPORTED_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", lbp.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lbp_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_struct_layout_matches_c_compiler(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text('''
#include <stdio.h>
#include <stddef.h>
#include "lbp.h"
int main(void) {
  printf("%zu %zu %zu\\n", sizeof(lbp_config), offsetof(lbp_config, sm_scale),
         offsetof(lbp_config, kv_dtype));
  printf("%zu %zu %zu %zu\\n", sizeof(lbp_plan_info), offsetof(lbp_plan_info, plan_bytes),
         offsetof(lbp_plan_info, page_table_dev), offsetof(lbp_plan_info, page_table_stride));
  printf("%zu\\n", sizeof(lbp_plan_offsets));
  printf("%zu %zu %zu %zu\\n", sizeof(lbp_prologue_args), offsetof(lbp_prologue_args, max_position),
         offsetof(lbp_prologue_args, q_out), offsetof(lbp_prologue_args, v_scale));
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    a = [int(x) for x in lines[0].split()]
    b = [int(x) for x in lines[1].split()]
    c = int(lines[2])
    assert a == [ctypes.sizeof(lbp.lbp_config), lbp.lbp_config.sm_scale.offset,
                 lbp.lbp_config.kv_dtype.offset]
    assert b == [ctypes.sizeof(lbp.lbp_plan_info), lbp.lbp_plan_info.plan_bytes.offset,
                 lbp.lbp_plan_info.page_table_dev.offset,
                 lbp.lbp_plan_info.page_table_stride.offset]
    assert c == ctypes.sizeof(lbp.lbp_plan_offsets)
    d = [int(x) for x in lines[3].split()]
    P = lbp.lbp_prologue_args
    assert d == [ctypes.sizeof(P), P.max_position.offset, P.q_out.offset, P.v_scale.offset]


def cfg(**kw):
    base = dict(num_q_heads=64, num_kv_heads=8, max_batch=64, max_pages_per_seq=1024,
                num_workgroups=256, min_tiles_per_bin=4)
    base.update(kw)
    return lbp.make_config(**base)


def query(c, policy=0, param=0):
    pb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    st = lbp.load().lbp_query_workspace(ctypes.byref(c), policy, param, ctypes.byref(pb),
                                        ctypes.byref(sb))
    return st, pb.value, sb.value


def test_version_and_status_strings(lib):
    assert lbp.lbp_version() == 2
    for s, name in lbp._STATUS_NAMES.items():
        assert lbp.lbp_status_string(s) == name


def test_q_len_workspace(lib):
    _, _, sb1 = query(cfg())
    st, _, sb2 = query(cfg(q_len=2))
    assert st == lbp.LBP_OK and sb2 >= 2 * sb1 - 512      # twice the columns per slot
    assert query(cfg(num_q_heads=8, num_kv_heads=8, q_len=64))[0] == lbp.LBP_OK
    st, _, sb6 = query(cfg(q_len=6))                        # 48 columns: three blocks
    assert st == lbp.LBP_OK and sb6 >= 6 * sb1 - 512


def test_workspace_sizes(lib):
    st, pb, sb = query(cfg())
    assert st == lbp.LBP_OK
    max_desc = 8 * 64 + 256 - 1
    G = 8
    assert sb >= max_desc * G * 128 * 4 + max_desc * G * 4
    assert pb >= 64 + 4 * 257 + 16 * max_desc + 3 * 4 * 512
    st, pb2, sb2 = query(cfg(), lbp.LBP_POLICY_STATIC_SPLITS, 4)
    assert st == lbp.LBP_OK and sb2 >= 8 * 64 * 4 * G * 128 * 4
    st, _, sb3 = query(cfg(), lbp.LBP_POLICY_STATIC_CHUNK, 16)
    assert st == lbp.LBP_OK and sb3 >= 8 * 64 * (1024 // 16) * G * 128 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), lbp.LBP_ERR_UNSUPPORTED),
    (dict(page_size=16), lbp.LBP_ERR_UNSUPPORTED),
    (dict(num_q_heads=64, num_kv_heads=2), lbp.LBP_ERR_UNSUPPORTED),   # group 32
    (dict(num_q_heads=60, num_kv_heads=8), lbp.LBP_ERR_INVALID_ARG),   # not divisible
    (dict(max_batch=0), lbp.LBP_ERR_INVALID_ARG),
    (dict(max_pages_per_seq=0), lbp.LBP_ERR_INVALID_ARG),
    (dict(num_workgroups=-1), lbp.LBP_ERR_INVALID_ARG),
    (dict(kv_dtype=7), lbp.LBP_ERR_UNSUPPORTED),
    (dict(sm_scale=0.0), lbp.LBP_ERR_INVALID_ARG),
    (dict(sm_scale=float("nan")), lbp.LBP_ERR_INVALID_ARG),
    (dict(max_pages_per_seq=1 << 30), lbp.LBP_ERR_UNSUPPORTED),
    (dict(q_len=9), lbp.LBP_ERR_UNSUPPORTED),                             # 8 * 9 > 64
    (dict(num_q_heads=16, num_kv_heads=1, q_len=5), lbp.LBP_ERR_UNSUPPORTED),  # 80 > 64
    (dict(q_len=-1), lbp.LBP_ERR_INVALID_ARG),
])
def test_config_guards(lib, kw, status):
    assert query(cfg(**kw))[0] == status


def test_policy_guards(lib):
    assert query(cfg(), 9, 1)[0] == lbp.LBP_ERR_INVALID_ARG
    assert query(cfg(), lbp.LBP_POLICY_STATIC_SPLITS, 0)[0] == lbp.LBP_ERR_INVALID_ARG
    assert query(cfg(), lbp.LBP_POLICY_STATIC_CHUNK, -3)[0] == lbp.LBP_ERR_INVALID_ARG


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails its guard first


def plan(c, seq=FAKE, batch=4, pt=FAKE, stride=1024, ws=FAKE, ws_bytes=1 << 30):
    info = lbp.lbp_plan_info()
    st = lbp.load().lbp_plan(ctypes.byref(c), seq, batch, pt, stride, ws, ws_bytes,
                             ctypes.byref(info), None)
    return st, info


def test_plan_guards(lib):
    c = cfg()
    assert plan(c, seq=None)[0] == lbp.LBP_ERR_INVALID_ARG
    assert plan(c, pt=None)[0] == lbp.LBP_ERR_INVALID_ARG
    assert plan(c, ws=None)[0] == lbp.LBP_ERR_INVALID_ARG
    assert plan(c, batch=0)[0] == lbp.LBP_ERR_INVALID_ARG
    assert plan(c, batch=65)[0] == lbp.LBP_ERR_INVALID_ARG
    assert plan(c, stride=1000)[0] == lbp.LBP_ERR_INVALID_ARG
    assert plan(c, ws_bytes=100)[0] == lbp.LBP_ERR_WORKSPACE_TOO_SMALL
    assert plan(cfg(head_dim=96))[0] == lbp.LBP_ERR_UNSUPPORTED
    info = lbp.lbp_plan_info()
    st = lib.lbp_plan_static(ctypes.byref(c), lbp.LBP_POLICY_DYNAMIC, 4, FAKE, 4, FAKE, 1024,
                             FAKE, 1 << 30, ctypes.byref(info), None)
    assert st == lbp.LBP_ERR_INVALID_ARG


def good_info(c, batch=4, max_desc=None):
    info = lbp.lbp_plan_info()
    info.magic = lbp.LBP_PLAN_MAGIC
    info.policy = 0
    info.param = 4
    info.batch = batch
    info.num_kv_heads = c.num_kv_heads
    info.num_q_heads = c.num_q_heads
    info.num_bins = 256
    info.max_desc = max_desc if max_desc is not None else c.num_kv_heads * batch + 255
    info.page_table_dev = 0x1000
    info.page_table_stride = 1024
    return info


def attend(c, info, plan_ws=FAKE, q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, split=FAKE,
           split_bytes=1 << 34, out=FAKE):
    return lbp.load().lbp_attend(ctypes.byref(c), ctypes.byref(info), plan_ws, q, k, v, ks, vs,
                                 split, split_bytes, out, None)


def test_attend_guards(lib):
    c = cfg()
    info = good_info(c)
    bad = good_info(c)
    bad.magic = 0
    assert attend(c, bad) == lbp.LBP_ERR_MISMATCH
    other = good_info(c)
    other.num_kv_heads = 4
    assert attend(c, other) == lbp.LBP_ERR_MISMATCH
    big = good_info(c, batch=65)
    assert attend(c, big) == lbp.LBP_ERR_MISMATCH
    assert attend(c, info, q=None) == lbp.LBP_ERR_INVALID_ARG
    assert attend(c, info, out=None) == lbp.LBP_ERR_INVALID_ARG
    assert attend(c, info, split_bytes=1024) == lbp.LBP_ERR_WORKSPACE_TOO_SMALL
    c8 = cfg(kv_dtype="fp8_e4m3")
    assert attend(c8, good_info(c8)) == lbp.LBP_ERR_INVALID_ARG       # FP8 without scales
    assert attend(cfg(head_dim=256), info) == lbp.LBP_ERR_UNSUPPORTED
    st = lib.lbp_combine(ctypes.byref(c), ctypes.byref(bad), FAKE, FAKE, 1 << 34, FAKE, None)
    assert st == lbp.LBP_ERR_MISMATCH


def test_noalloc_guards(lib):
    """lbp_attend_noalloc checks everything lbp_attend checks, then the split
    buffer the plan needs against its fixed array, before any device call."""
    c = cfg()
    info = good_info(c)

    def call(config=c, inf=info, plan_ws=FAKE, q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, out=FAKE):
        return lib.lbp_attend_noalloc(ctypes.byref(config), ctypes.byref(inf), plan_ws, q, k, v,
                                      ks, vs, out, None)
    bad = good_info(c)
    bad.magic = 0
    assert call(inf=bad) == lbp.LBP_ERR_MISMATCH
    assert call(q=None) == lbp.LBP_ERR_INVALID_ARG
    assert call(out=None) == lbp.LBP_ERR_INVALID_ARG
    assert call(plan_ws=None) == lbp.LBP_ERR_INVALID_ARG
    c8 = cfg(kv_dtype="fp8_e4m3")
    assert call(config=c8, inf=good_info(c8)) == lbp.LBP_ERR_INVALID_ARG   # FP8 without scales
    assert call(config=cfg(head_dim=64)) == lbp.LBP_ERR_UNSUPPORTED
    # 64 columns per slot: 1016 slots fit in 32 MiB, 1100 do not
    c64 = cfg(q_len=8)
    assert call(config=c64, inf=good_info(c64, max_desc=1100)) == lbp.LBP_ERR_SCRATCH_LIMIT
    assert lbp.lbp_status_string(lbp.LBP_ERR_SCRATCH_LIMIT) == "LBP_ERR_SCRATCH_LIMIT"
    # the decode workloads' plans fit: FP8 (128 requests x 8 KV heads + 255 slots of 8 columns)
    st, _, sb = query(cfg(max_batch=128))
    assert st == lbp.LBP_OK and sb <= lbp.NOALLOC_SCRATCH_BYTES


def test_fp8q_guards(lib):
    c = cfg()
    info = good_info(c)
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 34, FAKE, None)
    assert lib.lbp_attend_fp8q(ctypes.byref(c), ctypes.byref(info), *args) == \
        lbp.LBP_ERR_UNSUPPORTED                                   # BF16 KV
    c8 = cfg(kv_dtype="fp8_e4m3")
    i8 = good_info(c8)
    no_scale = (FAKE, FAKE, None) + args[3:]
    assert lib.lbp_attend_fp8q(ctypes.byref(c8), ctypes.byref(i8), *no_scale) == \
        lbp.LBP_ERR_INVALID_ARG
    no_kv_scale = args[:5] + (None, None) + args[7:]
    assert lib.lbp_attend_fp8q(ctypes.byref(c8), ctypes.byref(i8), *no_kv_scale) == \
        lbp.LBP_ERR_INVALID_ARG
    bad = good_info(c8)
    bad.magic = 0
    assert lib.lbp_attend_fp8q(ctypes.byref(c8), ctypes.byref(bad), *args) == lbp.LBP_ERR_MISMATCH


def test_plan_layout(lib):
    c = cfg()
    info = good_info(c)
    off = lbp.lbp_plan_layout(info)
    assert off.header == 0
    assert off.bin_offset >= 64 and off.bin_first >= off.bin_offset + 4 * 257
    assert off.bin_first % 16 == 0 and off.desc >= off.bin_first + 32 * 256
    assert off.desc % 16 == 0
    assert off.pair_first >= off.desc + 16 * info.max_desc
    assert off.pair_count >= off.pair_first + 4 * 32
    assert off.split_list >= off.scratch + 4 * 32 and off.split_list % 16 == 0
    assert off.arrive >= off.split_list + 16 * min(32, 256 - 1)
    assert off.total >= off.arrive + 4 * 2 * info.max_desc       # two counters per slot
    static = good_info(c)
    static.policy = lbp.LBP_POLICY_STATIC_SPLITS
    soff = lbp.lbp_plan_layout(static)
    assert soff.total - soff.arrive < 256                          # no counters
    bad = good_info(c)
    bad.magic = 1
    with pytest.raises(lbp.LbpError):
        lbp.lbp_plan_layout(bad)


def test_binding_rejects_host_tensors(lib):
    import torch
    c = cfg()
    with pytest.raises(ValueError):
        lbp.lbp_plan(c, torch.zeros(4, dtype=torch.int32), torch.zeros(4, 1024, dtype=torch.int32),
                     torch.zeros(1 << 20, dtype=torch.uint8))


def prologue_args(**kw):
    a = lbp.lbp_prologue_args()
    for f, _ in lbp.lbp_prologue_args._fields_:
        setattr(a, f, FAKE.value if f not in ("page_table_stride", "max_position", "norm_eps",
                                              "q_fp8") else 0)
    a.page_table_stride = 1024
    a.max_position = 4096
    a.norm_eps = 1e-6
    a.q_fp8 = 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_prologue_guards(lib):
    c = cfg()

    def st(args, batch=4, config=c):
        return lib.lbp_prologue(ctypes.byref(config), batch, ctypes.byref(args), None)
    assert st(prologue_args(), batch=0) == lbp.LBP_ERR_INVALID_ARG
    assert st(prologue_args(), batch=65) == lbp.LBP_ERR_INVALID_ARG
    for f in ("qkv", "seq_lens", "page_table", "q_norm_weight", "k_norm_weight", "rope_cos_sin",
              "q_out", "k_cache", "v_cache"):
        assert st(prologue_args(**{f: None})) == lbp.LBP_ERR_INVALID_ARG, f
    assert st(prologue_args(q_fp8=1, q_scale_out=None)) == lbp.LBP_ERR_INVALID_ARG
    assert st(prologue_args(q_fp8=2)) == lbp.LBP_ERR_INVALID_ARG
    assert st(prologue_args(max_position=0)) == lbp.LBP_ERR_INVALID_ARG
    assert st(prologue_args(norm_eps=-1.0)) == lbp.LBP_ERR_INVALID_ARG
    assert st(prologue_args(norm_eps=float("inf"))) == lbp.LBP_ERR_INVALID_ARG
    assert st(prologue_args(page_table_stride=1000)) == lbp.LBP_ERR_INVALID_ARG
    c8 = cfg(kv_dtype="fp8_e4m3")
    assert st(prologue_args(k_scale=None), config=c8) == lbp.LBP_ERR_INVALID_ARG
    assert st(prologue_args(v_scale=None), config=c8) == lbp.LBP_ERR_INVALID_ARG
    assert st(prologue_args(), config=cfg(head_dim=64)) == lbp.LBP_ERR_UNSUPPORTED
    assert lib.lbp_prologue(ctypes.byref(c), 4, None, None) == lbp.LBP_ERR_INVALID_ARG


def test_read_stream_guards(lib):
    """The read-stream reference rejects bad arguments before any launch."""
    P = ctypes.c_void_p
    aligned, odd = P(1 << 20), P((1 << 20) + 4)
    assert lib.lbp_read_stream(None, 1024, FAKE, 8, None) == lbp.LBP_ERR_INVALID_ARG
    assert lib.lbp_read_stream(aligned, 1024, None, 8, None) == lbp.LBP_ERR_INVALID_ARG
    assert lib.lbp_read_stream(aligned, 1024, FAKE, 0, None) == lbp.LBP_ERR_INVALID_ARG
    assert lib.lbp_read_stream(aligned, 1000, FAKE, 8, None) == lbp.LBP_ERR_INVALID_ARG
    assert lib.lbp_read_stream(odd, 1024, FAKE, 8, None) == lbp.LBP_ERR_INVALID_ARG


def test_taskmap_to_host_guards(lib):
    """lbp_taskmap_to_host rejects bad arguments before any copy."""
    c = cfg()
    info = good_info(c)
    total = lbp.lbp_plan_layout(info).total
    buf = ctypes.create_string_buffer(int(total))
    call = lib.lbp_taskmap_to_host
    assert call(None, FAKE, buf, total, None) == lbp.LBP_ERR_INVALID_ARG
    assert call(ctypes.byref(info), None, buf, total, None) == lbp.LBP_ERR_INVALID_ARG
    assert call(ctypes.byref(info), FAKE, None, total, None) == lbp.LBP_ERR_INVALID_ARG
    assert call(ctypes.byref(info), FAKE, buf, total - 1, None) == lbp.LBP_ERR_WORKSPACE_TOO_SMALL
    bad = good_info(c)
    bad.magic = 0
    assert call(ctypes.byref(bad), FAKE, buf, total, None) == lbp.LBP_ERR_MISMATCH
