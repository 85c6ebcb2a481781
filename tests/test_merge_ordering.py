"""Build-time guard for the in-kernel merge's ordering (CPU only).

The single-launch form merges split pairs inside the attention kernel.  A
workgroup publishes its partials by waiting for its own stores
(`s_waitcnt vmcnt(0)`) and passing a barrier, and only then counts its
arrival with a returning atomic add; the workgroup whose add completes the
count reads every partial.  That order rests on the ISA (a store has
completed at the device coherence point once vmcnt drops to zero), not on
the language's memory model, so a compiler that moved the wait, dropped it
or sank a store past it would break the merge silently.  This test compiles
the attention kernel for gfx950 with the library's own flags and checks the
generated code of every instance:

* each single-launch instance holds the two publish sequences (the bin's
  arrivals and the first level of a two-level merge): a wait for vmcnt(0)
  directly followed by a barrier;
* after each of them the next returning atomic add comes before any
  vector-memory store;
* the other instances hold no such sequence (they carry none of the merge).

The GPU tests check the merge's results; this one checks, without a GPU,
that the compiled order they rely on is still there.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "load_balanced_paged_amd", "csrc", "attend_kernel.hip")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    from load_balanced_paged_amd import build
    out = str(tmp_path_factory.mktemp("asm") / "attend.s")
    flags = [f for f in build.HIP_FLAGS if f != "-fPIC"]
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", f"-I{build.INCLUDE}", f"-I{build.CSRC}",
           SRC, "-o", out]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout[-4000:]
    lines = open(out).read().split("\n")
    funcs, start = {}, None
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\S*attend_kernel\S*):", line)
        if m:
            start = (m.group(1), i)
        elif start and line.startswith(".Lfunc_end"):
            body = [l.strip() for l in lines[start[1]:i]]
            funcs[start[0]] = [l for l in body if l and not l.startswith((";", "."))]
            start = None
    assert funcs, "no attention kernel instances found"
    return funcs


def _fused(name):
    # template arguments <Kv, kCausal, kNB, kTileW, kFuse>: kFuse is the last
    return re.search(r"ELb1EEEvNS_10AttendArgs", name) is not None


def _publishes(body):
    """Indices of barriers directly preceded by a wait for vmcnt(0)."""
    found = []
    for i, ins in enumerate(body[:-1]):
        if ins.startswith("s_waitcnt") and "vmcnt(0)" in ins:
            j = i + 1
            while j < len(body) and body[j].startswith("s_nop"):
                j += 1
            if j < len(body) and body[j].startswith("s_barrier"):
                found.append(j)
    return found


def test_every_instance_found(kernels):
    fused = [n for n in kernels if _fused(n)]
    # three KV forms x (decode + four causal tile forms), with and without the merge
    assert len(fused) == 15 and len(kernels) == 30, sorted(kernels)


def _order_violations(body):
    """Problems with the publish-then-count order in one instance's code."""
    bad = []
    pubs = _publishes(body)
    if len(pubs) < 2:
        bad.append(f"{len(pubs)} publish sequence(s)")
    for j in pubs:
        k = j + 1
        while k < len(body) and not (body[k].startswith("global_atomic_add") and " sc0" in body[k]):
            if re.match(r"(global|buffer|flat)_store", body[k]):
                bad.append(f"store after a publish: {body[k]}")
            k += 1
        if k == len(body):
            bad.append("no arrival after a publish")
    return bad


def test_checker_rejects_planted_orders():
    """The checker itself: a store between the barrier and the count, a
    missing wait and a missing count are all reported."""
    good = ["global_store_dwordx4 v[0:1], v[2:5], off", "s_waitcnt vmcnt(0)", "s_barrier",
            "v_mov_b32 v0, 1", "global_atomic_add v1, v0, v0, s[0:1] sc0"]
    assert _order_violations(good + good) == []
    sunk = good[:3] + ["buffer_store_dword v0, v1, s[4:7], 0 offen"] + good[3:]
    assert any("store after" in b for b in _order_violations(sunk + good))
    no_wait = [i for i in good if not i.startswith("s_waitcnt")]
    assert _order_violations(no_wait + good) == ["1 publish sequence(s)"]
    no_count = good[:-1]
    assert "no arrival after a publish" in _order_violations(good + no_count)


def test_single_launch_instances_publish_before_counting(kernels):
    for name, body in kernels.items():
        if _fused(name):
            assert _order_violations(body) == [], name


def test_other_instances_carry_no_merge(kernels):
    for name, body in kernels.items():
        if not _fused(name):
            assert not _publishes(body), name
