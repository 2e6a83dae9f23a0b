"""The boundary from plain C (CPU only): ``tests/c_abi_client.c`` includes
``include/wf.h`` and ``include/wf_dit.h``, links ``libwf.so`` and walks a
request with host-only calls -- no Python, no torch in that process.  The
headers must compile as strict C99 and as C++; what the client prints must
equal the oracle's plans bit for bit (WF §3.1 Eq. 3-5, App. B.2-B.3) and the
Python binding's layout and split for the same config."""

import json
import os
import shutil
import subprocess

import pytest

from chunk_causal_dit_round_amd import wf
from oracle import wf_plan as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi_client.c")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.dirname(wf.LIB_PATH)

CASES = [
    # S, W, W_store, anchor, n_chunk, F, Hh, Ww, heads, head_dim, layers, dtype, mask
    (2, 2, -1, 1, 6, 3, 4, 6, 2, 64, 1, wf.WF_F32, wf.WF_MASK_WAVE),
    (4, 4, -1, 1, 30, 3, 30, 52, 12, 128, 30, wf.WF_BF16, wf.WF_MASK_WAVE),
    (5, 6, -1, 1, 25, 3, 30, 52, 12, 128, 30, wf.WF_BF16, wf.WF_MASK_ROLLING),
    (3, 2, 4, 0, 12, 2, 8, 8, 2, 128, 2, wf.WF_FP8, wf.WF_MASK_WAVE),
    (4, 4, -1, 1, 20, 3, 30, 52, 12, 128, 30, wf.WF_FP8K, wf.WF_MASK_WAVE),
]


def _compile(tmp_path, compiler, std_flags):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    exe = str(tmp_path / f"client_{compiler.replace('+', 'x')}")
    cmd = [compiler, *std_flags, "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE, SRC,
           "-o", exe, "-L", LIBDIR, "-lwf", f"-Wl,-rpath,{LIBDIR}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    return _compile(tmp_path_factory.mktemp("c_abi"), "gcc", ["-std=c99"])


def test_headers_compile_as_cxx(tmp_path):
    _compile(tmp_path, "g++", ["-x", "c++", "-std=c++11"])


def _oracle_plan_json(c, k):
    p = P.plan(c, k)
    groups = [[[kd, ch, sl] for kd, ch, sl in g["entries"]] for g in p["groups"]]
    cells = [[x["stage"], x["chunk"], int(x["active"]), x["slot"], x["frame0"]] for x in p["cells"]]
    a = p["anchor"]
    return dict(k=k, n_active=p["n_active"], evict=p["evict"], kv_tokens=p["kv_tokens"],
                flops=p["flops"], anchor=[int(a["present"]), a["slot"], a["frame0"], int(a["capture"])],
                cells=cells, groups=groups)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"S{c[0]}W{c[1]}N{c[4]}d{c[11]}m{c[12]}")
def test_c_client_matches_oracle_and_binding(client, case):
    r = subprocess.run([client, *map(str, case)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [json.loads(x) for x in r.stdout.splitlines()]
    S, W, Ws, A, n, F, Hh, Ww, H, D, L, dtype, mask = case
    oc = P.Config(S=S, W=W, W_store=Ws, anchor=A, n_chunk=n, F=F, Hh=Hh, Ww=Ww, n_heads=H,
                  head_dim=D, n_layers=L, mask=mask)
    plans, layout, split, errors = lines[:oc.n_rounds], lines[-3], lines[-2], lines[-1]
    assert len(lines) == oc.n_rounds + 3
    for k, got in enumerate(plans):
        assert got == _oracle_plan_json(oc, k), k

    cfg = wf.make_config(S, W, n, F, Hh, Ww, H, D, L, W_store=Ws, anchor=A, mask=mask, dtype=dtype)
    lay = wf.wf_page_layout(cfg)
    assert layout["layout"] == [lay.n_slots, lay.page_bytes, lay.pool_bytes, lay.anchor_bytes,
                                lay.table_bytes]
    assert layout["bytes"] == list(wf.wf_pool_bytes(cfg))
    assert lay.n_slots == oc.n_slots

    h = wf.wf_create(cfg)
    try:
        want = wf.wf_attention_split_choice(h, wf.wf_round_plan(h, split["split_k"]))
    finally:
        wf.wf_destroy(h)
    assert [tuple(x) for x in split["split"]] == want
    if dtype == wf.WF_F32:
        assert want == []

    assert errors["errors"] == [wf.WF_ERANGE, wf.WF_EINVAL, wf.WF_EORDER, wf.WF_EINVAL,
                                wf.WF_EINVAL, 0]
    assert errors["text"] == wf.wf_strerror(wf.WF_ERANGE)
