"""CPU tests of the C ABI boundary: the library loads, exports every entry
point declared in include/*.h, and rejects bad arguments before any HIP
call (so no GPU is needed). Also checks the build and bench host logic."""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def attn():
    from software_pipelined_amd import attn as a, build
    if not os.path.exists(a.LIB_PATH):
        build.build_library()
    a.load_library()
    return a


def declared_functions(headers=None):
    """Names of the functions declared in the given headers (default: every
    include/*.h), comments and preprocessor lines removed."""
    names = set()
    for h in headers or HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        text = "\n".join(line for line in text.splitlines() if not line.lstrip().startswith("#"))
        names.update(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attn_fwd", "attn_strerror", "attn_num_variants", "attn_variant_name",
              "attn_variant_info", "attn_default_variant", "attn_fwd_variant", "attn_decode_workspace_size",
              "attn_fwd_decode", "attn_decode_static_max_bytes", "attn_fwd_decode_static",
              "attn_bwd_workspace_size", "attn_bwd", "chunk_scan", "mla_decode_workspace_size", "mla_decode",
              "attn_probe_mfma"):
        assert n in names, n


def test_probe_validation_happens_before_any_hip_call(attn):
    P = 1 << 20
    assert attn.attn_probe_mfma(4, 1, 1, P, None) == attn.ATTN_ERR_BAD_SHAPE
    assert attn.attn_probe_mfma(-1, 1, 1, P, None) == attn.ATTN_ERR_BAD_SHAPE
    assert attn.attn_probe_mfma(0, 0, 1, P, None) == attn.ATTN_ERR_BAD_SHAPE
    assert attn.attn_probe_mfma(1, 1, 0, P, None) == attn.ATTN_ERR_BAD_SHAPE
    assert attn.attn_probe_mfma(0, 1, 1, 0, None) == attn.ATTN_ERR_NULL_PTR


def test_library_exports_every_declared_symbol(attn):
    out = subprocess.run(["nm", "-D", "--defined-only", attn.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"


def test_validation_happens_before_any_hip_call(attn):
    P = 1 << 20  # a fake 16-byte-aligned address; never dereferenced on these paths
    good = (P, P, P, P, P)
    assert attn.attn_fwd(0, P, P, P, P, 1, 1, 16, 128, 0, 0.1, None) == attn.ATTN_ERR_NULL_PTR
    assert attn.attn_fwd(*good, -1, 1, 16, 128, 0, 0.1, None) == attn.ATTN_ERR_BAD_SHAPE
    assert attn.attn_fwd(*good, 1, -2, 16, 128, 0, 0.1, None) == attn.ATTN_ERR_BAD_SHAPE
    assert attn.attn_fwd(*good, 1, 1, -16, 128, 0, 0.1, None) == attn.ATTN_ERR_BAD_SHAPE
    for d in (0, 32, 96, 192, 512):
        assert attn.attn_fwd(*good, 1, 1, 16, d, 0, 0.1, None) == attn.ATTN_ERR_HEAD_DIM
    for s in (float("nan"), float("inf"), float("-inf")):
        assert attn.attn_fwd(*good, 1, 1, 16, 128, 0, s, None) == attn.ATTN_ERR_BAD_SCALE
    # zero and negative scales pass validation (the next check, alignment, fires)
    for s in (0.0, -0.0, -0.5):
        assert attn.attn_fwd(P + 2, P, P, P, P, 1, 1, 16, 128, 0, s, None) == attn.ATTN_ERR_MISALIGNED
    # lse needs only 4-byte alignment, every other buffer 16
    assert attn.attn_fwd(P, P, P, P, P + 2, 1, 1, 16, 128, 0, 0.1, None) == attn.ATTN_ERR_MISALIGNED
    assert attn.attn_fwd(P + 2, P, P, P, P, 1, 1, 16, 128, 0, 0.1, None) == attn.ATTN_ERR_MISALIGNED
    assert attn.attn_fwd(P, P, P, P + 8, P, 1, 1, 16, 128, 0, 0.1, None) == attn.ATTN_ERR_MISALIGNED
    # empty problems are a no-op success, even with null pointers
    assert attn.attn_fwd(0, 0, 0, 0, 0, 0, 4, 16, 128, 1, 0.1, None) == attn.ATTN_OK
    assert attn.attn_fwd(0, 0, 0, 0, 0, 2, 4, 0, 64, 0, 0.1, None) == attn.ATTN_OK
    # size overflow is a shape error
    big = 1 << 30
    assert attn.attn_fwd(*good, big, big, big, 128, 0, 0.1, None) == attn.ATTN_ERR_BAD_SHAPE


def test_decode_validation_happens_before_any_hip_call(attn):
    P = 1 << 20
    st, need = attn.attn_decode_workspace_size(1, 32, 1, 4096, 128)
    assert st == attn.ATTN_OK and need > 0
    # the workspace holds one fp32 row of d + 1 values per chunk and query row
    assert need % (4 * 129) == 0
    assert attn.attn_decode_workspace_size(0, 32, 1, 4096, 128) == (attn.ATTN_OK, 0)
    assert attn.attn_decode_workspace_size(1, 32, 0, 4096, 128) == (attn.ATTN_OK, 0)
    assert attn.attn_decode_workspace_size(1, 32, 1, 4096, 96)[0] == attn.ATTN_ERR_HEAD_DIM
    assert attn.attn_decode_workspace_size(1, -1, 1, 4096, 128)[0] == attn.ATTN_ERR_BAD_SHAPE
    assert attn.attn_decode_workspace_size(1, 1, 1, 0, 128)[0] == attn.ATTN_ERR_BAD_SHAPE
    big = 1 << 30
    assert attn.attn_decode_workspace_size(big, big, 1, big, 128)[0] == attn.ATTN_ERR_BAD_SHAPE

    def call(q=P, k=P, v=P, o=P, l=P, B=1, H=32, Nq=1, Nkv=4096, d=128, s=0.1, ws=P, wsb=None):
        return attn.attn_fwd_decode(q, k, v, o, l, B, H, Nq, Nkv, d, s, ws, need if wsb is None else wsb,
                                    None)

    assert call(q=0) == attn.ATTN_ERR_NULL_PTR
    assert call(ws=0) == attn.ATTN_ERR_NULL_PTR
    assert call(d=192) == attn.ATTN_ERR_HEAD_DIM
    assert call(Nkv=0) == attn.ATTN_ERR_BAD_SHAPE
    assert call(s=float("nan")) == attn.ATTN_ERR_BAD_SCALE
    assert call(s=0.0, k=P + 4) == attn.ATTN_ERR_MISALIGNED  # a zero scale is valid
    assert call(k=P + 4) == attn.ATTN_ERR_MISALIGNED
    assert call(ws=P + 8) == attn.ATTN_ERR_MISALIGNED
    assert call(wsb=need - 1) == attn.ATTN_ERR_WORKSPACE
    assert call(q=0, k=0, v=0, o=0, l=0, ws=0, B=0) == attn.ATTN_OK  # empty: nothing launched


def test_bwd_validation_happens_before_any_hip_call(attn):
    P = 1 << 20
    st, need = attn.attn_bwd_workspace_size(2, 16, 1000, 128)
    # 256 bytes of statistics per 32 query rows of each head
    assert st == attn.ATTN_OK and need == 2 * 16 * 32 * 256
    assert attn.attn_bwd_workspace_size(0, 16, 1000, 128) == (attn.ATTN_OK, 0)
    assert attn.attn_bwd_workspace_size(1, 1, 1000, 256) == (attn.ATTN_OK, 32 * 256)
    assert attn.attn_bwd_workspace_size(1, 1, 1000, 96)[0] == attn.ATTN_ERR_HEAD_DIM
    assert attn.attn_bwd_workspace_size(1, -1, 1000, 64)[0] == attn.ATTN_ERR_BAD_SHAPE
    big = 1 << 30
    assert attn.attn_bwd_workspace_size(big, big, big, 64)[0] == attn.ATTN_ERR_BAD_SHAPE

    def call(ptrs=None, B=2, H=16, N=1000, d=128, causal=0, s=0.1, ws=P, wsb=None, **over):
        p = dict(q=P, k=P, v=P, o=P, l=P, do=P, dq=P, dk=P, dv=P)
        p.update(over)
        return attn.attn_bwd(p["q"], p["k"], p["v"], p["o"], p["l"], p["do"], p["dq"], p["dk"], p["dv"],
                             B, H, N, d, causal, s, ws, need if wsb is None else wsb, None)

    for name in ("q", "k", "v", "o", "l", "do", "dq", "dk", "dv"):
        assert call(**{name: 0}) == attn.ATTN_ERR_NULL_PTR, name
    assert call(ws=0) == attn.ATTN_ERR_NULL_PTR
    assert call(d=96) == attn.ATTN_ERR_HEAD_DIM
    assert call(N=-1) == attn.ATTN_ERR_BAD_SHAPE
    for sc in (float("nan"), float("inf")):
        assert call(s=sc) == attn.ATTN_ERR_BAD_SCALE
    assert call(s=0.0, do=P + 2) == attn.ATTN_ERR_MISALIGNED  # a zero scale is valid
    assert call(do=P + 2) == attn.ATTN_ERR_MISALIGNED
    assert call(dk=P + 8) == attn.ATTN_ERR_MISALIGNED
    assert call(l=P + 2) == attn.ATTN_ERR_MISALIGNED
    assert call(ws=P + 8) == attn.ATTN_ERR_MISALIGNED
    assert call(wsb=need - 1) == attn.ATTN_ERR_WORKSPACE
    assert call(N=0, q=0, dq=0, ws=0) == attn.ATTN_OK  # empty: nothing launched


def test_chunk_scan_validation_happens_before_any_hip_call(attn):
    P = 1 << 20

    def call(x=P, cb=P, dt=P, da=P, o=P, B=2, S=1000, H=8, Pd=64, L=256):
        return attn.chunk_scan(x, cb, dt, da, o, B, S, H, Pd, L, None)

    for kw in ("x", "cb", "dt", "da", "o"):
        assert call(**{kw: 0}) == attn.ATTN_ERR_NULL_PTR, kw
    assert call(Pd=128) == attn.ATTN_ERR_HEAD_DIM
    for L in (0, 16, 48, 288, 512):
        assert call(L=L) == attn.ATTN_ERR_BAD_SHAPE, L
    assert call(S=-1) == attn.ATTN_ERR_BAD_SHAPE
    assert call(H=0) == attn.ATTN_ERR_BAD_SHAPE
    assert call(dt=P + 4) == attn.ATTN_ERR_MISALIGNED
    assert call(x=P + 2) == attn.ATTN_ERR_MISALIGNED
    big = 1 << 30
    assert call(B=big, S=big) == attn.ATTN_ERR_BAD_SHAPE
    assert call(S=0, x=0, o=0) == attn.ATTN_OK  # empty: nothing launched


def test_mla_validation_happens_before_any_hip_call(attn):
    P = 1 << 20
    st, need = attn.mla_decode_workspace_size(32, 128, 4096)
    assert st == attn.ATTN_OK and need > 0 and need % (4 * 513) == 0
    assert attn.mla_decode_workspace_size(0, 128, 4096) == (attn.ATTN_OK, 0)
    assert attn.mla_decode_workspace_size(1, 96, 4096)[0] == attn.ATTN_ERR_BAD_SHAPE
    assert attn.mla_decode_workspace_size(1, 128, 0)[0] == attn.ATTN_ERR_BAD_SHAPE

    def call(q=P, kv=P, o=P, l=P, B=32, H=128, N=4096, s=0.07, ws=P, wsb=None):
        return attn.mla_decode(q, kv, o, l, B, H, N, s, ws, need if wsb is None else wsb, None)

    for kw in ("q", "kv", "o", "l", "ws"):
        assert call(**{kw: 0}) == attn.ATTN_ERR_NULL_PTR, kw
    assert call(H=64 + 32) == attn.ATTN_ERR_BAD_SHAPE
    assert call(s=float("nan")) == attn.ATTN_ERR_BAD_SCALE
    assert call(s=0.0, kv=P + 8) == attn.ATTN_ERR_MISALIGNED  # a zero scale is valid
    assert call(kv=P + 8) == attn.ATTN_ERR_MISALIGNED
    assert call(l=P + 2) == attn.ATTN_ERR_MISALIGNED
    assert call(wsb=need - 1) == attn.ATTN_ERR_WORKSPACE
    assert call(B=0, q=0, kv=0, o=0, l=0, ws=0) == attn.ATTN_OK


def test_variant_table(attn):
    n = attn.attn_num_variants()
    assert n >= 3
    seen_d = set()
    for i in range(n):
        info = attn.attn_variant_info(i)
        name = attn.attn_variant_name(i)
        assert name and f"d{info['head_dim']}" in name
        assert info["block_m"] % (32 * info["waves"]) == 0  # 32-row query tiles per wave
        assert info["lds_bytes"] <= 160 * 1024
        seen_d.add(info["head_dim"])
    assert seen_d == {64, 128, 256}
    assert attn.attn_variant_name(n) is None and attn.attn_variant_name(-1) is None
    with pytest.raises(attn.AttnError):
        attn.attn_variant_info(n)
    for d in (64, 128, 256):
        for c in (0, 1):
            vid = attn.attn_default_variant(d, c)
            assert 0 <= vid < n and attn.attn_variant_info(vid)["head_dim"] == d
    assert attn.attn_default_variant(96, 0) == -1
    P = 1 << 20
    assert attn.attn_fwd_variant(n, P, P, P, P, P, 1, 1, 16, 128, 0, 0.1, None) == attn.ATTN_ERR_BAD_SHAPE
    d128 = attn.attn_default_variant(128, 0)
    assert attn.attn_fwd_variant(d128, P, P, P, P, P, 1, 1, 16, 64, 0, 0.1, None) == attn.ATTN_ERR_BAD_SHAPE


def header_status_codes():
    text = open(HEADER).read()
    enum = text[text.index("enum attn_status"):]
    enum = re.sub(r"/\*.*?\*/", "", enum[:enum.index("};")], flags=re.S)
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(ATTN_\w+)\s*=\s*(\d+)", enum)}


def test_status_codes_match_the_header(attn):
    codes = header_status_codes()
    # the codes of the boundary contract, plus the workspace code of the
    # entries that take one
    assert codes == {"ATTN_OK": 0, "ATTN_ERR_NULL_PTR": 1, "ATTN_ERR_BAD_SHAPE": 2, "ATTN_ERR_HEAD_DIM": 3,
                     "ATTN_ERR_BAD_SCALE": 4, "ATTN_ERR_MISALIGNED": 5, "ATTN_ERR_HIP": 6,
                     "ATTN_ERR_WORKSPACE": 8, "ATTN_ERR_TOO_LARGE": 9}
    for name, value in codes.items():
        assert getattr(attn, name) == value, name
    assert not hasattr(attn, "ATTN_ERR_BAD_VARIANT")


def test_strerror_covers_every_status(attn):
    for st in header_status_codes().values():
        assert attn.attn_strerror(st) and attn.attn_strerror(st) != "unknown status"
    assert attn.attn_strerror(7) == "unknown status"
    assert attn.attn_strerror(99) == "unknown status"
    # the workspace message names no single entry point
    assert "decode" not in attn.attn_strerror(attn.ATTN_ERR_WORKSPACE)


def test_binding_refuses_to_run_without_library(tmp_path, monkeypatch):
    import software_pipelined_amd.attn as a
    monkeypatch.setattr(a, "_lib", None)
    monkeypatch.setattr(a, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(FileNotFoundError):
        a.attn_fwd(0, 0, 0, 0, 0, 1, 1, 1, 64, 0, 1.0, None)


def test_library_shares_torchs_hip_runtime(attn):
    """Loading the library in a fresh process leaves exactly one HIP runtime
    mapped: the library must bind torch's, whose pointers and streams it is
    handed (with two runtimes every launch fails)."""
    code = ("from software_pipelined_amd import attn; attn.load_library(); "
            "print('\\n'.join(sorted({l.split()[-1] for l in open('/proc/self/maps') "
            "if 'libamdhip64' in l})))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    runtimes = r.stdout.split()
    assert len(runtimes) == 1, runtimes


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
    assert r.stdout == ""


def test_product_path_never_imports_the_oracle():
    """The HIP binding, build step and kernel sources never import, load or
    link anything under oracle/."""
    pkg = os.path.join(ROOT, "software_pipelined_amd")
    pat = re.compile(r"^\s*(from|import)\s+oracle|attn_oracle|liboracle|oracle/", re.M)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not pat.search(text), f"{f} references the oracle"
