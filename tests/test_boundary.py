"""The C ABI library on the CPU: it loads, exports every function include/*.h declares, sizes workspaces on the host, and rejects invalid or unsupported arguments with
the documented status codes before touching any device (no compute call is made here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_index.h")
BENCH_HEADER = os.path.join(ROOT, "include", "dsa_bench.h")


@pytest.fixture(scope="module")
def lib():
    import sparse_attention_indexer_dsa_amd as dsa
    return dsa.load()


def test_exports_every_declared_symbol(lib):
    text = open(HEADER).read()
    names = sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(dsa_\w+)\s*\(", text, re.M)))
    assert {"dsa_index_preprocess", "dsa_index_kpool", "dsa_index_workspace_size", "dsa_index_score_topk",
            "dsa_index_score", "dsa_index_topk", "dsa_index_forward", "dsa_index_forward_workspace_size",
            "dsa_index_score_fused", "dsa_index_selection_softmax", "dsa_index_sparse_attention",
            "dsa_last_error", "dsa_index_score_topk_noalloc"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_exports_measurement_symbols(lib):
    text = open(BENCH_HEADER).read()
    names = sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(dsa_\w+)\s*\(", text, re.M)))
    assert {"dsa_bench_mfma", "dsa_bench_mfma_flops", "dsa_bench_stream"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_measurement_validation(lib):
    # host-side checks only: every call below is rejected before anything is launched
    assert lib.dsa_bench_mfma(7, 8, 8, FAKE, None) == 2
    assert lib.dsa_bench_mfma(1, 0, 8, FAKE, None) == 1
    assert lib.dsa_bench_mfma(1, 8, 0, FAKE, None) == 1
    assert lib.dsa_bench_mfma(1, 70000, 8, FAKE, None) == 1
    assert lib.dsa_bench_mfma(1, 8, 8, None, None) == 1
    assert lib.dsa_bench_stream(FAKE, FAKE, 0, 0, None) == 1
    assert lib.dsa_bench_stream(FAKE, FAKE, 24, 0, None) == 1
    assert lib.dsa_bench_stream(FAKE + 8, FAKE, 32, 0, None) == 1
    assert lib.dsa_bench_stream(FAKE, None, 32, 1, None) == 1
    assert lib.dsa_bench_stream(FAKE, FAKE, 32, 2, None) == 1
    # flops per call: blocks x 4 waves x iters x 4 chains x flops per instruction
    assert lib.dsa_bench_mfma_flops(0, 10, 100) == 10 * 4 * 100 * 4 * 32 * 32 * 16 * 2
    assert lib.dsa_bench_mfma_flops(1, 10, 100) == 10 * 4 * 100 * 4 * 32 * 32 * 64 * 2
    assert lib.dsa_bench_mfma_flops(2, 10, 100) == lib.dsa_bench_mfma_flops(1, 10, 100)
    assert lib.dsa_bench_mfma_flops(5, 10, 100) == 0.0


def test_workspace_size(lib):
    ws = lib.dsa_index_workspace_size
    # fp32 scores at a row stride rounded up to 64 candidates, plus 256 bytes
    assert ws(8192, 64, 128, 2, 4096, 512, 1, 1) == 8192 * 4096 * 4 + 256
    assert ws(32768, 64, 128, 12, 6144, 2048, 1, 2) == 32768 * 6144 * 4 + 256
    assert ws(65536, 64, 128, 1, 65536, 2048, 4, 0) == 65536 * 16384 * 4 + 256
    assert ws(10, 16, 64, 1, 100, 8, 1, 0) == 10 * 128 * 4 + 256
    assert ws(-1, 16, 64, 1, 100, 8, 1, 0) == 0


FAKE = 1 << 20          # an aligned host integer that is never dereferenced: validation fails first


def _score(lib, **kw):
    a = dict(q_op=FAKE, q_scale=FAKE, k_op=FAKE, k_scale=FAKE, w=FAKE, w_dtype=1, T=64, S=64, H=64, D=128,
             cu=FAKE, B=1, max_seqlen=64, kpool=1, cu_pools=None, tail=1, topk=8, sm=1.0, prec=0,
             oi=FAKE, os=FAKE, ol=FAKE, op=None, ws=FAKE, wsb=10, stream=None)
    a.update(kw)
    return lib.dsa_index_score_topk(a["q_op"], a["q_scale"], a["k_op"], a["k_scale"], a["w"], a["w_dtype"],
                                    a["T"], a["S"], a["H"], a["D"], a["cu"], a["B"], a["max_seqlen"], a["kpool"],
                                    a["cu_pools"], a["tail"], a["topk"], a["sm"], a["prec"], a["oi"], a["os"],
                                    a["ol"], a["op"], a["ws"], a["wsb"], a["stream"])


def test_score_topk_validation(lib):
    assert _score(lib, prec=7) == 2
    assert b"unsupported DSA indexer scoring precision 7" in lib.dsa_last_error()
    assert _score(lib, H=48) == 2
    assert _score(lib, D=96) == 2
    assert _score(lib, topk=0) == 1
    assert _score(lib, cu=None) == 1
    assert _score(lib, kpool=4, cu_pools=None) == 1
    assert _score(lib, kpool=65) == 2
    assert _score(lib, w_dtype=5) == 1
    assert _score(lib, prec=1, q_scale=None) == 1
    assert _score(lib, q_op=FAKE + 8) == 1                  # misaligned operand
    assert _score(lib, max_seqlen=1 << 17) == 2             # more candidates than the LDS selection holds
    assert _score(lib, topk=32768, max_seqlen=32768) == 2   # selection buffer beyond LDS
    assert _score(lib, wsb=10) == 3                         # everything valid but the workspace
    assert b"workspace" in lib.dsa_last_error()
    assert _score(lib, T=0) == 0                            # empty problem: nothing to do


def test_score_topk_noalloc_validation(lib):
    # host-side checks of the entry point that allocates nothing: the same argument checks as
    # dsa_index_score_topk, then the fixed scratch bound, all before any device call
    import sparse_attention_indexer_dsa_amd as dsa
    text = open(HEADER).read()
    assert f"DSA_NOALLOC_SCRATCH_BYTES ((size_t){dsa.NOALLOC_SCRATCH_BYTES})" in text

    def call(**kw):
        a = dict(q_op=FAKE, q_scale=FAKE, k_op=FAKE, k_scale=FAKE, w=FAKE, w_dtype=1, T=64, S=64, H=64, D=128,
                 cu=FAKE, B=1, max_seqlen=64, kpool=1, cu_pools=None, tail=1, topk=8, sm=1.0, prec=0,
                 oi=FAKE, os=FAKE, ol=FAKE, op=None)
        a.update(kw)
        return lib.dsa_index_score_topk_noalloc(
            a["q_op"], a["q_scale"], a["k_op"], a["k_scale"], a["w"], a["w_dtype"], a["T"], a["S"], a["H"], a["D"],
            a["cu"], a["B"], a["max_seqlen"], a["kpool"], a["cu_pools"], a["tail"], a["topk"], a["sm"], a["prec"],
            a["oi"], a["os"], a["ol"], a["op"], None)
    assert call(prec=7) == 2
    assert call(H=48) == 2
    assert call(topk=0) == 1
    assert call(oi=None) == 1
    assert call(q_op=FAKE + 8) == 1
    assert call(T=0) == 0
    # 8192 rows x 8192 candidates: 256 MiB of score rows > the 128 MiB + 4 KiB scratch
    assert call(T=8192, S=8192, max_seqlen=8192) == 2
    assert b"scratch" in lib.dsa_last_error()
    # 16384 rows of 4 x 4096 tokens pooled by 4 (1024 candidates): 64 MiB, accepted up to the
    # device call, which the host-only fake pointers never reach: check the size rule alone
    need = lib.dsa_index_workspace_size(16384, 64, 128, 1, 4096, 8, 4, 0)
    assert need <= dsa.NOALLOC_SCRATCH_BYTES
    assert lib.dsa_index_workspace_size(8192, 64, 128, 2, 4096, 512, 1, 1) <= dsa.NOALLOC_SCRATCH_BYTES


def test_score_only_candidate_bound(lib):
    def score(max_seqlen, kpool=1):
        return lib.dsa_index_score(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 128, FAKE, 1, max_seqlen, kpool,
                                   FAKE if kpool > 1 else None, 1.0, 0, FAKE, 10, None)
    assert score(1 << 23) == 2                  # byte offsets inside a document would pass 32 bits
    assert b"candidates per row" in lib.dsa_last_error()
    assert score(1 << 23, kpool=2) == 3         # 2^22 pools: only the workspace is missing
    assert score(1 << 20) == 3


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, dt=0, w=FAKE, wdt=1, T=64, H=64, D=128, cu=FAKE, B=1, maxlen=64, g=None, b=None,
             eps=1e-6, cos=None, sin=None, R=0, maxpos=0, inter=0, f32=0, topk=8, sm=1.0, prec=1, oi=FAKE,
             os=FAKE, ol=FAKE, qo=None, qs=None, ws=FAKE, wsb=10)
    a.update(kw)
    return lib.dsa_index_forward(a["q"], a["k"], a["dt"], a["w"], a["wdt"], a["T"], a["H"], a["D"], a["cu"], a["B"],
                                 a["maxlen"], a["g"], a["b"], a["eps"], a["cos"], a["sin"], a["R"], a["maxpos"],
                                 a["inter"], a["f32"], a["topk"], a["sm"], a["prec"], a["oi"], a["os"], a["ol"],
                                 a["qo"], a["qs"], a["ws"], a["wsb"], None)


def test_forward_validation(lib):
    ws = lib.dsa_index_forward_workspace_size
    # score rows, then keys and scales, each rounded up to 256 bytes, plus 256
    assert ws(8192, 128, 4096, 1) == 8192 * 4096 * 4 + 8192 * 128 + 8192 + 256
    assert ws(100, 64, 100, 0) == 100 * 128 * 4 + 12800 + 0 + 256
    assert ws(100, 96, 100, 0) == 0
    assert _fwd(lib, prec=3) == 2
    assert _fwd(lib, H=48) == 2
    assert _fwd(lib, R=32, cos=FAKE, sin=FAKE, maxpos=10) == 2          # fp8 rotate-half over 32 dims
    assert b"rope_dim % 64" in lib.dsa_last_error()
    assert _fwd(lib, R=32, cos=FAKE, sin=FAKE, maxpos=10, prec=0) == 3   # bf16 fuses it: only the workspace
    assert _fwd(lib, R=32, cos=FAKE, sin=FAKE, maxpos=10, inter=1) == 3  # interleaved pairs are in-lane
    assert _fwd(lib, topk=0) == 1
    assert _fwd(lib, q=None) == 1
    assert _fwd(lib, qo=FAKE + 4) == 1                                  # misaligned operand copy
    assert _fwd(lib) == 3
    assert b"workspace" in lib.dsa_last_error()
    assert _fwd(lib, T=0) == 0


def test_score_fused_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, dt=0, k=FAKE, ks=FAKE, w=FAKE, wdt=1, T=64, S=64, H=64, D=128, cu=FAKE, B=1, maxlen=64,
                 cos=None, sin=None, R=0, maxpos=0, inter=0, f32=0, sm=1.0, prec=1, qo=None, qs=None, ws=FAKE,
                 wsb=10)
        a.update(kw)
        return lib.dsa_index_score_fused(a["q"], a["dt"], a["k"], a["ks"], a["w"], a["wdt"], a["T"], a["S"], a["H"],
                                         a["D"], a["cu"], a["B"], a["maxlen"], a["cos"], a["sin"], a["R"],
                                         a["maxpos"], a["inter"], a["f32"], a["sm"], a["prec"], a["qo"], a["qs"],
                                         a["ws"], a["wsb"], None)
    assert call(dt=7) == 1
    assert call(ks=None) == 1                                           # fp8 keys need scales
    assert call(R=32, cos=FAKE, sin=FAKE, maxpos=10) == 2
    assert call(R=64, cos=FAKE, sin=FAKE, maxpos=10) == 3               # all valid but the workspace
    assert call(qo=FAKE + 2, wsb=1 << 30) == 1
    assert call(T=0) == 0


def _pre(lib, **kw):
    a = dict(q=FAKE, k=FAKE, dt=0, T=64, S=64, H=64, D=128, cu=FAKE, B=1, g=None, b=None, eps=1e-6, cos=None,
             sin=None, R=0, maxpos=0, inter=0, f32=0, prec=0, qo=FAKE, qs=FAKE, ko=FAKE, ks=FAKE, qf=None, kf=None)
    a.update(kw)
    return lib.dsa_index_preprocess(a["q"], a["k"], a["dt"], a["T"], a["S"], a["H"], a["D"], a["cu"], a["B"],
                                    a["g"], a["b"], a["eps"], a["cos"], a["sin"], a["R"], a["maxpos"], a["inter"],
                                    a["f32"], a["prec"], a["qo"], a["qs"], a["ko"], a["ks"], a["qf"], a["kf"], None)


def test_preprocess_validation(lib):
    assert _pre(lib, prec=3) == 2
    assert b"expected bf16" in lib.dsa_last_error()
    assert _pre(lib, q=None, k=None) == 1
    assert _pre(lib, S=65) == 1                             # queries and keys share cu_seqlens
    assert _pre(lib, R=63, cos=FAKE, sin=FAKE, maxpos=10) == 2
    assert _pre(lib, R=48, cos=FAKE, sin=FAKE, maxpos=10) == 2   # rotate-half needs a multiple of 32
    assert _pre(lib, R=64, cos=None, sin=None, maxpos=10) == 1
    assert _pre(lib, R=64, cos=FAKE + 4, sin=FAKE, maxpos=10) == 1     # tables must be 16-byte aligned
    assert _pre(lib, R=130, cos=FAKE, sin=FAKE, maxpos=10, inter=1) == 2
    assert _pre(lib, prec=1, qs=None) == 1
    assert _pre(lib, dt=9) == 1
    assert _pre(lib, H=8) == 2
    assert _pre(lib, cu=None) == 1


def test_kpool_validation(lib):
    f = lib.dsa_index_kpool
    assert f(FAKE, 0, 64, 128, FAKE, 1, FAKE, FAKE, 0, 0, FAKE, None, FAKE, None) == 2
    assert f(FAKE, 0, 64, 128, FAKE, 1, FAKE, FAKE, 4, 9, FAKE, None, FAKE, None) == 2
    assert f(FAKE, 0, 64, 100, FAKE, 1, FAKE, FAKE, 4, 0, FAKE, None, FAKE, None) == 2
    assert f(FAKE, 0, 64, 128, None, 1, FAKE, FAKE, 4, 0, FAKE, None, FAKE, None) == 1
    assert f(FAKE, 0, 64, 128, FAKE, 1, FAKE, FAKE, 4, 1, FAKE, None, FAKE, None) == 1   # fp8 needs scales


def test_selection_softmax_validation(lib):
    f = lib.dsa_index_selection_softmax
    assert f(FAKE, -1, 8, FAKE, None) == 1
    assert f(FAKE, 4, 0, FAKE, None) == 1
    assert f(None, 4, 8, FAKE, None) == 1
    assert f(FAKE, 4, 8, None, None) == 1
    assert f(FAKE + 2, 4, 8, FAKE, None) == 1               # misaligned
    assert b"aligned" in lib.dsa_last_error()
    assert f(None, 0, 8, None, None) == 0                   # empty problem: nothing to do


def test_sparse_attention_validation(lib):
    f = lib.dsa_index_sparse_attention
    ok = dict(q=FAKE, kv=FAKE, idx=FAKE, lens=None, T=4, H=64, S=100, topk=32, dk=576, dv=512, sc=0.1, out=FAKE,
              lse=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["kv"], a["idx"], a["lens"], a["T"], a["H"], a["S"], a["topk"], a["dk"], a["dv"], a["sc"],
                 a["out"], a["lse"], None)

    assert call(T=-1) == 1 and call(S=-1) == 1 and call(H=0) == 1 and call(topk=0) == 1
    assert call(sc=float("inf")) == 1 and call(sc=float("nan")) == 1
    assert call(dk=512) == 2 and call(dv=448) == 2                    # widths other than 576 / 512
    assert b"576" in lib.dsa_last_error()
    assert call(H=24) == 2                                             # heads in groups of 16
    assert call(S=1 << 21) == 2                                        # latent tensor of 2 GiB or more
    assert call(q=None) == 1 and call(idx=None) == 1 and call(out=None) == 1
    assert call(kv=None) == 1
    assert call(q=FAKE + 8) == 1 and call(out=FAKE + 4) == 1 and call(lse=FAKE + 2) == 1
    assert call(lens=FAKE + 2) == 1
    assert b"aligned" in lib.dsa_last_error()
    assert call(T=0, q=None, idx=None, out=None, lse=None, kv=None) == 0   # empty problem: nothing to do


def test_python_binding_maps_errors():
    import sparse_attention_indexer_dsa_amd as dsa
    with pytest.raises(ValueError, match="unsupported DSA indexer scoring precision"):
        dsa._prec("fp4")
    with pytest.raises(ValueError):
        dsa._check(2, "x")
    with pytest.raises(RuntimeError):
        dsa._check(3, "x")
