"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments synchronously before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

from sampling_spec_verify_amd import specverify as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["sv_status_string", "sv_chain_workspace_bytes", "sv_chain_verify",
                            "sv_chain_verify_noalloc",
                            "sv_chain_acceptance_workspace_bytes", "sv_chain_acceptance_rate",
                            "sv_chain_row_stats", "sv_chain_accept_resample",
                            "sv_chain_row_stats_timed", "sv_chain_verify_ex",
                            "sv_tree_workspace_bytes", "sv_tree_verify_greedy",
                            "sv_tree_row_argmax", "sv_tree_greedy_walk",
                            "sv_tree_row_argmax_timed", "sv_tree_verify_greedy_timed",
                            "sv_tree_attention_mask",
                            "sv_tree_attention_mask_timed", "sv_tree_verify_path",
                            "sv_tree_verify_path_ex", "sv_tree_multi_workspace_bytes",
                            "sv_tree_verify_multi", "sv_tree_verify_multi_ex",
                            "sv_read_stream"])


def test_library_exports_every_declared_symbol():
    L = sv.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(sv.SIGNATURES)


def test_status_strings():
    for code in range(8):
        s = sv.status_string(code)
        assert s.startswith("SV_")
    assert "unknown" in sv.status_string(99)


def _header_enum(name):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef enum \{([^}]*)\} " + name + ";", text).group(1)
    # names ending in "_" only widen the type to the range of int
    return {k: int(v) for k, v in re.findall(r"(SV_[A-Z0-9_]+)\s*=\s*(\d+)", body) if not k.endswith("_")}


def test_status_codes_and_data_bits():
    """The return codes and data-status bits the header fixes.  There is no
    separate shape code (a bad size is SV_EINVAL); null pointers, misaligned
    logits and the no-alloc call's size limit have codes of their own
    (SV_ENULL, SV_EALIGN, SV_ETOOBIG); data errors are OR-ed bits of one
    status word, so that a call reports every kind it met, not only the
    first."""
    codes = _header_enum("sv_status")
    assert codes == {"SV_OK": 0, "SV_EINVAL": 1, "SV_ENULL": 2, "SV_EALIGN": 3,
                     "SV_EWORKSPACE": 4, "SV_EDTYPE": 5, "SV_EHIP": 6, "SV_ETOOBIG": 7}
    for k, v in codes.items():
        assert getattr(sv, k) == v, k
        assert sv.status_string(v).startswith(k + ":"), k
    bits = dict(re.findall(r"#define (SV_DATA_[A-Z_]+)\s+(0x[0-9a-fA-F]+)", open(HEADER).read()))
    assert {k[8:]: int(v, 16) for k, v in bits.items()} == {n: b for b, n in sv.DATA_FLAGS.items()}
    vals = sorted(int(v, 16) for v in bits.values())
    assert vals == [1 << i for i in range(len(vals))]          # one bit each: they OR together


def test_noalloc_rejects_oversize_before_any_hip_call():
    B, K, V = 2048, 64, 128256
    assert sv.chain_workspace_bytes(B, K, V) > sv.SV_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(16)
    code = sv.lib().sv_chain_verify_noalloc(p, V, p, V, sv.SV_BF16, B, K, V, p, None, p, p, 0.0,
                                            1.0, p, p, None, None, None)
    assert code == sv.SV_ETOOBIG
    # argument errors still come first
    assert sv.lib().sv_chain_verify_noalloc(p, V, p, V, sv.SV_BF16, B, K, V, p, None, p, p, 2.0,
                                            1.0, p, p, None, None, None) == sv.SV_EINVAL
    assert sv.lib().sv_chain_verify_noalloc(p, V, p, V, 9, B, K, V, p, None, p, p, 0.0,
                                            1.0, p, p, None, None, None) == sv.SV_EDTYPE


def test_workspace_sizes():
    L = sv.lib()
    assert L.sv_chain_workspace_bytes(-1, 4, 100) == 0
    assert L.sv_chain_workspace_bytes(1, 65, 100) == 0
    assert L.sv_chain_workspace_bytes(1, 4, 0) == 0
    a = L.sv_chain_workspace_bytes(1, 8, 128256)
    b = L.sv_chain_workspace_bytes(64, 8, 128256)
    assert 0 < a < b and a % 256 == 0
    assert L.sv_tree_workspace_bytes(8, 26, 128256) > 0
    assert L.sv_tree_workspace_bytes(8, 1025, 128256) == 0


FAKE = 1 << 20          # an aligned non-null address; never dereferenced (calls fail validation)


def chain_call(fn="sv_chain_verify", **kw):
    args = dict(t=FAKE, ld_t=128, d=FAKE, ld_q=128, dtype=sv.SV_BF16, B=2, K=4, V=128,
                tok=FAKE, dl=None, ua=FAKE, us=FAKE, lam=0.0, T=1.0, acc=FAKE, out=FAKE,
                ap=FAKE, st=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    args.update(kw)
    L = sv.lib()
    timed = (FAKE, FAKE) if fn.endswith("_timed") else ()
    if fn == "sv_chain_verify_ex":
        timed = (args.get("space", sv.SV_MIX_LOGIT), args.get("stages", 3), None, None)
    return getattr(L, fn)(args["t"], args["ld_t"], args["d"], args["ld_q"], args["dtype"], args["B"],
                          args["K"], args["V"], args["tok"], args["dl"], args["ua"], args["us"],
                          args["lam"], args["T"], args["acc"], args["out"], args["ap"], args["st"],
                          args["ws"], args["wsb"], args["stream"], *timed)


@pytest.mark.parametrize("fn", ["sv_chain_verify", "sv_chain_row_stats", "sv_chain_accept_resample",
                                "sv_chain_row_stats_timed", "sv_chain_verify_ex"])
@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), sv.SV_EDTYPE),
    (dict(B=-1), sv.SV_EINVAL),
    (dict(K=-1), sv.SV_EINVAL),
    (dict(K=65), sv.SV_EINVAL),
    (dict(V=0), sv.SV_EINVAL),
    (dict(lam=1.5), sv.SV_EINVAL),
    (dict(lam=-0.1), sv.SV_EINVAL),
    (dict(lam=float("nan")), sv.SV_EINVAL),
    (dict(T=0.0), sv.SV_EINVAL),
    (dict(T=-1.0), sv.SV_EINVAL),
    (dict(T=float("inf")), sv.SV_EINVAL),
    (dict(T=float("nan")), sv.SV_EINVAL),
    (dict(T=1e36), sv.SV_EINVAL),
    (dict(T=1e-42), sv.SV_EINVAL),
    (dict(t=None), sv.SV_ENULL),
    (dict(d=None), sv.SV_ENULL),
    (dict(tok=None), sv.SV_ENULL),
    (dict(ua=None), sv.SV_ENULL),
    (dict(us=None), sv.SV_ENULL),
    (dict(acc=None), sv.SV_ENULL),
    (dict(out=None), sv.SV_ENULL),
    (dict(t=FAKE + 8), sv.SV_EALIGN),
    (dict(d=FAKE + 2), sv.SV_EALIGN),
    (dict(ld_t=100), sv.SV_EALIGN),              # ld < V
    (dict(ld_t=132), sv.SV_EALIGN),              # 264-byte rows are not 16-byte multiples
    (dict(dtype=sv.SV_F32, ld_q=130), sv.SV_EALIGN),
    (dict(ws=None), sv.SV_EWORKSPACE),
    (dict(ws=FAKE + 4), sv.SV_EWORKSPACE),
    (dict(wsb="short"), sv.SV_EWORKSPACE),
])
def test_chain_argument_errors(fn, kw, code):
    if kw.get("wsb") == "short":
        kw = dict(wsb=sv.lib().sv_chain_workspace_bytes(2, 4, 128) - 16)
    assert chain_call(fn, **kw) == code


@pytest.mark.parametrize("kw", [dict(space=2), dict(space=-1), dict(stages=0), dict(stages=4)])
def test_chain_ex_rejects_unknown_mode_or_stages(kw):
    assert chain_call("sv_chain_verify_ex", **kw) == sv.SV_EINVAL


def test_chain_empty_batch_is_a_no_op():
    assert chain_call(B=0, t=None, d=None, tok=None, ua=None, us=None, acc=None, out=None,
                      ws=None, wsb=0) == sv.SV_OK


def test_chain_without_drafts_needs_no_draft_tensor():
    # K = 0 still needs the workspace: a too-small one is reported, no launch happens
    assert chain_call(K=0, d=None, tok=None, ua=None, wsb=16) == sv.SV_EWORKSPACE


GREEDY_ENTRIES = ["sv_tree_verify_greedy", "sv_tree_row_argmax", "sv_tree_greedy_walk",
                  "sv_tree_row_argmax_timed", "sv_tree_verify_greedy_timed"]


def greedy_call(fn="sv_tree_verify_greedy", **kw):
    args = dict(t=FAKE, ld=128, dtype=sv.SV_BF16, B=2, N=5, V=128, par=FAKE, tok=FAKE, acc=FAKE,
                out=FAKE, nodes=FAKE, Dmax=6, st=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    args.update(kw)
    timed = (FAKE, FAKE) if fn.endswith("_timed") else ()
    return getattr(sv.lib(), fn)(args["t"], args["ld"], args["dtype"], args["B"], args["N"],
                                 args["V"], args["par"], args["tok"], args["acc"], args["out"],
                                 args["nodes"], args["Dmax"], args["st"], args["ws"], args["wsb"],
                                 args["stream"], *timed)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), sv.SV_EDTYPE), (dict(B=-2), sv.SV_EINVAL), (dict(N=-1), sv.SV_EINVAL),
    (dict(N=1025), sv.SV_EINVAL), (dict(V=0), sv.SV_EINVAL), (dict(Dmax=-1), sv.SV_EINVAL),
    (dict(t=None), sv.SV_ENULL), (dict(par=None), sv.SV_ENULL), (dict(tok=None), sv.SV_ENULL),
    (dict(acc=None), sv.SV_ENULL), (dict(out=None), sv.SV_ENULL), (dict(nodes=None), sv.SV_ENULL),
    (dict(t=FAKE + 2), sv.SV_EALIGN), (dict(ld=127), sv.SV_EALIGN),
    (dict(ws=None), sv.SV_EWORKSPACE), (dict(wsb=100), sv.SV_EWORKSPACE),
])
@pytest.mark.parametrize("fn", GREEDY_ENTRIES)
def test_greedy_argument_errors(fn, kw, code):
    # the split launches validate exactly like the whole call
    assert greedy_call(fn, **kw) == code


def path_call(**kw):
    args = dict(t=FAKE, ld_t=128, d=FAKE, ld_q=128, dtype=sv.SV_BF16, B=2, N=5, V=128, tok=FAKE,
                path=FAKE, Dmax=4, ua=FAKE, us=FAKE, lam=0.0, T=1.0, acc=FAKE, out=FAKE, ap=FAKE,
                st=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    args.update(kw)
    return sv.lib().sv_tree_verify_path(*args.values())


def test_path_ex_rejects_unknown_mode():
    args = dict(t=FAKE, ld_t=128, d=FAKE, ld_q=128, dtype=sv.SV_BF16, B=2, N=5, V=128, tok=FAKE,
                path=FAKE, Dmax=4, ua=FAKE, us=FAKE, lam=0.3, T=1.0, acc=FAKE, out=FAKE, ap=FAKE,
                st=FAKE, ws=FAKE, wsb=16, stream=None)
    L = sv.lib()
    assert L.sv_tree_verify_path_ex(*args.values(), 5) == sv.SV_EINVAL
    assert L.sv_tree_verify_path_ex(*args.values(), sv.SV_MIX_LOGIT) == sv.SV_EWORKSPACE


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=9), sv.SV_EDTYPE), (dict(Dmax=65), sv.SV_EINVAL), (dict(N=2000), sv.SV_EINVAL),
    (dict(T=0.0), sv.SV_EINVAL), (dict(lam=2.0), sv.SV_EINVAL), (dict(path=None), sv.SV_ENULL),
    (dict(tok=None), sv.SV_ENULL), (dict(d=None), sv.SV_ENULL), (dict(d=FAKE + 4), sv.SV_EALIGN),
    (dict(wsb=16), sv.SV_EWORKSPACE),
])
def test_path_argument_errors(kw, code):
    assert path_call(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), sv.SV_EINVAL), (dict(N=-1), sv.SV_EINVAL), (dict(N=1025), sv.SV_EINVAL),
    (dict(W=0), sv.SV_EINVAL), (dict(N=32, W=1), sv.SV_EINVAL), (dict(par=None), sv.SV_ENULL),
    (dict(mask=None), sv.SV_ENULL),
])
@pytest.mark.parametrize("fn", ["sv_tree_attention_mask", "sv_tree_attention_mask_timed"])
def test_mask_argument_errors(kw, code, fn):
    args = dict(par=FAKE, B=2, N=5, mask=FAKE, W=1, depth=None, st=None, stream=None)
    args.update(kw)
    timed = (FAKE, FAKE) if fn.endswith("_timed") else ()
    assert getattr(sv.lib(), fn)(*args.values(), *timed) == code


def test_mask_empty_batch_and_rootless_tree_need_no_parent():
    L = sv.lib()
    assert L.sv_tree_attention_mask(None, 0, 5, None, 1, None, None, None) == sv.SV_OK


def alpha_call(**kw):
    args = dict(t=FAKE, ld_t=128, d=FAKE, ld_q=128, dtype=sv.SV_BF16, B=2, K=4, V=128, dl=None,
                lam=0.3, T=1.0, space=sv.SV_MIX_PROB, alpha=FAKE, st=None, ws=FAKE, wsb=1 << 30,
                stream=None)
    args.update(kw)
    return sv.lib().sv_chain_acceptance_rate(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(space=3), sv.SV_EINVAL), (dict(dtype=5), sv.SV_EDTYPE), (dict(B=-1), sv.SV_EINVAL),
    (dict(K=65), sv.SV_EINVAL), (dict(V=0), sv.SV_EINVAL), (dict(lam=-1.0), sv.SV_EINVAL),
    (dict(T=0.0), sv.SV_EINVAL), (dict(alpha=None), sv.SV_ENULL), (dict(t=None), sv.SV_ENULL),
    (dict(d=FAKE + 2), sv.SV_EALIGN), (dict(ld_q=100), sv.SV_EALIGN), (dict(ws=None), sv.SV_EWORKSPACE),
    (dict(wsb="short"), sv.SV_EWORKSPACE), (dict(B=0, t=None, alpha=None), sv.SV_OK),
    (dict(K=0, d=None, alpha=None), sv.SV_OK),
])
def test_acceptance_rate_argument_errors(kw, code):
    if kw.get("wsb") == "short":
        kw = dict(wsb=sv.lib().sv_chain_acceptance_workspace_bytes(2, 4, 128) - 16)
    assert alpha_call(**kw) == code


def test_acceptance_workspace_covers_the_chain_layout():
    L = sv.lib()
    for B, K, V in [(1, 8, 128256), (64, 8, 128256), (3, 0, 10)]:
        assert L.sv_chain_acceptance_workspace_bytes(B, K, V) >= L.sv_chain_workspace_bytes(B, K, V)
    assert L.sv_chain_acceptance_workspace_bytes(1, 65, 10) == 0


def multi_call(**kw):
    args = dict(t=FAKE, ld_t=128, d=FAKE, ld_q=128, dtype=sv.SV_BF16, B=2, N=5, V=128, par=FAKE,
                tok=FAKE, ua=FAKE, us=FAKE, lam=0.2, T=1.0, space=sv.SV_MIX_PROB, acc=FAKE, out=FAKE,
                nodes=FAKE, ap=None, Dmax=4, st=None, ws=FAKE, wsb=1 << 30, stream=None)
    ex = kw.pop("ex", None)
    args.update(kw)
    if ex is None:
        return sv.lib().sv_tree_verify_multi(*args.values())
    return sv.lib().sv_tree_verify_multi_ex(*args.values(), ex)


@pytest.mark.parametrize("kw,code", [
    (dict(space=2), sv.SV_EINVAL), (dict(dtype=4), sv.SV_EDTYPE), (dict(B=-1), sv.SV_EINVAL),
    (dict(N=1025), sv.SV_EINVAL), (dict(V=0), sv.SV_EINVAL), (dict(Dmax=65), sv.SV_EINVAL),
    (dict(Dmax=-1), sv.SV_EINVAL), (dict(T=-1.0), sv.SV_EINVAL), (dict(lam=1.5), sv.SV_EINVAL),
    (dict(us=None), sv.SV_ENULL), (dict(acc=None), sv.SV_ENULL), (dict(out=None), sv.SV_ENULL),
    (dict(nodes=None), sv.SV_ENULL), (dict(par=None), sv.SV_ENULL), (dict(tok=None), sv.SV_ENULL),
    (dict(ua=None), sv.SV_ENULL), (dict(t=FAKE + 4), sv.SV_EALIGN), (dict(ld_q=127), sv.SV_EALIGN),
    (dict(ws=None), sv.SV_EWORKSPACE), (dict(wsb="short"), sv.SV_EWORKSPACE),
    (dict(B=0, t=None, acc=None), sv.SV_OK),
])
def test_multi_argument_errors(kw, code):
    if kw.get("wsb") == "short":
        kw = dict(wsb=sv.lib().sv_tree_multi_workspace_bytes(2, 5, 128) - 16)
    assert multi_call(**kw) == code
    for g in (0, 1, sv.SV_MAX_BLOCKS_PER_TREE):
        assert multi_call(ex=g, **kw) == code


@pytest.mark.parametrize("g", [-1, sv.SV_MAX_BLOCKS_PER_TREE + 1, 1 << 20])
def test_multi_ex_rejects_block_counts_outside_the_range(g):
    assert multi_call(ex=g) == sv.SV_EINVAL
    assert multi_call(ex=g, B=0, t=None, acc=None) == sv.SV_EINVAL


def test_read_stream_rejects_bad_arguments():
    L = sv.lib()
    buf = ctypes.c_void_p(0x10000)      # never dereferenced: every call fails validation
    sink = ctypes.c_void_p(0x20000)
    assert L.sv_read_stream(None, 1024, sink, None, None, None) == sv.SV_EINVAL
    assert L.sv_read_stream(buf, 1024, None, None, None, None) == sv.SV_EINVAL
    assert L.sv_read_stream(buf, 0, sink, None, None, None) == sv.SV_EINVAL
    assert L.sv_read_stream(buf, 1000, sink, None, None, None) == sv.SV_EINVAL
    assert L.sv_read_stream(ctypes.c_void_p(0x10008), 1024, sink, None, None, None) == sv.SV_EINVAL


def test_data_flags_match_the_header():
    text = open(HEADER).read()
    macros = {int(v, 16): n for n, v in re.findall(r"#define SV_DATA_([A-Z_]+)\s+(0x[0-9a-fA-F]+)", text)}
    assert macros == sv.DATA_FLAGS
    assert sv.decode_flags(0x82) == ["BAD_ROW", "SYNC"]


def test_header_constants_match_the_binding():
    text = open(HEADER).read()
    assert int(re.search(r"#define SV_MAX_POSITIONS\s+(\d+)", text).group(1)) == sv.SV_MAX_POSITIONS
    assert int(re.search(r"#define SV_MAX_TREE_NODES\s+(\d+)", text).group(1)) == sv.SV_MAX_TREE_NODES
    assert int(re.search(r"#define SV_MAX_VOCAB_BF16\s+(\d+)", text).group(1)) == sv.SV_MAX_VOCAB_BF16
    assert int(re.search(r"#define SV_MAX_VOCAB_F32\s+(\d+)", text).group(1)) == sv.SV_MAX_VOCAB_F32
    assert int(re.search(r"#define SV_MAX_BLOCKS_PER_TREE\s+(\d+)", text).group(1)) == sv.SV_MAX_BLOCKS_PER_TREE


@pytest.mark.parametrize("fn", ["sv_chain_verify", "sv_chain_row_stats", "sv_chain_accept_resample",
                                "sv_chain_verify_ex"])
@pytest.mark.parametrize("dtype,per", [(sv.SV_BF16, 8), (sv.SV_F32, 4)])
def test_chain_vocabulary_limit(fn, dtype, per):
    """One element past the largest vocabulary is refused before any launch."""
    vmax = sv.SV_MAX_VOCAB_BF16 if dtype == sv.SV_BF16 else sv.SV_MAX_VOCAB_F32
    ld = vmax + per
    assert chain_call(fn, dtype=dtype, V=vmax + 1, ld_t=ld, ld_q=ld) == sv.SV_EINVAL
    assert sv.lib().sv_chain_workspace_bytes(2, 4, vmax) > 0


def test_multi_empty_slot_marker_cannot_be_a_published_value():
    """The multi-branch walk's barrier reads a slot as empty while it holds a
    fixed signalling-NaN bit pattern.  A published value is an fp64 result of
    arithmetic (a quiet NaN at worst), an fp32 value widened (low 29 bits
    zero), or an integer converted to fp64 (never NaN): none can carry it."""
    text = open(os.path.join(ROOT, "sampling_spec_verify_amd", "csrc", "sv_multi.hip")).read()
    marker = int(re.search(r"kEmpty = (0x[0-9A-Fa-f]+)ull", text).group(1), 16)
    exp, frac = (marker >> 52) & 0x7FF, marker & ((1 << 52) - 1)
    assert exp == 0x7FF and frac != 0              # a NaN ...
    assert not (frac >> 51) & 1                     # ... with the quiet bit clear
    assert marker & ((1 << 29) - 1) != 0            # not a widened fp32 value
    # every fp32 NaN pattern (quiet and signalling, both signs), widened
    payload = np.arange(1, 1 << 23, dtype=np.uint32)
    for sign in (0, 1):
        bits = (np.uint32(sign << 31) | np.uint32(0xFF << 23) | payload).view(np.float32)
        with np.errstate(invalid="ignore"):
            wide = bits.astype(np.float64).view(np.uint64)
        assert not (wide == np.uint64(marker)).any()
