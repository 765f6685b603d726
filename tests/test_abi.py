"""The C ABI: libengram.so loads without a GPU, exports every entry point that
include/engram.h declares, and validates arguments on the host (statuses come
back before anything is enqueued, so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

import gram_hash_embedding_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "engram.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(engram_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) >= {"engram_hash", "engram_hash_gather_packed", "engram_gather_dequant", "engram_gather_dequant_packed",
                          "engram_pack_table", "engram_wkv", "engram_gate_dot",
                          "engram_gate_output", "engram_wkv_gate", "engram_wkv_gate_workspace_bytes",
                          "engram_gate_residual", "engram_wkv_gate_layers", "engram_status_string", "engram_last_error",
                          "engram_abi_version"}
    L = g.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    L = g.lib()
    assert L.engram_abi_version() == 1
    for s in range(4):
        assert L.engram_status_string(s)
    assert L.engram_status_string(99) == b"unknown status"


P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first


def _err():
    return g.lib().engram_last_error().decode()


@pytest.mark.parametrize("args,status,msg", [
    (dict(B=-1), 1, "negative"),
    (dict(N=1), 1, "N=1"),
    (dict(N=9), 1, "N=9"),
    (dict(E=0), 1, "E=0"),
    (dict(E=9), 1, "E=9"),
    (dict(H=0), 1, "H=0"),
    (dict(H=400), 1, "columns"),
    (dict(cache_B=1), 2, "cache"),
    (dict(cache_L=63), 2, "cache"),
    (dict(start_pos=1), 2, "cache"),
    (dict(input_ids=None), 1, "null"),
    (dict(out=None), 1, "null"),
    (dict(input_ids=ctypes.c_void_p(0x100004)), 1, "aligned"),
])
def test_hash_validation(args, status, msg):
    a = dict(input_ids=FAKE, B=2, L=64, start_pos=0, mask=None, token_map=FAKE, vocab=10, cache=FAKE, cache_B=2,
             cache_L=64, mult=FAKE, primes=FAKE, offsets=FAKE, E=1, N=4, H=2, pad=2, dead=-1, out=FAKE)
    a.update(args)
    rc = g.lib().engram_hash(a["input_ids"], a["B"], a["L"], a["start_pos"], a["mask"], a["token_map"], a["vocab"],
                             a["cache"], a["cache_B"], a["cache_L"], a["mult"], a["primes"], a["offsets"], a["E"],
                             a["N"], a["H"], a["pad"], a["dead"], a["out"], None)
    assert rc == status
    assert msg in _err()


def test_zero_tokens_is_a_valid_no_op():
    L = g.lib()
    assert L.engram_hash(None, 0, 5, 0, None, None, 10, None, 0, 5, None, None, None, 1, 4, 2, 2, -1, None, None) == 0
    assert L.engram_hash_gather_packed(None, 0, 5, 0, None, None, 10, None, 0, 5, None, None, None, 1, 4, 2, 2, -1,
                                       None, None, None, None, 64, 32, None, None) == 0
    assert L.engram_gather_dequant(None, 0, 24, 24, None, None, 10, 0, 64, 32, None, None, None, None) == 0
    assert L.engram_gather_dequant_packed(None, 0, 24, 24, None, 10, 0, 64, 32, None, None, None, None) == 0
    assert L.engram_pack_table(None, None, 0, 64, 32, None, None) == 0
    assert L.engram_wkv(None, None, None, 0, 64, 64, None) == 0
    assert L.engram_gate_dot(None, None, 64, None, None, 1e-20, None, 0, 4, 16, None) == 0
    assert L.engram_gate_output(None, None, 80, None, None, 1e-20, None, None, None, 0, 4, 16, None) == 0
    assert L.engram_wkv_gate(None, None, None, None, None, 1e-20, None, 256, None, None, 0, 0, 64, 4, 256, None) == 0
    assert L.engram_gate_residual(None, None, 16, None, None, None, 0, 4, 16, None) == 0
    assert L.engram_wkv_gate_layers(2, None, None, None, None, None, 1e-20, None, 256, None, None, 0, 0, 64, 4, 256,
                                    None) == 0


def _hash_gather(**kw):
    a = dict(input_ids=FAKE, B=2, L=64, start_pos=0, mask=None, token_map=FAKE, vocab=10, cache=FAKE, cache_B=2,
             cache_L=64, mult=FAKE, primes=FAKE, offsets=FAKE, E=2, N=4, H=2, pad=2, dead=-1, ids=None,
             tables=[FAKE.value, FAKE.value], rows=[100, 100], row_starts=None, D=64, blk=32,
             outs=[FAKE.value, FAKE.value])
    a.update(kw)
    arr = lambda t, v: None if v is None else (t * len(v))(*v)
    return g.lib().engram_hash_gather_packed(
        a["input_ids"], a["B"], a["L"], a["start_pos"], a["mask"], a["token_map"], a["vocab"], a["cache"],
        a["cache_B"], a["cache_L"], a["mult"], a["primes"], a["offsets"], a["E"], a["N"], a["H"], a["pad"], a["dead"],
        a["ids"], arr(ctypes.c_void_p, a["tables"]), arr(ctypes.c_int64, a["rows"]),
        arr(ctypes.c_int64, a["row_starts"]), a["D"], a["blk"], arr(ctypes.c_void_p, a["outs"]), None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(D=48), 1, "D=48"), (dict(blk=8), 1, "blk=8"), (dict(blk=48), 1, "blk=48"), (dict(E=0), 1, "E=0"),
    (dict(E=9), 1, "E=9"), (dict(N=1), 1, "N=1"), (dict(cache_L=63), 2, "cache"), (dict(tables=None), 1, "null"),
    (dict(outs=None), 1, "null"), (dict(rows=[100, 0]), 1, "layer 1: R < 1"),
    (dict(tables=[FAKE.value, None]), 1, "layer 1: null"), (dict(outs=[None, FAKE.value]), 1, "layer 0: null"),
    (dict(tables=[FAKE.value, 0x100040]), 1, "layer 1: misaligned"),  # a 128-byte record needs 128
    (dict(outs=[FAKE.value, 0x100008]), 1, "layer 1: misaligned"),
    (dict(input_ids=None), 1, "null"), (dict(ids=ctypes.c_void_p(0x100004)), 1, "aligned"),
    (dict(E=8, N=8, H=100, tables=[FAKE.value] * 8, rows=[100] * 8, outs=[FAKE.value] * 8), 1, "at most 4096"),
])
def test_hash_gather_validation(kw, status, msg):
    assert _hash_gather(**kw) == status
    assert msg in _err()
    assert "engram_hash_gather_packed" in _err()


@pytest.mark.parametrize("kw,msg", [
    (dict(D=48), "D=48"),
    (dict(blk=8), "blk=8"),
    (dict(blk=48), "blk=48"),
    (dict(C=0), "C=0"),
    (dict(stride=3), "stride"),
    (dict(R=0), "R < 1"),
    (dict(weight=None), "null"),
    (dict(weight=ctypes.c_void_p(0x100008)), "misaligned"),
])
def test_gather_validation(kw, msg):
    a = dict(ids=FAKE, T=10, stride=24, C=24, weight=FAKE, scale=FAKE, R=100, row_start=0, D=64, blk=32, out=FAKE)
    a.update(kw)
    rc = g.lib().engram_gather_dequant(a["ids"], a["T"], a["stride"], a["C"], a["weight"], a["scale"], a["R"],
                                       a["row_start"], a["D"], a["blk"], a["out"], None, None, None)
    assert rc == 1
    assert msg in _err()


@pytest.mark.parametrize("kw,msg", [
    (dict(D=48), "D=48"),
    (dict(blk=8), "blk=8"),
    (dict(C=0), "C=0"),
    (dict(R=0), "R < 1"),
    (dict(table=None), "null"),
    (dict(table=ctypes.c_void_p(0x100040)), "misaligned"),  # 64-byte aligned, a 128-byte record needs 128
])
def test_gather_packed_validation(kw, msg):
    a = dict(ids=FAKE, T=10, stride=24, C=24, table=FAKE, R=100, row_start=0, D=64, blk=32, out=FAKE)
    a.update(kw)
    rc = g.lib().engram_gather_dequant_packed(a["ids"], a["T"], a["stride"], a["C"], a["table"], a["R"],
                                              a["row_start"], a["D"], a["blk"], a["out"], None, None, None)
    assert rc == 1
    assert msg in _err()
    assert "engram_gather_dequant_packed" in _err()


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("kw,msg", [
    (dict(D=48), "D=48"),
    (dict(blk=8), "blk=8"),
    (dict(C=3, stride=3), "C*D=192"),  # the MX scale layout needs whole 128-column groups
    (dict(R=0), "R < 1"),
    (dict(q=None), "null"),
    (dict(q_scale=None), "null"),
    (dict(q=ctypes.c_void_p(0x100008)), "misaligned"),
])
def test_gather_mx_validation(kw, msg, packed):
    a = dict(ids=FAKE, T=10, stride=24, C=24, weight=FAKE, scale=FAKE, R=100, row_start=0, D=64, blk=32, q=FAKE,
             q_scale=FAKE)
    a.update(kw)
    L = g.lib()
    if packed:
        rc = L.engram_gather_mx_packed(a["ids"], a["T"], a["stride"], a["C"], a["weight"], a["R"], a["row_start"],
                                       a["D"], a["blk"], a["q"], a["q_scale"], None)
    else:
        rc = L.engram_gather_mx(a["ids"], a["T"], a["stride"], a["C"], a["weight"], a["scale"], a["R"],
                                a["row_start"], a["D"], a["blk"], a["q"], a["q_scale"], None)
    assert rc == 1
    assert msg in _err()
    assert ("engram_gather_mx_packed" if packed else "engram_gather_mx") in _err()


@pytest.mark.parametrize("kw,msg", [(dict(D=40), "D=40"), (dict(blk=24), "blk=24"), (dict(R=-1), "R < 0"),
                                    (dict(packed=None), "null"), (dict(packed=ctypes.c_void_p(0x100040)), "misaligned")])
def test_pack_table_validation(kw, msg):
    a = dict(weight=FAKE, scale=FAKE, R=100, D=64, blk=32, packed=FAKE)
    a.update(kw)
    assert g.lib().engram_pack_table(a["weight"], a["scale"], a["R"], a["D"], a["blk"], a["packed"], None) == 1
    assert msg in _err()


@pytest.mark.parametrize("K,N,msg", [(0, 64, "K=0"), (12, 64, "K=12"), (64, 4, "Nout=4"), (64, 36, "Nout=36")])
def test_wkv_validation(K, N, msg):
    assert g.lib().engram_wkv(FAKE, FAKE, FAKE, 10, K, N, None) == 1
    assert msg in _err()


@pytest.mark.parametrize("ld,hc,dim,msg", [(64, 0, 16, "hc=0"), (64, 65, 16, "hc=65"), (64, 4, 12, "dim=12"),
                                           (60, 4, 16, "ld_kv"), (68, 4, 16, "ld_kv")])
def test_gate_validation(ld, hc, dim, msg):
    assert g.lib().engram_gate_dot(FAKE, FAKE, ld, FAKE, FAKE, 1e-20, FAKE, 10, hc, dim, None) == 1
    assert msg in _err()


@pytest.mark.parametrize("ld,hc,dim,msg", [(80, 0, 16, "hc=0"), (80, 65, 16, "hc=65"), (80, 4, 12, "dim=12"),
                                           (16392, 1, 8200, "dim=8200"), (64, 4, 16, "ld_kv"),
                                           (84, 4, 16, "ld_kv")])
def test_gate_output_validation(ld, hc, dim, msg):
    assert g.lib().engram_gate_output(FAKE, FAKE, ld, FAKE, FAKE, 1e-20, None, FAKE, None, 10, hc, dim, None) == 1
    assert msg in _err()


def test_gate_output_pointer_checks():
    L = g.lib()
    assert L.engram_gate_output(FAKE, FAKE, 80, FAKE, FAKE, 1e-20, None, None, None, 10, 4, 16, None) == 1
    assert "null" in _err()
    bad = ctypes.c_void_p(0x100008)
    assert L.engram_gate_output(FAKE, FAKE, 80, FAKE, FAKE, 1e-20, None, bad, None, 10, 4, 16, None) == 1
    assert "misaligned" in _err()
    assert L.engram_gate_output(FAKE, FAKE, 80, FAKE, FAKE, 1e-20, None, FAKE, ctypes.c_void_p(0x100002), 10, 4,
                                16, None) == 1
    assert "misaligned" in _err()


def test_wkv_gate_workspace_bytes():
    L = g.lib()
    assert L.engram_wkv_gate_workspace_bytes(65536, 4, 5120) == 4 * 40 * 3 * 65536 * 4
    assert L.engram_wkv_gate_workspace_bytes(1, 1, 256) == 1 * 2 * 3 * 1 * 4
    assert L.engram_wkv_gate_workspace_bytes(0, 4, 256) == 0
    for T, hc, dim in [(-1, 4, 256), (10, 0, 256), (10, 65, 256), (10, 4, 320), (10, 4, 128)]:
        assert L.engram_wkv_gate_workspace_bytes(T, hc, dim) == -1
    with pytest.raises(ValueError):
        g.engram_wkv_gate_workspace_bytes(10, 4, 320)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(K=96), 1, "K=96"), (dict(K=0), 1, "K=0"), (dict(hc=0), 1, "hc=0"), (dict(dim=320), 1, "dim=320"),
    (dict(dim=128), 1, "dim=128"), (dict(ld_value=200), 1, "ld_value"), (dict(ld_value=260), 1, "ld_value"),
    (dict(ws_bytes=10 * 4 * 2 * 3 * 4 - 4), 2, "workspace"), (dict(a=None), 1, "null"), (dict(ws=None), 1, "null"),
    (dict(value=ctypes.c_void_p(0x100008)), 1, "misaligned"), (dict(ws=ctypes.c_void_p(0x100004)), 1, "misaligned"),
])
def test_wkv_gate_validation(kw, status, msg):
    a = dict(a=FAKE, w=FAKE, x=FAKE, q=FAKE, k=FAKE, value=FAKE, ld_value=256, dot=FAKE, ws=FAKE,
             ws_bytes=10 * 4 * 2 * 3 * 4, T=10, K=128, hc=4, dim=256)
    a.update(kw)
    rc = g.lib().engram_wkv_gate(a["a"], a["w"], a["x"], a["q"], a["k"], 1e-20, a["value"], a["ld_value"], a["dot"],
                                 a["ws"], a["ws_bytes"], a["T"], a["K"], a["hc"], a["dim"], None)
    assert rc == status
    assert msg in _err()


@pytest.mark.parametrize("ld,hc,dim,msg", [(16, 0, 16, "hc=0"), (16, 65, 16, "hc=65"), (16, 4, 12, "dim=12"),
                                           (8, 4, 16, "ld_value"), (20, 4, 16, "ld_value")])
def test_gate_residual_validation(ld, hc, dim, msg):
    assert g.lib().engram_gate_residual(FAKE, FAKE, ld, FAKE, None, FAKE, 10, hc, dim, None) == 1
    assert msg in _err()
    assert g.lib().engram_gate_residual(FAKE, FAKE, 16, None, None, FAKE, 10, 4, 16, None) == 1
    assert "null" in _err()


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(g, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(g, "_lib", None)
    with pytest.raises(ImportError):
        g.lib()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(layers=0), 1, "layers=0"), (dict(layers=9), 1, "layers=9"), (dict(a=None), 1, "null pointer array"),
    (dict(dot=None), 1, "null pointer array"), (dict(K=96), 1, "K=96"), (dict(dim=320), 1, "dim=320"),
    (dict(ws_bytes=2 * 10 * 4 * 2 * 3 * 4 - 4), 2, "workspace"), (dict(ws=None), 1, "null"),
    (dict(value=[FAKE.value, 0x100008]), 1, "layer 1: misaligned"), (dict(x=[FAKE.value, None]), 1, "layer 1: null"),
])
def test_wkv_gate_layers_validation(kw, status, msg):
    a = dict(layers=2, a=[FAKE.value] * 2, w=[FAKE.value] * 2, x=[FAKE.value] * 2, q=[FAKE.value] * 2,
             k=[FAKE.value] * 2, value=[FAKE.value] * 2, ld_value=256, dot=[FAKE.value] * 2, ws=FAKE,
             ws_bytes=2 * 10 * 4 * 2 * 3 * 4, T=10, K=128, hc=4, dim=256)
    a.update(kw)
    arr = lambda v: None if v is None else (ctypes.c_void_p * len(v))(*v)
    rc = g.lib().engram_wkv_gate_layers(a["layers"], arr(a["a"]), arr(a["w"]), arr(a["x"]), arr(a["q"]), arr(a["k"]),
                                        1e-20, arr(a["value"]), a["ld_value"], arr(a["dot"]), a["ws"], a["ws_bytes"],
                                        a["T"], a["K"], a["hc"], a["dim"], None)
    assert rc == status
    assert msg in _err()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(layers=0), 1, "layers=0"), (dict(a=None), 1, "null pointer array"), (dict(K=96), 1, "K=96"),
    (dict(dim=320), 1, "dim=320"), (dict(ld_value=200), 1, "ld_value"),
    (dict(value=[FAKE.value, 0x100008]), 1, "layer 1: misaligned"),
    # 2 layers x 4370 tokens x 4 copies x 40 slice pairs x 3 floats x 4 bytes = 16,780,800 > 16 MiB of scratch
    (dict(T=4370, dim=5120), 2, "scratch"),
])
def test_wkv_gate_layers_noalloc_validation(kw, status, msg):
    """The allocation-free entry point checks every argument, and its scratch limit, before it looks up the
    scratch's device address (no HIP call happens here)."""
    a = dict(layers=2, a=[FAKE.value] * 2, w=[FAKE.value] * 2, x=[FAKE.value] * 2, q=[FAKE.value] * 2,
             k=[FAKE.value] * 2, value=[FAKE.value] * 2, ld_value=256, dot=[FAKE.value] * 2, T=10, K=128, hc=4,
             dim=256)
    a.update(kw)
    if a["dim"] == 5120:
        a["ld_value"] = 5120
    arr = lambda v: None if v is None else (ctypes.c_void_p * len(v))(*v)
    rc = g.lib().engram_wkv_gate_layers_noalloc(a["layers"], arr(a["a"]), arr(a["w"]), arr(a["x"]), arr(a["q"]),
                                                arr(a["k"]), 1e-20, arr(a["value"]), a["ld_value"], arr(a["dot"]),
                                                a["T"], a["K"], a["hc"], a["dim"], None)
    assert rc == status
    assert msg in _err()
    assert g.NOALLOC_SCRATCH_BYTES == 16 << 20
    # 2 layers x 4369 tokens fit
    assert 2 * g.lib().engram_wkv_gate_workspace_bytes(4369, 4, 5120) <= g.NOALLOC_SCRATCH_BYTES


def test_mx_validation():
    L = g.lib()
    assert L.engram_mx_scale_bytes(10, 256) == 2 * 12 * 4
    assert L.engram_mx_scale_bytes(0, 128) == 0
    assert L.engram_mx_scale_bytes(10, 192) == -1 and L.engram_mx_scale_bytes(10, 0) == -1
    assert L.engram_mx_quant(FAKE, 10, 192, FAKE, FAKE, None) == 1 and "K=192" in _err()
    assert L.engram_mx_quant(FAKE, -1, 128, FAKE, FAKE, None) == 1 and "rows" in _err()
    assert L.engram_mx_quant(None, 10, 128, FAKE, FAKE, None) == 1 and "null" in _err()
    assert L.engram_mx_quant(ctypes.c_void_p(0x100008), 10, 128, FAKE, FAKE, None) == 1 and "misaligned" in _err()
    assert L.engram_mx_quant(None, 0, 128, None, None, None) == 0
    assert L.engram_wkv_mx(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 64, 256, None) == 1 and "K=64" in _err()
    assert L.engram_wkv_mx(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 128, 12, None) == 1 and "Nout=12" in _err()
    assert L.engram_wkv_mx(FAKE, None, FAKE, FAKE, FAKE, 10, 128, 256, None) == 1 and "null" in _err()
    assert L.engram_wkv_mx(FAKE, FAKE, FAKE, ctypes.c_void_p(0x100004), FAKE, 10, 128, 256, None) == 1
    assert "misaligned" in _err()
    assert L.engram_wkv_mx(None, None, None, None, None, 0, 128, 256, None) == 0


def test_formats_validation():
    L = g.lib()
    args = lambda **kw: dict(dict(ids=FAKE, idb=8, T=10, stride=24, C=24, w=FAKE, s=FAKE, fmt=1, R=100, rs=0, D=64,
                                  blk=32, out=FAKE, o8=None, os=None), **kw)
    call = lambda a: L.engram_gather_dequant_fmt(a["ids"], a["idb"], a["T"], a["stride"], a["C"], a["w"], a["s"],
                                                 a["fmt"], a["R"], a["rs"], a["D"], a["blk"], a["out"], a["o8"],
                                                 a["os"], None)
    assert call(args(idb=2)) == 1 and "id_bytes" in _err()
    assert call(args(fmt=3)) == 1 and "scale_format" in _err()
    assert call(args(blk=24)) == 1 and "blk" in _err()
    assert call(args(ids=ctypes.c_void_p(0x100004))) == 1 and "misaligned" in _err()  # int64 ids need 8 bytes
    assert call(args(s=None)) == 1 and "null" in _err()
    assert call(args(T=0, ids=None, w=None, s=None, out=None)) == 0
    assert L.engram_hash_i32(FAKE, 1, 64, 0, None, FAKE, 10, FAKE, 1, 64, FAKE, FAKE, FAKE, 1, 4, 2, 2, -1, None,
                             None) == 1
    assert "null" in _err()
    assert L.engram_hash_i32(FAKE, 1, 64, 0, None, FAKE, 10, FAKE, 1, 64, FAKE, FAKE, FAKE, 1, 4, 2, 2, -1,
                             ctypes.c_void_p(0x100002), None) == 1
    assert "aligned" in _err()


def test_probe_library_exports_and_validates():
    """libengram_probe.so (the measured ceilings) loads without a GPU, exports what include/engram_probe.h
    declares, and rejects bad arguments on the host before any launch."""
    from gram_hash_embedding_amd import build as engram_build

    text = open(os.path.join(ROOT, "include", "engram_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(engram_probe_\w+)\s*\(", text)))
    assert set(names) == {"engram_probe_mfma", "engram_probe_read", "engram_probe_copy", "engram_probe_read_grid"}
    L = ctypes.CDLL(engram_build.PROBE_LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    L.engram_probe_mfma.argtypes = [ctypes.c_int32, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]
    L.engram_probe_read.argtypes = [P, ctypes.c_int64, P, P]
    L.engram_probe_copy.argtypes = [P, P, ctypes.c_int64, P]
    assert L.engram_probe_read_grid() > 0
    assert L.engram_probe_mfma(5, FAKE, FAKE, 256, 8, 10, None) != 0   # unknown kind
    assert L.engram_probe_mfma(-1, FAKE, FAKE, 256, 8, 10, None) != 0
    assert L.engram_probe_mfma(0, FAKE, FAKE, 256, 9, 10, None) != 0   # more than 8 waves
    assert L.engram_probe_mfma(0, None, FAKE, 256, 8, 10, None) != 0
    assert L.engram_probe_read(FAKE, 24, FAKE, None) != 0              # not a multiple of 16
    assert L.engram_probe_read(ctypes.c_void_p(0x100008), 32, FAKE, None) != 0  # misaligned
    assert L.engram_probe_copy(FAKE, None, 32, None) != 0


def test_mx_gate_validation():
    L = g.lib()
    need = L.engram_wkv_gate_workspace_bytes(10, 4, 256)
    args = lambda **kw: dict(dict(a=FAKE, as_=FAKE, w=FAKE, ws=FAKE, x=FAKE, q=FAKE, k=FAKE, value=FAKE, ld=256,
                                  dot=FAKE, ws_buf=FAKE, ws_bytes=need, T=10, K=384, hc=4, dim=256), **kw)
    call = lambda a: L.engram_wkv_mx_gate(a["a"], a["as_"], a["w"], a["ws"], a["x"], a["q"], a["k"], 1e-20,
                                          a["value"], a["ld"], a["dot"], a["ws_buf"], a["ws_bytes"], a["T"], a["K"],
                                          a["hc"], a["dim"], None)
    assert call(args(K=256)) == 1 and "K=256" in _err()  # at least three 128-column slabs
    assert call(args(K=400)) == 1 and "K=400" in _err()
    assert call(args(hc=0)) == 1 and "hc=0" in _err()
    assert call(args(dim=320)) == 1 and "dim=320" in _err()
    assert call(args(hc=64, dim=65536, ld=65536, ws_bytes=1 << 40)) == 1 and "2^22" in _err()  # 128 rows of x < 2 GiB
    assert call(args(ld=128)) == 1 and "ld_value" in _err()
    assert call(args(ws_bytes=need - 4)) == 2 and "workspace" in _err()
    assert call(args(x=None)) == 1 and "null" in _err()
    assert call(args(dot=ctypes.c_void_p(0x100002))) == 1 and "misaligned" in _err()
    assert call(args(T=0, a=None, as_=None, w=None, ws=None, x=None, q=None, k=None, value=None, dot=None,
                     ws_buf=None, ws_bytes=0)) == 0
