"""Host-side checks of the C ABI (CPU only, no GPU compute).

The library loads, exports every entry point the header declares, and rejects invalid
arguments on the host before anything is enqueued (these calls return before any HIP
call is made, so they are safe without a GPU).
"""

import ctypes
import os
import re

import pytest

from ragged_verify_acceptance_amd import rva

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rva.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x100000)  # non-null, 256-aligned; never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rva_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = rva.lib()
    names = declared_functions()
    assert "rva_verify_attention" in names and len(names) == 18
    for n in names:
        assert hasattr(L, n), f"{n} declared in rva.h but not exported"
    assert set(names) == set(rva.EXPORTED)


def test_version():
    assert rva.version() == 100


def _sched(**kw):
    args = dict(B=4, gamma=6, mode=0, hidden=None, hd=1, H=0, head_w=None, head_b=0.0,
                conf_in=FAKE, sts_T=None, bias=20.0, alpha=FAKE, alpha_len=5, theta=FAKE,
                theta_len=25, out=FAKE)
    args.update(kw)
    a = args
    return rva.lib().rva_schedule_windows(a["B"], a["gamma"], a["mode"], a["hidden"], a["hd"], a["H"],
                                          a["head_w"], a["head_b"], a["conf_in"], a["sts_T"], a["bias"],
                                          a["alpha"], a["alpha_len"], a["theta"], a["theta_len"],
                                          a["out"], a["out"], a["out"], a["out"], a["out"], None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), INVALID),
    (dict(gamma=1), INVALID),
    (dict(gamma=65), INVALID),
    (dict(B=1000, gamma=6), INVALID),          # B*(gamma-1) > 4096
    (dict(mode=7), INVALID),
    (dict(conf_in=None), INVALID),             # neither hidden nor conf_in
    (dict(hidden=FAKE, H=16, head_w=FAKE), INVALID),  # both given
    (dict(sts_T=FAKE), INVALID),               # temperatures need the head's logits
    (dict(alpha_len=4), INVALID),              # alpha_len must exceed B
    (dict(theta_len=24), INVALID),             # theta_len must exceed B*gamma
    (dict(out=None), INVALID),
])
def test_schedule_validation(kw, code):
    assert _sched(**kw) == code
    assert rva.lib().rva_last_error().decode() != ""


def _pack(B=3, gamma=6, tiers=(4, 8, 12, 18), max_rows=18, src=None, dst=None, windows=FAKE):
    t = (ctypes.c_int32 * len(tiers))(*tiers)
    return rva.lib().rva_pack_ragged(B, gamma, windows, FAKE, ctypes.cast(t, ctypes.c_void_p), len(tiers),
                                     src, 16 if src else 0, dst, max_rows, FAKE, FAKE, FAKE, FAKE, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), INVALID),
    (dict(tiers=(4, 12, 8, 18)), INVALID),     # not ascending
    (dict(tiers=(4, 8, 12, 16)), INVALID),     # largest tier below B*gamma = 18
    (dict(max_rows=17), INVALID),
    (dict(src=FAKE), INVALID),                 # src without dst
    (dict(windows=None), INVALID),
])
def test_pack_validation(kw, code):
    assert _pack(**kw) == code


def _sched_pack(B=3, gamma=6, mode=0, conf_in=FAKE, alpha_len=4, theta_len=19, tiers=(4, 8, 12, 18),
                max_rows=18, src=None, dst=None, windows=FAKE):
    t = (ctypes.c_int32 * len(tiers))(*tiers)
    return rva.lib().rva_schedule_and_pack(B, gamma, mode, None, 1, 0, None, 0.0, conf_in, None, 20.0, FAKE,
                                           alpha_len, FAKE, theta_len, FAKE, FAKE, windows, FAKE, FAKE, FAKE,
                                           ctypes.cast(t, ctypes.c_void_p), len(tiers), src, 16 if src else 0,
                                           dst, max_rows, FAKE, FAKE, FAKE, FAKE, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), INVALID),                      # both stages reject it
    (dict(gamma=65), INVALID),                 # the schedule's limit
    (dict(mode=3), INVALID),
    (dict(conf_in=None), INVALID),             # neither hidden nor conf_in
    (dict(alpha_len=3), INVALID),              # alpha_len must exceed B
    (dict(tiers=(4, 12, 8, 18)), INVALID),     # the pack's checks: tiers not ascending
    (dict(max_rows=17), INVALID),
    (dict(src=FAKE), INVALID),                 # src without dst
    (dict(windows=None), INVALID),
])
def test_schedule_and_pack_validation(kw, code):
    assert _sched_pack(**kw) == code
    assert rva.lib().rva_last_error().decode() != ""


def _attn(B=2, max_window=6, max_rows=16, Hq=32, Hkv=8, D=128, page=64, num_pages=10, max_pages=5,
          dtype=1, ws=None, ws_bytes=0, q=FAKE):
    return rva.lib().rva_verify_attention(B, max_window, max_rows, Hq, Hkv, D, page, num_pages, max_pages,
                                          dtype, q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1,
                                          FAKE, None, ws, ws_bytes, None)


def test_attention_validation():
    need = rva.verify_attention_workspace_size(2, 6, 32, 8, 128, 64, 5, 1)
    assert need > 0
    assert _attn(Hq=30) == INVALID                        # Hq % Hkv != 0
    assert _attn(D=96) == UNSUPPORTED
    assert _attn(max_window=1025) == UNSUPPORTED          # 1025 * 4 > 4096 columns per kv head
    assert _attn(dtype=5) == INVALID
    assert _attn(q=None) == INVALID
    assert _attn(q=ctypes.c_void_p(0x100002)) == INVALID  # misaligned
    assert _attn(ws=None) == WS_SMALL
    assert _attn(ws=FAKE, ws_bytes=need - 1) == WS_SMALL
    # the float32 generic path needs no workspace
    assert rva.verify_attention_workspace_size(2, 6, 4, 2, 64, 16, 5, 0) == 0


def _attn_noalloc(B=2, max_window=6, max_rows=16, Hq=32, Hkv=8, D=128, page=64, num_pages=10,
                  max_pages=5, dtype=1, q=FAKE):
    return rva.lib().rva_verify_attention_noalloc(B, max_window, max_rows, Hq, Hkv, D, page,
                                                  num_pages, max_pages, dtype, q, FAKE, FAKE, FAKE,
                                                  FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, None)


def test_attention_noalloc_validation():
    """The no-workspace variant validates its arguments before it looks up the library's
    scratch, with the same codes as the workspace variant (no GPU needed for these)."""
    assert _attn_noalloc(Hq=30) == INVALID
    assert _attn_noalloc(D=96) == UNSUPPORTED
    assert _attn_noalloc(max_window=1025) == UNSUPPORTED
    assert _attn_noalloc(dtype=5) == INVALID
    assert _attn_noalloc(q=None) == INVALID
    assert _attn_noalloc(q=ctypes.c_void_p(0x100002)) == INVALID


def _accept(B=2, gamma=6, V=1024, dtype=1, max_rows=16, ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = rva.accept_workspace_size(B, max(gamma, 2), V, max_rows)
    return rva.lib().rva_accept_and_commit(B, gamma, V, dtype, max_rows, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           FAKE, FAKE, FAKE, None, None, None, None, ws, ws_bytes, None)


def test_accept_validation():
    assert _accept(B=0) == INVALID
    assert _accept(gamma=1) == INVALID
    assert _accept(V=0) == INVALID
    assert _accept(dtype=3) == INVALID
    assert _accept(ws_bytes=0) == WS_SMALL
    assert _accept(ws=None) == WS_SMALL
    assert _accept(max_rows=70000) == INVALID   # grid rows beyond 65535
    big = rva.accept_workspace_size(256, 16, 151936, 4096)
    assert big > rva.accept_workspace_size(64, 8, 151936, 512) > 0


def _capped(cap=FAKE, full=FAKE, B=2, gamma=6, V=1024, ws=FAKE):
    ws_bytes = rva.accept_workspace_size(B, gamma, V, 16)
    return rva.lib().rva_accept_capped(B, gamma, V, 1, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, cap,
                                       FAKE, full, FAKE, FAKE, None, None, None, None, ws, ws_bytes,
                                       None)


def test_accept_capped_validation():
    assert _capped(cap=None) == INVALID            # the commit cap is required
    assert _capped(full=None) == INVALID           # so is the uncapped accept length
    assert _capped(B=0) == INVALID
    assert _capped(gamma=65) == INVALID
    assert _capped(ws=None) == WS_SMALL


def test_pack_binding_row_bytes(monkeypatch):
    """The binding derives the packed row size from the source's trailing shape, also when
    only the first B blocks of a larger source are packed."""
    import types

    import torch

    seen = {}

    class FakeLib:
        def rva_pack_ragged(self, *args):
            seen["row_bytes"] = args[7]
            return 0

        def rva_last_error(self):
            return b""

    monkeypatch.setattr(rva, "lib", lambda: FakeLib())
    # host tensors stand in for device ones: nothing is dereferenced
    monkeypatch.setattr(rva, "_ptr", lambda t: None if t is None else ctypes.c_void_p(t.data_ptr()))
    st = types.SimpleNamespace(cuda_stream=0)
    i32 = torch.zeros(64, dtype=torch.int32)
    src = torch.zeros((64, 8, 4096), dtype=torch.bfloat16)
    dst = torch.zeros((512, 4096), dtype=torch.bfloat16)
    for B in (1, 48, 64):
        rva.pack_ragged(B, 8, i32, i32, [8, 512], src, dst, 512, i32, i32, i32, i32, stream=st)
        assert seen["row_bytes"] == 8192
    with pytest.raises(ValueError):
        rva.pack_ragged(65, 8, i32, i32, [8, 520], src, dst, 512, i32, i32, i32, i32, stream=st)
    with pytest.raises(ValueError):   # destination rows of another size
        rva.pack_ragged(4, 8, i32, i32, [8, 32], src, dst[:, :100], 512, i32, i32, i32, i32,
                        stream=st)
    with pytest.raises(ValueError):   # block length mismatch
        rva.pack_ragged(4, 6, i32, i32, [8, 32], src, dst, 512, i32, i32, i32, i32, stream=st)


def test_calibration_validation():
    L = rva.lib()
    ws = rva.sts_fit_workspace_size(1000)
    assert ws > 1000 * 8 and rva.sts_fit_workspace_size(0) == 0

    def fit(N=1000, G1=7, z=FAKE, n=FAKE, T_out=FAKE, lo=0.05, hi=20.0, w=FAKE, wb=ws):
        return L.rva_sts_fit(N, G1, z, n, None, lo, hi, T_out, None, w, wb, None)

    assert fit(N=0) == INVALID
    assert fit(G1=64) == INVALID
    assert fit(z=None) == INVALID
    assert fit(T_out=None) == INVALID
    assert fit(lo=0.0) == INVALID
    assert fit(lo=2.0, hi=1.0) == INVALID
    assert fit(w=None) == WS_SMALL
    assert fit(wb=ws - 1) == WS_SMALL
    assert fit(w=ctypes.c_void_p(0x100010)) == INVALID   # not 256-byte aligned

    we = rva.calibration_ece_workspace_size(1000, 7, 15)
    assert we > 0 and rva.calibration_ece_workspace_size(1000, 63, 64) == 0  # 63*64 > 3840

    def ece(N=1000, G1=7, nb=15, out=FAKE, w=FAKE, wb=we):
        return L.rva_calibration_ece(N, G1, FAKE, FAKE, None, None, nb, out, None, w, wb, None)

    assert ece(nb=0) == INVALID
    assert ece(nb=65) == INVALID
    assert ece(G1=63, nb=61) == INVALID
    assert ece(out=None) == INVALID
    assert ece(w=None) == WS_SMALL
    assert ece(wb=we - 1) == WS_SMALL


def test_markov_validation():
    L = rva.lib()
    ws = rva.markov_workspace_size(64, 151936)
    assert ws > 0 and rva.markov_workspace_size(0, 10) == 0

    def mk(B=64, G1=7, V=151936, r=256, dt=1, base=FAKE, out=ctypes.c_void_p(0x200000), w1=FAKE,
           w=FAKE, wb=ws):
        return L.rva_markov_sample(B, G1, V, r, dt, base, FAKE, FAKE, w1, FAKE, FAKE, FAKE, out,
                                   FAKE, None, None, w, wb, None)

    assert mk(B=0) == INVALID
    assert mk(G1=64) == INVALID
    assert mk(r=96) == INVALID
    assert mk(dt=4) == INVALID
    assert mk(base=None) == INVALID
    assert mk(out=FAKE) == INVALID                        # aliasing the base logits
    assert mk(w1=ctypes.c_void_p(0x100008)) == INVALID    # not 16-byte aligned
    assert mk(w=None) == WS_SMALL
    assert mk(wb=ws - 1) == WS_SMALL
