"""The Python binding checks every tensor it hands to the C ABI before any
launch: the library sees only pointers, so a short, wrong-dtype, strided or
host-resident output, gradient or workspace buffer would otherwise become an
out-of-bounds device write.  These run on the CPU: device residency is
stubbed to true for CPU tensors and the library is replaced by a stub that
fails the test if any entry point (other than a pure size query) is called."""

import numpy as np
import pytest
import torch

import exact_attention_17_amd as fa
from exact_attention_17_amd import build

bf16, f32, i32 = torch.bfloat16, torch.float32, torch.int32
class FakeStream:
    cuda_stream = 0          # a null HIP stream handle; only the stub library receives it


STREAM = FakeStream()


class NoLaunchLib:
    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name.endswith("_workspace_size"):
            return getattr(self._real, name)

        def launched(*a):
            raise AssertionError(f"{name} reached the C ABI despite an invalid argument")
        return launched


@pytest.fixture
def stub(monkeypatch):
    if not __import__("os").path.exists(build.LIB_PATH):
        build.build_library()
    real = fa.load_library()
    monkeypatch.setattr(fa, "_is_device", lambda t: True)
    monkeypatch.setattr(fa, "load_library", lambda path=None: NoLaunchLib(real))


def z(*shape, dtype=bf16):
    return torch.zeros(shape, dtype=dtype)


def dense(B=2, Lq=5, Lk=7, Hq=4, Hkv=2, d=64):
    return z(B, Lq, Hq, d), z(B, Lk, Hkv, d), z(B, Lk, Hkv, d)


@pytest.mark.parametrize("bad", [
    dict(out=z(2, 5, 4, 63)),                       # short
    dict(out=z(2, 5, 4, 64, dtype=f32)),            # wrong dtype
    dict(out=z(2, 5, 4, 128)[..., :64]),            # not contiguous
    dict(out=z(2, 5, 4, 64), lse=z(2, 4, 4, dtype=f32)),
    dict(out=z(2, 5, 4, 64), lse=z(2, 4, 5)),       # bf16 lse
    dict(out=z(2, 5, 4, 64), lse=z(4, 2, 5, dtype=f32)),
])
def test_fwd_rejects_bad_outputs(stub, bad):
    q, k, v = dense()
    kw = dict(out=None, lse=None)
    kw.update(bad)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, v, stream=STREAM, **kw)


def test_fwd_rejects_host_output_and_mixed_devices(monkeypatch, stub):
    q, k, v = dense()
    out = z(2, 5, 4, 64)
    monkeypatch.setattr(fa, "_is_device", lambda t: t is not out)
    with pytest.raises(ValueError, match="device tensor"):
        fa.fa_fwd(q, k, v, out=out, lse=z(2, 4, 5, dtype=f32), stream=STREAM)
    monkeypatch.setattr(fa, "_is_device", lambda t: True)
    with pytest.raises(ValueError, match="expected"):
        fa.fa_fwd(q, k, v.to("meta"), out=out, lse=z(2, 4, 5, dtype=f32), stream=STREAM)


@pytest.mark.parametrize("which", ["out", "lse", "k", "v"])
def test_varlen_rejects_bad_buffers(stub, which):
    T, Tk, Hq, Hkv, d = 9, 11, 4, 2, 128
    a = dict(q=z(T, Hq, d), k=z(Tk, Hkv, d), v=z(Tk, Hkv, d), out=z(T, Hq, d),
             lse=z(Hq, T, dtype=f32))
    a[which] = {"out": z(T - 1, Hq, d), "lse": z(T, Hq, dtype=f32), "k": z(Tk, Hkv, 64),
                "v": z(Tk - 1, Hkv, d)}[which]
    cu = torch.tensor([0, 4, 9], dtype=i32)
    cuk = torch.tensor([0, 5, 11], dtype=i32)
    with pytest.raises(ValueError):
        fa.fa_fwd_varlen(a["q"], a["k"], a["v"], cu, cuk, 5, 6, out=a["out"], lse=a["lse"],
                         stream=STREAM)
    plan = torch.zeros((3, 2), dtype=i32)
    with pytest.raises(ValueError):
        fa.fa_fwd_varlen_run(a["q"], a["k"], a["v"], cu, cuk, plan, 5, 6, out=a["out"],
                             lse=a["lse"], stream=STREAM)


def paged(B=3, Hq=8, Hkv=2, d=128, pages=20, ps=16, mb=6):
    return (z(B, 1, Hq, d), z(pages, ps, Hkv, d), z(pages, ps, Hkv, d),
            torch.zeros((B, mb), dtype=i32), torch.zeros(B, dtype=i32))


@pytest.mark.parametrize("bad", ["out", "lse", "ws_short", "ws_strided", "seqlens", "v_cache"])
def test_decode_rejects_bad_buffers(stub, bad):
    q, kc, vc, bt, sl = paged()
    need = fa.fa_decode_paged_workspace_size(3, 8, 128, 6, 16, 0)
    out, lse = z(3, 1, 8, 128), z(3, 8, dtype=f32)
    ws = torch.zeros(need, dtype=torch.uint8)
    if bad == "out":
        out = z(3, 8, 128)
    elif bad == "lse":
        lse = z(3, 8, 1, dtype=f32)
    elif bad == "ws_short":
        ws = torch.zeros(need - 1, dtype=torch.uint8)
    elif bad == "ws_strided":
        ws = torch.zeros(2 * need, dtype=torch.uint8)[::2]
    elif bad == "seqlens":
        sl = torch.zeros(2, dtype=i32)
    else:
        vc = z(20, 16, 2, 64)
    with pytest.raises(ValueError):
        fa.fa_decode_paged(q, kc, vc, bt, sl, out=out, lse=lse, workspace=ws, stream=STREAM)
    with pytest.raises(ValueError):
        fa.fa_decode_paged_run(q, kc, vc, bt, sl, torch.zeros((1, 2), dtype=i32), out=out,
                               lse=lse, workspace=ws, stream=STREAM)


@pytest.mark.parametrize("bad", ["out", "lse", "knew"])
def test_kvcache_rejects_bad_buffers(stub, bad):
    q = z(3, 4, 8, 128)
    _, kc, vc, bt, sl = paged()
    out, lse, kn = z(3, 4, 8, 128), z(3, 8, 4, dtype=f32), z(3, 4, 2, 128)
    if bad == "out":
        out = z(3, 4, 8, 64)
    elif bad == "lse":
        lse = z(3, 4, 8, dtype=f32)
    else:
        kn = z(3, 5, 2, 128)
    with pytest.raises(ValueError):
        fa.fa_fwd_kvcache(q, kc, vc, bt, sl, kn, kn.clone(), out=out, lse=lse, stream=STREAM)


@pytest.mark.parametrize("which", ["dq", "dk", "dv", "ws", "lse", "dout"])
def test_bwd_rejects_bad_buffers(stub, which):
    q, k, v = dense()
    a = dict(dq=z(2, 5, 4, 64), dk=z(2, 7, 2, 64), dv=z(2, 7, 2, 64),
             ws=torch.zeros(fa.fa_bwd_workspace_size(2, 4, 5), dtype=torch.uint8),
             lse=z(2, 4, 5, dtype=f32), dout=z(2, 5, 4, 64))
    a[which] = {"dq": z(2, 5, 4, 64, dtype=f32), "dk": z(2, 7, 4, 64), "dv": z(2, 6, 2, 64),
                "ws": torch.zeros(16, dtype=torch.uint8), "lse": z(2, 5, 4, dtype=f32),
                "dout": z(2, 5, 4, 32)}[which]
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, z(2, 5, 4, 64), a["lse"], a["dout"], dq=a["dq"], dk=a["dk"],
                  dv=a["dv"], workspace=a["ws"], stream=STREAM)


@pytest.mark.parametrize("which", ["dq", "dk", "ws"])
def test_bwd_varlen_rejects_bad_buffers(stub, which):
    T, Tk, Hq, Hkv, d = 9, 11, 4, 2, 64
    q, k, v = z(T, Hq, d), z(Tk, Hkv, d), z(Tk, Hkv, d)
    cu = torch.tensor([0, 4, 9], dtype=i32)
    cuk = torch.tensor([0, 5, 11], dtype=i32)
    a = dict(dq=z(T, Hq, d), dk=z(Tk, Hkv, d),
             ws=torch.zeros(fa.fa_bwd_varlen_workspace_size(2, Hq, T), dtype=torch.uint8))
    a[which] = {"dq": z(T, Hq, d + 1), "dk": z(Tk, Hq, d), "ws": torch.zeros(8, dtype=torch.uint8)}[which]
    with pytest.raises(ValueError):
        fa.fa_bwd_varlen(q, k, v, z(T, Hq, d), z(Hq, T, dtype=f32), z(T, Hq, d), cu, cuk, 5, 6,
                         dq=a["dq"], dk=a["dk"], dv=z(Tk, Hkv, d), workspace=a["ws"],
                         stream=STREAM)


def test_valid_arguments_reach_the_library(stub):
    """The same checks accept correct buffers (the stub then sees the launch)."""
    q, k, v = dense()
    with pytest.raises(AssertionError, match="reached the C ABI"):
        fa.fa_fwd(q, k, v, out=z(2, 5, 4, 64), lse=z(2, 4, 5, dtype=f32), stream=STREAM)
