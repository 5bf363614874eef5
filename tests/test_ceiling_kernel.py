"""The benchmark's streaming-ceiling kernel (libboundary_ceiling.so).

It is a context figure, not part of the boundary path; these tests only make sure it streams
what it claims (every output element is the XOR of the nine inputs, nothing outside the rows'
streamed elements is written) and that bad launch shapes are refused before any launch.
"""
import ctypes

import pytest
import torch

from reduce_residual_rmsnorm_bnd_amd import _build

VP = ctypes.c_void_p


def _lib():
    L = ctypes.CDLL(_build.CEILING_LIB_PATH)
    L.bnd_ceiling_mix_9r2w.argtypes = [ctypes.POINTER(VP), VP, VP, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int, ctypes.c_int, VP]
    L.bnd_ceiling_mix_9r2w.restype = ctypes.c_int
    L.bnd_ceiling_mix.argtypes = [ctypes.POINTER(VP), ctypes.c_int, VP, VP, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_int, ctypes.c_int, VP]
    L.bnd_ceiling_mix.restype = ctypes.c_int
    L.bnd_ceiling_mix_byte_out1.argtypes = L.bnd_ceiling_mix.argtypes
    L.bnd_ceiling_mix_byte_out1.restype = ctypes.c_int
    for fn in (L.bnd_ceiling_empty, L.bnd_ceiling_empty_args):
        fn.argtypes = [ctypes.c_int64, ctypes.c_int, VP]
        fn.restype = ctypes.c_int
    L.bnd_ceiling_gather_9r2w.argtypes = [VP, ctypes.c_int64, VP, VP, VP, VP, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int, ctypes.c_int, VP]
    L.bnd_ceiling_gather_9r2w.restype = ctypes.c_int
    return L


def test_ceiling_refuses_bad_shapes():
    # fake, never dereferenced addresses: every call below fails validation before a launch
    L = _lib()
    a = 0x7F0000000000
    src = (VP * 9)(*[a + (i << 24) for i in range(9)])
    o0, o1 = VP(a + (20 << 24)), VP(a + (21 << 24))
    bad = [
        (src, o0, o1, 0, 4096, 4096, 256, 2),        # no rows
        (src, o0, o1, 4, 4096, 4096, 32, 2),         # threads below a wavefront
        (src, o0, o1, 4, 4096, 4096, 96 + 1, 2),     # threads not a multiple of 64
        (src, o0, o1, 4, 4096, 4096, 2048, 1),       # threads above 1024
        (src, o0, o1, 4, 4096, 4096, 256, 3),        # vectors per thread not 1, 2, 4 or 8
        (src, o0, o1, 4, 4096, 4096, 64, 16),
        (src, o0, o1, 4, 4096, 4096, 128, 2),        # 128 x 2 x 8 < 4096: cannot cover the row
        (src, o0, o1, 4, 4096, 4100, 512, 1),        # row elements not a multiple of 8
        (src, o0, o1, 4, 4092, 4096, 512, 1),        # ld shorter than the row
        (src, o0, o1, 4, 4100, 4096, 512, 1),        # ld not a multiple of 8
        (src, VP(a + 8), o1, 4, 4096, 4096, 512, 1),  # misaligned output
        (src, None, o1, 4, 4096, 4096, 512, 1),      # null output
        (None, o0, o1, 4, 4096, 4096, 512, 1),       # null source table
    ]
    for args in bad:
        assert L.bnd_ceiling_mix_9r2w(*args, None) == -1, args
    src[4] = a + 2  # a misaligned source
    assert L.bnd_ceiling_mix_9r2w(src, o0, o1, 4, 4096, 4096, 512, 1, None) == -1
    src16 = (VP * 16)(*[a + (i << 24) for i in range(16)])
    for n in (0, 17):  # source counts outside 1..16
        assert L.bnd_ceiling_mix(src16, n, o0, None, 4, 4096, 4096, 512, 1, None) == -1, n
    assert L.bnd_ceiling_mix_9r2w(src, o0, None, 4, 4096, 4096, 512, 1, None) == -1  # 9:2 needs two outputs
    # a byte-wide second output is required and 8-byte aligned
    assert L.bnd_ceiling_mix_byte_out1(src16, 9, o0, None, 4, 4096, 4096, 512, 1, None) == -1
    assert L.bnd_ceiling_mix_byte_out1(src16, 9, o0, VP(a + (21 << 24) + 4), 4, 4096, 4096, 512, 1, None) == -1
    for wg, threads in ((0, 64), (1, 32), (1, 100), (1, 2048), (1 << 31, 64), (1 << 26, 128)):
        assert L.bnd_ceiling_empty(wg, threads, None) == -1, (wg, threads)
        assert L.bnd_ceiling_empty_args(wg, threads, None) == -1, (wg, threads)
    E, idx, s8 = VP(a), VP(a + (30 << 24)), VP(a + (31 << 24))
    bad_gather = [
        (None, 64, idx, s8, o0, o1, 4, 4096, 4096, 64, 8),    # no source rows
        (E, 0, idx, s8, o0, o1, 4, 4096, 4096, 64, 8),        # empty source rows
        (E, 64, None, s8, o0, o1, 4, 4096, 4096, 64, 8),      # no index
        (E, 64, VP(a + 2), s8, o0, o1, 4, 4096, 4096, 64, 8),  # misaligned index
        (E, 64, idx, VP(a + 8), o0, o1, 4, 4096, 4096, 64, 8),  # misaligned ninth source
        (E, 64, idx, s8, o0, o1, 0, 4096, 4096, 64, 8),       # no rows
        (E, 64, idx, s8, o0, o1, 4, 4096, 4096, 64, 4),       # 64 x 4 x 8 < 4096
    ]
    for args in bad_gather:
        assert L.bnd_ceiling_gather_9r2w(*args, None) == -1, args


@pytest.mark.gpu
def test_empty_kernel_launches():
    L = _lib()
    assert L.bnd_ceiling_empty(1, 512, torch.cuda.current_stream().cuda_stream) == 0
    assert L.bnd_ceiling_empty(300, 64, torch.cuda.current_stream().cuda_stream) == 0
    assert L.bnd_ceiling_empty_args(1, 512, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()


@pytest.mark.gpu
@pytest.mark.parametrize("rows,H,ld,threads,vpt", [(37, 4096, 4096, 256, 2), (5, 1000, 1016, 64, 2),
                                                   (3, 8, 8, 64, 1), (9, 4096, 4104, 128, 4),
                                                   (11, 3600, 3600, 64, 8)])
def test_ceiling_streams_the_xor(rows, H, ld, threads, vpt):
    L = _lib()
    g = torch.Generator().manual_seed(rows * 7 + vpt)
    host = [torch.randint(-32768, 32768, (rows, ld), dtype=torch.int16, generator=g) for _ in range(9)]
    srcs = [h.to("cuda:0") for h in host]
    out = [torch.full((rows, ld), 7, dtype=torch.int16, device="cuda:0") for _ in range(2)]
    print(f"\n  ceiling rows={rows} H={H} ld={ld} {threads}x{vpt}", flush=True)
    rc = L.bnd_ceiling_mix_9r2w((VP * 9)(*[s.data_ptr() for s in srcs]), out[0].data_ptr(),
                                out[1].data_ptr(), rows, ld, H, threads, vpt,
                                torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    expect = host[0].clone()
    for h in host[1:]:
        expect ^= h
    for o in out:
        o = o.cpu()
        assert torch.equal(o[:, :H], expect[:, :H])
        assert bool((o[:, H:] == 7).all())


@pytest.mark.gpu
@pytest.mark.parametrize("rows,H,threads,vpt", [(37, 4096, 64, 8), (5, 1000, 128, 1), (9, 4096, 256, 2)])
def test_gather_streams_the_xor(rows, H, threads, vpt):
    L = _lib()
    g = torch.Generator().manual_seed(rows + vpt)
    n_src = 3 * rows
    E = torch.randint(-32768, 32768, (n_src, H), dtype=torch.int16, generator=g)
    s8 = torch.randint(-32768, 32768, (rows, H), dtype=torch.int16, generator=g)
    idx = torch.randint(0, n_src, (rows * 8,), dtype=torch.int32, generator=g)
    idx[3] = -1          # outside the rows: reads zeros
    idx[11] = n_src
    dE, ds8, didx = E.to("cuda:0"), s8.to("cuda:0"), idx.to("cuda:0")
    out = [torch.full((rows, H), 7, dtype=torch.int16, device="cuda:0") for _ in range(2)]
    print(f"\n  gather ceiling rows={rows} H={H} {threads}x{vpt}", flush=True)
    rc = L.bnd_ceiling_gather_9r2w(dE.data_ptr(), n_src, didx.data_ptr(), ds8.data_ptr(), out[0].data_ptr(),
                                   out[1].data_ptr(), rows, H, H, threads, vpt,
                                   torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    expect = s8.clone()
    for t in range(rows):
        for j in range(8):
            e = int(idx[t * 8 + j])
            if 0 <= e < n_src:
                expect[t] ^= E[e]
    for o in out:
        assert torch.equal(o.cpu(), expect)


@pytest.mark.gpu
@pytest.mark.parametrize("n_src,two_outputs", [(8, False), (9, False), (1, True), (16, False)])
def test_mix_streams_the_xor(n_src, two_outputs):
    L = _lib()
    rows, H, threads, vpt = 13, 4096, 64, 8
    g = torch.Generator().manual_seed(n_src)
    host = [torch.randint(-32768, 32768, (rows, H), dtype=torch.int16, generator=g) for _ in range(n_src)]
    srcs = [h.to("cuda:0") for h in host]
    out = [torch.full((rows, H), 7, dtype=torch.int16, device="cuda:0") for _ in range(2)]
    print(f"\n  mix {n_src}:{2 if two_outputs else 1} rows={rows} H={H}", flush=True)
    rc = L.bnd_ceiling_mix((VP * n_src)(*[s.data_ptr() for s in srcs]), n_src, out[0].data_ptr(),
                           out[1].data_ptr() if two_outputs else None, rows, H, H, threads, vpt,
                           torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    expect = host[0].clone()
    for h in host[1:]:
        expect ^= h
    assert torch.equal(out[0].cpu(), expect)
    if two_outputs:
        assert torch.equal(out[1].cpu(), expect)
    else:
        assert bool((out[1] == 7).all()), "one output: the second buffer is untouched"


@pytest.mark.gpu
@pytest.mark.parametrize("threads,vpt,H", [(64, 8, 4096), (128, 8, 7168), (1024, 1, 7168), (256, 4, 3600)])
def test_mix_byte_second_output(threads, vpt, H):
    """The second output one byte per element: each 16-byte vector's first 8 bytes at half its
    offset; the bf16 output and everything past the row untouched otherwise."""
    L = _lib()
    rows, n_src = 11, 9
    g = torch.Generator().manual_seed(threads + H)
    host = [torch.randint(-32768, 32768, (rows, H), dtype=torch.int16, generator=g) for _ in range(n_src)]
    srcs = [h.to("cuda:0") for h in host]
    out0 = torch.full((rows, H), 7, dtype=torch.int16, device="cuda:0")
    out1 = torch.full((rows, H + 64), 9, dtype=torch.uint8, device="cuda:0")  # ld = H elements; tail canary
    print(f"\n  mix {n_src}:1.5 rows={rows} H={H} {threads}x{vpt}", flush=True)
    rc = L.bnd_ceiling_mix_byte_out1((VP * n_src)(*[s.data_ptr() for s in srcs]), n_src, out0.data_ptr(),
                                     out1.data_ptr(), rows, H, H, threads, vpt, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    expect = host[0].clone()
    for h in host[1:]:
        expect ^= h
    assert torch.equal(out0.cpu(), expect)
    b = out1.cpu()
    first8 = expect.view(torch.uint8).reshape(rows, H // 8, 16)[:, :, :8].reshape(rows, H)
    flat = b.reshape(-1)
    got = torch.stack([flat[r * H:(r + 1) * H] for r in range(rows)])  # rows at ld = H bytes
    assert torch.equal(got, first8)
    assert bool((flat[rows * H:] == 9).all()), "nothing past the last row"
