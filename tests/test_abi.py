"""Host-only checks of the C-ABI library: it loads, exports every function
that include/kdkl.h declares, sizes workspaces, and rejects bad arguments with
the documented status before any HIP call (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

from chunked_kl_loss_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULL, SHAPE, VALUE, DTYPE, WORKSPACE, OVERFLOW, HIP, ALIGN, OPTION = range(10)
FAKE = 0x10000  # 16-byte aligned, never dereferenced on the host


@pytest.fixture(scope="module")
def lib():
    return L.load()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "kdkl.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kdkl_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("kdkl_forward", "kdkl_backward", "kdkl_workspace_size", "kdkl_status_string",
              "kdkl_abi_version", "kdkl_profile_begin", "kdkl_profile_end"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"libkdkl.so does not export {n}"
    assert set(declared_functions()) <= set(L.SIGNATURES)


def test_version_and_status_strings(lib):
    assert lib.kdkl_abi_version() == 2
    for s in list(range(10)) + [99, -1]:
        v = lib.kdkl_status_string(s)
        assert v is not None and len(v) > 0
    assert lib.kdkl_status_string(WORKSPACE).startswith(b"KDKL_ERR_WORKSPACE")


def opts(**kw):
    o = L.Options()
    for k, v in kw.items():
        if k == "reserved":
            o.reserved[0] = v
        else:
            setattr(o, k, v)
    return C.byref(o)


def ws(lib, N, d, V, K, chunk, dt, o=None):
    f, b = C.c_size_t(), C.c_size_t()
    st = lib.kdkl_workspace_size(N, d, V, K, chunk, dt, o, C.byref(f), C.byref(b))
    return st, f.value, b.value


def test_workspace_size_arithmetic(lib):
    # gpt-oss-like head at 32K: the bf16 backward workspace holds the
    # token-major dZ of one group of chunks over one vocabulary slice (about
    # as many elements as one chunk over the whole vocabulary), the group's
    # H^T, the dH split partials, the group's fp32 dH sum and (unless the
    # build reads W in place) W^T; nothing scales with N except the
    # forward's per-row KL scratch.
    st, f, b = ws(lib, 32768, 2880, 201088, 100, 2048, L.KDKL_BF16)
    assert st == OK
    Vp = (201088 + 255) // 256 * 256
    p = plan(lib, 32768, 2880, 201088, 100, 2048, L.KDKL_BF16)
    rows = p.chunks_per_group * 2048
    vpart = -(-201088 // p.vocab_slices) // 768 * 768 + (768 if -(-201088 // p.vocab_slices) % 768 else 0)
    assert b >= rows * vpart * 2 and rows * vpart * 2 <= 4 * 2**30  # the dZ buffer, within its budget
    assert b < 4 * 2**30 + 2880 * Vp * 2 + 2**30
    # d not a multiple of 64: the generic path also keeps W^T, H_c^T and a
    # vocabulary-major copy of dZ
    _, _, bg = ws(lib, 32768, 2888, 201088, 100, 2048, L.KDKL_BF16)
    assert bg >= 2 * 2048 * Vp * 2 + 2888 * Vp * 2
    assert f < 512 * 2**20  # per-group teacher products and split partials (32768 rows)
    # memory is independent of N apart from O(N) scratch
    _, f2, b2 = ws(lib, 262144, 2880, 201088, 100, 2048, L.KDKL_BF16)
    assert b2 == b and f2 - f == (262144 - 32768) * 4
    # fp32 storage doubles the element-sized regions (against bf16 at the
    # fp32 path's blocking: one chunk at a time, the whole vocabulary)
    _, _, b32 = ws(lib, 32768, 2880, 201088, 100, 2048, L.KDKL_F32)
    _, _, b1 = ws(lib, 32768, 2880, 201088, 100, 2048, L.KDKL_BF16, opts(chunks_per_group=1, vocab_slices=1))
    assert b32 > b1
    # outputs may be NULL
    assert lib.kdkl_workspace_size(10, 8, 16, 2, 4, L.KDKL_BF16, None, None, None) == OK


@pytest.mark.parametrize("args,status", [
    ((-1, 64, 100, 4, 8, 1), SHAPE),      # N < 0
    ((8, 0, 100, 4, 8, 1), SHAPE),        # d = 0
    ((8, 12, 100, 4, 8, 1), SHAPE),       # bf16 d not a multiple of 8
    ((8, 6, 100, 4, 8, 0), SHAPE),        # fp32 d not a multiple of 4
    ((8, 64, 100, 0, 8, 1), SHAPE),       # K = 0
    ((8, 64, 3, 4, 8, 1), SHAPE),         # K > V
    ((8, 64, 4096, 1025, 8, 1), SHAPE),   # K > 1024
    ((8, 64, 100, 4, 0, 1), SHAPE),       # chunk = 0
    ((8, 64, 100, 4, 8, 2), DTYPE),       # unknown dtype
    ((8, 64, 0, 1, 8, 1), SHAPE),         # V = 0
    ((2**40, 64, 100, 4, 8, 1), OVERFLOW),
])
def test_workspace_size_rejects(lib, args, status):
    st, _, _ = ws(lib, *args)
    assert st == status


def fwd(lib, **kw):
    a = dict(H=FAKE, W=FAKE, ids=FAKE, lg=FAKE, N=64, d=64, V=1000, K=8, T=1.0, chunk=16,
             dt=L.KDKL_BF16, o=None, loss=FAKE, lse=FAKE, kl=None, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.kdkl_forward(a["H"], a["W"], a["ids"], a["lg"], a["N"], a["d"], a["V"], a["K"],
                            a["T"], a["chunk"], a["dt"], a["o"], a["loss"], a["lse"], a["kl"], a["ws"],
                            a["wsb"], a["stream"])


def bwd(lib, **kw):
    a = dict(H=FAKE, W=FAKE, ids=FAKE, lg=FAKE, N=64, d=64, V=1000, K=8, T=1.0, chunk=16,
             dt=L.KDKL_BF16, o=None, lse=FAKE, g=None, dH=FAKE, dW=FAKE, acc=0, ws=FAKE, wsb=1 << 40,
             stream=None)
    a.update(kw)
    return lib.kdkl_backward(a["H"], a["W"], a["ids"], a["lg"], a["N"], a["d"], a["V"], a["K"],
                             a["T"], a["chunk"], a["dt"], a["o"], a["lse"], a["g"], a["dH"], a["dW"],
                             a["acc"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("call", [fwd, bwd], ids=["forward", "backward"])
@pytest.mark.parametrize("kw,status", [
    (dict(W=None), NULL),
    (dict(H=None), NULL),
    (dict(ids=None), NULL),
    (dict(lg=None), NULL),
    (dict(ws=None), NULL),
    (dict(T=0.0), VALUE),
    (dict(T=-1.0), VALUE),
    (dict(T=float("inf")), VALUE),
    (dict(T=float("nan")), VALUE),
    (dict(d=60), SHAPE),
    (dict(K=0), SHAPE),
    (dict(K=2000), SHAPE),
    (dict(chunk=0), SHAPE),
    (dict(dt=7), DTYPE),
    (dict(wsb=16), WORKSPACE),
    (dict(H=FAKE + 8), ALIGN),
    (dict(W=FAKE + 2), ALIGN),
    (dict(ws=FAKE + 4), ALIGN),
    (dict(o=opts(loss=7)), OPTION),
    (dict(o=opts(chunks_per_group=-1)), OPTION),
    (dict(o=opts(vocab_slices=1025)), OPTION),
    (dict(o=opts(dh_w_in_place=3)), OPTION),
    (dict(o=opts(reserved=1)), OPTION),
    (dict(o=opts(dh_w_in_place=1), dt=L.KDKL_F32), OPTION),      # in place needs the bf16 main loop
    (dict(o=opts(chunks_per_group=2), dt=L.KDKL_F32), OPTION),   # so do groups of chunks
    (dict(o=opts(chunks_per_group=2), d=72), OPTION),
])
def test_compute_calls_reject_bad_arguments(lib, call, kw, status):
    assert call(lib, **kw) == status


def test_forward_output_pointers_checked(lib):
    assert fwd(lib, loss=None) == NULL
    assert fwd(lib, lse=None) == NULL


def test_backward_output_pointers_checked(lib):
    assert bwd(lib, dW=None) == NULL
    assert bwd(lib, dH=None) == NULL
    assert bwd(lib, lse=None) == NULL
    assert bwd(lib, dW=FAKE + 4) == ALIGN


def test_profile_calls_without_launches(lib):
    assert lib.kdkl_profile_begin() == OK
    n = C.c_int(-1)
    assert lib.kdkl_profile_end(None, 0, C.byref(n)) == OK
    assert n.value == 0


def test_binding_refuses_cpu_tensors():
    import torch

    import chunked_kl_loss_amd as kd

    H = torch.zeros(4, 8, dtype=torch.bfloat16)
    W = torch.zeros(16, 8, dtype=torch.bfloat16)
    ids = torch.zeros(4, 2, dtype=torch.int32)
    lg = torch.zeros(4, 2)
    with pytest.raises(ValueError):
        kd.kdkl_forward(H, W, ids, lg, 1.0, 2)


# --- forward-chunked KL entry points ------------------------------------------

def lfwd(lib, **kw):
    a = dict(Z=FAKE, ids=FAKE, lg=FAKE, N=64, V=1000, K=8, T=1.0, dt=L.KDKL_BF16, loss=FAKE,
             lse=FAKE, kl=FAKE, stream=None)
    a.update(kw)
    return lib.kdkl_logits_forward(a["Z"], a["ids"], a["lg"], a["N"], a["V"], a["K"], a["T"],
                                   a["dt"], a["loss"], a["lse"], a["kl"], a["stream"])


def lbwd(lib, **kw):
    a = dict(Z=FAKE, ids=FAKE, lg=FAKE, N=64, V=1000, K=8, T=1.0, dt=L.KDKL_BF16, lse=FAKE, g=None,
             dZ=FAKE, ws=FAKE, wsb=256, stream=None)
    a.update(kw)
    return lib.kdkl_logits_backward(a["Z"], a["ids"], a["lg"], a["N"], a["V"], a["K"], a["T"],
                                    a["dt"], a["lse"], a["g"], a["dZ"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("call", [lfwd, lbwd], ids=["logits_forward", "logits_backward"])
@pytest.mark.parametrize("kw,status", [
    (dict(Z=None), NULL),
    (dict(ids=None), NULL),
    (dict(lg=None), NULL),
    (dict(lse=None), NULL),
    (dict(T=0.0), VALUE),
    (dict(T=float("nan")), VALUE),
    (dict(K=0), SHAPE),
    (dict(K=1025), SHAPE),
    (dict(K=1001), SHAPE),  # K > V
    (dict(V=0), SHAPE),
    (dict(N=-1), SHAPE),
    (dict(N=1 << 41), OVERFLOW),
    (dict(N=1 << 40, V=1 << 40), OVERFLOW),  # each size in range, the grid not
    (dict(N=1 << 31, V=1 << 30), OVERFLOW),
    (dict(dt=3), DTYPE),
    (dict(Z=FAKE + 2), ALIGN),
])
def test_logits_calls_reject_bad_arguments(lib, call, kw, status):
    assert call(lib, **kw) == status


def test_logits_output_pointers_checked(lib):
    assert lfwd(lib, loss=None) == NULL
    assert lfwd(lib, kl=None) == NULL
    assert lbwd(lib, dZ=None) == NULL
    assert lbwd(lib, dZ=FAKE + 8) == ALIGN
    assert lbwd(lib, ws=None) == NULL
    assert lbwd(lib, ws=FAKE + 4) == ALIGN
    assert lbwd(lib, wsb=255) == WORKSPACE
    # nothing to do for N == 0 on the backward: returns before any HIP call
    assert lbwd(lib, N=0, Z=None, ids=None, lg=None, lse=None, dZ=None, ws=None, wsb=0) == OK


def test_logits_binding_refuses_cpu_tensors():
    import torch

    import chunked_kl_loss_amd as kd

    Z = torch.zeros(4, 16, dtype=torch.bfloat16)
    ids = torch.zeros(4, 2, dtype=torch.int32)
    lg = torch.zeros(4, 2)
    with pytest.raises(ValueError):
        kd.logits_forward(Z, ids, lg, 1.0)


# --- dense baseline entry points ------------------------------------------------

def test_dense_sizes(lib):
    f, sv, b = C.c_size_t(), C.c_size_t(), C.c_size_t()
    N, d, V, K = 32768, 2880, 201088, 100
    assert lib.kdkl_dense_sizes(N, d, V, K, L.KDKL_BF16, C.byref(f), C.byref(sv), C.byref(b)) == OK
    Vp = (V + 255) // 256 * 256
    assert sv.value >= 2 * N * Vp * 4 and sv.value < 2 * N * Vp * 4 + 4096  # both grids, fp32
    assert f.value >= N * Vp * 2                                            # the logit grid
    assert b.value >= N * Vp * 2                                            # the dZ grid
    assert lib.kdkl_dense_sizes(N, d, V, 0, L.KDKL_BF16, None, None, None) == SHAPE


def dfwd(lib, **kw):
    a = dict(H=FAKE, W=FAKE, ids=FAKE, lg=FAKE, N=64, d=64, V=1000, K=8, T=1.0, dt=L.KDKL_BF16,
             loss=FAKE, lse=FAKE, kl=None, sv=FAKE, svb=1 << 40, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.kdkl_dense_forward(a["H"], a["W"], a["ids"], a["lg"], a["N"], a["d"], a["V"], a["K"],
                                  a["T"], a["dt"], a["loss"], a["lse"], a["kl"], a["sv"], a["svb"],
                                  a["ws"], a["wsb"], a["stream"])


def dbwd(lib, **kw):
    a = dict(H=FAKE, W=FAKE, ids=FAKE, lg=FAKE, N=64, d=64, V=1000, K=8, T=1.0, dt=L.KDKL_BF16,
             sv=FAKE, svb=1 << 40, g=None, dH=FAKE, dW=FAKE, acc=0, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.kdkl_dense_backward(a["H"], a["W"], a["ids"], a["lg"], a["N"], a["d"], a["V"], a["K"],
                                   a["T"], a["dt"], a["sv"], a["svb"], a["g"], a["dH"], a["dW"], a["acc"],
                                   a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("call", [dfwd, dbwd], ids=["dense_forward", "dense_backward"])
@pytest.mark.parametrize("kw,status", [
    (dict(W=None), NULL),
    (dict(ids=None), NULL),
    (dict(sv=None), NULL),
    (dict(ws=None), NULL),
    (dict(T=0.0), VALUE),
    (dict(d=60), SHAPE),
    (dict(K=0), SHAPE),
    (dict(dt=5), DTYPE),
    (dict(svb=16), WORKSPACE),
    (dict(wsb=16), WORKSPACE),
    (dict(sv=FAKE + 4), ALIGN),
    (dict(H=FAKE + 8), ALIGN),
])
def test_dense_calls_reject_bad_arguments(lib, call, kw, status):
    assert call(lib, **kw) == status


# --- teacher-id validation entry point -------------------------------------------

def chk(lib, **kw):
    a = dict(ids=FAKE, N=64, K=8, V=1000, counts=FAKE, ws=FAKE, wsb=16384, stream=None)
    a.update(kw)
    return lib.kdkl_check_ids(a["ids"], a["N"], a["K"], a["V"], a["counts"], a["ws"], a["wsb"],
                              a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(ids=None), NULL),
    (dict(counts=None), NULL),
    (dict(ws=None), NULL),
    (dict(K=0), SHAPE),
    (dict(K=1025), SHAPE),
    (dict(V=0), SHAPE),
    (dict(N=-1), SHAPE),
    (dict(N=1 << 41), OVERFLOW),
    (dict(counts=FAKE + 4), ALIGN),
    (dict(ws=FAKE + 4), ALIGN),
    (dict(wsb=16383), WORKSPACE),
])
def test_check_ids_rejects_bad_arguments(lib, kw, status):
    assert chk(lib, **kw) == status


def test_check_ids_binding_refuses_cpu_tensors():
    import torch

    import chunked_kl_loss_amd as kd

    with pytest.raises(ValueError):
        kd.check_ids(torch.zeros(4, 2, dtype=torch.int32), 16)


def test_binding_output_checks():
    """Caller-provided outputs are written through raw pointers: the binding
    refuses any whose shape, dtype or layout differs from what the call
    writes (host-side check, no device needed)."""
    import torch

    import chunked_kl_loss_amd as kd

    cpu = torch.device("cpu")
    kd._want(torch.zeros(4, 3), (4, 3), torch.float32, cpu, "ok")
    for bad in (torch.zeros(3, 4), torch.zeros(4, 3, dtype=torch.bfloat16), torch.zeros(3, 4).t()):
        with pytest.raises(ValueError):
            kd._want(bad, (4, 3), torch.float32, cpu, "dW")
    assert kd._nbytes(torch.zeros(5, dtype=torch.float32)) == 20


def test_dh_reading_w_in_place_drops_the_transposed_copy(lib):
    # the bf16 backward at gpt-oss 32K keeps W^T [d, Vp]; with dh_w_in_place=1
    # its dH product reads W in place and the workspace shrinks by that copy
    N, d, V, K, chunk = 32768, 2880, 201088, 100, 2048
    _, f0, b0 = ws(lib, N, d, V, K, chunk, L.KDKL_BF16)
    _, f1, b1 = ws(lib, N, d, V, K, chunk, L.KDKL_BF16, opts(dh_w_in_place=1))
    Vp = (V + 383) // 384 * 384
    assert f1 == f0
    assert b0 - b1 >= d * Vp * 2 and b0 - b1 < d * Vp * 2 + 512
    # the generic path (d not a multiple of 64) always keeps W^T and cannot
    # read in place
    _, _, g0 = ws(lib, N, 2888, V, K, chunk, L.KDKL_BF16)
    _, _, g2 = ws(lib, N, 2888, V, K, chunk, L.KDKL_BF16, opts(dh_w_in_place=2))
    assert g2 == g0
    assert ws(lib, N, 2888, V, K, chunk, L.KDKL_BF16, opts(dh_w_in_place=1))[0] == OPTION


def plan(lib, N, d, V, K, chunk, dt, o=None):
    p = L.Plan()
    st = lib.kdkl_plan_info(N, d, V, K, chunk, dt, o, C.byref(p))
    assert st == OK, L_status(lib, st)
    return p


def L_status(lib, st):
    return lib.kdkl_status_string(st).decode()


@pytest.mark.parametrize("sizes,groups,slices", [
    # the GPU parity cases for backward groups: each must exercise its size
    ((150, 64, 131001, 16, 64), 2, 1),
    ((148, 64, 262001, 12, 32), 4, 1),
    ((133, 64, 524001, 20, 16), 8, 1),
    ((261, 64, 524001, 20, 16), 16, 1),
    # the named workloads (N, d, V, K, chunk): the largest group of 16, 8, 4
    # or 2 chunks with a vocabulary slicing whose dZ buffer fits 4 GiB and
    # whose slices fill dW's rounds to 95%, with its fewest slices. gpt-oss
    # at 32K: all 16 chunks, quarters of the vocabulary (32768 x 50688 bf16,
    # 3.3 GB; halves would take 6.6 GB). At 256K (chunks of 4096): 16 chunks
    # would need eighths, whose dW leaves the last of four rounds 48% empty,
    # so 8 chunks over quarters. Llama at 8K and the 2K workload: all chunks,
    # the whole vocabulary.
    ((32768, 2880, 201088, 100, 2048), 16, 4),
    ((262144, 2880, 201088, 100, 4096), 8, 4),
    ((8192, 3072, 128256, 100, 1024), 8, 1),
    ((2048, 1024, 32000, 100, 256), 8, 1),
])
def test_plan_groups(lib, sizes, groups, slices):
    p = plan(lib, *sizes, L.KDKL_BF16)
    assert (p.chunks_per_group, p.vocab_slices) == (groups, slices)
    assert p.dh_splits >= 1 and p.bf16_main_loop == 1


def test_plan_groups_never_exceed_the_chunks(lib):
    # two chunks only: a group never spans more chunks than there are
    p = plan(lib, 128, 64, 524001, 20, 64, L.KDKL_BF16)
    assert p.chunks_per_group <= 2


def test_plan_fp32_takes_one_chunk_at_a_time(lib):
    p = plan(lib, 128, 256, 4096, 16, 32, L.KDKL_F32)
    assert (p.chunks_per_group, p.vocab_slices, p.bf16_main_loop, p.dh_w_in_place) == (1, 1, 0, 0)


def test_plan_dh_splits_fill_the_rounds(lib):
    # gpt-oss at 32K: 32768-row groups by 2880 columns on 256 x 320 tiles is
    # 1152 tiles; two splits fill nine rounds of 256 workgroups exactly. With
    # 8192-row groups (288 tiles) six splits fill 96.4% of seven rounds.
    p = plan(lib, 32768, 2880, 201088, 100, 2048, L.KDKL_BF16)
    assert p.dh_splits == 2 and p.hidden_tile == 320 and p.vocab_tile == 384
    assert plan(lib, 32768, 2880, 201088, 100, 2048, L.KDKL_BF16, opts(chunks_per_group=4)).dh_splits == 6


def test_plan_info_validates_like_the_compute_calls(lib):
    p = L.Plan()
    assert lib.kdkl_plan_info(10, 8, 16, 0, 4, L.KDKL_BF16, None, C.byref(p)) == SHAPE
    assert lib.kdkl_plan_info(10, 8, 16, 2, 4, L.KDKL_BF16, None, None) == NULL
    assert lib.kdkl_plan_info(10, 8, 16, 2, 4, L.KDKL_BF16, None, C.byref(p)) == OK
    assert lib.kdkl_plan_info(10, 8, 16, 2, 4, L.KDKL_BF16, opts(vocab_slices=-2), C.byref(p)) == OPTION
    # the sizes it reports are kdkl_workspace_size's
    q = plan(lib, 32768, 2880, 201088, 100, 2048, L.KDKL_BF16)
    assert (q.fwd_bytes, q.bwd_bytes) == ws(lib, 32768, 2880, 201088, 100, 2048, L.KDKL_BF16)[1:]


def test_options_select_the_blocking(lib):
    sizes = (32768, 2880, 201088, 100, 2048)
    base = plan(lib, *sizes, L.KDKL_BF16)
    # vocabulary slices apart from the chunks per group: the dZ buffer holds
    # group rows x V/slices columns, slices starting on 768-row boundaries
    # (16 slices of the 16-chunk group: 32768 rows x 13056 columns, 856 MB,
    # against 32768 x 50688, 3.3 GB, for the default 4 slices)
    assert (base.chunks_per_group, base.vocab_slices) == (16, 4)
    p16 = plan(lib, *sizes, L.KDKL_BF16, opts(vocab_slices=16))
    assert (p16.chunks_per_group, p16.vocab_slices) == (16, 16)
    assert p16.dh_splits == base.dh_splits
    assert base.bwd_bytes - p16.bwd_bytes == 32768 * (50688 - 13056) * 2
    # a set group size keeps its own fewest slices within the budget
    p4 = plan(lib, *sizes, L.KDKL_BF16, opts(chunks_per_group=4))
    assert (p4.chunks_per_group, p4.vocab_slices) == (4, 1)
    p1 = plan(lib, *sizes, L.KDKL_BF16, opts(chunks_per_group=1))
    assert (p1.chunks_per_group, p1.vocab_slices) == (1, 1)
    # a set slicing too large for the budget at 16 chunks takes a smaller group
    p2s = plan(lib, *sizes, L.KDKL_BF16, opts(vocab_slices=2))
    assert (p2s.chunks_per_group, p2s.vocab_slices) == (8, 2)
    # both set: kept as given, whatever the dZ buffer (16 chunks over halves: 6.6 GB)
    p16_2 = plan(lib, *sizes, L.KDKL_BF16, opts(chunks_per_group=16, vocab_slices=2))
    assert (p16_2.chunks_per_group, p16_2.vocab_slices) == (16, 2)
    p8 = plan(lib, *sizes, L.KDKL_BF16, opts(chunks_per_group=8, vocab_slices=32))
    # 32 slices asked: ceil(V/32) = 6284 rows rounded up to 6912 give 30
    assert (p8.chunks_per_group, p8.vocab_slices) == (8, 30)
    # the forward's workspace follows the group size
    assert base.fwd_bytes > p8.fwd_bytes > p4.fwd_bytes > p1.fwd_bytes
    # explicit W layouts
    assert plan(lib, *sizes, L.KDKL_BF16, opts(dh_w_in_place=1)).dh_w_in_place == 1
    assert plan(lib, *sizes, L.KDKL_BF16, opts(dh_w_in_place=2)).dh_w_in_place == 0
    # zero-filled options are the defaults
    z = plan(lib, *sizes, L.KDKL_BF16, opts())
    assert (z.chunks_per_group, z.vocab_slices, z.dh_splits, z.dh_w_in_place, z.bwd_bytes) == \
        (base.chunks_per_group, base.vocab_slices, base.dh_splits, base.dh_w_in_place, base.bwd_bytes)


@pytest.mark.parametrize("sizes,in_place", [
    ((8192, 3072, 128256, 100, 1024), True),     # Llama-like head, 8K: 1 dH launch per call
    ((16384, 2880, 201088, 100, 2048), True),    # gpt-oss-like head, 16K: one group over halves, 2 launches
    ((16385, 2880, 201088, 100, 2048), False),   # one position more: a second group, 4 launches
    ((32768, 2880, 201088, 100, 2048), False),   # gpt-oss-like head, 32K: one group over quarters, 4 launches
    ((262144, 2880, 201088, 100, 4096), False),  # the same head at 256K: 8 groups over quarters, 32 launches
])
def test_w_copy_chosen_per_shape(lib, sizes, in_place):
    # by default the dH product reads W in place unless the copy saves at
    # least about 0.3 ms per call by the library's model; the options force
    # either. The backward workspace steps up by the copy where the choice
    # flips (gpt-oss-like head with chunks of 2048: between 16384 and 16385).
    assert plan(lib, *sizes, L.KDKL_BF16).dh_w_in_place == int(in_place)
    _, _, b_default = ws(lib, *sizes, L.KDKL_BF16)
    _, _, b_in_place = ws(lib, *sizes, L.KDKL_BF16, opts(dh_w_in_place=1))
    _, _, b_copy = ws(lib, *sizes, L.KDKL_BF16, opts(dh_w_in_place=2))
    d, V = sizes[1], sizes[2]
    assert b_copy - b_in_place >= d * V * 2
    assert b_default == (b_in_place if in_place else b_copy)


def test_library_reads_no_environment(lib):
    # the library is configured by arguments only
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", L.LIB_PATH], capture_output=True, text=True)
    assert out.returncode == 0
    assert "getenv" not in out.stdout


# --- allocation-free forward ------------------------------------------------------

def fna(lib, **kw):
    a = dict(H=FAKE, W=FAKE, ids=FAKE, lg=FAKE, N=64, d=64, V=1000, K=8, T=1.0, chunk=16,
             dt=L.KDKL_BF16, o=None, loss=FAKE, lse=FAKE, kl=FAKE, stream=None)
    a.update(kw)
    return lib.kdkl_forward_noalloc(a["H"], a["W"], a["ids"], a["lg"], a["N"], a["d"], a["V"], a["K"],
                                    a["T"], a["chunk"], a["dt"], a["o"], a["loss"], a["lse"], a["kl"],
                                    a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), NULL),
    (dict(H=None), NULL),
    (dict(kl=None), NULL),       # the per-row KL is the caller's: no scratch grows with N
    (dict(lse=None), NULL),
    (dict(loss=None), NULL),
    (dict(T=0.0), VALUE),
    (dict(d=60), SHAPE),
    (dict(dt=9), DTYPE),
    (dict(H=FAKE + 8), ALIGN),
    (dict(o=opts(vocab_slices=-1)), OPTION),
    # one chunk of 8192 positions over gpt-oss's vocabulary needs 8192 x 524
    # vocabulary tiles x 16 bytes of split partials alone: more than the array
    (dict(N=8192, d=2880, V=201088, K=100, chunk=8192), WORKSPACE),
    # the options fix four chunks of 2048 per launch: 84 MB of scratch
    (dict(N=32768, d=2880, V=201088, K=100, chunk=2048, o=opts(chunks_per_group=4)), WORKSPACE),
])
def test_forward_noalloc_rejects_before_any_hip_call(lib, kw, status):
    assert fna(lib, **kw) == status


def test_forward_noalloc_scratch_is_modest():
    # the static array is 64 MiB per GPU; the library's default forward
    # blocking at the gpt-oss-like 32K and 256K workloads needs more, and the
    # allocation-free entry point halves the chunks per launch to fit
    assert L.NOALLOC_SCRATCH_BYTES == 64 << 20
    lib = L.load()
    for sizes in ((32768, 2880, 201088, 100, 2048), (262144, 2880, 201088, 100, 4096)):
        full = plan(lib, *sizes, L.KDKL_BF16)
        assert full.fwd_bytes > L.NOALLOC_SCRATCH_BYTES
        half = plan(lib, *sizes, L.KDKL_BF16, opts(chunks_per_group=full.chunks_per_group // 2))
        one = plan(lib, *sizes, L.KDKL_BF16, opts(chunks_per_group=1))
        assert one.fwd_bytes - sizes[0] * 4 < L.NOALLOC_SCRATCH_BYTES
        assert half.fwd_bytes < full.fwd_bytes


def test_library_never_allocates_device_memory():
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", L.LIB_PATH], capture_output=True, text=True)
    assert out.returncode == 0
    for sym in ("hipMalloc", "hipFree", "hipMallocAsync", "hipExtMallocWithFlags", "hipHostMalloc"):
        assert sym not in out.stdout, sym


def test_jsd_options(lib):
    sizes = (32768, 2880, 201088, 100, 2048)
    assert ws(lib, *sizes, L.KDKL_BF16, opts(loss=L.KDKL_LOSS_JSD))[0] == OPTION             # beta 0
    assert ws(lib, *sizes, L.KDKL_BF16, opts(loss=L.KDKL_LOSS_JSD, beta=1.0))[0] == OPTION
    assert ws(lib, *sizes, L.KDKL_BF16, opts(loss=L.KDKL_LOSS_JSD, beta=float("nan")))[0] == OPTION
    assert ws(lib, *sizes, L.KDKL_BF16, opts(loss=5, beta=0.5))[0] == OPTION
    assert ws(lib, *sizes, L.KDKL_BF16, opts(loss=-1, beta=0.5))[0] == OPTION
    st, f, b = ws(lib, *sizes, L.KDKL_BF16, opts(loss=L.KDKL_LOSS_JSD, beta=0.5))
    _, f0, b0 = ws(lib, *sizes, L.KDKL_BF16)
    assert st == OK
    # the student logits at the sorted teacher entries [group rows, K] fp32 in
    # the forward's workspace, the per-row coefficient of q in the backward's
    g = plan(lib, *sizes, L.KDKL_BF16).chunks_per_group * 2048
    assert f - f0 == g * 100 * 4
    assert b - b0 == g * 4
    # beta is ignored by the KL
    assert ws(lib, *sizes, L.KDKL_BF16, opts(beta=7.0))[1:] == (f0, b0)
    assert fwd(lib, o=opts(loss=L.KDKL_LOSS_JSD, beta=-0.5)) == OPTION
    assert bwd(lib, o=opts(loss=L.KDKL_LOSS_JSD, beta=1.5)) == OPTION


def test_skew_loss_options(lib):
    """The skew KL takes 0 <= alpha < 1, the skew reverse KL 0 < alpha <= 1
    (kdkl_options.beta); both keep the JSD's extra workspace."""
    sizes = (32768, 2880, 201088, 100, 2048)
    _, fj, bj = ws(lib, *sizes, L.KDKL_BF16, opts(loss=L.KDKL_LOSS_JSD, beta=0.5))
    for loss, good, bad in ((L.KDKL_LOSS_SKL, (0.0, 0.1, 0.999), (1.0, -0.1, float("nan"), 2.0)),
                            (L.KDKL_LOSS_SRKL, (1.0, 0.1, 1e-6), (0.0, -0.1, float("nan"), 1.5))):
        for a in good:
            assert ws(lib, *sizes, L.KDKL_BF16, opts(loss=loss, beta=a)) == (OK, fj, bj), (loss, a)
        for a in bad:
            assert ws(lib, *sizes, L.KDKL_BF16, opts(loss=loss, beta=a))[0] == OPTION, (loss, a)
        assert fwd(lib, o=opts(loss=loss, beta=bad[0])) == OPTION
        assert bwd(lib, o=opts(loss=loss, beta=bad[1])) == OPTION


def test_topk_rkl_options(lib):
    """The reverse KL over the top-K support takes no parameter (beta is
    ignored) and keeps the KL's forward workspace; its backward needs no dZ
    buffer, W^T or dH partials (the entry gradients and a counting sort of
    them by id instead), so for a given group size its workspace does not
    depend on the vocabulary slices, and it is a small part of the KL's."""
    sizes = (32768, 2880, 201088, 100, 2048)
    _, f0, b0 = ws(lib, *sizes, L.KDKL_BF16)
    st, f, b = ws(lib, *sizes, L.KDKL_BF16, opts(loss=L.KDKL_LOSS_TRKL))
    assert (st, f) == (OK, f0) and b < b0 // 16
    for beta in (0.5, -3.0, float("nan")):
        assert ws(lib, *sizes, L.KDKL_BF16, opts(loss=L.KDKL_LOSS_TRKL, beta=beta)) == (OK, f, b), beta
    b8 = {ws(lib, *sizes, L.KDKL_BF16, opts(loss=L.KDKL_LOSS_TRKL, chunks_per_group=8, vocab_slices=v))[2]
          for v in (1, 3, 8)}
    assert len(b8) == 1  # for a given group size
    assert ws(lib, *sizes, L.KDKL_F32, opts(loss=L.KDKL_LOSS_TRKL))[0] == OK
    p = plan(lib, *sizes, L.KDKL_BF16, opts(loss=L.KDKL_LOSS_TRKL, chunks_per_group=4))
    assert p.chunks_per_group == 4


@pytest.mark.parametrize("N,d,V,K,chunk,dt", [
    (N, d, V, 16, chunk, dt)
    for N in (1, 700, 5000, 40000, 300000)
    for d, V in ((64, 1000), (1024, 32000), (2880, 201088), (3072, 128256), (2888, 50000), (4096, 262144))
    for chunk in (32, 1024, 4096)
    for dt in (L.KDKL_BF16, L.KDKL_F32)
    if not (dt == L.KDKL_BF16 and d % 8) and not (dt == L.KDKL_F32 and d % 4)
])
def test_default_blocking_invariants(lib, N, d, V, K, chunk, dt):
    """The library's own blocking over a grid of shapes: groups never span
    more chunks than there are, the dZ buffer (group rows x slice rows x
    element bytes) stays within 4 GiB, the generic path keeps one chunk and
    the whole vocabulary, and the workspace query agrees with the plan."""
    p = plan(lib, N, d, V, K, chunk, dt)
    chunks = max(1, -(-N // chunk))
    c = min(chunk, max(N, 1))
    if not p.bf16_main_loop:
        assert (p.chunks_per_group, p.vocab_slices) == (1, 1)
        return
    assert 1 <= p.chunks_per_group <= max(1, min(16, chunks))
    vt = p.vocab_tile
    align = vt if vt % 256 == 0 else 2 * vt
    s = p.vocab_slices
    vpart = -(-V // vt) * vt if s <= 1 else -(-(-(-V // s)) // align) * align
    rows = -(-(p.chunks_per_group * c) // 256) * 256
    assert rows * vpart * 2 <= 4 * 2 ** 30, (rows, vpart)
    assert -(-V // vpart) == s  # the reported count is the slices the backward visits
    st, f, b = ws(lib, N, d, V, K, chunk, dt)
    assert st == OK and (f, b) == (p.fwd_bytes, p.bwd_bytes)


@pytest.mark.parametrize("N,d,V,chunk", [
    (8192, 2880, 201088, 2048), (32768, 2880, 201088, 2048), (262144, 2880, 201088, 4096),
    (8192, 3072, 128256, 1024), (2048, 1024, 32000, 256), (20000, 512, 50000, 512), (3000, 256, 100000, 64),
])
def test_blocking_options_keep_the_vocabulary_tile(lib, N, d, V, chunk):
    """The vocabulary tile depends on the sizes only: every group size and
    slice count a caller (or the allocation-free forward, which takes fewer
    chunks per launch) may set gives the same tile, hence the same per-tile
    partials and the same rounding of the forward's results."""
    base = plan(lib, N, d, V, 100, chunk, L.KDKL_BF16).vocab_tile
    for cpg in (1, 2, 4, 8, 16):
        for vs in (0, 1, 3):
            p = L.Plan()
            st = lib.kdkl_plan_info(N, d, V, 100, chunk, L.KDKL_BF16, opts(chunks_per_group=cpg, vocab_slices=vs),
                                    C.byref(p))
            if st == OK:
                assert p.vocab_tile == base, (cpg, vs, p.vocab_tile, base)
