"""The C ABI on a host without a GPU: the library loads, exports every symbol the
header declares, and its host-side logic (argument checks, launch-shape policy,
source-store state machine) behaves as documented.  No kernel is launched:
every call here fails its checks before the first HIP call, or has T = 0 where
that launches nothing, or passes its checks and stops at the device query --
a call made only where no GPU is visible (``passes_host_checks``)."""

import ctypes
import math
import os
import re

import pytest
import torch

from depth_wise_attention_block_amd import binding as B

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(REPO, "include", "attnres.h")

# Fake, 16-byte aligned, non-overlapping device addresses: never dereferenced,
# because every call below is rejected on the host (or has nothing to do).
SRC, W, OUT, WTS = 0x10000000, 0x20000000, 0x30000000, 0x40000000

# Counting devices initialises no GPU.  With one visible, a call that passes
# every host check would launch on the fake addresses above.
NO_GPU = torch.cuda.device_count() == 0


def passes_host_checks(call):
    """``call()`` passes every host check: on a host without a GPU it then stops
    at the device query (ATTNRES_ELAUNCH).  Where a GPU is visible the call is
    not made."""
    if NO_GPU:
        assert call() == B.ELAUNCH


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libattnres.so is not built; run python -m depth_wise_attention_block_amd.build")
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"ATTNRES_API\s+[\w\s\*]+?\b(attnres_\w+)\s*\(", text)


def test_header_symbols_are_exported(lib):
    names = declared_functions()
    assert len(names) == 20, names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(B._SIGNATURES)


def test_version_and_strerror(lib):
    assert B.version() == 10000
    codes = [B.OK, B.EINVAL, B.EUNSUPPORTED, B.EALIAS, B.ELAUNCH, B.ESTATE]
    texts = [B.strerror(c) for c in codes]
    assert len(set(texts)) == len(codes)
    assert B.strerror(-99) == "unknown status"


def agg(S=9, T=4, d=7168, stride=0, src=SRC, w=W, out=OUT, wts=WTS, eps=1e-5, dtype=B.BF16):
    return B.lib().attnres_aggregate(src, S, T, d, stride, w, out, wts, eps, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(S=0), B.EINVAL), (dict(S=257), B.EINVAL), (dict(S=-1), B.EINVAL),
    (dict(T=-1), B.EINVAL), (dict(d=0), B.EINVAL),
    (dict(d=7164), B.EUNSUPPORTED), (dict(d=6, dtype=B.F32), B.EUNSUPPORTED),
    (dict(d=16392), B.EUNSUPPORTED), (dict(d=8196, dtype=B.F32), B.EUNSUPPORTED),
    (dict(dtype=2), B.EUNSUPPORTED),
    (dict(eps=float("nan")), B.EINVAL), (dict(eps=-1e-5), B.EINVAL), (dict(eps=float("inf")), B.EINVAL),
    (dict(stride=4 * 7168 - 8), B.EINVAL), (dict(stride=-8), B.EINVAL), (dict(stride=4 * 7168 + 4), B.EUNSUPPORTED),
    (dict(src=None), B.EINVAL), (dict(w=None), B.EINVAL), (dict(out=None), B.EINVAL),
    (dict(src=SRC + 8), B.EUNSUPPORTED), (dict(w=W + 4), B.EUNSUPPORTED), (dict(out=OUT + 2), B.EUNSUPPORTED),
    (dict(wts=WTS + 2), B.EUNSUPPORTED),
    (dict(out=SRC + 16), B.EALIAS), (dict(out=SRC + 8 * 4 * 7168 * 2), B.EALIAS),
    (dict(S=94, out=SRC + 93 * 4 * 7168 * 2), B.EALIAS), (dict(S=256, stride=4 * 7168 - 8), B.EINVAL),
    (dict(out=W - 16), B.EALIAS), (dict(wts=SRC + 64), B.EALIAS), (dict(wts=OUT + 4 * 7168 * 2 - 4), B.EALIAS),
    (dict(wts=W + 16), B.EALIAS),
])
def test_aggregate_rejects_before_any_launch(lib, kwargs, status):
    assert agg(**kwargs) == status


def test_aggregate_empty_batch_is_ok_without_pointers(lib):
    assert agg(T=0, src=None, w=None, out=None, wts=None) == B.OK
    assert agg(T=0, S=0) == B.EINVAL  # shape checks still apply


def test_last_source_end_is_the_alias_boundary(lib):
    # sources end exactly where out begins: touching, not overlapping -> only the
    # launch would remain, which needs a GPU; so check the neighbour byte instead
    end = SRC + (8 * 4 * 7168 + 4 * 7168) * 2
    assert agg(out=end - 16) == B.EALIAS


@pytest.mark.parametrize("S,T,d,dtype,threads,vpl", [
    (9, 262144, 7168, B.BF16, 448, 2),
    (9, 4096, 7168, B.BF16, 448, 2),
    (4, 64, 256, B.F32, 64, 1),
    (9, 5, 264, B.BF16, 64, 1),
    (9, 5, 7176, B.BF16, 512, 2),
    (9, 5, 4096, B.BF16, 512, 1),
    (9, 5, 7168, B.F32, 448, 4),
    (1, 1, 16384, B.BF16, 512, 4),
    (2, 3, 8, B.BF16, 64, 1),
])
def test_launch_shape_policy(lib, S, T, d, dtype, threads, vpl):
    cfg = B.aggregate_config(S, T, d, {B.BF16: B.torch.bfloat16, B.F32: B.torch.float32}[dtype], 256)
    assert cfg["threads"] == threads and cfg["vecs_per_lane"] == vpl
    epv = 8 if dtype == B.BF16 else 4
    assert cfg["threads"] * cfg["vecs_per_lane"] >= d // epv  # every vector has a lane
    assert cfg["threads"] % 64 == 0 and cfg["threads"] <= 512
    run = 32 if T >= 4096 else 1
    span = -(-T // (8 * run)) * 8 * run if run > 1 else T
    assert cfg["grid"] == min(span, 256 * 4096) and cfg["tokens_per_group"] == 1 and cfg["xcd_run"] == run


def test_launch_grid_caps_and_loops(lib):
    cfg = B.aggregate_config(2, 5_000_000, 8, B.torch.bfloat16, 256)
    assert cfg["grid"] == 256 * 4096 and cfg["xcd_run"] == 32


@pytest.mark.parametrize("T,run,grid", [
    (4095, 1, 4095),              # small batches: one token per XCD in turn
    (4096, 32, 4096),             # runs of 32 tokens per XCD
    (4097, 32, 4096 + 256),       # the virtual range is T rounded up to 8 runs
    (262144, 32, 262144),
    (256 * 4096 + 1, 32, 256 * 4096),  # grid-stride beyond the cap (a multiple of 8)
])
def test_launch_xcd_runs(lib, T, run, grid):
    cfg = B.aggregate_config(9, T, 7168, B.torch.bfloat16, 256)
    assert cfg["xcd_run"] == run and cfg["grid"] == grid
    assert run == 1 or cfg["grid"] % 8 == 0
    # the many-source kernel takes the same runs (its workgroups loop past the cap)
    many = B.aggregate_config(10, T, 7168, B.torch.bfloat16, 256)
    assert many["xcd_run"] == run and many["grid"] == grid


def xcd_token(b: int, run_log2: int) -> int:
    """The device's token of virtual workgroup index b (restated for the host test)."""
    x, k = b & 7, b >> 3
    return ((((k >> run_log2) << 3) | x) << run_log2) | (k & ((1 << run_log2) - 1))


@pytest.mark.parametrize("run_log2", [0, 1, 5])
def test_xcd_token_map_is_a_bijection(run_log2):
    span = 8 << run_log2
    for rounds in (1, 3):
        n = span * rounds
        got = sorted(xcd_token(b, run_log2) for b in range(n))
        assert got == list(range(n))
        # each XCD's tokens come in runs of 2^run_log2 consecutive tokens
        for b in range(0, n, 8):
            assert xcd_token(b + 8, run_log2) - xcd_token(b, run_log2) in (1, 8 * (1 << run_log2) - (1 << run_log2) + 1)


def _store(T=0, d=8, s_max=9, base=SRC, stride=0, dtype=B.BF16):
    st = B.attnres_store_t()
    rc = B.lib().attnres_store_init(ctypes.byref(st), base, s_max, T, d, stride, dtype)
    return rc, st


@pytest.mark.parametrize("kwargs,status", [
    (dict(s_max=1), B.EINVAL), (dict(s_max=10), B.EINVAL), (dict(T=4, base=None), B.EINVAL),
    (dict(T=0, base=None), B.OK),
    (dict(base=SRC + 2), B.EUNSUPPORTED), (dict(d=12), B.EUNSUPPORTED), (dict(dtype=7), B.EUNSUPPORTED),
    (dict(T=4, d=8, stride=24), B.EINVAL), (dict(T=4, d=8, stride=36), B.EUNSUPPORTED),
])
def test_store_init_checks(lib, kwargs, status):
    assert _store(**kwargs)[0] == status


def test_empty_store_without_memory(lib):
    """T = 0 with no memory behind the slots (an empty tensor's null pointer):
    the store's calls only update the counters."""
    rc, st = _store(T=0, base=None)
    assert rc == B.OK
    assert B.lib().attnres_accumulate(ctypes.byref(st), None, 0, None) == B.OK
    assert B.lib().attnres_accumulate_aggregate(ctypes.byref(st), None, 1, None, None, None, 1e-5, None) == B.OK
    assert (st.n_completed, st.partial_valid) == (1, 0)
    assert B.lib().attnres_store_sources(ctypes.byref(st)) == 2


def test_store_state_machine_follows_the_block_rule(lib):
    """93 layers in blocks of 12 through the C bookkeeping (T = 0, so nothing is
    enqueued): live-source counts before each layer, and the full store."""
    rc, st = _store(T=0)
    assert rc == B.OK
    counts = []
    for l in range(1, 94):
        counts.append(B.lib().attnres_store_sources(ctypes.byref(st)))
        finalize = l % 12 == 0 or l == 93
        assert B.lib().attnres_accumulate(ctypes.byref(st), None, int(finalize), None) == B.OK
    hist = {s: counts.count(s) for s in sorted(set(counts))}
    assert counts[0] == 1 and hist == {1: 1, 2: 12, 3: 12, 4: 12, 5: 12, 6: 12, 7: 12, 8: 12, 9: 8}
    assert st.n_completed == 8 and st.partial_valid == 0
    assert B.lib().attnres_store_sources(ctypes.byref(st)) == 9
    # no slot left for a ninth block
    before = (st.n_completed, st.partial_valid)
    assert B.lib().attnres_accumulate(ctypes.byref(st), None, 0, None) == B.ESTATE
    assert (st.n_completed, st.partial_valid) == before


def test_accumulate_argument_checks(lib):
    rc, st = _store(T=4, d=8)
    assert rc == B.OK
    acc = lambda ptr, fin=0: B.lib().attnres_accumulate(ctypes.byref(st), ptr, fin, None)
    assert acc(None) == B.EINVAL
    assert acc(OUT, fin=2) == B.EINVAL
    assert acc(OUT + 8) == B.EUNSUPPORTED
    assert acc(SRC + 16) == B.EALIAS
    assert acc(SRC + 9 * 4 * 8 * 2 - 16) == B.EALIAS
    assert (st.n_completed, st.partial_valid) == (0, 0)
    st.partial_valid = 3
    assert acc(OUT) == B.ESTATE
    st.partial_valid, st.n_completed = 1, 8
    assert acc(OUT) == B.ESTATE
    assert B.lib().attnres_accumulate(None, OUT, 0, None) == B.EINVAL


def test_fused_update_aggregate_checks(lib):
    """attnres_accumulate_aggregate rejects bad arguments before any HIP call and
    leaves the store untouched."""
    rc, st = _store(T=4, d=8)
    assert rc == B.OK
    F, Wq, O, A = OUT, W, 0x50000000, WTS

    def call(f=F, fin=0, w=Wq, out=O, wts=A, eps=1e-5):
        return B.lib().attnres_accumulate_aggregate(ctypes.byref(st), f, fin, w, out, wts, eps, None)

    assert call(f=None) == B.EINVAL
    assert call(w=None) == B.EINVAL
    assert call(out=None) == B.EINVAL
    assert call(fin=3) == B.EINVAL
    assert call(eps=float("nan")) == B.EINVAL
    assert call(f=F + 8) == B.EUNSUPPORTED
    assert call(out=O + 4) == B.EUNSUPPORTED
    assert call(wts=A + 1) == B.EUNSUPPORTED
    assert call(out=SRC + 32) == B.EALIAS          # residual into the store
    assert call(wts=SRC + 64) == B.EALIAS          # weights into the store
    assert call(out=F + 16) == B.EALIAS            # residual over the layer output
    assert call(wts=O + 16) == B.EALIAS            # weights over the residual
    assert call(w=SRC + 16) == B.EALIAS            # query inside the store
    assert (st.n_completed, st.partial_valid) == (0, 0)
    st.n_completed, st.partial_valid = 8, 0
    assert call() == B.ESTATE
    assert (st.n_completed, st.partial_valid) == (8, 0)


def test_fused_update_aggregate_bookkeeping_without_tokens(lib):
    """With T = 0 the fused call only advances the store, exactly like
    attnres_accumulate."""
    rc, st = _store(T=0)
    assert rc == B.OK
    counts = []
    for l in range(1, 94):
        fin = int(l % 12 == 0 or l == 93)
        assert B.lib().attnres_accumulate_aggregate(ctypes.byref(st), None, fin, None, None, None, 1e-5, None) == B.OK
        counts.append(B.lib().attnres_store_sources(ctypes.byref(st)))
    # sources seen by layers 2..93 and the output layer
    assert counts[-1] == 9 and st.n_completed == 8 and counts[0] == 2


def test_two_phase_checks_and_bookkeeping(lib):
    """attnres_block_prepare / attnres_block_merge argument checks (no launch) and
    their effect on the store with T = 0."""
    rc, st = _store(T=4, d=8)
    assert rc == B.OK
    INTER, LOG, W0 = 0x60000000, 0x70000000, 0x78000000

    def prep(f=OUT, close=0, w=W, nb=12, inter=INTER, stride=0, lg=LOG, w0=W0, eps=1e-5):
        return B.lib().attnres_block_prepare(ctypes.byref(st), f, close, w, nb, inter, stride, lg, w0, eps, None)

    assert prep(nb=0) == B.EINVAL and prep(nb=17) == B.EINVAL
    assert prep(close=2) == B.EINVAL
    assert prep(w=None) == B.EINVAL and prep(inter=None) == B.EINVAL and prep(lg=None) == B.EINVAL
    assert prep(close=1, f=None) == B.EINVAL
    assert prep(inter=INTER + 8) == B.EUNSUPPORTED and prep(lg=LOG + 2) == B.EUNSUPPORTED
    assert prep(stride=4 * 8 - 8) == B.EINVAL
    assert prep(inter=SRC + 16) == B.EALIAS and prep(lg=INTER + 64) == B.EALIAS and prep(w0=LOG) == B.EALIAS
    st.partial_valid = 1
    assert prep() == B.ESTATE          # an open partial must be closed first
    st.partial_valid, st.n_completed = 0, 7
    assert prep(close=1) == B.EUNSUPPORTED or prep(close=1) == B.ESTATE   # 9 inter sources: too many
    st.n_completed = 0
    rcf, stf = _store(T=4, d=8, dtype=B.F32)
    assert B.lib().attnres_block_prepare(ctypes.byref(stf), None, 0, W, 4, INTER, 0, LOG, None, 1e-5,
                                         None) == B.EUNSUPPORTED

    def merge(f=OUT, w=W, inter=INTER, lg=LOG, out=0x58000000, wts=W0):
        return B.lib().attnres_block_merge(ctypes.byref(st), f, w, inter, lg, out, wts, 1e-5, None)

    assert merge(f=None) == B.EINVAL and merge(out=None) == B.EINVAL
    assert merge(out=SRC) == B.EALIAS and merge(out=INTER + 16) == B.EALIAS and merge(wts=LOG) == B.EALIAS
    assert (st.n_completed, st.partial_valid) == (0, 0)

    split = B.lib().attnres_split_queries
    assert split(None, 2, 8, OUT, None) == B.EINVAL and split(W, -1, 8, OUT, None) == B.EINVAL
    assert split(W + 2, 2, 8, OUT, None) == B.EUNSUPPORTED and split(W, 2, 8, W + 16, None) == B.EALIAS
    assert split(None, 0, 8, None, None) == B.OK
    assert split(W, 2, 12, OUT, None) == B.EUNSUPPORTED and split(W, 2, 8, OUT + 8, None) == B.EUNSUPPORTED

    rc, st0 = _store(T=0)
    call = lambda: B.lib().attnres_block_prepare(ctypes.byref(st0), None, 0, None, 12, None, 0, None, None,
                                                 1e-5, None)
    assert call() == B.OK and (st0.n_completed, st0.partial_valid) == (0, 0)
    assert B.lib().attnres_block_merge(ctypes.byref(st0), None, None, None, None, None, None, 1e-5, None) == B.OK
    assert st0.partial_valid == 1
    assert B.lib().attnres_block_prepare(ctypes.byref(st0), None, 1, None, 12, None, 0, None, None, 1e-5,
                                         None) == B.OK
    assert (st0.n_completed, st0.partial_valid) == (1, 0)


def test_backward_host_checks(lib):
    """attnres_aggregate_backward rejects bad arguments before touching the GPU."""
    GS, GL, GW, WS = 0x60000000, 0x68000000, 0x6C000000, 0x70000000

    CF = 0x74000000

    def bwd(S=3, T=4, d=8, src=SRC, w=W, g=OUT, gs=GS, gstride=0, gl=None, gw=GW, ws=WS, wsb=1 << 20, eps=1e-5,
            dtype=B.BF16, src_stride=0, last=None, defer=0, cf=None, cfs=0):
        return B.lib().attnres_aggregate_backward(src, S, T, d, src_stride, last, w, g, gs, gstride, 0, defer, cf,
                                                  cfs, gl, gw, ws, wsb, eps, dtype, None)

    assert bwd(S=0) == B.EINVAL and bwd(S=10) == B.EINVAL          # Block AttnRes sizes only
    assert bwd(T=-1) == B.EINVAL and bwd(d=12) == B.EUNSUPPORTED
    assert bwd(eps=-1.0) == B.EINVAL and bwd(eps=float("nan")) == B.EINVAL
    assert bwd(gw=None) == B.EINVAL and bwd(gw=GW + 2) == B.EUNSUPPORTED
    assert bwd(src=None) == B.EINVAL and bwd(g=None) == B.EINVAL and bwd(gs=None) == B.EINVAL
    assert bwd(ws=None) == B.EINVAL and bwd(wsb=0) == B.EINVAL
    assert bwd(gstride=8) == B.EINVAL and bwd(gstride=4 * 8 + 2) == B.EUNSUPPORTED
    assert bwd(gs=GS + 8) == B.EUNSUPPORTED and bwd(gl=GL + 8) == B.EUNSUPPORTED
    assert bwd(gs=SRC + 32) == B.EALIAS and bwd(gl=OUT) == B.EALIAS and bwd(gw=W) == B.EALIAS
    assert bwd(ws=GS + 64) == B.EALIAS and bwd(gl=GS + 16) == B.EALIAS
    assert bwd(last=SRC + 8) == B.EUNSUPPORTED and bwd(last=GS) == B.EALIAS
    assert bwd(S=1, src=None) == B.EINVAL
    assert bwd(defer=0b011, cf=None, cfs=9) == B.EINVAL and bwd(defer=0b011, cf=CF, cfs=8) == B.EINVAL
    assert bwd(defer=0b011, cf=CF + 2, cfs=9) == B.EUNSUPPORTED
    assert bwd(defer=0b100, cf=CF, cfs=9, gl=GL) == B.EINVAL          # the last source is deferred
    assert bwd(defer=0b011, cf=GS + 4, cfs=9) == B.EALIAS and bwd(defer=0b011, cf=SRC, cfs=9) == B.EALIAS
    assert bwd(defer=0b011, cf=CF, cfs=1 << 40) == B.EINVAL           # coefficient offsets beyond 2^40
    # no grad_w: dL/dw left to the caller, every source's coefficients written, no workspace
    assert bwd(gw=None, cf=CF, cfs=8) == B.EINVAL and bwd(gw=None, cf=CF + 2, cfs=9) == B.EUNSUPPORTED
    assert bwd(gw=None, cf=GS + 4, cfs=9) == B.EALIAS                  # coefficients of all three sources
    assert bwd(gw=None, cf=CF + 64, cfs=9, gs=CF) == B.EALIAS
    passes_host_checks(lambda: bwd(gw=None, cf=CF, cfs=9, ws=None, wsb=0))
    assert bwd(T=0, gw=None, cf=CF, cfs=9, ws=None, wsb=0) == B.OK     # nothing to launch
    assert bwd(T=0, gw=None, cf=None, cfs=9) == B.EINVAL

    Arr = ctypes.c_void_p * 2
    G2, W2, DW2 = Arr(OUT, OUT + 4096), Arr(W, W + 4096), Arr(GW, GW + 4096)

    def blk(n=3, T=4, d=8, src=SRC, Bl=2, gs_=G2, ws_=W2, cf=CF, cls=0, grads=GS, gl=None, dtype=B.BF16,
            gstride=0, dws=DW2, wk=WS, wkb=1 << 20):
        return B.lib().attnres_block_backward(src, n, T, d, 0, Bl, gs_, ws_, cf, cls, grads, gstride, 0, gl, dws,
                                              wk, wkb, dtype, None)

    assert blk(n=0) == B.EINVAL and blk(n=9) == B.EINVAL and blk(Bl=0) == B.EINVAL and blk(Bl=17) == B.EINVAL
    assert blk(T=0) == B.OK and blk(d=12) == B.EUNSUPPORTED and blk(gstride=8) == B.EINVAL
    assert blk(src=None) == B.EINVAL and blk(cf=None) == B.EINVAL and blk(grads=None) == B.EINVAL
    assert blk(dws=None) == B.EINVAL and blk(wk=None) == B.EINVAL and blk(dws=Arr(GW, 0)) == B.EINVAL
    assert blk(gs_=Arr(OUT, 0)) == B.EINVAL and blk(ws_=Arr(W, W + 8)) == B.EUNSUPPORTED
    assert blk(grads=GS + 8) == B.EUNSUPPORTED and blk(cf=CF + 2) == B.EUNSUPPORTED
    assert blk(dws=Arr(GW, GW + 8)) == B.EUNSUPPORTED and blk(wk=WS + 8) == B.EUNSUPPORTED
    assert blk(grads=SRC) == B.EALIAS and blk(gl=OUT + 4096) == B.EALIAS and blk(grads=CF) == B.EALIAS
    assert blk(dws=Arr(GW, W)) == B.EALIAS and blk(dws=Arr(GW, GW)) == B.EALIAS and blk(wk=GS) == B.EALIAS
    assert blk(dws=Arr(GW, WS + 64)) == B.EALIAS
    assert blk(cls=8) == B.EINVAL and blk(cls=-9) == B.EINVAL          # fewer floats per layer than 3n
    assert blk(cls=1 << 40) == B.EUNSUPPORTED                          # T * B * m * 4 beyond 32-bit offsets
    assert blk(cls=12, grads=CF + 4 * 2 * 12 * 4 - 16) == B.EALIAS     # the coefficients span T * B * m floats
    passes_host_checks(lambda: blk(cls=12, grads=CF + 4 * 2 * 12 * 4))
    passes_host_checks(lambda: blk(cls=12))

    add = B.lib().attnres_add_rows
    assert add(None, None, W, 4, 8, B.BF16, None) == B.EINVAL and add(None, OUT, None, 4, 8, B.BF16, None) == B.EINVAL
    assert add(SRC + 8, OUT, W, 4, 8, B.BF16, None) == B.EUNSUPPORTED and add(None, OUT, OUT, 4, 8, B.BF16, None) == B.EALIAS
    assert add(SRC, OUT, SRC + 16, 4, 8, B.BF16, None) == B.EALIAS and add(None, OUT, W, 0, 8, B.BF16, None) == B.OK
    out = ctypes.c_int64()
    assert B.lib().attnres_aggregate_backward_workspace(0, 8, B.BF16, ctypes.byref(out)) == B.OK and out.value == 0
    assert B.lib().attnres_aggregate_backward_workspace(4, 8, B.BF16, None) == B.EINVAL
    wsb = B.lib().attnres_block_backward_workspace
    assert wsb(0, 8, 3, B.BF16, ctypes.byref(out)) == B.OK and out.value == 0
    assert wsb(4, 8, 0, B.BF16, ctypes.byref(out)) == B.EINVAL and wsb(4, 8, 17, B.BF16, ctypes.byref(out)) == B.EINVAL
    assert wsb(4, 12, 3, B.BF16, ctypes.byref(out)) == B.EUNSUPPORTED and wsb(4, 8, 3, B.BF16, None) == B.EINVAL


def test_partial_dw_host_checks(lib):
    """attnres_partial_dw rejects bad arguments before touching the GPU."""
    Arr = ctypes.c_void_p * 3
    R0, R1, CF, DW, WS = 0x60000000, 0x61000000, 0x62000000, 0x63000000, 0x64000000
    ROWS, DWS = Arr(None, R0, R1), Arr(DW, DW + 4096, DW + 8192)

    def pdw(rows=ROWS, Bl=3, T=4, d=8, cf=CF, cs=6, cls=3, dws=DWS, ws=WS, wsb=1 << 20, dtype=B.BF16):
        return B.lib().attnres_partial_dw(rows, Bl, T, d, cf, cs, cls, dws, ws, wsb, dtype, None)

    assert pdw(Bl=0) == B.EINVAL and pdw(Bl=17) == B.EINVAL and pdw(T=-1) == B.EINVAL
    assert pdw(d=12) == B.EUNSUPPORTED and pdw(dtype=2) == B.EUNSUPPORTED
    assert pdw(rows=None) == B.EINVAL and pdw(dws=None) == B.EINVAL and pdw(dws=Arr(DW, None, DW + 64)) == B.EINVAL
    assert pdw(cs=-1) == B.EINVAL and pdw(cls=-1) == B.EINVAL and pdw(cs=1 << 40) == B.EINVAL
    assert pdw(cls=(1 << 40) + 1) == B.EINVAL
    assert pdw(cf=None) == B.EINVAL and pdw(cf=CF + 2) == B.EUNSUPPORTED          # rows need coefficients
    assert pdw(rows=Arr(None, R0 + 8, R1)) == B.EUNSUPPORTED and pdw(dws=Arr(DW, DW + 2, DW + 64)) == B.EUNSUPPORTED
    assert pdw(ws=None) == B.EINVAL and pdw(ws=WS + 8) == B.EUNSUPPORTED
    assert pdw(dws=Arr(DW, R0 + 16, DW + 64)) == B.EALIAS and pdw(dws=Arr(DW, CF + 8, DW + 64)) == B.EALIAS
    assert pdw(dws=Arr(DW, DW + 16, DW + 64)) == B.EALIAS and pdw(ws=R1) == B.EALIAS and pdw(ws=DW) == B.EALIAS
    passes_host_checks(lambda: pdw(dws=Arr(DW, CF + 4 * (3 * 6 + 2 * 3) + 4, DW + 64)))  # past the last coefficient
    passes_host_checks(lambda: pdw(rows=Arr(None, None, None), cf=None))    # nothing to read
    passes_host_checks(lambda: pdw(T=0, cf=None, ws=None))                  # T = 0 still zeroes the rows
    out = ctypes.c_int64()
    wsq = B.lib().attnres_partial_dw_workspace
    assert wsq(0, 8, 3, B.BF16, ctypes.byref(out)) == B.OK and out.value == 0
    assert wsq(4, 8, 0, B.BF16, ctypes.byref(out)) == B.EINVAL and wsq(4, 8, 17, B.BF16, ctypes.byref(out)) == B.EINVAL
    assert wsq(4, 12, 3, B.BF16, ctypes.byref(out)) == B.EUNSUPPORTED and wsq(4, 8, 3, B.BF16, None) == B.EINVAL


def test_backward_static_checks_like_the_workspace_entry_point(lib):
    """attnres_aggregate_backward_static takes the same arguments minus the
    workspace and rejects the same mistakes before any HIP call; a valid call
    gets as far as the device query (which fails on a host without a GPU)."""
    GS, GW, GL, G, CF = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xA0000000

    def bs(src=SRC, S=3, T=4, d=7168, w=W, g=G, gs=GS, gw=GW, gl=GL, acc=0, defer=0, cf=None, cs=0, eps=1e-5,
           dtype=B.BF16):
        return B.lib().attnres_aggregate_backward_static(src, S, T, d, 0, None, w, g, gs, 0, acc, defer, cf, cs,
                                                         gl, gw, eps, dtype, None)

    assert bs(S=0) == B.EINVAL and bs(S=10) == B.EINVAL and bs(d=7164) == B.EUNSUPPORTED
    assert bs(eps=float("nan")) == B.EINVAL and bs(gw=None) == B.EINVAL and bs(g=None) == B.EINVAL
    assert bs(src=SRC + 8) == B.EUNSUPPORTED and bs(gw=GW + 2) == B.EUNSUPPORTED
    assert bs(gs=SRC + 32) == B.EALIAS and bs(gl=G) == B.EALIAS and bs(gw=W) == B.EALIAS
    assert bs(defer=1) == B.EINVAL                                 # deferred sources need coef
    assert bs(gw=None, cf=None) == B.EINVAL
    passes_host_checks(lambda: bs(gw=None, cf=0xB0000000, cs=9))
    passes_host_checks(bs)


def test_partial_sums_host_checks(lib):
    Arr = ctypes.c_void_p * 3
    F3 = Arr(SRC, SRC + 4096, SRC + 8192)

    def ps(arr=F3, count=3, T=4, d=8, out=OUT, stride=0, dtype=B.BF16):
        return B.lib().attnres_partial_sums(arr, count, T, d, out, stride, dtype, None)

    assert ps(count=0) == B.EINVAL and ps(count=17) == B.EINVAL and ps(d=12) == B.EUNSUPPORTED
    assert ps(T=0) == B.OK and ps(stride=8) == B.EINVAL and ps(out=None) == B.EINVAL
    assert ps(out=OUT + 8) == B.EUNSUPPORTED and ps(arr=Arr(SRC, 0, SRC)) == B.EINVAL
    assert ps(arr=Arr(SRC, SRC + 8, SRC)) == B.EUNSUPPORTED and ps(out=SRC + 4096) == B.EALIAS


def test_binding_limits_match_the_header():
    """The binding's size limits are the header's #defines."""
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                             "attnres.h")).read()
    defines = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (ATTNRES_\w+) (\d+)", text)}
    assert defines["ATTNRES_MAX_SOURCES"] == B.MAX_SOURCES
    assert defines["ATTNRES_MAX_SOURCES_FULL"] == B.MAX_SOURCES_FULL
    assert defines["ATTNRES_MAX_INTER_SOURCES"] == B.MAX_INTER_SOURCES
    assert defines["ATTNRES_MAX_BLOCK_QUERIES"] == B.MAX_BLOCK_QUERIES
    assert defines["ATTNRES_MAX_D_BF16"] == B.MAX_D_BF16 and defines["ATTNRES_MAX_D_F32"] == B.MAX_D_F32
    assert re.search(r"#define ATTNRES_STATIC_SCRATCH_BYTES \(16 << 20\)", text) and B.STATIC_SCRATCH_BYTES == 16 << 20


def test_binding_refuses_host_tensors():
    """The C ABI cannot tell host pointers from device pointers, so the binding
    refuses tensors that are not on a GPU before anything reaches the library --
    also when a stream handle is given explicitly."""
    import torch
    S, T, d = 3, 4, 16
    H = torch.zeros((S, T, d), dtype=torch.bfloat16)
    w = torch.zeros(d, dtype=torch.float32)
    for stream in (None, 0):
        with pytest.raises(ValueError, match="GPU"):
            B.aggregate(H, w, stream=stream)
        with pytest.raises(ValueError, match="GPU"):
            B.add_rows(H[0], H[1], torch.empty((T, d), dtype=torch.bfloat16), stream=stream)
        with pytest.raises(ValueError, match="GPU"):
            B.split_queries(torch.zeros((2, d), dtype=torch.float32), stream=stream)
        with pytest.raises(ValueError, match="GPU"):
            B.aggregate_backward(H, w, H[0], torch.zeros((S, T, d), dtype=torch.float32),
                                 workspace=torch.zeros(64, dtype=torch.float32), stream=stream)


class _OnGpu:
    """A host tensor that reports a GPU device: enough for the binding's
    argument checks, which must refuse a call before any pointer reaches the
    library.  Slicing keeps the disguise."""

    def __init__(self, t):
        self._t = t

    @property
    def device(self):
        import torch
        return torch.device("cuda", 0)

    def __getitem__(self, k):
        return _OnGpu(self._t[k])

    def __getattr__(self, name):
        return getattr(self._t, name)


class _HostOnlyLib:
    """The real library for its host-only calls; any launching entry point fails the test."""
    HOST = {"attnres_store_init", "attnres_store_sources", "attnres_strerror", "attnres_version"}

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in self.HOST:
            return getattr(self._real, name)
        raise AssertionError(f"{name} was called with a host tensor among its arguments")


def _mixed_calls():
    """(label, argument index, call) for every binding entry point that
    launches work: call(k) disguises every tensor argument as a GPU tensor
    except the k-th, which stays on the host."""
    import torch
    S, T, d, Bq = 3, 4, 16, 2
    bf, f32 = torch.bfloat16, torch.float32

    def mk(*shape, dtype=bf):
        return torch.zeros(shape, dtype=dtype)

    def pick(args, k):
        return [a if i == k else (_OnGpu(a) if a is not None else None) for i, a in enumerate(args)]

    calls = []

    def add(label, args, fn):
        for k in range(len(args)):
            calls.append((label, k, lambda k=k, args=args, fn=fn: fn(*pick(args, k))))

    add("aggregate", [mk(S, T, d), mk(d, dtype=f32), mk(T, d), mk(T, S, dtype=f32)],
        lambda H, w, o, a: B.aggregate(H, w, o, a))
    add("add_rows", [mk(T, d), mk(T, d), mk(T, d)], lambda a, b, o: B.add_rows(a, b, o))
    add("aggregate_backward",
        [mk(S - 1, T, d), mk(T, d), mk(d, dtype=f32), mk(T, d), mk(S, T, d, dtype=f32), mk(T, 3 * S, dtype=f32),
         mk(d, dtype=f32), mk(T, d), mk(64, dtype=f32)],
        lambda H, last, w, g, gs, cf, gw, gl, ws: B.aggregate_backward(
            H, w, g, gs, last_source=last, defer=1, coef=cf, coef_stride=3 * S, grad_w=gw, grad_last=gl,
            workspace=ws))
    add("partial_sums", [mk(T, d), mk(T, d), mk(2, T, d)], lambda a, b, o: B.partial_sums([a, b], o))
    add("block_backward",
        [mk(S, T, d), mk(T, d), mk(T, d), mk(d, dtype=f32), mk(d, dtype=f32), mk(T, Bq, S, 3, dtype=f32),
         mk(S, T, d, dtype=f32), mk(d, dtype=f32), mk(d, dtype=f32), mk(T, d), mk(64, dtype=f32)],
        lambda H, g0, g1, w0, w1, cf, gs, dw0, dw1, gl, ws: B.block_backward(
            H, [g0, g1], [w0, w1], cf, gs, [dw0, dw1], grad_last=gl, workspace=ws))
    add("split_queries", [mk(Bq, d, dtype=f32), mk(*B.prepared_query_shape(Bq, d))],
        lambda w, o: B.split_queries(w, o))
    add("partial_dw", [mk(T, d), mk(T, d), mk(T * Bq * 3, dtype=f32), mk(d, dtype=f32), mk(d, dtype=f32),
                       mk(64, dtype=f32)],
        lambda r0, r1, cf, dw0, dw1, ws: B.partial_dw([r0, r1], cf, Bq * 3, 3, [dw0, dw1], workspace=ws))

    def store(slots):
        st = B.SourceStore(T, d, s_max=4, slots=slots)
        st.set_state(1, True)
        return st

    add("SourceStore.accumulate", [mk(4, T, d), mk(T, d)], lambda sl, F: store(sl).accumulate(F))
    add("SourceStore.accumulate_aggregate", [mk(4, T, d), mk(T, d), mk(d, dtype=f32), mk(T, d), mk(T, 3, dtype=f32)],
        lambda sl, F, w, o, a: store(sl).accumulate_aggregate(F, False, w, o, a))
    add("SourceStore.block_prepare",
        [mk(4, T, d), mk(T, d), mk(*B.prepared_query_shape(Bq, d)), mk(Bq, T, d), mk(Bq, T, 3, dtype=f32),
         mk(T, 3, dtype=f32)],
        lambda sl, F, ws, inter, lg, w0: store(sl).block_prepare(F, True, ws, inter, lg, w0))
    add("SourceStore.block_merge",
        [mk(4, T, d), mk(T, d), mk(d, dtype=f32), mk(T, d), mk(T, 2, dtype=f32), mk(T, d), mk(T, 3, dtype=f32)],
        lambda sl, F, w, inter, lg, o, a: store(sl).block_merge(F, w, inter, lg, o, a))
    return calls


@pytest.mark.parametrize("label,k,call", _mixed_calls(), ids=lambda v: str(v) if not callable(v) else "")
def test_binding_refuses_one_host_tensor_among_gpu_tensors(monkeypatch, label, k, call):
    """Every launching entry point checks the device of every tensor argument:
    one host tensor among (disguised) GPU tensors is refused with ValueError
    before the library sees a pointer."""
    real = B.lib()
    monkeypatch.setattr(B, "lib", lambda: _HostOnlyLib(real))
    with pytest.raises(ValueError, match="GPU|must be on"):
        call()


def test_binding_refuses_a_short_coefficient_buffer(monkeypatch):
    """The kernels write (backward) or read (partial_dw) coefficients at
    t * coef_stride + ... from the buffer's first element, which the C ABI
    cannot bound: the binding refuses a buffer one element short, and lets
    the exact size through to the library."""
    import torch
    real = B.lib()
    monkeypatch.setattr(B, "lib", lambda: _HostOnlyLib(real))
    S, T, d = 3, 4, 16

    def g(*shape, dtype=torch.bfloat16):
        return _OnGpu(torch.zeros(shape, dtype=dtype))

    def bwd(n, defer, form_dw):
        kw = dict(grad_w=g(d, dtype=torch.float32), workspace=g(64, dtype=torch.float32)) if form_dw else {}
        B.aggregate_backward(g(S, T, d), g(d, dtype=torch.float32), g(T, d), g(S, T, d, dtype=torch.float32),
                             defer=defer, coef=g(n, dtype=torch.float32), coef_stride=9, form_dw=form_dw, **kw)

    # every source's triple without dL/dw; up to the highest deferred source's with it
    for defer, form_dw, need in ((0b011, False, 3 * 9 + 9), (0b011, True, 3 * 9 + 6), (0b001, True, 3 * 9 + 3)):
        with pytest.raises(ValueError, match="coef"):
            bwd(need - 1, defer, form_dw)
        with pytest.raises(AssertionError, match="was called"):
            bwd(need, defer, form_dw)

    def pdw(n):
        B.partial_dw([None, g(T, d), g(T, d)], g(n, dtype=torch.float32), 9, 3,
                     [g(d, dtype=torch.float32) for _ in range(3)], workspace=g(64, dtype=torch.float32))

    need = 3 * 9 + 2 * 3 + 1
    with pytest.raises(ValueError, match="coef"):
        pdw(need - 1)
    with pytest.raises(AssertionError, match="was called"):
        pdw(need)


def test_c_client_checks_its_input_before_any_gpu_call(tmp_path):
    """The plain C caller refuses bad usage and a bad header before it makes
    any HIP call (so this runs without a GPU)."""
    import struct
    import subprocess
    client = os.path.join(os.path.dirname(B.LIB_PATH), "capi_client")
    r = subprocess.run([client], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
    bad = tmp_path / "bad.bin"
    bad.write_bytes(struct.pack("<4i", 0, 4, 16, 0))
    r = subprocess.run([client, str(bad), str(tmp_path / "out.bin")], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "bad header" in r.stderr


# ---- property-based sweep of the argument checks ---------------------------
# Random sizes, strides (from edge values: negative, zero, tiny, the largest
# accepted, just past it, near int64's end) and fake pointers (aligned,
# misaligned, overlapping each other, null): every call must return one of the
# documented statuses, and -- in the sanitized child run of this file -- do so
# without an out-of-bounds access or an integer overflow in the range and
# alias arithmetic.  Calls that pass their checks stop at the device query, so
# the sweep runs only where no GPU is visible.

from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

STATUSES = {B.OK, B.EINVAL, B.EUNSUPPORTED, B.EALIAS, B.ELAUNCH}
EDGE = [-(1 << 62), -1, 0, 1, 2, 3, 4, 7, 8, 9, 12, 16, 17, 27, 255, 256, 4096, 7168, 7176, 8192, 16384, 16392,
        (1 << 31) - 1, 1 << 31, 1 << 37, (1 << 40) // 8, 1 << 40, (1 << 40) + 1, 1 << 62, (1 << 63) - 1]
PTRS = [None, 0x10000000, 0x10000008, 0x10000010, 0x10000400, 0x20000000, 0x30000000, 0x30000004, 0x7FFFFFFFFFF0]
ints = st.sampled_from(EDGE)
small = st.integers(min_value=-2, max_value=18)
ptrs = st.sampled_from(PTRS)
FUZZ = settings(max_examples=300, deadline=None, derandomize=True, suppress_health_check=list(HealthCheck))
no_gpu = pytest.mark.skipif(not NO_GPU, reason="a call that passes its checks would launch on fake addresses")


def _arr(items):
    return (ctypes.c_void_p * max(len(items), 1))(*items)


@no_gpu
@FUZZ
@given(S=small, T=ints, d=ints, src_stride=ints, grad_stride=ints, coef_stride=ints, ws_bytes=ints,
       acc=st.integers(0, 0x3FF), defer=st.integers(0, 0x3FF), dtype=st.sampled_from([0, 1, 2]),
       p=st.lists(ptrs, min_size=9, max_size=9), static=st.booleans())
def test_fuzz_aggregate_backward(lib, S, T, d, src_stride, grad_stride, coef_stride, ws_bytes, acc, defer, dtype, p,
                                 static):
    src, last, w, g, gs, cf, gl, gw, ws = p
    if static:
        rc = B.lib().attnres_aggregate_backward_static(src, S, T, d, src_stride, last, w, g, gs, grad_stride, acc,
                                                       defer, cf, coef_stride, gl, gw, 1e-5, dtype, None)
    else:
        rc = B.lib().attnres_aggregate_backward(src, S, T, d, src_stride, last, w, g, gs, grad_stride, acc, defer,
                                                cf, coef_stride, gl, gw, ws, ws_bytes, 1e-5, dtype, None)
    assert rc in STATUSES


@no_gpu
@FUZZ
@given(n=small, Bl=small, T=ints, d=ints, src_stride=ints, grad_stride=ints, cls=ints, ws_bytes=ints,
       dtype=st.sampled_from([0, 1, 2]), p=st.lists(ptrs, min_size=5, max_size=5),
       rows=st.lists(ptrs, min_size=16, max_size=16), qs=st.lists(ptrs, min_size=16, max_size=16),
       dws=st.lists(ptrs, min_size=16, max_size=16))
def test_fuzz_block_backward(lib, n, Bl, T, d, src_stride, grad_stride, cls, ws_bytes, dtype, p, rows, qs, dws):
    src, cf, gs, gl, ws = p
    rc = B.lib().attnres_block_backward(src, n, T, d, src_stride, Bl, _arr(rows), _arr(qs), cf, cls, gs, grad_stride,
                                        0xFF, gl, _arr(dws), ws, ws_bytes, dtype, None)
    assert rc in STATUSES


@no_gpu
@FUZZ
@given(Bl=small, T=ints, d=ints, cs=ints, cls=ints, ws_bytes=ints, dtype=st.sampled_from([0, 1, 2]),
       cf=ptrs, ws=ptrs, rows=st.lists(ptrs, min_size=16, max_size=16), dws=st.lists(ptrs, min_size=16, max_size=16))
def test_fuzz_partial_dw(lib, Bl, T, d, cs, cls, ws_bytes, dtype, cf, ws, rows, dws):
    rc = B.lib().attnres_partial_dw(_arr(rows), Bl, T, d, cf, cs, cls, _arr(dws), ws, ws_bytes, dtype, None)
    assert rc in STATUSES


@no_gpu
@FUZZ
@given(S=st.sampled_from([-1, 0, 1, 2, 9, 10, 94, 256, 257]), T=ints, d=ints, stride=ints,
       dtype=st.sampled_from([0, 1, 2]), p=st.lists(ptrs, min_size=4, max_size=4),
       count=small, outs=st.lists(ptrs, min_size=16, max_size=16), out=ptrs, out_stride=ints)
def test_fuzz_aggregate_and_partial_sums(lib, S, T, d, stride, dtype, p, count, outs, out, out_stride):
    src, w, o, wts = p
    assert B.lib().attnres_aggregate(src, S, T, d, stride, w, o, wts, 1e-5, dtype, None) in STATUSES
    assert B.lib().attnres_partial_sums(_arr(outs), count, T, d, out, out_stride, dtype, None) in STATUSES


STORE_FIELDS = ("base", "T", "slot_stride", "d", "s_max", "dtype", "n_completed", "partial_valid", "reserved")


@no_gpu
@FUZZ
@given(base=ptrs, T=ints, stride=ints, d=ints, s_max=small, dtype=st.sampled_from([0, 1, 2]),
       n_done=small, pv=st.integers(-1, 2), which=st.integers(0, 4), fin=st.integers(-1, 2), nb=small,
       inter_stride=ints, p=st.lists(ptrs, min_size=6, max_size=6))
def test_fuzz_store_calls(lib, base, T, stride, d, s_max, dtype, n_done, pv, which, fin, nb, inter_stride, p):
    """Any store, including one no attnres_store_init would produce: each call
    returns a documented status, and a rejected call leaves the store as it was."""
    s = B.attnres_store_t(base=base, T=T, slot_stride=stride, d=d, s_max=s_max, dtype=dtype, n_completed=n_done,
                          partial_valid=pv, reserved=0)
    before = tuple(getattr(s, f) for f in STORE_FIELDS)
    f, w, inter, lg, out, wts = p
    ref = ctypes.byref(s)
    if which == 0:
        rc = B.lib().attnres_accumulate(ref, f, fin, None)
    elif which == 1:
        rc = B.lib().attnres_accumulate_aggregate(ref, f, fin, w, out, wts, 1e-5, None)
    elif which == 2:
        rc = B.lib().attnres_block_prepare(ref, f, fin, w, nb, inter, inter_stride, lg, wts, 1e-5, None)
    elif which == 3:
        rc = B.lib().attnres_block_merge(ref, f, w, inter, lg, out, wts, 1e-5, None)
    else:
        rc = B.lib().attnres_store_sources(ref)
        assert rc in STATUSES | {B.ESTATE} or 1 <= rc <= 9
        rc = B.OK
    assert rc in STATUSES | {B.ESTATE}
    if rc not in (B.OK, B.ELAUNCH):
        assert tuple(getattr(s, f) for f in STORE_FIELDS) == before, "a rejected call changed the store"


@no_gpu
@FUZZ
@given(n=st.sampled_from([-1, 0, 1, 4, 5, 16, 17, 1 << 20]), T=ints, d=ints, dtype=st.sampled_from([0, 1, 2]),
       p=st.lists(ptrs, min_size=3, max_size=3))
def test_fuzz_split_queries_and_add_rows(lib, n, T, d, dtype, p):
    a, b, out = p
    assert B.lib().attnres_split_queries(a, n, d, out, None) in STATUSES
    assert B.lib().attnres_add_rows(a, b, out, T, d, dtype, None) in STATUSES
