"""Host-side checks of the C ABI: exports, workspace sizing and validation.

These run without a GPU.  Every call here fails validation (or is the batch = 0
no-op) before the library touches the HIP runtime, so fake, aligned, never
dereferenced pointer values are enough.
"""
import ctypes
import re

import pytest

import newton_schulz_03_amd as nsa
from newton_schulz_03_amd._binding import NsParams, StepParams, _i64_array, _ptr_array

FAKE = 0x7f0000000000  # aligned, never dereferenced


def header_functions():
    text = open(nsa.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return nsa.load_library()


def test_every_declared_function_is_exported(lib):
    names = header_functions()
    assert set(names) == set(nsa.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_kernel_names_follow_the_header_enum():
    text = open(nsa.HEADER_PATH).read()
    ids = {m.group(1).lower(): int(m.group(2))
           for m in re.finditer(r"MUON_K_([A-Z0-9_]+)\s*=\s*(\d+)", text)}
    count = ids.pop("count")
    assert count == len(nsa.KERNELS)
    assert {name: k for k, name in enumerate(nsa.KERNELS)} == ids


def test_status_strings(lib):
    for code, name in [(0, "MUON_OK"), (1, "MUON_ERR_INVALID_ARG"), (2, "MUON_ERR_UNSUPPORTED"),
                       (3, "MUON_ERR_WORKSPACE"), (4, "MUON_ERR_HIP")]:
        assert nsa.status_string(code) == name
    assert nsa.status_string(99) == "MUON_UNKNOWN_STATUS"


def expected_workspace(shapes, esize):
    """Workspace layout restated from the header's description of the buffers."""
    def up(x, a):
        return (x + a - 1) // a * a

    batch = len(shapes)
    desc = 112  # sizeof(MatDesc)
    total = up(desc * batch, 256) + up(4 * 7 * (batch + 1), 256)  # 7 phase prefix arrays
    total += up(4 * batch, 256)  # per-matrix 1 / (||U|| + eps)
    total += up(4 * 2 * 16, 256)  # two sets of 16 tile-claim counters
    # one partial sum of squares per momentum-pass tile of the padded wide
    # iterate: 32 x 256 for a wide matrix (rows <= cols), 256 x 64 for a tall one
    blocks = sum((up(r, 256) // 32) * (up(c, 256) // 256) if r <= c else
                 (up(c, 256) // 256) * (up(r, 256) // 64) for r, c in shapes)
    total += up(4 * blocks, 256)
    for r, c in shapes:
        s, l = min(r, c), max(r, c)
        sp, lp = up(s, 256), up(l, 256)
        total += 2 * up(sp * lp * esize, 256) + 2 * up(sp * sp * esize, 256)
    total += up(4 * 4 * 2048, 256)  # last, the claim-queue order table: 4 launch kinds x 2048
    return total


@pytest.mark.parametrize("dtype,esize", [(nsa.MUON_BF16, 2), (nsa.MUON_FP32, 4)])
def test_workspace_bytes(dtype, esize):
    for shapes in [[(256, 512)], [(2048, 6144)] * 3, [(257, 771), (771, 257), (1, 5)],
                   [(6144, 6144), (6144, 1024)], [(300, 200)] * 60 + [(2048, 6144)] * 3]:
        assert nsa.workspace_bytes(shapes, dtype) == expected_workspace(shapes, esize)
    assert nsa.workspace_bytes([], dtype) == 0


def test_workspace_bytes_invalid(lib):
    assert lib.muon_workspace_bytes(1, _i64_array([0]), _i64_array([5]), 0) == nsa._binding.SIZE_MAX
    assert "shape" in nsa.last_error_detail()
    assert lib.muon_workspace_bytes(1, _i64_array([5]), _i64_array([5]), 7) == nsa._binding.SIZE_MAX
    assert lib.muon_workspace_bytes(-1, None, None, 0) == nsa._binding.SIZE_MAX


def ns_call(lib, batch=1, rows=(64,), cols=(96,), x=(FAKE,), out=(FAKE + 4096,), dtype=0,
            steps=5, coeffs=(3.4445, -4.775, 2.0315), eps=1e-7, ws=FAKE + (1 << 20),
            ws_bytes=1 << 40, params=True, budget=0):
    p = NsParams(steps, *coeffs, eps, budget)
    return lib.muon_ns_batched(batch, _i64_array(rows) if rows is not None else None,
                               _i64_array(cols) if cols is not None else None,
                               _ptr_array(x) if x is not None else None,
                               _ptr_array(out) if out is not None else None, dtype,
                               ctypes.byref(p) if params else None, ctypes.c_void_p(ws),
                               ws_bytes, None)


def step_call(lib, w=FAKE, g=FAKE + 8192, m=FAKE + 16384, rows=(64,), cols=(96,), nesterov=0,
              lr=0.02, beta=0.95, ws=FAKE + (1 << 20), ws_bytes=1 << 40, steps=5, mhost=0):
    p = StepParams(lr, beta, nesterov, NsParams(steps, 3.4445, -4.775, 2.0315, 1e-7), mhost)
    return lib.muon_step_batched(1, _i64_array(rows), _i64_array(cols), _ptr_array([w]),
                                 _ptr_array([g]), _ptr_array([m]), 0, ctypes.byref(p),
                                 ctypes.c_void_p(ws), ws_bytes, None)


def test_ns_validation(lib):
    E = nsa
    assert ns_call(lib, batch=0, rows=None, cols=None, x=None, out=None) == E.MUON_OK
    assert ns_call(lib, batch=-1) == E.MUON_ERR_INVALID_ARG
    assert ns_call(lib, rows=None) == E.MUON_ERR_INVALID_ARG
    assert ns_call(lib, rows=(0,)) == E.MUON_ERR_INVALID_ARG
    assert ns_call(lib, cols=(-3,)) == E.MUON_ERR_INVALID_ARG
    assert ns_call(lib, rows=(E.MAX_DIM + 1,)) == E.MUON_ERR_UNSUPPORTED
    assert ns_call(lib, dtype=2) == E.MUON_ERR_INVALID_ARG
    assert ns_call(lib, steps=-1) == E.MUON_ERR_INVALID_ARG
    assert ns_call(lib, params=False) == E.MUON_ERR_INVALID_ARG
    assert ns_call(lib, coeffs=(float("nan"), 0.0, 0.0)) == E.MUON_ERR_INVALID_ARG
    assert ns_call(lib, eps=-1.0) == E.MUON_ERR_INVALID_ARG
    assert ns_call(lib, budget=-1) == E.MUON_ERR_INVALID_ARG
    assert ns_call(lib, x=None) == E.MUON_ERR_INVALID_ARG
    assert ns_call(lib, x=(0,)) == E.MUON_ERR_INVALID_ARG
    assert ns_call(lib, out=(FAKE + 2,)) == E.MUON_ERR_INVALID_ARG
    assert "aligned" in nsa.last_error_detail()
    assert ns_call(lib, ws=0) == E.MUON_ERR_WORKSPACE
    need = nsa.workspace_bytes([(64, 96)], 0)
    assert ns_call(lib, ws_bytes=need - 1) == E.MUON_ERR_WORKSPACE
    assert str(need) in nsa.last_error_detail()
    assert ns_call(lib, ws=FAKE + 128) == E.MUON_ERR_INVALID_ARG


def test_step_validation(lib):
    E = nsa
    assert step_call(lib, w=FAKE, g=FAKE) == E.MUON_ERR_INVALID_ARG  # aliasing
    assert step_call(lib, m=FAKE + 8192) == E.MUON_ERR_INVALID_ARG
    assert step_call(lib, nesterov=2) == E.MUON_ERR_INVALID_ARG
    assert step_call(lib, lr=float("inf")) == E.MUON_ERR_INVALID_ARG
    assert step_call(lib, steps=-2) == E.MUON_ERR_INVALID_ARG
    assert step_call(lib, g=0) == E.MUON_ERR_INVALID_ARG
    assert step_call(lib, ws_bytes=16) == E.MUON_ERR_WORKSPACE
    assert step_call(lib, mhost=2) == E.MUON_ERR_INVALID_ARG


def adamw_call(lib, batch=1, numel=(100,), p=(FAKE,), g=(FAKE + 4096,), m=(FAKE + 8192,),
               v=(FAKE + 12288,), dtype=0, lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1, step=1,
               ws=FAKE + (1 << 20), ws_bytes=1 << 40, params=True):
    prm = nsa.AdamWParams(lr, b1, b2, eps, wd, step)
    return lib.muon_adamw_batched(batch, _i64_array(numel) if numel is not None else None,
                                  _ptr_array(p) if p is not None else None,
                                  _ptr_array(g) if g is not None else None,
                                  _ptr_array(m) if m is not None else None,
                                  _ptr_array(v) if v is not None else None, dtype,
                                  ctypes.byref(prm) if params else None, ctypes.c_void_p(ws),
                                  ws_bytes, None)


def test_adamw_workspace_bytes(lib):
    def up(x, a):
        return (x + a - 1) // a * a
    for numels in [[1], [0, 5, 8192 * 4 + 1], [6144] * 223]:
        b = len(numels)
        assert nsa.adamw_workspace_bytes(numels) == up(40 * b, 256) + up(4 * (b + 1), 256)
    assert nsa.adamw_workspace_bytes([]) == 0
    assert lib.muon_adamw_workspace_bytes(1, _i64_array([-1])) == nsa._binding.SIZE_MAX
    assert "negative" in nsa.last_error_detail()


def test_adamw_validation(lib):
    E = nsa
    assert adamw_call(lib, batch=0, numel=None, p=None, g=None, m=None, v=None) == E.MUON_OK
    assert adamw_call(lib, batch=-1) == E.MUON_ERR_INVALID_ARG
    assert adamw_call(lib, numel=(-4,)) == E.MUON_ERR_INVALID_ARG
    assert adamw_call(lib, dtype=3) == E.MUON_ERR_INVALID_ARG
    assert adamw_call(lib, step=0) == E.MUON_ERR_INVALID_ARG
    assert adamw_call(lib, b1=1.0) == E.MUON_ERR_INVALID_ARG
    assert adamw_call(lib, b2=-0.1) == E.MUON_ERR_INVALID_ARG
    assert adamw_call(lib, eps=-1.0) == E.MUON_ERR_INVALID_ARG
    assert adamw_call(lib, lr=float("nan")) == E.MUON_ERR_INVALID_ARG
    assert adamw_call(lib, params=False) == E.MUON_ERR_INVALID_ARG
    assert adamw_call(lib, p=None) == E.MUON_ERR_INVALID_ARG
    assert adamw_call(lib, v=(0,)) == E.MUON_ERR_INVALID_ARG
    assert adamw_call(lib, m=(FAKE + 8,)) == E.MUON_ERR_INVALID_ARG
    assert "aligned" in nsa.last_error_detail()
    assert adamw_call(lib, g=(FAKE,)) == E.MUON_ERR_INVALID_ARG
    assert "distinct" in nsa.last_error_detail()
    assert adamw_call(lib, ws=0) == E.MUON_ERR_WORKSPACE
    assert adamw_call(lib, ws_bytes=8) == E.MUON_ERR_WORKSPACE
    assert adamw_call(lib, ws=FAKE + (1 << 20) + 16) == E.MUON_ERR_INVALID_ARG


def test_hbm_stream_validation(lib):
    """The measurement stream rejects bad counts, sizes and pointers before any
    launch; zero bytes is a no-op."""
    ins = _ptr_array([FAKE, FAKE + 16384])
    outs = _ptr_array([FAKE + 2 * 16384, FAKE + 3 * 16384])
    for n_in, n_out, nbytes, args in [(0, 1, 16384, (ins, outs)), (3, 1, 16384, (ins, outs)),
                                      (1, 0, 16384, (ins, outs)), (1, 3, 16384, (ins, outs)),
                                      (1, 1, 16000, (ins, outs)), (1, 1, 16384, (None, outs)),
                                      (1, 1, 16384, (_ptr_array([FAKE + 8]), outs)),
                                      (2, 2, 16384, (ins, _ptr_array([FAKE, 0])))]:
        st = lib.muon_hbm_stream(n_in, args[0], n_out, args[1], nbytes, 0, None)
        assert st == nsa.MUON_ERR_INVALID_ARG, (n_in, n_out, nbytes)
    assert lib.muon_hbm_stream(2, ins, 2, outs, 0, 1, None) == nsa.MUON_OK


def test_ns_noalloc_validation(lib):
    """The allocation-free call validates like muon_ns_batched, and refuses a batch
    whose workspace exceeds the library's array (MUON_NOALLOC_MAX_WORKSPACE)
    before any HIP call."""
    p = NsParams(5, 3.4445, -4.775, 2.0315, 1e-7, 0)
    ptrs = _ptr_array([FAKE])
    assert lib.muon_ns_batched_noalloc(0, None, None, None, None, 0, ctypes.byref(p), None) == \
        nsa.MUON_OK
    st = lib.muon_ns_batched_noalloc(1, _i64_array([64]), _i64_array([96]), None, ptrs, 0,
                                     ctypes.byref(p), None)
    assert st == nsa.MUON_ERR_INVALID_ARG
    st = lib.muon_ns_batched_noalloc(1, _i64_array([64]), _i64_array([96]), _ptr_array([FAKE + 8]),
                                     ptrs, 0, ctypes.byref(p), None)
    assert st == nsa.MUON_ERR_INVALID_ARG
    bad = NsParams(-1, 3.4445, -4.775, 2.0315, 1e-7, 0)
    st = lib.muon_ns_batched_noalloc(1, _i64_array([64]), _i64_array([96]), ptrs, ptrs, 0,
                                     ctypes.byref(bad), None)
    assert st == nsa.MUON_ERR_INVALID_ARG
    big = 8192  # bf16 workspace 2 * 8192^2 * 2 * 2 bytes = 512 MiB
    assert nsa.workspace_bytes([(big, big)], nsa.MUON_BF16) > nsa.NOALLOC_MAX_WORKSPACE
    st = lib.muon_ns_batched_noalloc(1, _i64_array([big]), _i64_array([big]), ptrs, ptrs, 0,
                                     ctypes.byref(p), None)
    assert st == nsa.MUON_ERR_WORKSPACE and "allocation-free" in nsa.last_error_detail()


def test_fp8_steps_validation(lib):
    """fp8_steps: bf16 only, fewer than steps, no CU budget; the workspace of such
    a call is muon_workspace_bytes_fp8() (two e4m3 buffers per matrix more)."""
    shapes = [(300, 700), (700, 300)]
    rows, cols = _i64_array([r for r, _ in shapes]), _i64_array([c for _, c in shapes])
    plain = nsa.workspace_bytes(shapes, nsa.MUON_BF16)
    fp8 = nsa.workspace_bytes(shapes, nsa.MUON_BF16, fp8=True)
    up = lambda x, a: -(-x // a) * a
    extra = 0
    for r, c in shapes:
        n = up(min(r, c), 256) * up(max(r, c), 256)
        extra += 2 * up(n + n // 32, 256)  # two e4m3 buffers: values, then a scale per 32
    assert fp8 == plain + extra
    ptrs = _ptr_array([FAKE, FAKE + (1 << 24)])
    for dtype, steps, f8, budget, ws in [(nsa.MUON_FP32, 5, 2, 0, fp8), (nsa.MUON_BF16, 5, 5, 0, fp8),
                                         (nsa.MUON_BF16, 5, -1, 0, fp8), (nsa.MUON_BF16, 5, 2, 8, fp8),
                                         (nsa.MUON_BF16, 0, 1, 0, fp8)]:
        p = NsParams(steps, 3.4445, -4.775, 2.0315, 1e-7, budget, f8)
        st = lib.muon_ns_batched(2, rows, cols, ptrs, ptrs, dtype, ctypes.byref(p),
                                 ctypes.c_void_p(FAKE), ws, None)
        assert st == nsa.MUON_ERR_INVALID_ARG, (dtype, steps, f8, budget)
    # a valid e4m3 call with the plain workspace size is refused as too small
    p = NsParams(5, 3.4445, -4.775, 2.0315, 1e-7, 0, 2)
    st = lib.muon_ns_batched(2, rows, cols, ptrs, ptrs, nsa.MUON_BF16, ctypes.byref(p),
                             ctypes.c_void_p(FAKE), plain, None)
    assert st == nsa.MUON_ERR_WORKSPACE


def test_workspace_bytes_ex(lib):
    """flags = 0 is the plain size; momentum in host memory adds the chunks' own
    tables and two staging slots of a chunk each (at most 16 chunks: at least a
    sixteenth of the momentum bytes, less than that plus one matrix);
    unknown flags, or e4m3 steps with fp32, are refused."""
    shapes = [(2048, 6144)] * 20 + [(300, 700), (700, 300)]
    rows, cols = _i64_array([r for r, _ in shapes]), _i64_array([c for _, c in shapes])
    plain = nsa.workspace_bytes(shapes, nsa.MUON_BF16)
    assert lib.muon_workspace_bytes_ex(len(shapes), rows, cols, nsa.MUON_BF16, 0) == plain
    host = nsa.workspace_bytes(shapes, nsa.MUON_BF16, momentum_host=True)
    mbytes = sum(2 * r * c for r, c in shapes)
    biggest = max(2 * r * c for r, c in shapes)
    # each chunk has its own tables (descriptors, prefixes, the 32 KiB order table)
    assert plain + 2 * mbytes // 16 <= host <= (plain + 2 * (mbytes // 16 + biggest)
                                                 + 16 * (4096 + 4 * 4 * 2048))
    both = nsa.workspace_bytes(shapes, nsa.MUON_BF16, fp8=True, momentum_host=True)
    assert both - host == nsa.workspace_bytes(shapes, nsa.MUON_BF16, fp8=True) - plain
    assert lib.muon_workspace_bytes_ex(len(shapes), rows, cols, nsa.MUON_BF16, 4) == ctypes.c_size_t(-1).value
    assert lib.muon_workspace_bytes_ex(len(shapes), rows, cols, nsa.MUON_FP32, 1) == ctypes.c_size_t(-1).value
    # a step with the momentum in host memory and the plain workspace is refused
    ptrs = _ptr_array([FAKE + (k << 26) for k in range(len(shapes))])
    gp = _ptr_array([FAKE + (1 << 40) + (k << 26) for k in range(len(shapes))])
    mp = _ptr_array([FAKE + (2 << 40) + (k << 26) for k in range(len(shapes))])
    p = StepParams(0.02, 0.95, 0, NsParams(5, 3.4445, -4.775, 2.0315, 1e-7), 1)
    st = lib.muon_step_batched(len(shapes), rows, cols, ptrs, gp, mp, nsa.MUON_BF16,
                               ctypes.byref(p), ctypes.c_void_p(FAKE), plain, None)
    assert st == nsa.MUON_ERR_WORKSPACE and "host memory" in nsa.last_error_detail()
