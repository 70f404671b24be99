"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/mx4.h, sizes and plans are what the layout says, and bad
arguments are rejected on the host before any HIP call (fake pointers are
never dereferenced because validation fails first)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

from microscaled_mxfp4_block_amd import binding as B
from microscaled_mxfp4_block_amd.inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mx4.h")

FAKE = 1 << 40          # an aligned, never-dereferenced address
FAKE_ODD = FAKE + 2      # misaligned for 16-byte loads


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int)\s+(mx_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = set(re.findall(r"\bT (mx_\w+)", out))
    assert set(names) <= exported
    assert set(B.EXPORTS) == set(names)


def test_strerror_codes():
    for c in (0, -1, -2, -3, -4, -5):
        assert B.strerror(c) and B.strerror(c) != "unknown error code"
    assert B.strerror(-99) == "unknown error code"


def size_of(N, K):
    out = ctypes.c_size_t()
    rc = B.lib().mx_packed_weight_bytes(N, K, ctypes.byref(out))
    return rc, out.value


@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name)
def test_packed_bytes_of_workloads_are_algorithmic(w):
    # every workload has N % 32 == 0 and K % 256 == 0: no padding at all,
    # exactly N*K/2 code bytes plus N*K/32 scale bytes
    rc, n = size_of(w.N, w.K)
    assert rc == 0
    assert n == w.N * w.K // 2 + w.N * w.K // 32


def test_packed_bytes_padding():
    # 33 rows -> 2 row blocks of 32; K=96 -> 2 K steps of 64, 1 scale word
    rc, n = size_of(33, 96)
    assert rc == 0 and n == 2 * 2 * 1024 + 2 * 1 * 256


@pytest.mark.parametrize("N,K", [(0, 64), (-1, 64), (16, 0), (16, 48), (16, 33), (1 << 25, 64)])
def test_packed_bytes_rejects_bad_shapes(N, K):
    assert size_of(N, K)[0] == B.MX_EINVAL


def test_pack_weight_validation():
    L = B.lib()
    nbytes = size_of(64, 512)[1]
    assert L.mx_pack_weight(FAKE, 64, 500, 512, FAKE, nbytes, None) == B.MX_EINVAL      # K % 32
    assert L.mx_pack_weight(FAKE, 64, 512, 256, FAKE, nbytes, None) == B.MX_EINVAL      # ldb < K
    assert L.mx_pack_weight(FAKE, 64, 512, 516, FAKE, nbytes, None) == B.MX_EINVAL      # ldb % 8
    assert L.mx_pack_weight(None, 64, 512, 512, FAKE, nbytes, None) == B.MX_EALIGN
    assert L.mx_pack_weight(FAKE_ODD, 64, 512, 512, FAKE, nbytes, None) == B.MX_EALIGN
    assert L.mx_pack_weight(FAKE, 64, 512, 512, FAKE, nbytes - 1, None) == B.MX_ESPACE


def test_import_weight_validation():
    L = B.lib()
    nbytes = size_of(64, 512)[1]
    assert L.mx_import_weight(FAKE, FAKE, 64, 500, FAKE, nbytes, None) == B.MX_EINVAL      # K % 32
    assert L.mx_import_weight(FAKE, FAKE, 0, 512, FAKE, nbytes, None) == B.MX_EINVAL
    assert L.mx_import_weight(FAKE_ODD, FAKE, 64, 512, FAKE, nbytes, None) == B.MX_EALIGN  # codes 16-B
    assert L.mx_import_weight(FAKE, None, 64, 512, FAKE, nbytes, None) == B.MX_EALIGN
    assert L.mx_import_weight(FAKE, FAKE + 1, 64, 512, FAKE_ODD, nbytes, None) == B.MX_EALIGN
    assert L.mx_import_weight(FAKE, FAKE + 1, 64, 512, FAKE, nbytes - 1, None) == B.MX_ESPACE
    with pytest.raises(ValueError):
        B.mx_import_weight(torch.zeros((64, 256), dtype=torch.uint8), torch.zeros((64, 15), dtype=torch.uint8),
                           64, 512)


def test_quant_act_validation():
    L = B.lib()
    assert L.mx_quant_act(FAKE, 0, 512, 512, FAKE, FAKE, None) == B.MX_EINVAL
    assert L.mx_quant_act(FAKE, 4, 520, 520, FAKE, FAKE, None) == B.MX_EINVAL
    assert L.mx_quant_act(FAKE, 4, 512, 504, FAKE, FAKE, None) == B.MX_EINVAL
    assert L.mx_quant_act(FAKE_ODD, 4, 512, 512, FAKE, FAKE, None) == B.MX_EALIGN
    assert L.mx_quant_act(FAKE, 4, 512, 512, None, FAKE, None) == B.MX_EALIGN
    assert L.mx_quant_act(FAKE, 4, 512, 512, FAKE, None, None) == B.MX_EALIGN


def test_gemm_validation():
    L = B.lib()
    M, N, K = 16, 2112, 7168
    ws = ctypes.c_size_t()
    assert L.mx_gemm_workspace_bytes(M, N, K, ctypes.byref(ws)) == 0
    args = dict(A=FAKE, M=M, K=K, lda=K, P=FAKE, N=N, C=FAKE, ldc=N, ws=FAKE, wsb=ws.value)

    def call(**kw):
        a = dict(args, **kw)
        return L.mx_gemm(a["A"], a["M"], a["K"], a["lda"], a["P"], a["N"], a["C"], a["ldc"], a["ws"], a["wsb"],
                         None)

    assert call(M=0) == B.MX_EINVAL
    assert call(N=-3) == B.MX_EINVAL
    assert call(K=7160) == B.MX_EINVAL
    assert call(lda=K - 8) == B.MX_EINVAL
    assert call(ldc=N - 4) == B.MX_EINVAL
    assert call(C=FAKE + 1) == B.MX_EALIGN
    assert call(A=None) == B.MX_EALIGN
    assert call(A=FAKE_ODD) == B.MX_EALIGN
    assert call(P=None) == B.MX_EALIGN
    assert call(C=None) == B.MX_EALIGN
    if ws.value > 0:
        assert call(ws=None) == B.MX_EALIGN
        assert call(wsb=ws.value - 1) == B.MX_ESPACE


def test_plans_for_workloads():
    for w in WORKLOADS:
        p = B.mx_gemm_plan(w.M, w.N, w.K)
        assert p["amode"] in (B.MX_AMODE_LDS, B.MX_AMODE_PREQUANT, B.MX_AMODE_DIRECT, B.MX_AMODE_SHARED)
        assert p["finish"] in (B.MX_FINISH_KERNEL, B.MX_FINISH_LAST_ARRIVAL)
        if p["amode"] == B.MX_AMODE_SHARED:
            # wn MFMA waves + wk quantiser waves
            assert (p["mb"], p["nb"], p["wn"], p["wk"]) in ((1, 1, 2, 2), (1, 1, 3, 4), (1, 1, 3, 8), (1, 1, 4, 4),
                                                            (1, 1, 4, 8), (1, 2, 2, 2), (1, 2, 4, 4))
        else:
            assert p["mb"] in (1, 2) and p["nb"] in (1, 2) and p["wn"] in (1, 2)
            assert p["wk"] in (1, 2, 4, 8, 16) and p["wn"] * p["wk"] <= 16
        assert p["splits"] >= 1
        ws = B.mx_gemm_workspace_bytes(w.M, w.N, w.K)
        if p["splits"] == 1 and p["amode"] != B.MX_AMODE_PREQUANT:
            assert ws == 0
        else:
            assert ws > 0


def test_measured_plans_are_accepted():
    """Every plan of the measured tables (both products, all shapes) passes
    the planner's register, LDS and grid checks."""
    from microscaled_mxfp4_block_amd.inputs import EXTRA_WORKLOADS
    for w in list(WORKLOADS) + list(EXTRA_WORKLOADS):
        for plan in (B.mx_gemm_plan(w.M, w.N, w.K), B.mx_gemm_a16w4_plan(w.M, w.N, w.K)):
            assert B.mx_gemm_workspace_bytes(w.M, w.N, w.K, plan) >= 0


def test_plan_model_for_other_shapes():
    for (M, N, K) in [(1, 32, 32), (5, 200, 320), (33, 1000, 4096), (300, 5000, 8192), (1024, 1024, 1024)]:
        p = B.mx_gemm_plan(M, N, K)
        assert p["splits"] >= 1
        assert B.mx_gemm_workspace_bytes(M, N, K, p) >= 0


def test_explicit_plan_rejections():
    bad = [dict(mb=3, nb=1, wn=1, wk=1, splits=1, amode=0),      # no such tile
           dict(mb=1, nb=1, wn=1, wk=3, splits=1, amode=1),      # no such wave count
           dict(mb=1, nb=1, wn=4, wk=8, splits=4, amode=0),      # no such wave count along N
           dict(mb=1, nb=1, wn=2, wk=16, splits=4, amode=2),     # more than 16 waves
           dict(mb=1, nb=1, wn=1, wk=4, splits=4, amode=5),      # no such activation mode
           dict(mb=2, nb=1, wn=1, wk=4, splits=1, amode=4),      # stream mode: one M block per workgroup
           dict(mb=1, nb=1, wn=2, wk=4, splits=1, amode=4),      # stream mode: one wave along N
           dict(mb=1, nb=4, wn=1, wk=16, splits=1, amode=4),     # stream mode: nb <= 2 at 16 waves
           dict(mb=1, nb=4, wn=1, wk=4, splits=1, amode=0),      # nb = 4 only in the stream mode
           dict(mb=1, nb=1, wn=1, wk=1, splits=1, amode=5),      # shared mode: no such wave split
           dict(mb=1, nb=1, wn=4, wk=4, splits=2, amode=5),      # shared mode: 56 K steps > 24 per split
           dict(mb=1, nb=1, wn=4, wk=4, splits=4, amode=5, finish=1),   # shared mode: no last-arrival finish
           dict(mb=1, nb=1, wn=1, wk=4, splits=4, amode=0, finish=2),   # no such split-K finish
           dict(mb=1, nb=1, wn=1, wk=4, splits=0, amode=1),
           dict(mb=1, nb=1, wn=1, wk=4, splits=1000, amode=1),   # more splits than K steps
           dict(mb=1, nb=1, wn=1, wk=8, splits=1, amode=1),      # 14 K steps per wave > register budget
           dict(mb=2, nb=1, wn=1, wk=16, splits=1, amode=0),     # activation slice over the 160 KiB LDS
           dict(mb=8, nb=8, wn=4, wk=2, splits=2, amode=6, finish=1),   # tile mode: reduce_kernel finish only
           dict(mb=8, nb=8, wn=2, wk=4, splits=1, amode=6),      # tile mode: no such wave split
           dict(mb=2, nb=1, wn=1, wk=8, splits=1, amode=6)]      # tile mode: no such tile
    for p in bad:
        with pytest.raises(B.MxError) as e:
            B.mx_gemm_workspace_bytes(16, 2112, 7168, p)
        assert e.value.code == B.MX_EPLAN


@pytest.mark.parametrize("shape,expect", [
    ((160, 3072, 1536), dict(amode=5, wn=3)),              # shared mode, one round of 5 x 32 workgroups
    ((288, 3072, 1536), dict(amode=5, wn=4)),              # four MFMA waves: 9 x 24 fits one round, 9 x 32 not
    ((320, 2880, 1536), dict(amode=5, wn=4)),              # a ragged last N tile when only that fits one round
    ((4, 672, 4096), dict(amode=2, wk=4, splits=8)),       # N of 21 blocks past K = 2048: split toward 256
    ((74, 544, 1024), dict(amode=2, wk=8, splits=1)),      # ... but not at K <= 2048
    ((4, 3456, 768), dict(amode=2, wk=4, splits=1)),       # four register waves at 12 K steps
    ((128, 2112, 4096), dict(amode=6, mb=2, nb=2)),        # the 64 x 64 tile past M = 64 at K > 2048
    ((64, 4096, 4096), dict(amode=2)),                     # ... not at M = 64
])
def test_model_rules_off_the_grid(shape, expect):
    """The model's rules between and beyond the grid's shapes (measured in
    graph replay against the candidate plans; host-only plan queries)."""
    plan = B.mx_gemm_plan(*shape)
    assert {k: plan[k] for k in expect} == expect, (shape, plan)


def test_random_regret_summary_from_synthetic_results(tmp_path, monkeypatch):
    """The off-grid regret summary renders from synthetic sweep results, for
    the default seed and another (its own file), without a GPU."""
    import bench
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    plan = dict(mb=1, nb=1, wn=1, wk=4, splits=1, amode=2, finish=0)
    res = [{"M": 4, "N": 672, "K": 4096, "plan": plan, "us": 5.0, "best_plan": plan, "best_us": 4.0, "regret": 1.25,
            "candidates": 3, "all": []}]
    bench.regret_summary(res, "`cmd`", random=True)
    bench.regret_summary(res, "`cmd`", random=True, seed=7)
    text = (tmp_path / "profiles" / "plan_regret_random.md").read_text()
    assert "seed 2024" in text and "geometric mean 1.250, worst 1.250" in text and "| 4 | 672 | 4096 |" in text
    assert "seed 7" in (tmp_path / "profiles" / "plan_regret_random_seed7.md").read_text()


def test_random_regret_shapes_are_seeded_and_in_range():
    import bench
    g1, g2 = bench.random_regret_groups(), bench.random_regret_groups()
    assert g1 == g2 and sum(len(ms) for _, ms in g1) >= 35
    for (N, K), ms in g1:
        assert 256 <= N <= 8192 and N % 32 == 0 and 256 <= K <= 8192 and K % 256 == 0
        assert all(1 <= m <= 1024 for m in ms)


def test_tile_splits_take_the_reduction_kernel():
    """The tile mode splits K at multiples of 4 steps, its partials summed by
    reduce_kernel; its plans with the last-arrival finish are refused."""
    plan = dict(mb=2, nb=2, wn=2, wk=2, splits=3, amode=6, finish=0)
    assert B.mx_gemm_workspace_bytes(130, 2112, 7168, plan) >= 3 * 130 * 2112 * 4
    with pytest.raises(B.MxError) as e:
        B.mx_gemm_workspace_bytes(130, 2112, 7168, dict(plan, finish=1))
    assert e.value.code == B.MX_EPLAN


def test_binding_without_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        B.lib()


def test_fast_call_extension_validates_without_gpu():
    ext = B.ext()
    # same validation path as the C entry points: no HIP call is reached
    assert ext.gemm(FAKE, 0, 512, 512, FAKE, 64, FAKE, 64, 0, 0, 0) == B.MX_EINVAL
    assert ext.gemm(FAKE, 4, 512, 512, None, 64, FAKE, 64, 0, 0, 0) == B.MX_EALIGN
    assert ext.gemm_with_plan(FAKE, 4, 512, 512, FAKE, 64, FAKE, 64, 0, 0, 3, 1, 1, 1, 1, 0, 0, 0) == B.MX_EPLAN
    assert ext.gemm_with_plan(FAKE, 4, 512, 512, FAKE, 64, FAKE, 64, 0, 0, 1, 1, 1, 1, 2, 0, 5, 0) == B.MX_EPLAN
    with pytest.raises(TypeError):
        ext.gemm(1, 2, 3)
    with pytest.raises(OverflowError):
        ext.gemm(FAKE, 1 << 40, 512, 512, FAKE, 64, FAKE, 64, 0, 0, 0)


def test_workspace_layout_reserves_counters():
    """A non-empty workspace always starts with the 16 KiB counter block, so
    that shapes sharing one workspace never overlap a counter."""
    p = dict(mb=1, nb=1, wn=1, wk=4, splits=1, amode=B.MX_AMODE_LDS, finish=0)
    assert B.mx_gemm_workspace_bytes(32, 4096, 512, p) == 0
    pre = dict(p, amode=B.MX_AMODE_PREQUANT)
    codes = 32 * 512 // 2 + 32 * 512 // 32
    assert B.mx_gemm_workspace_bytes(32, 4096, 512, pre) == 16384 + (codes + 255) // 256 * 256
    split = dict(p, splits=2, finish=1)
    assert B.mx_gemm_workspace_bytes(32, 4096, 512, split) == 16384 + 2 * 32 * 4096 * 4
    # more output tiles than counters: only the reduction kernel can finish
    big = dict(p, splits=2, finish=1)
    with pytest.raises(B.MxError) as e:
        B.mx_gemm_workspace_bytes(32 * 65, 32 * 64, 512, big)
    assert e.value.code == B.MX_EPLAN
    assert B.mx_gemm_workspace_bytes(32 * 65, 32 * 64, 512, dict(big, finish=0)) > 0


def test_planner_rejects_every_spilling_kernel():
    """Every kernel instantiation whose gfx950 code spills VGPRs (read from the
    build's device assembly) is refused by the planner, so no accepted plan
    runs one."""
    import glob
    build = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "_build")
    asms = glob.glob(os.path.join(build, "mx4_gemm_kr*.s"))
    if not asms:
        pytest.skip("no device assembly under _build (run the package build first)")
    checked = 0
    for path in asms:
        kr = int(re.search(r"kr(\d+)\.s$", path).group(1))
        text = open(path).read()
        for block in text.split("  - .agpr_count:")[1:]:
            name = re.search(r"\.name:\s+(\S+)", block).group(1)
            spills = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", block).group(1))
            m = re.match(r"_ZN3mx411gemm_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", name)
            if not m:
                continue
            mb, nb, wn, wk, am, kr_t = map(int, m.groups())
            assert kr_t == kr
            plan = dict(mb=mb, nb=nb, wn=wn, wk=wk, splits=1, amode=am, finish=0)
            # a shape whose single split gives each wave exactly KR steps
            M, N, K = 32 * mb, 32 * nb * wn, 64 * kr * wk
            try:
                B.mx_gemm_workspace_bytes(M, N, K, plan)
                accepted = True
            except B.MxError as e:
                assert e.code == B.MX_EPLAN
                accepted = False
            if spills:
                assert not accepted, "planner accepts spilling kernel %s" % (plan,)
            checked += 1
    assert checked > 100


def test_gemm_kernels_take_preloaded_arguments():
    """Every GEMM kernel's descriptor asks for its 14 leading argument SGPRs
    (pointers and shape) to be preloaded at wave launch, and its whole
    argument segment is the 72 bytes of its thirteen scalars (no parameter
    block, no hidden arguments); the reduction kernel's is the 48 bytes of
    its ten scalars, all preloaded."""
    import glob
    build = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "_build")
    asms = glob.glob(os.path.join(build, "mx4_gemm_kr*.s"))
    if not asms:
        pytest.skip("no device assembly under _build (run the package build first)")
    seen = 0
    for path in asms:
        text = open(path).read()
        for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
            name, body = m.group(1), m.group(2)
            n = int(re.search(r"\.amdhsa_user_sgpr_kernarg_preload_length (\d+)", body).group(1))
            if "gemm_kernel" in name:
                assert n == 14, (name, n)
                size = int(re.search(r"\.amdhsa_kernarg_size (\d+)", body).group(1))
                assert size == 72, (name, size)
                seen += 1
            elif "reduce_kernel" in name:
                size = int(re.search(r"\.amdhsa_kernarg_size (\d+)", body).group(1))
                assert (n, size) == (12, 48), (name, n, size)
    assert seen > 100


def test_quantiser_kernels_have_no_hidden_arguments():
    """The quantisation kernels (the per-call activation quantisers among
    them) read no blockDim or gridDim, so their argument segments hold only
    their own scalars (at most 64 bytes), with no hidden-argument block."""
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "_build", "mx4_quant.s")
    if not os.path.exists(path):
        pytest.skip("no device assembly under _build (run the package build first)")
    text = open(path).read()
    seen = 0
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
        size = int(re.search(r"\.amdhsa_kernarg_size (\d+)", m.group(2)).group(1))
        assert size <= 64, (m.group(1), size)
        seen += 1
    assert seen == 4


def test_lds_dma_tiles_are_read_only_after_their_loads_land():
    """In every GEMM kernel that loads activation tiles straight into LDS, no
    LDS read and no vector store comes after the last such load before a
    vmcnt wait that covers it: a wait whose count is at most the number of
    vector loads issued after that last tile load.  Vector-memory operations
    of one wave complete in issue order, so such a wait implies that every
    tile has landed (a wait with a larger count, for loads issued before the
    tiles, does not)."""
    import glob
    build = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "_build")
    asms = glob.glob(os.path.join(build, "mx4_gemm_kr*.s"))
    if not asms:
        pytest.skip("no device assembly under _build (run the package build first)")
    vmem_load = re.compile(r"^\s*(buffer|global|flat|scratch)_load\w*")
    vmem_store = re.compile(r"^\s*(buffer|global|flat|scratch)_(store|atomic)\w*")
    checked = 0
    for path in asms:
        text = open(path).read()
        for m in re.finditer(r"^(_ZN3mx411gemm_kernel\S*):.*?s_endpgm", text, re.S | re.M):
            body = m.group(0).splitlines()
            dma = [k for k, ln in enumerate(body) if vmem_load.match(ln) and ln.rstrip().endswith(" lds")]
            if not dma:
                continue
            loads = 0
            for ln in body[dma[-1] + 1:]:
                assert not vmem_store.match(ln), (m.group(1), ln)
                assert not ln.strip().startswith("ds_read"), (m.group(1), "LDS read before the tiles landed")
                w = re.search(r"s_waitcnt\s.*vmcnt\((\d+)\)", ln)
                if w and int(w.group(1)) <= loads:
                    break
                if vmem_load.match(ln):
                    assert not ln.rstrip().endswith(" lds")
                    loads += 1
            else:
                raise AssertionError("%s: no vmcnt wait covers its LDS loads" % m.group(1))
            checked += 1
    assert checked > 50


def test_shared_kernels_keep_weight_loads_in_flight_across_barriers():
    """In every shared-mode kernel: the barrier between the quantiser waves'
    loads to LDS and the MFMA waves' weight loads waits for no vector memory
    (no vmcnt wait between the last load to LDS and it); the first LDS read
    of the quantisers comes after a vmcnt wait that covers their first step
    and no more (rq (KL - 1) loads left outstanding for rq = 4, 2 or 1 loaded
    row chunks per step, KL = KR / QW steps per wave); and the slice barrier after the quantisation
    waits only for LDS (it is preceded by `s_waitcnt lgkmcnt(0)` alone), so
    the weight loads stay in flight across it."""
    build = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "_build")
    path = os.path.join(build, "mx4_shared.s")
    if not os.path.exists(path):
        pytest.skip("no device assembly under _build (run the package build first)")
    text = open(path).read()
    checked = 0
    for m in re.finditer(r"^(_ZN3mx418gemm_shared_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E\S*):.*?^\.Lfunc_end",
                         text, re.S | re.M):
        name = m.group(1)
        QW, KR = int(m.group(4)), int(m.group(5))
        KL = KR // QW
        body = [ln for ln in m.group(0).splitlines() if not ln.strip().startswith(";")]
        dma = [k for k, ln in enumerate(body)
               if re.match(r"^\s*buffer_load_dwordx4\b", ln) and ln.rstrip().endswith(" lds")]
        bars = [k for k, ln in enumerate(body) if ln.strip() == "s_barrier"]
        assert len(dma) == (4 + 2 + 1) * KL and bars, name   # the 4-, 2- and 1-chunk copies
        b1 = next(k for k in bars if k > dma[-1])
        assert not any("vmcnt" in ln for ln in body[dma[-1]:b1]), (name, "vmcnt wait before the first barrier")
        r1 = next(k for k in range(b1, len(body)) if body[k].strip().startswith("ds_read"))
        waits = [int(w.group(1)) for ln in body[b1:r1] for w in [re.search(r"vmcnt\((\d+)\)", ln)] if w]
        assert waits and max(waits) <= 4 * (KL - 1), (name, waits)
        # the waits for the first step under each count of loaded row chunks
        # (rq loads per step): rq (KL - 1) loads of the later steps left
        # outstanding, and none of them waits for all the loads
        allw = {int(w) for w in re.findall(r"vmcnt\((\d+)\)", "\n".join(body[b1:]))}
        assert {rq * (KL - 1) for rq in (1, 2, 4)} <= allw, (name, sorted(allw))
        b2 = next(k for k in bars if k > r1)
        assert body[b2 - 1].strip() == "s_waitcnt lgkmcnt(0)", (name, body[b2 - 1])
        checked += 1
    assert checked == 19, checked


def test_tile_kernels_keep_their_ring_of_loads_in_flight():
    """In every tile-mode kernel (MB x NB blocks, WM x WN waves, S ring
    stages, one barrier per G K steps; LPW = (MB + NB) / (WM WN) blocks
    loaded per wave and step, plus one scale word load per block every 4
    steps): before the first barrier the kernel waits only for step 0, with
    the tiles of steps 1 .. S - G and their word groups still in flight, and
    each barrier of the K loop waits only for the steps up to t + G, leaving
    steps t + G + 1 .. t + S - G in flight: for the loop position u = t mod 4,
    LPW (S - 2G) tile loads plus LPW per word group starting in that range.
    Every barrier waits for the wave's own LDS reads first, and only the
    epilogue waits for every load."""
    build = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "_build")
    path = os.path.join(build, "mx4_tile.s")
    if not os.path.exists(path):
        pytest.skip("no device assembly under _build (run the package build first)")
    text = open(path).read()

    def starts(lo, hi):   # word groups (first step a multiple of 4) among steps lo .. hi
        return sum(1 for x in range(lo, hi + 1) if x % 4 == 0)
    checked = 0
    pat = r"^(_ZN3mx416gemm_tile_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E\S*):.*?^\.Lfunc_end"
    for m in re.finditer(pat, text, re.S | re.M):
        name = m.group(1)
        MB, NB, WM, WN, S, G = (int(m.group(k)) for k in range(2, 8))
        lpw = (MB + NB) // (WM * WN)
        body = [ln.strip() for ln in m.group(0).splitlines() if not ln.strip().startswith(";")]
        bars = [k for k, ln in enumerate(body) if ln == "s_barrier"]
        assert len(bars) >= 3, name
        for k in bars:
            assert body[k - 1] == "s_waitcnt lgkmcnt(0)", (name, body[k - 1])
        waits = [(k, int(w.group(1))) for k, ln in enumerate(body) for w in [re.search(r"vmcnt\((\d+)\)", ln)] if w]
        first = [v for k, v in waits if k < bars[0]]
        assert first == [lpw * (S - G) + lpw * starts(1, S - G)], (name, first)
        inner = [(k, v) for k, v in waits if bars[0] < k < bars[-1]]
        assert inner and inner[-1][1] == 0, name            # the epilogue's wait for every load
        loop = {v for k, v in inner[:-1]}
        expected = {lpw * (S - 2 * G) + lpw * starts(u + G + 1, u + S - G) for u in range(0, 4, G)}
        assert loop == expected, (name, sorted(loop), sorted(expected))
        assert not [v for k, v in waits if k > bars[-1]], name
        checked += 1
    assert checked == 7, checked


def test_shapes_past_the_addressing_limit_are_refused():
    """rows * K * 2 >= 2^31 for an operand (32-bit buffer offsets) is refused
    before any launch; just below it is accepted."""
    with pytest.raises(B.MxError) as e:
        B.mx_gemm_workspace_bytes(1, 32768, 32768)
    assert e.value.code == B.MX_EINVAL
    assert B.mx_gemm_workspace_bytes(64, 32768, 32736) > 0


def test_bench_algorithmic_bytes_of_the_workloads():
    """The roofline numerator of bench.py: A bf16 in + packed B (e2m1 codes
    and e8m0 scales) + C bf16 out per call, counted by hand from the five
    shapes (2MK + NK/2 + NK/32 + 2MN)."""
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("mx4_bench", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    expected = {(4, 2880, 512): 4096 + 737280 + 46080 + 23040,
                (32, 4096, 512): 32768 + 1048576 + 65536 + 262144,
                (16, 2112, 7168): 229376 + 7569408 + 473088 + 67584,
                (64, 7168, 2048): 262144 + 7340032 + 458752 + 917504,
                (256, 3072, 1536): 786432 + 2359296 + 147456 + 1572864}
    assert [bench.algorithmic_bytes(w.M, w.N, w.K) for w in WORKLOADS] == \
        [expected[(w.M, w.N, w.K)] for w in WORKLOADS]
    assert sorted(expected.values()) == sorted([810496, 1409024, 8339456, 8978432, 4866048])


def test_bench_names_every_function_it_calls():
    """Every plain name that bench.py calls resolves to a module-level
    definition, an import or a builtin: the offline subcommands
    (--summarize, --stats-md, --regret-merge) run without a GPU and are
    otherwise exercised only when profiles are rewritten."""
    import ast
    import builtins
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    tree = ast.parse(open(os.path.join(root, "bench.py")).read())
    defined = set(dir(builtins))
    for node in ast.walk(tree):
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            defined.add(node.name)
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            defined.update((a.asname or a.name).split(".")[0] for a in node.names)
        elif isinstance(node, ast.Name) and isinstance(node.ctx, ast.Store):
            defined.add(node.id)
        elif isinstance(node, ast.arg):
            defined.add(node.arg)
    called = {n.func.id for n in ast.walk(tree) if isinstance(n, ast.Call) and isinstance(n.func, ast.Name)}
    assert called - defined == set(), sorted(called - defined)
    assert {"stats_markdown", "regret_summary", "summarize_profiles", "plan_regret"} <= defined


def test_split_k_partials_complete_before_arrival():
    """In every GEMM kernel, the last-arrival split-K finish counts a
    workgroup's arrival (the agent-scope atomic add on the tile counter) only
    after a full vmcnt(0) wait that follows the wave's last agent-scope
    (sc1) partial store: a workgroup barrier does not wait for vector
    memory, so without that wait the last workgroup could sum partials that
    have not landed."""
    import glob
    build = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "_build")
    asms = glob.glob(os.path.join(build, "mx4_gemm_kr*.s"))
    if not asms:
        pytest.skip("no device assembly under _build (run the package build first)")
    checked = 0
    for path in asms:
        text = open(path).read()
        for m in re.finditer(r"^(_ZN3mx411gemm_kernel\S*):.*?s_endpgm", text, re.S | re.M):
            body = m.group(0).splitlines()
            atomics = [k for k, ln in enumerate(body) if re.match(r"^\s*global_atomic_add\b", ln)]
            if not atomics:
                continue
            stores = [k for k, ln in enumerate(body[:atomics[0]])
                      if re.match(r"^\s*global_store\w*\s.*\bsc1\b", ln)]
            assert stores, (m.group(1), "no agent-scope partial store before the arrival atomic")
            between = body[stores[-1] + 1:atomics[0]]
            assert any(re.search(r"s_waitcnt\s.*vmcnt\(0\)", ln) for ln in between), \
                (m.group(1), "arrival counted before the partial stores completed")
            checked += 1
    assert checked > 50


def test_hwcheck_library_exports_its_header():
    """libmx4hw.so (the tests' hardware checks) exports every function that
    include/mx4_hwcheck.h declares, and libmx4.so exports none of them."""
    hdr = open(os.path.join(ROOT, "include", "mx4_hwcheck.h")).read()
    names = sorted(set(re.findall(r"^\s*int\s+(mxhw_\w+)\s*\(", hdr, re.M)))
    assert len(names) == 5
    hwlib = os.path.join(ROOT, "microscaled_mxfp4_block_amd", "libmx4hw.so")
    out = subprocess.run(["nm", "-D", "--defined-only", hwlib], stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, re.M))
    assert set(names) <= exported
    main = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], stdout=subprocess.PIPE, text=True,
                          check=True).stdout
    assert "mxhw_" not in main


def xcd_fetch_cost(mt, nt, K, cols):
    """Bytes the 8 XCDs' L2s fetch when workgroup lin runs on XCD lin % 8:
    per XCD, its distinct M tiles' bf16 activation rows (32 x K x 2 bytes)
    and its distinct N tiles' packed weight (cols x (K/2 + K/32))."""
    lin = np.arange(mt.size)
    cost = 0.0
    for x in range(8):
        sel = lin % 8 == x
        cost += np.unique(mt[sel]).size * 64.0 * K + np.unique(nt[sel]).size * cols * (K / 2 + K / 32)
    return cost


def test_shared_xcd_map_places_every_tile_once_and_fetches_no_more():
    """The GEMM's placement of tiles on the XCDs (library code, through
    libmx4hw.so's host-only hook), as the shared mode uses it (all
    workgroups resident at once): every (M tile, N tile) goes to exactly one
    workgroup for every grid, the dispatcher's order is kept where no
    rectangle fits, the chosen placement never makes the XCDs fetch more
    than the dispatcher's order would, and 256 x 3072 x 1536 (8 x 32 tiles of
    96 columns) gets 4 M tiles x 8 N tiles per XCD."""
    place = xcd_placer()
    remapped = 0
    for mtiles in (1, 2, 3, 4, 5, 6, 8, 12, 16, 32):
        for ntiles in range(1, 66):
            for K, cols in ((1536, 96), (512, 128), (7168, 64)):
                mp, mt, nt = place(mtiles, ntiles, 1, 64.0 * K, cols * (K / 2 + K / 32), 0)
                T = mtiles * ntiles
                assert mt.min() >= 0 and mt.max() < mtiles and nt.min() >= 0 and nt.max() < ntiles
                assert np.unique(mt.astype(np.int64) * ntiles + nt).size == T, (mtiles, ntiles, mp)
                lin = np.arange(T)
                d_mt, d_nt = lin // ntiles, lin % ntiles
                if mp == 0:
                    assert np.array_equal(mt, d_mt) and np.array_equal(nt, d_nt)
                else:
                    remapped += 1
                    assert T % 8 == 0
                    assert xcd_fetch_cost(mt, nt, K, cols) <= xcd_fetch_cost(d_mt, d_nt, K, cols) + 1e-6
    assert remapped > 100
    mp, mt, nt = place(8, 32, 1, 64.0 * 1536, 96 * (1536 / 2 + 1536 / 32), 0)
    for x in range(8):
        sel = np.arange(256) % 8 == x
        assert np.unique(mt[sel]).size == 4 and np.unique(nt[sel]).size == 8
    assert place(8, 32, 2, 64.0 * 1536, 96 * 816.0, 0)[0] == 0       # K splits keep the dispatcher's order
    assert placement_hook().mxhw_xcd_map(0, 32, 1, 1.0, 1.0, 0, 0, None, None, None) == -1
    assert placement_hook().mxhw_xcd_map(8, 32, 1, 1.0, 1.0, 0, 3, None, None, None) == -1


def placement_hook():
    """libmx4hw.so with the argument types of its host-only placement hook."""
    hw = ctypes.CDLL(os.path.join(ROOT, "microscaled_mxfp4_block_amd", "libmx4hw.so"))
    I, P, D = ctypes.c_int, ctypes.c_void_p, ctypes.c_double
    hw.mxhw_xcd_map.argtypes = [I, I, I, D, D, I, I, P, P, P]
    return hw


def xcd_placer():
    hw = placement_hook()

    def place(mtiles, ntiles, splits, a_bytes, b_bytes, conc, runs=0):
        T = mtiles * ntiles
        mt, nt, mp = (ctypes.c_int * T)(), (ctypes.c_int * T)(), ctypes.c_int(-1)
        assert hw.mxhw_xcd_map(mtiles, ntiles, splits, a_bytes, b_bytes, conc, runs, ctypes.byref(mp), mt, nt) == 0
        return mp.value, np.frombuffer(mt, np.int32).copy(), np.frombuffer(nt, np.int32).copy()
    return place


def round_fetch_cost(mt, nt, a_bytes, b_bytes, conc):
    """Bytes the XCDs' L2s fetch when each XCD runs its workgroups (linear id
    x mod 8) in dispatch order, conc at a time: per round, its distinct M
    tiles times a_bytes plus its distinct N tiles times b_bytes."""
    lin = np.arange(mt.size)
    cost = 0.0
    for x in range(8):
        idx = lin[lin % 8 == x]
        for r in range(0, idx.size, conc):
            sel = idx[r:r + conc]
            cost += np.unique(mt[sel]).size * a_bytes + np.unique(nt[sel]).size * b_bytes
    return cost


def test_tile_xcd_map_scores_rounds_when_an_xcd_runs_its_tiles_in_turn():
    """The rectangles of the tile mode's placement (at most 32 workgroups of
    an XCD at once; the runs left out):
    every tile goes to exactly one workgroup, and where the grid runs in
    several rounds per XCD the chosen rectangle fetches, round by round as
    the dispatcher runs them, no more than the rectangle chosen for an
    all-resident grid; at 8192^3 (32 x 32 tiles of 256 x 256, equal bytes)
    each XCD takes 8 M tiles x 16 N tiles, so each round covers 8 x 4."""
    place = xcd_placer()
    checked = 0
    for mtiles in (4, 8, 16, 32, 64):
        for ntiles in (8, 16, 24, 28, 32, 56, 64):
            for a_bytes, b_bytes in ((1.0, 1.0), (2.0, 1.0), (1.0, 2.0)):
                mp, mt, nt = place(mtiles, ntiles, 1, a_bytes, b_bytes, 32)
                T = mtiles * ntiles
                assert np.unique(mt.astype(np.int64) * ntiles + nt).size == T, (mtiles, ntiles, mp)
                if T <= 8 * 32:
                    continue
                mp0, mt0, nt0 = place(mtiles, ntiles, 1, a_bytes, b_bytes, 0)
                assert round_fetch_cost(mt, nt, a_bytes, b_bytes, 32) <= \
                    round_fetch_cost(mt0, nt0, a_bytes, b_bytes, 32) + 1e-9, (mtiles, ntiles, a_bytes, b_bytes)
                checked += 1
    assert checked > 30
    mp, mt, nt = place(32, 32, 1, 1.0, 1.0, 32)
    for x in range(8):
        sel = np.arange(1024) % 8 == x
        assert np.unique(mt[sel]).size == 8 and np.unique(nt[sel]).size == 16
        first = np.arange(1024)[sel][:32]
        assert np.unique(mt[first]).size == 8 and np.unique(nt[first]).size == 4
    assert round_fetch_cost(mt, nt, 1.0, 1.0, 32) < round_fetch_cost(*place(32, 32, 1, 1.0, 1.0, 0)[1:], 1.0, 1.0, 32)


def test_tile_xcd_runs_cover_every_grid_and_fetch_no_more():
    """The tile mode's placement with the runs among the candidates: for
    every grid (tile counts not a multiple of 8 included) each tile goes to
    exactly one workgroup; where the runs are chosen (code 128), XCD x's
    workgroups, in dispatch order, take consecutive tiles t = nt * mtiles + mt
    from x * q + min(x, r) on (q, r = tiles / 8, tiles mod 8); the fetches,
    round by round as the dispatcher runs them, are never above those of the
    placement without the runs; and 512 x 2112 (8 x 33 tiles of 64 x 64, all
    resident) takes runs that touch at most 8 M and 5 N tiles per XCD instead
    of 1 x 33."""
    place = xcd_placer()
    chosen = 0
    for mtiles in (1, 2, 3, 4, 5, 8, 12, 16, 32):
        for ntiles in range(1, 71):
            for conc in (0, 32, 64, 128):
                for a_bytes, b_bytes in ((1.0, 1.0), (2.0, 1.0), (1.0, 2.0)):
                    T = mtiles * ntiles
                    mp, mt, nt = place(mtiles, ntiles, 1, a_bytes, b_bytes, conc, 1)
                    assert mt.min() >= 0 and mt.max() < mtiles and nt.min() >= 0 and nt.max() < ntiles
                    assert np.unique(mt.astype(np.int64) * ntiles + nt).size == T, (mtiles, ntiles, mp)
                    if mp != 128:
                        continue
                    chosen += 1
                    q, r = T // 8, T % 8
                    lin = np.arange(T)
                    for x in range(8):
                        t = (nt * mtiles + mt)[lin % 8 == x]
                        start = x * q + min(x, r)
                        assert np.array_equal(t, np.arange(start, start + t.size)), (mtiles, ntiles, x)
                    rounds = conc if conc else T
                    mp0, mt0, nt0 = place(mtiles, ntiles, 1, a_bytes, b_bytes, conc, 0)
                    assert round_fetch_cost(mt, nt, a_bytes, b_bytes, rounds) <= \
                        round_fetch_cost(mt0, nt0, a_bytes, b_bytes, rounds) + 1e-9, (mtiles, ntiles, conc, mp0)
    assert chosen > 500
    mp, mt, nt = place(8, 33, 1, 1.0, 1.0, 128, 1)
    assert mp == 128
    for x in range(8):
        sel = np.arange(264) % 8 == x
        assert np.unique(mt[sel]).size == 8 and np.unique(nt[sel]).size <= 5
    assert place(8, 33, 1, 1.0, 1.0, 128, 0)[0] == 1 + 16 * 3      # 1 x 33 per XCD without the runs
    # runs only in place of a rectangle (2): 8 x 33 takes them, 4 x 33 (no rectangle) keeps the dispatcher's order
    assert place(8, 33, 1, 1.0, 1.0, 128, 2)[0] == 128
    assert place(4, 33, 1, 1.0, 1.0, 128, 1)[0] == 128 and place(4, 33, 1, 1.0, 1.0, 128, 2)[0] == 0


def test_noalloc_validates_before_any_hip_call():
    """mx_gemm_noalloc rejects a bad shape (MX_EINVAL) and a shape whose
    workspace exceeds its static array (MX_ESPACE: 4096^3 pre-quantises an
    8.4 MB activation) on the host, with fake pointers, before any HIP call;
    the workloads' workspaces fit."""
    L = B.lib()
    assert B.mx_gemm_workspace_bytes(4096, 4096, 4096) > B.MX_NOALLOC_SCRATCH_BYTES
    assert L.mx_gemm_noalloc(FAKE, 4096, 4096, 4096, FAKE, 4096, FAKE, 4096, None) == B.MX_ESPACE
    assert L.mx_gemm_noalloc(FAKE, 4, 33, 40, FAKE, 64, FAKE, 64, None) == B.MX_EINVAL
    for w in WORKLOADS:
        assert B.mx_gemm_workspace_bytes(w.M, w.N, w.K) <= B.MX_NOALLOC_SCRATCH_BYTES
    hdr = open(HEADER).read()
    assert "#define MX_NOALLOC_SCRATCH_BYTES (8u << 20)" in hdr and B.MX_NOALLOC_SCRATCH_BYTES == 8 << 20


@pytest.mark.parametrize("src,kname,count", [("mx4_stream.s", "gemm_stream_kernel", 42),
                                              ("mx4_shared.s", "gemm_shared_kernel", 19),
                                              ("mx4_tile.s", "gemm_tile_kernel", 7)])
def test_mode_kernels_preload_arguments_and_never_spill(src, kname, count):
    """The K-looped stream-mode kernels, the quantiser-wave shared-mode
    kernels and the LDS-tiled tile-mode kernels take the GEMM kernels'
    72-byte scalar argument segment with its
    14 leading SGPRs preloaded, and none spills VGPRs or uses scratch
    memory."""
    path = os.path.join(ROOT, "_build", src)
    if not os.path.exists(path):
        pytest.skip("no device assembly under _build (run the package build first)")
    text = open(path).read()
    seen = 0
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
        name, body = m.group(1), m.group(2)
        if kname not in name:
            continue
        assert int(re.search(r"\.amdhsa_user_sgpr_kernarg_preload_length (\d+)", body).group(1)) == 14, name
        assert int(re.search(r"\.amdhsa_kernarg_size (\d+)", body).group(1)) == 72, name
        assert int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body).group(1)) == 0, name
        seen += 1
    assert seen == count
    for block in text.split("  - .agpr_count:")[1:]:
        if kname in re.search(r"\.name:\s+(\S+)", block).group(1):
            assert int(re.search(r"\.vgpr_spill_count:\s+(\d+)", block).group(1)) == 0


def test_headers_are_plain_c():
    """include/*.h compile as C (gcc -std=c99 -Wall -Werror), on their own."""
    for h in ("mx4.h", "mx4_hwcheck.h"):
        r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c",
                            os.path.join(ROOT, "include", h)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                           text=True)
        assert r.returncode == 0, r.stdout


def test_library_under_test_is_the_one_named():
    """The binding loads MX4_LIBRARY when it is set (the sanitizer run), else
    the library built next to the package."""
    want = os.environ.get("MX4_LIBRARY") or os.path.join(ROOT, "microscaled_mxfp4_block_amd", "libmx4.so")
    assert B.LIB_PATH == want


def test_library_plans_are_accepted_for_random_shapes():
    """For 3000 seeded random shapes (M up to 600, N up to 3000, K up to
    9600) and the pages' shape grid, the plan each product picks passes the
    planner's own checks (a plan the model picks must never be refused)."""
    import random
    rnd = random.Random(7)
    shapes = [(rnd.randint(1, 600), rnd.randint(1, 3000), 32 * rnd.randint(1, 300)) for _ in range(3000)]
    import importlib.util
    spec = importlib.util.spec_from_file_location("mx4_bench", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    shapes += [(M, N, K) for (N, K) in bench.GRID_DIM_PAIRS for M in bench.GRID_BATCH]
    for M, N, K in shapes:
        assert B.mx_gemm_workspace_bytes(M, N, K) >= 0
        assert B.mx_gemm_a16w4_workspace_bytes(M, N, K) >= 0


def test_bench_large_m_summary_from_synthetic_rocprof_output(tmp_path):
    """bench.py --summarize-large-m on hand-made rocprofv3 CSVs: the
    calibration copy sets the counter scales (FETCH_SIZE reads half the
    copied bytes, WRITE_SIZE all of them), each shape's segment drops its
    weight pack and ends at the reference dispatch, and the GEMM kernel's
    fp4 rate and byte ratio follow from the traced durations by hand."""
    import csv
    import importlib.util
    import json as _json
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("mx4_bench_lm", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    shapes = bench.LARGE_M_SHAPES
    calls = 3
    copy_kib = (256 << 20) // 1024

    def dispatches():
        d = [("copy_kernel", 1, 50.0, {"FETCH_SIZE": copy_kib // 2, "WRITE_SIZE": copy_kib})]
        for si, (M, N, K) in enumerate(shapes):
            d.append(("mx4::pack_kernel(a)", 999, 7.0, {"FETCH_SIZE": 1, "WRITE_SIZE": 1}))
            for c in range(calls):
                d.append(("mx4::pack_kernel(b)", 4096, 2.0 + si, {"FETCH_SIZE": 100, "WRITE_SIZE": 50}))
                # (the last shape's GEMM counts more than the calibration copy:
                # the calibration is the copy before the first library kernel)
                big = si == len(shapes) - 1
                d.append(("mx4::gemm_tile_kernel<8>(x)", 512, 10.0 * (si + 1) + c, {
                    "FETCH_SIZE": 4 * copy_kib if big else 1000, "WRITE_SIZE": 4 * copy_kib if big else 2000,
                    "SQ_INSTS_VALU_MFMA_MOPS_F6F4": 2.0 * M * N * K / 512, "SQ_VALU_MFMA_BUSY_CYCLES": 1.0e6}))
            d.append(("mx4::hw_stream_kernel(z)", 64, 1.0, {}))
        return d

    def write(sub, fname, counters):
        os.makedirs(tmp_path / sub)
        rows = []
        for i, (name, grid, us, cv) in enumerate(dispatches()):
            base = {"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": grid,
                    "Start_Timestamp": 10 ** 6 * (i + 1), "End_Timestamp": 10 ** 6 * (i + 1) + int(us * 1000)}
            picked = [c for c in counters if c in cv]
            rows += [dict(base, Counter_Name=c, Counter_Value=cv[c]) for c in picked] if counters else [base]
            if counters and not picked:
                rows.append(dict(base, Counter_Name="GRBM_COUNT", Counter_Value=0))
        with open(tmp_path / sub / fname, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=list(rows[0].keys()) if not counters else
                               ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp",
                                "Counter_Name", "Counter_Value"])
            w.writeheader()
            w.writerows(rows)
    write("t", "x_kernel_trace.csv", ())
    write("f", "x_counter_collection.csv", ("FETCH_SIZE",))
    write("w", "x_counter_collection.csv", ("WRITE_SIZE",))
    write("m", "x_counter_collection.csv", bench.MFMA_COUNTERS)
    out = tmp_path / "out"
    os.makedirs(out)
    bench.summarize_large_m(str(tmp_path / "t"), str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "m"),
                            calls, out_dir=str(out))
    rec = _json.load(open(out / "large_m_traffic.json"))
    assert list(rec["shapes"]) == ["%dx%dx%d" % s for s in shapes]
    for si, (M, N, K) in enumerate(shapes):
        r = rec["shapes"]["%dx%dx%d" % (M, N, K)]
        g = r["kernels"]["mx4::gemm_tile_kernel<8>"]
        avg = 10.0 * (si + 1) + 1.0                     # mean of 10(si+1) + {0, 1, 2}
        assert g["avg_us"] == round(avg, 3)
        assert set(r["kernels"]) == {"mx4::gemm_tile_kernel<8>", "mx4::pack_kernel"}   # weight pack dropped
        assert r["kernels"]["mx4::pack_kernel"]["avg_us"] == 2.0 + si
        assert r["gemm_tflops_traced"] == round(2.0 * M * N * K / avg / 1e6, 1)
        # counters: FETCH scaled x2, WRITE x1 (the calibration copy)
        if si == len(shapes) - 1:
            assert g["hbm_bytes"] == 4 * copy_kib * 1024 * 2 + 4 * copy_kib * 1024
        else:
            assert g["hbm_bytes"] == 1000 * 1024 * 2 + 2000 * 1024
        assert g["bytes_to_move"] == (M * K // 2 + M * K // 32) + (N * K // 2 + N * K // 32) + 2 * M * N
        assert r["traced_us_per_call"] == round(avg + 2.0 + si, 3)
    md = open(out / "large_m_trace.md").read()
    assert md.count("| 1.000 |") == len(shapes)     # MOPS x 512 / 2MNK
