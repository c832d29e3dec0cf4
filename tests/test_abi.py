"""C-ABI library: loads, exports every declared symbol, and rejects bad arguments on the host
(each call below fails validation before any HIP call, so no GPU is needed)."""

import ctypes
import os
import subprocess

import pytest

from mlra_latent_kv_amd import binding as B
from mlra_latent_kv_amd import inputs as I
from mlra_latent_kv_amd.harness import make_params

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from mlra_latent_kv_amd import build
        build.build()
    return B.load()


def test_exports_every_declared_symbol(lib):
    declared = B.header_functions()
    assert set(declared) == {"mla_workspace_size", "mla_num_splits", "mla_decode", "mlra_decode",
                             "mla_decode_timed", "mlra_decode_timed", "mla_decode_noalloc",
                             "mla_rope_rotate", "mla_status_str", "mla_append_workspace_size",
                             "mla_cache_append", "mla_decode_gated", "mlra_decode_gated",
                             "mla_prefill_workspace_size", "mla_prefill", "mla_prefill_timed"}
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)


def test_probe_library_exports_its_header(lib):
    """The probes (benchmark support) export what include/mla_probe.h declares."""
    from mlra_latent_kv_amd import build
    declared = B.header_functions(os.path.join(ROOT, "include", "mla_probe.h"))
    assert set(declared) == {"mla_probe_out_words", "mla_probe_read", "mla_probe_read_pages",
                             "mla_probe_issue_out_words", "mla_probe_issue"}
    out = subprocess.run(["nm", "-D", "--defined-only", build.PROBE_LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared) <= exported
    probe = ctypes.CDLL(build.PROBE_LIB)
    probe.mla_probe_out_words.restype = ctypes.c_size_t
    assert probe.mla_probe_out_words() == 512 * 4
    probe.mla_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_void_p]
    assert probe.mla_probe_read(None, 16, FAKE, None) == 1       # rejected before any launch
    assert probe.mla_probe_read(FAKE, 24, FAKE, None) == 1
    probe.mla_probe_read_pages.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert probe.mla_probe_read_pages(FAKE, 73728, None, 4, FAKE, None) == 1
    assert probe.mla_probe_read_pages(FAKE, 73720, FAKE, 4, FAKE, None) == 1
    assert probe.mla_probe_read_pages(FAKE, 73728, FAKE, 0, FAKE, None) == 1
    probe.mla_probe_issue_out_words.restype = ctypes.c_size_t
    assert probe.mla_probe_issue_out_words() == 256 * 512
    probe.mla_probe_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p]
    assert probe.mla_probe_issue(0, 0, 16, None, None) == 1      # rejected before any launch
    assert probe.mla_probe_issue(7, 0, 16, FAKE, None) == 1
    assert probe.mla_probe_issue(1, 1, 0, FAKE, None) == 1


def test_params_struct_layout_matches_header(tmp_path):
    """The ctypes mirror has the size and field offsets the C compiler gives the header's
    struct (a small C program prints them)."""
    # 16 int32, 5 int64, 3 float -> 64 + 40 + 12 = 116, padded to 120
    assert ctypes.sizeof(B.MlaParams) == 120
    assert B.MlaParams.flags.offset == 48 and B.MlaParams.num_pages.offset == 52
    assert B.MlaParams.num_queries.offset == 56 and B.MlaParams.latent_stride_tok.offset == 64
    assert B.MlaParams.softmax_scale.offset == 104
    names = [f[0] for f in B.MlaParams._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "mla_decode.h"\n'
                   "int main(void) {\n"
                   '  printf("%zu\\n", sizeof(mla_params));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(mla_params, {n}));\n' for n in names)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got == [ctypes.sizeof(B.MlaParams)] + [getattr(B.MlaParams, n).offset for n in names]


def params_for(wname, **over):
    w = I.WORKLOADS[wname]
    inp = I.make_inputs(w, seqlens=[5, 7])
    p = make_params(inp)
    for k, v in over.items():
        setattr(p, k, v)
    return p


FAKE = 1 << 20  # non-NULL, 256-aligned; never dereferenced because validation fails first


def call(lib, p, fn="mla_decode", ws_bytes=1 << 40, **ptr):
    args = dict(q_nope=FAKE, q_rope=FAKE, latent=FAKE, rope=FAKE, seqlens=FAKE, block_table=FAKE,
                w_uk=FAKE, w_uv=FAKE, out=FAKE, workspace=FAKE)
    args.update(ptr)
    return getattr(lib, fn)(ctypes.byref(p), *args.values(), ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    (dict(dtype=7), 5),
    (dict(batch=0), 2),
    (dict(d_rope=63), 2),
    (dict(max_seqlen=-1), 2),
    (dict(num_splits=-2), 2),
    (dict(page_size=16), 3),
    (dict(d_latent=256), 3),
    (dict(num_heads=48), 3),
    (dict(d_nope=64), 3),
    (dict(latent_stride_tok=500), 2),
    (dict(latent_stride_tok=580), 7),
    (dict(flags=8), 2),
    (dict(num_pages=-1), 2),
    (dict(softmax_scale=float("nan")), 2),
    (dict(rope_theta=0.0), 2),
    (dict(num_splits=1000), 2),
    (dict(num_queries=17), 2),
    (dict(num_queries=-1), 2),
    (dict(latent_format=2), 5),
    (dict(latent_format=1, latent_scale=0.0), 2),
    (dict(latent_format=1, latent_scale=float("inf")), 2),
])
def test_invalid_params_rejected(lib, over, status):
    p = params_for("mla_bf16_b32_h128_l4096", **over)
    assert call(lib, p) == status
    n = ctypes.c_size_t(0)
    st = lib.mla_workspace_size(ctypes.byref(p), ctypes.byref(n))
    assert st == status or (status in (1, 4, 7) and st == 0)


def test_noalloc_rejects_on_the_host(lib):
    """mla_decode_noalloc validates like mla_decode and refuses a call whose workspace would
    exceed its static scratch, all before any HIP call (so no GPU is needed here)."""
    def noalloc(p, **ptr):
        args = dict(q_nope=FAKE, q_rope=FAKE, latent=FAKE, rope=FAKE, seqlens=FAKE,
                    block_table=FAKE, w_uk=FAKE, w_uv=FAKE, out=FAKE)
        args.update(ptr)
        return lib.mla_decode_noalloc(ctypes.byref(p), *args.values(), None)
    big = params_for("mla_bf16_b32_h128_l4096", batch=256, max_seqlen=4096)
    assert B.workspace_size(big) > B.NOALLOC_SCRATCH_BYTES
    assert noalloc(big) == 4                                          # MLA_ERR_WORKSPACE
    assert noalloc(params_for("mla_bf16_b32_h128_l4096"), q_nope=None) == 1
    assert noalloc(params_for("mla_bf16_b32_h128_l4096"), w_uk=FAKE + 2) == 7
    assert noalloc(params_for("mlra4_bf16_b32_h32_l8192")) == 3        # MLA only (NB = 1)
    assert noalloc(params_for("mla_bf16_b32_h128_l4096", page_size=16)) == 3
    # every named workload fits the scratch
    for wname in I.WORKLOAD_ORDER:
        w = I.WORKLOADS[wname]
        p = params_for(wname, batch=w.batch, max_seqlen=w.seqlen,
                       max_pages_per_seq=-(-w.seqlen // 64), block_table_stride=-(-w.seqlen // 64))
        assert B.workspace_size(p) <= B.NOALLOC_SCRATCH_BYTES, wname


def test_branch_count_per_entry_point(lib):
    assert call(lib, params_for("mla_bf16_b32_h128_l4096"), fn="mlra_decode") == 3
    assert call(lib, params_for("mlra4_bf16_b32_h32_l8192"), fn="mla_decode") == 3


@pytest.mark.parametrize("name", ["q_nope", "q_rope", "latent", "rope", "seqlens", "w_uk", "w_uv",
                                  "out", "workspace"])
def test_null_pointer_rejected(lib, name):
    assert call(lib, params_for("mla_bf16_b32_h128_l4096"), **{name: None}) == 1


def test_paged_needs_block_table(lib):
    p = params_for("mla_bf16_paged_b64_h32_l1k-32k")
    assert call(lib, p, block_table=None) == 1
    p.max_pages_per_seq = 0
    assert call(lib, p) == 2


def test_workspace_and_alignment(lib):
    p = params_for("mla_bf16_b32_h128_l4096")
    need = B.workspace_size(p)
    assert call(lib, p, ws_bytes=need - 1) == 4
    assert call(lib, p, latent=FAKE + 8) == 7
    assert call(lib, p, workspace=FAKE + 64) == 7
    assert call(lib, p, w_uk=FAKE + 2) == 7     # bf16 weights need 16-byte alignment


def call_gated(lib, p, fn="mla_decode_gated", ws_bytes=1 << 40, **ptr):
    args = dict(q_nope=FAKE, q_rope=FAKE, latent=FAKE, rope=FAKE, seqlens=FAKE, block_table=FAKE,
                w_uk=FAKE, w_uv=FAKE, gate=FAKE, out=FAKE, workspace=FAKE)
    args.update(ptr)
    return getattr(lib, fn)(ctypes.byref(p), *args.values(), ws_bytes, None)


def test_folded_and_latent_flags_validation(lib):
    """MLA_FLAG_QUERY_LATENT drops the W_UK pointer and the d_nope rule, MLA_FLAG_OUTPUT_LATENT
    the W_UV pointer and the d_v rule; each call stops at the workspace check (MLA_ERR_WORKSPACE),
    past the pointer and shape checks, so nothing is launched."""
    QL, OL = B.MLA_FLAG_QUERY_LATENT, B.MLA_FLAG_OUTPUT_LATENT
    plain = params_for("mla_bf16_b32_h128_l4096")
    assert call(lib, plain, w_uk=None) == 1 and call(lib, plain, w_uv=None) == 1
    assert call(lib, params_for("mla_bf16_b32_h128_l4096", flags=QL), w_uk=None, ws_bytes=1) == 4
    assert call(lib, params_for("mla_bf16_b32_h128_l4096", flags=OL), w_uv=None, ws_bytes=1) == 4
    both = params_for("mlra4_bf16_b32_h32_l8192", flags=QL | OL)
    assert call(lib, both, fn="mlra_decode", w_uk=None, w_uv=None, ws_bytes=1) == 4
    assert call(lib, params_for("mla_bf16_b32_h128_l4096", d_nope=64)) == 3
    assert call(lib, params_for("mla_bf16_b32_h128_l4096", d_nope=64, flags=QL), ws_bytes=1) == 4
    assert call(lib, params_for("mla_bf16_b32_h128_l4096", d_v=64)) == 3
    assert call(lib, params_for("mla_bf16_b32_h128_l4096", d_v=64, flags=OL), ws_bytes=1) == 4
    assert call(lib, params_for("tiny_mla_f32_b1_h4_l64", d_nope=999, flags=QL),
                w_uk=None, ws_bytes=1) == 4


def test_fp8_latent_validation(lib):
    """MLA_LATENT_FP8: bf16 only, a finite positive scale, latent strides counted in bytes and
    16-byte aligned; the call passes validation up to the workspace check."""
    F8 = B.MLA_LATENT_FP8
    p = params_for("mla_bf16_paged_b64_h32_l1k-32k", latent_format=F8, latent_scale=0.01,
                   latent_stride_tok=512, latent_stride_seq=512 * 64)
    assert call(lib, p, ws_bytes=1) == 4
    assert call(lib, params_for("mlra4_bf16_b32_h32_l8192", latent_format=F8, latent_scale=0.5,
                                latent_stride_tok=512, latent_stride_seq=512 * 8192),
                fn="mlra_decode", ws_bytes=1) == 4
    # 128 heads with an fp8 latent run on the 32-head kernel: accepted
    assert call(lib, params_for("mla_bf16_b32_h128_l4096", latent_format=F8, latent_scale=1.0,
                                latent_stride_tok=512, latent_stride_seq=512 * 4096),
                ws_bytes=1) == 4
    bad = p.copy()
    bad.latent_stride_tok = 520  # 8 codes past a 16-byte boundary
    assert call(lib, bad) == 7
    assert call(lib, params_for("tiny_mla_f32_b1_h4_l64", latent_format=F8, latent_scale=1.0)) == 3


def test_several_query_tokens_validation(lib):
    """num_queries = s_q multiplies the query rows: accepted on every kernel family (the call
    stops at the workspace check), with a workspace that grows with s_q; a head count whose
    32-head groups would straddle two tokens is refused on bf16."""
    p1 = params_for("mla_bf16_paged_b64_h32_l1k-32k")
    p4 = params_for("mla_bf16_paged_b64_h32_l1k-32k", num_queries=4)
    assert call(lib, p4, ws_bytes=1) == 4
    assert B.workspace_size(p4) > B.workspace_size(p1)
    assert call(lib, params_for("mlra4_bf16_b32_h32_l8192", num_queries=3), fn="mlra_decode",
                ws_bytes=1) == 4
    assert call(lib, params_for("tiny_mla_f32_b1_h4_l64", num_queries=16), ws_bytes=1) == 4
    assert call(lib, params_for("mla_bf16_paged_b64_h32_l1k-32k", num_heads=16,
                                num_queries=2)) == 3


def test_gated_entry_points_validation(lib):
    p = params_for("mla_bf16_b32_h128_l4096")
    assert call_gated(lib, p, ws_bytes=1) == 4                       # passes pointer checks
    assert call_gated(lib, p, gate=None) == 1
    assert call_gated(lib, p, gate=FAKE + 2) == 7                    # bf16 gate: 16-byte aligned
    assert call_gated(lib, p, fn="mlra_decode_gated") == 3           # NB = 1 here
    assert call_gated(lib, params_for("mlra4_bf16_b32_h32_l8192"), fn="mlra_decode_gated",
                      ws_bytes=1) == 4
    lo = params_for("mla_bf16_b32_h128_l4096", flags=B.MLA_FLAG_OUTPUT_LATENT)
    assert call_gated(lib, lo) == 3                                  # no gate on a latent output
    assert call(lib, p, out=FAKE + 4) == 7                           # bf16 out: 16-byte aligned


def test_rope_rotate_validation(lib):
    f = lib.mla_rope_rotate
    assert f(FAKE, 64, FAKE, 10, 63, 1e4, 1, None) == 2
    assert f(FAKE, 32, FAKE, 10, 64, 1e4, 1, None) == 2
    assert f(FAKE, 64, FAKE, 10, 64, 1e4, 3, None) == 5
    assert f(None, 64, FAKE, 10, 64, 1e4, 1, None) == 1
    assert f(None, 64, None, 0, 64, 1e4, 1, None) == 0     # empty: nothing to do
    assert f(FAKE + 1, 64, FAKE, 10, 64, 1e4, 1, None) == 7


def test_status_strings(lib):
    for s in range(8):
        assert lib.mla_status_str(s).decode().startswith(B.STATUS[s])
    assert lib.mla_status_str(99).decode() == "unknown mla_status"


@pytest.mark.parametrize("wname", I.WORKLOAD_ORDER)
@pytest.mark.parametrize("forced", [0, 3])
def test_workspace_layout(lib, wname, forced):
    w = I.WORKLOADS[wname]
    lens = [w.seqlen] * 3
    inp = I.make_inputs(w, seqlens=[1, 2, 3]) if w.seqlen > 5000 else I.make_inputs(w, seqlens=lens)
    p = make_params(inp)
    p.max_seqlen = w.seqlen
    pages = (w.seqlen + 63) // 64
    if w.paged:
        p.max_pages_per_seq = p.block_table_stride = pages
    forced = min(forced, pages)
    p.num_splits = forced
    S = B.num_splits(p)
    wide = w.dtype == "bf16" and w.branches == 1 and w.heads % 128 == 0
    wg_per_item = w.heads // 128 if wide else w.heads // 32 if w.dtype == "bf16" else w.heads
    shard = w.dtype == "bf16" and w.branches == 1 and w.d_cb == 128   # four workgroups per CU
    target = max(1, -(-(256 if wide else 1024 if shard else 512) // wg_per_item))
    Bn, H, dc = 3, w.heads, w.d_c
    if forced:
        assert S == -(-pages // -(-pages // forced))
        cap = Bn * S
    else:
        assert S == min(pages, target)
        cap = max(target, Bn)
    slots = -(-cap // 8) * 8
    al = lambda x: (x + 255) // 256 * 256
    # plan (header, slot table, slot ends, item table, split offsets, device-check words),
    # queries, per-item partials (element type on the bf16 path), (m, l) in fp32, and the
    # fp32 merged latent; the workspace is sized for 256 compute units
    exp = al(32 + 16 * slots + 4 * slots + 16 * cap + 4 * (Bn + 1) + 4 * Bn) + \
        al(Bn * H * w.row * w.elem_bytes) + \
        al(cap * H * dc * w.elem_bytes) + al(cap * w.branches * H * 2 * 4) + \
        (al(Bn * H * dc * 4) if w.elem_bytes == 4 else 0)
    assert B.workspace_size(p) == exp


def test_split_bounds(lib):
    # bf16 MLA with H % 128 == 0: one workgroup per (work item, 128 heads), 256 items target
    p = params_for("mla_bf16_b32_h128_l4096", batch=32, max_seqlen=4096)
    assert B.num_splits(p) == 64         # one sequence may take up to all of its 64 pages
    p = params_for("mla_bf16_paged_b4_h128_l131072", batch=4, max_seqlen=131072,
                   max_pages_per_seq=2048, block_table_stride=2048)
    assert B.num_splits(p) == 256        # bounded by the item target
    p.num_splits = 7
    assert B.num_splits(p) == 7
    p.num_splits = 600                   # 4 pages per item: 512 items
    assert B.num_splits(p) == 512
    p.num_splits = 1000                  # 3 pages per item: 683 > 512 items
    with pytest.raises(B.MlaError):
        B.num_splits(p)
    # 32-head groups (two workgroups per CU): 512 items target
    p = params_for("mla_bf16_paged_b64_h32_l1k-32k", batch=64, max_seqlen=32768,
                   max_pages_per_seq=512, block_table_stride=512)
    assert B.num_splits(p) == 512
    p = params_for("mlra4_bf16_b32_h32_l8192", batch=32, max_seqlen=8192)
    assert B.num_splits(p) == 128
    p.num_splits = 129                   # more splits than pages
    with pytest.raises(B.MlaError):
        B.num_splits(p)


def test_plan_code_under_host_sanitizers(tmp_path):
    exe = tmp_path / "plan_fuzz"
    src = [os.path.join(ROOT, "tests", "plan_fuzz.cpp"),
           os.path.join(ROOT, "mlra_latent_kv_amd", "csrc", "plan.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "mlra_latent_kv_amd", "csrc"), *src, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "accepted" in r.stdout


def test_plan_checker_rejects_wrong_plans():
    """The GPU tests compare the device's split plan with plan_ref.expected_plan through
    plan_ref.check_plan; here that comparison is shown to reject plans with a plausible
    mistake (pages per item one too many, a shifted item, a wrong split offset, a missed idle
    slot, a wrong slot end, an item table entry cut short)."""
    import copy
    import numpy as np
    from plan_ref import check_plan, expected_plan
    lens = [0, 1, 64, 65, 4000, 0, 129, 3000, 77, 2048]
    good = expected_plan(lens, 4000, 256, 256, xcd_major=True)
    assert good["pages"] == 1 and good["items"] == 151  # 151 pages fit 256 items at c = 1
    check_plan(copy.deepcopy(good), good)
    forced = expected_plan(lens, 4000, 256, 80, forced=5)
    assert forced["pages"] == 13                        # ceil(63 / 5) pages per item
    # 63 pages at 5 forced splits: 13 pages per item; the 4000-token sequence gets 5 items
    assert np.array_equal(forced["split_off"][4:6], [3, 8])

    def bad_plans():
        p = copy.deepcopy(good); p["pages"] = 2; yield p, good
        p = copy.deepcopy(good); p["work"][0, 1] += 64; yield p, good
        p = copy.deepcopy(good); p["split_off"][3] += 1; yield p, good
        p = copy.deepcopy(good)
        p["work"][np.where(p["work"][:, 0] < 0)[0][0]] = (0, 0, 1, 0); yield p, good
        p = copy.deepcopy(good); p["slot_end"][0] += 1; yield p, good
        p = copy.deepcopy(forced); p["item_table"][3, 2] -= 32; yield p, forced

    for got, want in bad_plans():
        with pytest.raises(AssertionError):
            check_plan(got, want)


def append_params(**over):
    p = B.MlaAppendParams()
    p.batch, p.d_model, p.d_latent, p.d_rope = 64, 4096, 512, 64
    p.page_size, p.max_pages_per_seq, p.capacity, p.dtype = 64, 512, 0, B.MLA_BF16
    p.latent_stride_tok = p.rope_stride_tok = 576
    p.latent_stride_seq = p.rope_stride_seq = 576 * 64
    p.block_table_stride = 512
    p.rope_theta = 10000.0
    for k, v in over.items():
        setattr(p, k, v)
    return p


def test_append_params_layout_and_workspace(lib):
    # 8 int32, 5 int64, 1 float -> 32 + 40 + 4 = 76, padded to 80
    assert ctypes.sizeof(B.MlaAppendParams) == 88
    assert B.MlaAppendParams.latent_stride_tok.offset == 32
    assert B.MlaAppendParams.rope_theta.offset == 72
    assert B.MlaAppendParams.latent_format.offset == 76 and B.MlaAppendParams.latent_scale.offset == 80
    # fp32 partials [d_model / 256][B][d_latent + 64], then the page ranks [B]
    al = lambda x: (x + 255) // 256 * 256
    assert B.append_workspace_size(append_params()) == al(16 * 64 * 576 * 4) + al(64 * 4)
    assert B.append_workspace_size(append_params(d_latent=128, batch=3, d_model=256)) == \
        al(1 * 3 * 192 * 4) + al(3 * 4)


@pytest.mark.parametrize("over,status", [
    (dict(batch=0), 2), (dict(d_model=0), 2), (dict(rope_theta=0.0), 2),
    (dict(dtype=0), 3), (dict(dtype=9), 5), (dict(d_model=1000), 3), (dict(d_latent=256), 3),
    (dict(d_rope=32), 3), (dict(page_size=16), 3), (dict(max_pages_per_seq=0), 2),
    (dict(block_table_stride=100), 2), (dict(page_size=0, capacity=0), 2),
    (dict(latent_stride_tok=500), 2),
    (dict(latent_format=2), 5), (dict(latent_format=1, latent_scale=0.0), 2),
    (dict(latent_format=1, latent_scale=float("nan")), 2),
])
def test_append_invalid_params_rejected(lib, over, status):
    n = ctypes.c_size_t(0)
    assert lib.mla_append_workspace_size(ctypes.byref(append_params(**over)), ctypes.byref(n)) == status


def test_append_call_checks(lib):
    def call(p=None, n_free=1, ws_bytes=1 << 40, pages_used=FAKE, workspace=FAKE, **ptr):
        args = dict(hidden=FAKE, w_dkv=FAKE, w_kr=FAKE, latent=FAKE, rope=FAKE, seqlens=FAKE,
                    block_table=FAKE, free_pages=FAKE)
        args.update(ptr)
        p = p or append_params()
        return lib.mla_cache_append(ctypes.byref(p), *args.values(), n_free, pages_used,
                                    workspace, ws_bytes, None)
    assert call(hidden=None) == 1
    assert call(block_table=None) == 1
    assert call(free_pages=None) == 1
    # an empty free list needs no pointer, nor a contiguous cache a block table: those calls
    # get past the pointer checks and stop at the (too small) workspace, before any launch
    assert call(free_pages=None, n_free=0, ws_bytes=10) == 4
    assert call(p=append_params(page_size=0, capacity=8), block_table=None, ws_bytes=10) == 4
    assert call(n_free=-1) == 2
    assert call(ws_bytes=10) == 4
    assert call(w_dkv=FAKE + 8) == 7 and call(workspace=FAKE + 16) == 7
    assert call(pages_used=None) == 1


# ----------------------------------------------------------------------------- prefill
def test_prefill_workspace_size_and_validation(lib):
    """mla_prefill's workspace sizes (MLA and MLRA-4) and host checks: every call below fails
    validation before anything is launched (the pointers are never dereferenced)."""
    p = params_for("mla_bf16_b32_h128_l4096", num_queries=300, max_seqlen=300)
    # keys and values, B x H x L_pad x 128 bf16 each (L_pad = 300 rounded up to 512), and
    # the rotary keys, B x L_pad x 64 bf16
    assert B.prefill_workspace_size(p) == 2 * 2 * 128 * 512 * 128 * 2 + 2 * 512 * 64 * 2
    p1 = params_for("mla_bf16_b32_h128_l4096", num_queries=1, max_seqlen=1)
    assert B.prefill_workspace_size(p1) == 2 * 2 * 128 * 256 * 128 * 2 + 2 * 256 * 64 * 2
    # MLRA-4 (four 128-wide branches): keys and values per (head, branch), the rotary keys,
    # and the bf16 branch outputs B x s_q x H x 4 x 128
    p4 = params_for("mlra4_bf16_b32_h32_l8192", num_queries=300, max_seqlen=300)
    assert B.prefill_workspace_size(p4) == (2 * 2 * 32 * 4 * 512 * 128 * 2 + 2 * 512 * 64 * 2
                                            + 2 * 300 * 32 * 4 * 128 * 2)
    ws = B.prefill_workspace_size(p)
    assert call(lib, p, fn="mla_prefill", ws_bytes=ws - 1) == 4        # MLA_ERR_WORKSPACE
    assert call(lib, p, fn="mla_prefill", q_nope=None) == 1            # MLA_ERR_NULL
    assert call(lib, p, fn="mla_prefill", w_uv=None) == 1
    assert call(lib, p, fn="mla_prefill", q_rope=FAKE + 8) == 7        # MLA_ERR_ALIGN
    assert call(lib, p, fn="mla_prefill", out=FAKE + 2) == 7
    assert call(lib, p, fn="mla_prefill", workspace=FAKE + 16) == 7
    for over, status in [(dict(num_branches=4, d_latent=512), 3),     # MLRA-4 at 128 per branch
                         (dict(num_branches=2, d_latent=256), 3),
                         (dict(d_latent=256), 3), (dict(d_nope=64), 3),
                         (dict(flags=B.MLA_FLAG_QUERY_LATENT), 3),
                         (dict(dtype=B.MLA_F32), 3), (dict(dtype=9), 5),
                         (dict(page_size=16), 3), (dict(num_queries=-1), 2),
                         (dict(batch=70000), 2), (dict(latent_stride_tok=580), 7)]:
        q = params_for("mla_bf16_b32_h128_l4096", **{**dict(num_queries=300, max_seqlen=300), **over})
        assert call(lib, q, fn="mla_prefill") == status, over
    paged = params_for("mla_bf16_paged_b64_h32_l1k-32k", num_queries=5)
    assert call(lib, paged, fn="mla_prefill", block_table=None) == 1
