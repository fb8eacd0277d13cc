"""Host-side helpers of bench.py that need no GPU: the kernel-source hash that keys the committed
counter records, and the mapping of rocprofv3 kernel instances to the library's product names."""
import os

import bench


def _write(root, gemm, update):
    d = os.path.join(root, "sgd_cnns_amd", "csrc")
    os.makedirs(d, exist_ok=True)
    open(os.path.join(d, "gemm.hip"), "w").write(gemm)
    open(os.path.join(d, "update.hip"), "w").write(update)


def test_kernel_code_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    code = 'int f(int x) {\n  const char* s = "a // b /* c */";\n  return x + 1;\n}\n'
    commented = ('// header\nint f(int x) {  /* inline */\n\n  const char* s = "a // b /* c */";  // tail\n'
                 '  return x + 1;\n}\n/* trailing\n   block */\n')
    changed = code.replace("x + 1", "x + 2")
    in_string = code.replace('"a // b /* c */"', '"a // b /* d */"')
    hashes = []
    for gemm in (code, commented, changed, in_string):
        root = tmp_path / str(len(hashes))
        _write(str(root), gemm, "__global__ void k() {}\n")
        monkeypatch.setattr(bench, "ROOT", str(root))
        hashes.append(bench.kernel_code_sha256())
    assert hashes[0] == hashes[1]            # comments and blank lines only
    assert hashes[0] != hashes[2]            # code
    assert hashes[0] != hashes[3]            # comment markers inside a string literal are code


def test_bench_kernel_names():
    # the trailing template arguments of the kernel (pipelined loop, wavefront rows) do not change the name
    assert bench.bench_kernel_name(
        "void sgd::(anonymous namespace)::gemm_dma<128, 128, true, true, 5, false, true, false, 2>(KArgs, SkArgs)") == \
        "gemm_conv_dw_128x128"
    assert bench.bench_kernel_name(
        "void sgd::(anonymous namespace)::gemm_dma<64, 128, false, true, 3, false, false, false, 1>(KArgs, SkArgs)") \
        == "gemm_dma_64x128_nn"
    assert bench.bench_kernel_name(
        "void sgd::(anonymous namespace)::gemm_dma<128, 128, false, false, 2, false, false, true, 2>(KArgs, SkArgs)") \
        == "gemm_dma_128x128_nt"
    assert bench.bench_kernel_name("void sgd::(anonymous namespace)::dw_short<16, 2, 0>(KArgs, ShortArgs)") == \
        "gemm_dw_short_k32"
    assert bench.bench_kernel_name("sgd::(anonymous namespace)::dw_long_kernel(sgd::(anonymous namespace)::KArgs, "
                                   "float*, int)") == "gemm_staged_long_tn"
    assert bench.bench_kernel_name("void sgd::(anonymous namespace)::dw_short<8, 1, -1>(KArgs, ShortArgs)") == \
        "gemm_dw_short_k16"
    assert bench.bench_kernel_name(
        "void sgd::(anonymous namespace)::gemm_dma<128, 128, true, true, 5, false, true>(KArgs, SkArgs)") == \
        "gemm_conv_dw_128x128"
    assert bench.bench_kernel_name(
        "void sgd::(anonymous namespace)::gemm_dma<128, 128, false, true, 3, false, false>(KArgs, SkArgs)") == \
        "gemm_dma_128x128_nn"
    # the pipelined-loop instances carry one more template flag
    assert bench.bench_kernel_name(
        "void sgd::(anonymous namespace)::gemm_dma<128, 128, false, false, 2, true, false, true>(KArgs, SkArgs)") == \
        "gemm_conv_fwd_128x128"
    assert bench.bench_kernel_name(
        "void sgd::(anonymous namespace)::gemm_dma<128, 128, false, false, 2, false, false, false>(KArgs, SkArgs)") == \
        "gemm_dma_128x128_nt"
    assert bench.is_product("gemm_dw_short_k32") and not bench.is_product("softmax_ce")


def test_committed_traffic_records_name_each_dominant_kernel():
    """The committed counter record keys each kernel by the library's own name, so the bench line can
    attach HBM traffic to the dominant kernel it times (an instance that the name mapping misses would
    be filed under a bare template name)."""
    import json
    import os
    recs = json.load(open(os.path.join(bench.ROOT, "profiles", "traffic.json")))
    dominant = {"mlp5000": "gemm_dma_128x128_tn", "vgg16": "gemm_conv_dw_128x128",
                "vgg_cifar": "gemm_conv_dw_128x128", "ps_adagrad": "apply_kernel<2, 8>"}
    seen = set()
    for r in recs:
        kernels = r["kernels"]
        assert not {"gemm_dma", "gemm_staged"} & set(kernels), f"unmapped instance names in {r['workload']}"
        if r["workload"] in dominant:
            assert dominant[r["workload"]] in kernels
            assert kernels[dominant[r["workload"]]]["traffic_bytes"] > 0
            seen.add(r["workload"])
    assert seen == set(dominant)
