"""Host-side helpers of the measurement scripts (no GPU)."""
import bench_counters


def test_code_hash_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text('int f(int x) {\n  // one\n  return x + 1; /* two */\n}\nasm("s_nop 0 // kept");\n')
    b.write_text('int f(int x) {   return x + 1;\n\n}\n// other words\nasm("s_nop 0 // kept");\n')
    c.write_text('int f(int x) {\n  return x + 2;\n}\nasm("s_nop 0 // kept");\n')
    assert bench_counters.code_hash(str(a)) == bench_counters.code_hash(str(b))
    assert bench_counters.code_hash(str(a)) != bench_counters.code_hash(str(c))


def test_code_hash_keeps_string_literals(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    a.write_text('asm("s_nop 0 // x");\n')
    b.write_text('asm("s_nop 1 // x");\n')
    assert bench_counters.code_hash(str(a)) != bench_counters.code_hash(str(b))


def test_counter_labels_follow_the_step_order():
    """Dispatches are labelled by their place in a block step: the n-th GEMM
    of a step is the n-th projection, a split tail's fixup is added to the
    GEMM before it, steps 1-2 are the B = 2 block, 3-4 B = 1 and 5-6 the
    8-bit block (its two quantiser launches per step told apart); the
    weights' quantisation before the first step is set-up; the calibration
    copy is the first bf16 copy kernel."""
    def d(name, **c):
        return {"name": name, "grid": 1, "ns": 10, "counters": dict(c)}
    step = [d("dit::tmod_stage1(float)", X=1), d("dit::tmod_stage2_fewb(float)", X=1),
            d("_ZN3dit14modnorm_kernelIDF16b", X=1), d("_ZN3dit11gemm_kernelIDF16b", X=10),
            d("_ZN3dit13vtrans_kernelIDF16b", X=1), d("_ZN3dit11attn_kernelIDF16b", X=5),
            d("_ZN3dit11gemm_kernelIDF16b", X=20), d("_ZN3dit20resid_modnorm_kernelIDF16b", X=1),
            d("_ZN3dit11gemm_kernelIDF16b", X=30), d("_ZN3dit13gemm_sk_fixupIDF16b", X=3),
            d("_ZN3dit11gemm_kernelIDF16b", X=40), d("_ZN3dit13gemm_sk_fixupIDF16b", X=4),
            d("_ZN3dit12resid_kernelIfDF16b", X=1)]
    step8 = [d("dit::tmod_stage1(float)", X=1), d("dit::tmod_stage2_fewb(float)", X=1),
             d("_ZN3dit14modnorm_kernelIDF16bhLi8EEE", X=1), d("_ZN3dit15gemm_fp8_kernelILi0EEE", X=10),
             d("_ZN3dit11attn_kernelIDF16b", X=5), d("_ZN3dit21quantize_fp8_rows_regILi8EEE", X=2),
             d("_ZN3dit15gemm_fp8_kernelILi0EEE", X=20), d("_ZN3dit20resid_modnorm_kernelIDF16b", X=1),
             d("_ZN3dit15gemm_fp8_kernelILi1EEE", X=30), d("_ZN3dit21quantize_fp8_rows_regILi24EEE", X=3),
             d("_ZN3dit15gemm_fp8_kernelILi0EEE", X=40), d("_ZN3dit12resid_kernelIfDF16b", X=1)]
    setup = [d("_ZN3dit21quantize_fp8_rows_regILi8EEE", X=500)] * 4
    disp = [d("void at::native::vectorized_elementwise_kernel<4, at::native::bfloat16_copy_kernel_cuda", X=7),
            d("__amd_rocclr_copyBuffer", X=99)] + setup + step * 4 + step8 * 2
    rows = bench_counters._label(disp)
    assert not any(c.get("X") == 500 for _, _, c in rows)  # the weights' quantisation is set-up
    fp8 = [(w, k) for w, k, _ in rows if w == "1024px_B2_fp8"]
    assert fp8[:12] == [("1024px_B2_fp8", k) for k in ("tmod1", "tmod2", "modnorm1", "gemm_qkvg", "attn", "quant_og",
                                                        "gemm_o", "resid1+modnorm2", "gemm_w13", "quant_u",
                                                        "gemm_w2", "resid2")]
    assert len(fp8) == 24
    rows = [r for r in rows if r[0] != "1024px_B2_fp8"]
    assert rows[0][:2] == ("calib", "copy") and rows[0][2]["X"] == 7
    assert sum(1 for r in rows if r[0] == "calib") == 1
    labels = [(w, k) for w, k, _ in rows[1:]]
    assert labels[:11] == [("1024px_B2", k) for k in ("tmod1", "tmod2", "modnorm1", "gemm_qkvg", "vtrans", "attn",
                                                        "gemm_o", "resid1+modnorm2", "gemm_w13", "gemm_w2",
                                                        "resid2")]
    assert labels[22][0] == "1024px_B1" and labels[-2] == ("1024px_B1", "gemm_w2")
    w13 = [c for w, k, c in rows if k == "gemm_w13"][0]
    assert w13["X"] == 33 and w13["DURATION_NS"] == 20  # fixup added
