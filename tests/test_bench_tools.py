"""Host-side helpers of the measurement scripts (no GPU)."""
import bench_traffic


def test_code_hash_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text('int f(int x) {\n  // one\n  return x + 1; /* two */\n}\nasm("s_nop 0 // kept");\n')
    b.write_text('int f(int x) {   return x + 1;\n\n}\n// other words\nasm("s_nop 0 // kept");\n')
    c.write_text('int f(int x) {\n  return x + 2;\n}\nasm("s_nop 0 // kept");\n')
    assert bench_traffic.code_hash(str(a)) == bench_traffic.code_hash(str(b))
    assert bench_traffic.code_hash(str(a)) != bench_traffic.code_hash(str(c))


def test_code_hash_keeps_string_literals(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    a.write_text('asm("s_nop 0 // x");\n')
    b.write_text('asm("s_nop 1 // x");\n')
    assert bench_traffic.code_hash(str(a)) != bench_traffic.code_hash(str(b))
