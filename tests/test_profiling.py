"""Host logic of the profile tooling: the code hash that ties a stored
counter reading to the kernel source it was taken with."""
from roofline_driven_optimisation_amd.profiling import code_hash, source_hash


def test_code_hash_ignores_comments_and_blank_lines():
    a = "int f(int x) {\n    return x + 1;\n}\n"
    b = ("// header comment\n/* block\n   comment */\nint f(int x) {  // trailing\n\n"
         "    return x + 1;   \n}\n")
    assert code_hash(a) == code_hash(b)


def test_code_hash_sees_code_changes():
    assert code_hash("int f(int x) { return x + 1; }") != code_hash("int f(int x) { return x + 2; }")
    assert code_hash("a = b / c;") != code_hash("a = b;")


def test_source_hash_known_families():
    for fam in ("bf16_q4", "bf16_pp", "bf16_mfma", "f32_mfma", "f32_dma", "skinny", "naive"):
        h = source_hash(fam)
        assert len(h) == 16 and int(h, 16) >= 0
    assert source_hash("bf16_q4") == source_hash("bf16_pp")  # one source file
    assert source_hash("unknown_kernel") == ""
