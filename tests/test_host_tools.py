"""Host-side measurement helpers (CPU): the code hash that guards the committed
counter records, and the kernel names the rocprofv3 summariser reports."""
from layout_agnostic_latent_amd import rocprof_summary as rs


def test_code_tokens_ignore_comments_and_layout():
    a = "int x = 1; // one\n/* block\n comment */ float y  =\n  2.0f;"
    b = "int x = 1;\nfloat y = 2.0f; // two"
    assert rs._code_tokens(a) == rs._code_tokens(b)


def test_code_tokens_see_code_changes_and_keep_literals():
    assert rs._code_tokens("int x = 1;") != rs._code_tokens("int x = 2;")
    # comment markers inside string and character literals are code
    assert rs._code_tokens('const char* s = "a // b";') == 'const char* s = "a // b";'
    assert rs._code_tokens("char c = '/'; // x") == "char c = '/';"
    assert rs._code_tokens('s = "q\\"//";') == 's = "q\\"//";'


def test_kernel_source_hash_is_stable_and_short():
    h = rs.kernel_source_hash()
    assert len(h) == 16 and h == rs.kernel_source_hash()


def test_summariser_names_the_two_merges_apart():
    fp16 = "_ZN6splash12_GLOBAL__N_118split_merge_kernelIDF16_NS0_11ListedPartsEEEvPKT_PKfT0_iiPfS9_"
    fp32 = ("void splash::(anonymous namespace)::split_merge_kernel<float, splash::(anonymous namespace)::"
            "UniformParts>(float const*, float const*, splash::(anonymous namespace)::UniformParts, int, int, "
            "float*, float*)")
    assert rs.short(fp16).startswith("split_merge_kernel<fp16>")
    assert rs.short(fp32).startswith("split_merge_kernel<fp32>")
    dec = "void splash::(anonymous namespace)::decode_attn_kernel<576, 512, 4, 1>(splash::DecodeArgs)"
    assert rs.short(dec) == "decode_attn_kernel<576, 512, 4, 1>"
    dec16 = "void splash::(anonymous namespace)::decode_attn16_kernel<576, 512>(splash::DecodeArgs)"
    assert rs.short(dec16) == "decode_attn16_kernel<576, 512>"
