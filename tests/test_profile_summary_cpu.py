"""The source hash that ties a committed counter summary to the kernel
sources it was taken on ignores comments and layout, and nothing else."""

from matrix_roots_amd import profile_summary as P


def test_code_only_drops_comments_and_layout():
    a = 'int a = 1; // note\n/* block\n   note */ const char* s = "x // kept"; char c = \'"\';\n'
    b = 'int a = 1;   // another note\n   const char* s = "x // kept"; char c = \'"\';'
    assert P.code_only(a) == P.code_only(b) == 'int a = 1; const char* s = "x // kept"; char c = \'"\';'


def test_code_only_keeps_code_changes():
    a = "v = x * 2; // twice"
    assert P.code_only(a) != P.code_only("v = x * 3; // twice")
    assert P.code_only("a/*x*/b") == "a b"  # a comment still separates tokens
    assert P.code_only('s = "/* not a comment */";') == 's = "/* not a comment */";'


def test_every_family_hashes():
    hashes = {f: P.sources_sha256(f) for f in P.KERNEL_SOURCES}
    assert all(len(h) == 64 for h in hashes.values())
    assert len(set(hashes.values())) == len(hashes)
