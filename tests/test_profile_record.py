"""The counter record's source hash: comment edits keep it, code edits change it."""
from sparse_attention_video_tile_amd import profile_summary as ps


def test_strip_comments_keeps_strings_and_code():
    text = 'int a = 1; // note\n/* block\n  text */ const char* s = "//x/*y*/";\nchar c = \'"\';\n\n'
    assert ps.strip_comments(text) == 'int a = 1;\n  const char* s = "//x/*y*/";\nchar c = \'"\';\n'


def test_hash_ignores_comments_only():
    files = {f: open(f"{ps.ROOT}/{f}").read() for f in ps.KERNEL_SOURCES}
    base = ps.source_sha256(read=files.__getitem__)
    assert base == ps.source_sha256()
    first = ps.KERNEL_SOURCES[0]
    commented = dict(files, **{first: "// a new comment line\n" + files[first].replace("\n", "  // tail\n", 1)})
    assert ps.source_sha256(read=commented.__getitem__) == base
    changed = dict(files, **{first: files[first] + "\nstatic int extra_symbol;\n"})
    assert ps.source_sha256(read=changed.__getitem__) != base
