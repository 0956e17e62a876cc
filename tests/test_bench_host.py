"""Host-side pieces of bench.py that need no GPU: the code hash that keeps a
committed HBM-traffic record valid across comment edits, and the
algorithmic byte counts the roofline divides by."""
import bench


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = tmp_path / "k.hip"

    def h(text):
        src.write_text(text)
        return bench.source_hash(["k.hip"])

    base = h('int f(int a) { return a + 1; }  // one\nconst char* s = "x // y";\n')
    # comments and layout edited: same hash
    assert h('/* new */ int f(int a) {\n  return a + 1;  // two\n}\nconst char* s = "x // y";\n') == base
    # code edited: new hash, including inside a string literal that looks like a comment
    assert h('int f(int a) { return a + 2; }\nconst char* s = "x // y";\n') != base
    assert h('int f(int a) { return a + 1; }\nconst char* s = "x // z";\n') != base


def test_code_only_keeps_literals():
    text = "a = '\\'' ; b = \"/* not a comment */\"; // gone\n/* gone */ c"
    assert bench._code_only(text) == "a='\\'';b=\"/* not a comment */\";c"


def test_algorithmic_bytes_pages_shape():
    """The per-op byte counts at 8192 tokens x hidden 7168, top-8 of 256 with
    every selection valid: combine reads 65,536 rows and writes 8192, plus
    8 bytes of slot and weight per selection."""
    T, H, K, E = 8192, 7168, 8, 256
    n_sel = T * K
    got = bench.algorithmic_bytes(T, H, K, E, n_sel, 7392)
    assert got["combine"] == n_sel * H * 2 + T * K * 8 + T * H * 2 == 1_057_488_896


def test_more_than_one_gpu_is_refused(capsys):
    """bench.py measures one GPU's share; --gpus N > 1 exits with a message
    and a nonzero status before touching the GPU."""
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
