"""The C-ABI library loads, exports every symbol the header declares, its
struct layouts match the binding, and host-side validation rejects bad
arguments without touching a GPU."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec.h")


@pytest.fixture(scope="module")
def L():
    from draft_verification_spec_amd import _lib
    return _lib


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(spec_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    lib = L.load()
    names = declared_functions()
    assert set(names) == set(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.spec_abi_version() == 6
    assert lib.spec_strerror(-1).decode() == "invalid argument"


def test_struct_layout_matches_header(L, tmp_path):
    src = tmp_path / "layout.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "spec.h"', "int main(void) {"]
    for name, st in L.STRUCTS.items():
        lines.append(f'printf("{name} %zu\\n", sizeof({name}));')
        for f, _ in st._fields_:
            cf = "lambda" if f == "lam" else f
            lines.append(f'printf("{name}.{f} %zu\\n", offsetof({name}, {cf}));')
    lines.append("return 0; }")
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = dict(l.split() for l in subprocess.check_output([str(exe)]).decode().splitlines())
    for name, st in L.STRUCTS.items():
        assert int(got[name]) == C.sizeof(st), name
        for f, _ in st._fields_:
            assert int(got[f"{name}.{f}"]) == getattr(st, f).offset, (name, f)


def test_validation_rejects_bad_arguments_without_gpu(L):
    lib = L.load()
    assert lib.spec_ngram_draft(None, None) == L.SPEC_EINVAL
    assert lib.spec_allocate_budget(None, None) == L.SPEC_EINVAL
    assert lib.spec_verify_chain(None, None) == L.SPEC_EINVAL
    assert lib.spec_verify_tree(None, None) == L.SPEC_EINVAL
    fake = 0x1000  # never dereferenced: validation fails first
    a = L.NgramArgs(bs=1, nq=1, ctx=fake, ctx_stride=16, ctx_len=fake, n_min=3, n_max=2, max_draft=15,
                    copy_cap=256, draft=fake, draft_len=fake, feat=fake)
    assert lib.spec_ngram_draft(C.byref(a), None) == L.SPEC_EINVAL           # n_min > n_max
    a.n_max = 15
    a.max_draft = 40
    assert lib.spec_ngram_draft(C.byref(a), None) == L.SPEC_EINVAL           # draft too long
    a.max_draft = 15
    assert lib.spec_workspace_bytes(L.OP_NGRAM, C.byref(a)) == 0             # the drafter needs no scratch
    v = L.VerifyArgs(bs=2, vocab=100, temperature=-1.0, logits=fake, row_stride=100, row_base=fake,
                     n_logit_rows=4, tokens=fake, ld=3, n_slots=fake, out_tokens=fake, out_num=fake,
                     out_accepted=fake, out_flags=fake)
    assert lib.spec_verify_chain(C.byref(v), None) == L.SPEC_EINVAL          # T < 0
    v.temperature = 1.0
    assert lib.spec_verify_chain(C.byref(v), None) == L.SPEC_EINVAL          # T > 0 needs uniforms
    v.temperature = 0.0
    v.dtype = 7
    assert lib.spec_verify_chain(C.byref(v), None) == L.SPEC_EINVAL          # bad dtype
    v.dtype = 0
    assert lib.spec_workspace_bytes(L.OP_VERIFY_CHAIN, C.byref(v)) > 0
    assert lib.spec_verify_chain(C.byref(v), None) == L.SPEC_EWORKSPACE      # no workspace
    v.vocab = (1 << 23) + 1
    v.row_stride = v.vocab
    assert lib.spec_verify_chain(C.byref(v), None) == L.SPEC_EINVAL          # vocabulary too large
    al = L.AllocArgs(mode=5)
    assert lib.spec_allocate_budget(C.byref(al), None) == L.SPEC_EINVAL      # bad mode
    al.mode = L.ALLOC_CHAIN
    al.chain.bs = 4
    al.chain.ld = 15
    al.chain.K = 7
    al.chain.budget = -1
    assert lib.spec_allocate_budget(C.byref(al), None) == L.SPEC_EINVAL      # negative budget
    t = L.AllocArgs(mode=L.ALLOC_TREE)
    t.tree.bs, t.tree.c_max, t.tree.rows_cap = 2, 8, 4
    for f in ("node_token", "parent_row", "Q", "n_rows", "row_base", "total_rows", "forest_count", "out_flags"):
        setattr(t.tree, f, fake)
    t.tree.forest_token = fake
    assert lib.spec_allocate_budget(C.byref(t), None) == L.SPEC_EINVAL       # a forest without parents, q, n
    t.tree.forest_parent = t.tree.forest_q = t.tree.forest_n = fake
    t.tree.scores = fake
    assert lib.spec_allocate_budget(C.byref(t), None) == L.SPEC_EINVAL       # a given forest with scores
    t.tree.scores = None
    for c_max, rows_cap in ((0, 4), (1025, 4), (8, 0), (8, 65)):
        t.tree.c_max, t.tree.rows_cap = c_max, rows_cap
        assert lib.spec_allocate_budget(C.byref(t), None) == L.SPEC_EINVAL   # sizes out of range


def test_binding_fails_loudly_without_library(L, tmp_path):
    with pytest.raises(ImportError):
        L.load(str(tmp_path / "missing.so"))
