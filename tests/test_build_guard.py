"""The build's m0 guard (CPU only): kernels that write m0 from inline
assembly (the untracked HBM->LDS copies) must contain no compiler-generated
instruction that uses m0; m0_violations() reads a device assembly listing."""

from sequence_transformer_attention_rsa_amd.build import m0_violations

HEAD = """\t.text
\t.type\tkern_a,@function
\t.type\tkern_b,@function
"""

OURS = """\t;;#ASMSTART
\ts_mov_b32 m0, s38
\ts_nop 0
\tglobal_load_lds_dwordx4 v100, s[6:7]
\t;;#ASMEND
"""


def listing(body_a, body_b=""):
    return (HEAD + "kern_a:\n" + body_a + "\ts_endpgm\n.Lfunc_end0:\n"
            + "kern_b:\n" + body_b + "\ts_endpgm\n.Lfunc_end1:\n")


def test_untracked_copies_alone_pass():
    assert m0_violations(listing(OURS + "\tv_add_f32_e32 v1, v2, v3\n" + OURS)) == []


def test_compiler_m0_write_beside_untracked_copies_fails():
    bad = m0_violations(listing(OURS + "\ts_mov_b32 m0, -1\n\tds_read_b128 v[0:3], v4\n"))
    assert bad == ["kern_a: s_mov_b32 m0, -1"]


def test_implicit_m0_users_beside_untracked_copies_fail():
    for instr in ("v_movrels_b32_e32 v1, v2", "s_sendmsg sendmsg(MSG_DEALLOC_VGPRS)",
                  "global_load_lds_dword v3, s[4:5]", "buffer_load_dword v1, s[8:11], 0 offen lds",
                  "v_readlane_b32 s1, v2, m0"):
        assert m0_violations(listing(OURS + "\t" + instr + "\n")) == [f"kern_a: {instr}"], instr


def test_compiler_m0_use_without_untracked_copies_is_allowed():
    # the builtin copy alone (its m0 write is the compiler's own)
    body = "\ts_mov_b32 m0, s4\n\tglobal_load_lds_dwordx4 v1, s[2:3]\n"
    assert m0_violations(listing(body, OURS)) == []
