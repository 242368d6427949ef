"""The build-time check of the library's gfx950 assembly: a store of more than 64 bits
must not be followed directly by a write of its data registers."""
from depthwise_pointwise_convolution_amd.isa_check import store_data_overwrites

HEAD = "_ZN3fcm6kernelEv:\n"
TAIL = ".Lfunc_end0:\n"


def _asm(*lines):
    return HEAD + "".join(("" if l.endswith(":") else "\t") + l + "\n" for l in lines) + TAIL


def test_flags_next_write_of_store_data():
    asm = _asm("buffer_store_dwordx4 v[42:45], v46, s[40:43], s70 offen",
               "v_add_u32_e32 v42, s72, v99")
    hits = store_data_overwrites(asm)
    assert len(hits) == 1 and hits[0][0] == "_ZN3fcm6kernelEv"


def test_flags_global_store_and_fall_through_label():
    asm = _asm("global_store_dwordx4 v[2:3], v[10:13], off", ".LBB0_4:",
               "v_mov_b32_e32 v13, 0")
    assert len(store_data_overwrites(asm)) == 1


def test_wait_state_other_registers_and_narrow_stores_pass():
    nop = _asm("buffer_store_dwordx4 v[42:45], v46, s[40:43], 0 offen", "s_nop 0",
               "v_add_u32_e32 v42, s72, v99")
    addr_only = _asm("buffer_store_dwordx4 v[42:45], v16, s[40:43], 0 offen",
                     "v_add_u32_e32 v16, s72, v99")
    narrow = _asm("buffer_store_dwordx2 v[42:43], v46, s[40:43], s70 offen",
                  "v_add_u32_e32 v42, s72, v99")
    later = _asm("buffer_store_dwordx4 v[42:45], v46, s[40:43], s70 offen",
                 "v_add_u32_e32 v16, s72, v99", "v_mov_b32_e32 v42, 0")
    for asm in (nop, addr_only, narrow, later):
        assert store_data_overwrites(asm) == []
