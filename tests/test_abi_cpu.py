"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, and rejects bad arguments on the host before anything is
launched (no GPU needed: every call here fails its host checks)."""
import ctypes
import os
import re

import pytest

import hybrid_sliding_window_decode_amd as hswd
from hybrid_sliding_window_decode_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hswd.h")
MEASURE_HEADER = os.path.join(ROOT, "include", "hswd_measure.h")

A = ctypes.c_void_p(0x10000)       # aligned stand-in pointer (never dereferenced)
MIS = ctypes.c_void_p(0x10004)     # misaligned stand-in pointer


def declared(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|int32_t|size_t)\s+(hswd_\w+)\s*\(",
                                 text, re.M)))


def desc(**kw):
    d = dict(batch=2, n_heads=8, n_kv_heads=8, head_dim=256, n_slots=511, kv_dtype=2,
             scale=1 / 16, keys_per_split=0, chunks_per_workgroup=0, kv_scale=None)
    d.update(kw)
    return binding.AttnDesc(**d)


def test_exports_every_declared_symbol():
    L = binding.lib()
    names = declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(binding.SIGNATURES), set(names) ^ set(binding.SIGNATURES)


def test_measurement_library_exports_its_header_and_nothing_leaks_into_libhswd():
    M = binding.measure_lib()
    names = declared(MEASURE_HEADER)
    assert names == ["hswd_measure_stream_read"]
    for n in names:
        assert hasattr(M, n), n
    assert set(names) == set(binding.MEASURE_SIGNATURES)
    # the decode library exports no measurement entry
    assert not hasattr(binding.lib(), "hswd_measure_stream_read")
    assert not hasattr(binding.lib(), "hswd_stream_read")


def test_measurement_host_checks():
    M = binding.measure_lib()
    # null, size 0 or not a multiple of 16, workgroups, alignment
    assert M.hswd_measure_stream_read(None, 1 << 20, A, 64, None) == -1
    assert M.hswd_measure_stream_read(A, 0, A, 64, None) == -1
    assert M.hswd_measure_stream_read(A, 1000, A, 64, None) == -1
    assert M.hswd_measure_stream_read(A, 1 << 20, A, 0, None) == -1
    assert M.hswd_measure_stream_read(A, 1 << 20, A, 65537, None) == -1
    assert M.hswd_measure_stream_read(MIS, 1 << 20, A, 64, None) == -2
    assert M.hswd_measure_stream_read(A, 1 << 20, MIS, 64, None) == -2


def test_version_and_status_strings():
    assert hswd.version() >= 3
    for s in range(-6, 1):
        assert hswd.status_string(s) == binding.STATUS[s]
    assert hswd.status_string(-99) == "unknown status"


def test_workspace_and_splits():
    L = binding.lib()
    d = desc()
    # default chunk of a ring: 2^floor(log2(n_slots/32)) in [128, 512], at
    # least four quanta (quantum = 32768 / (D * element bytes) keys): 256 keys
    # for a bf16 ring.  An append cache's streams take their own chunk from
    # their n valid keys: the power of two at or above n / 32, at least four
    # quanta, at most 1024 keys below 131072 keys, 2048 below 524288 and from
    # there 1024 per kv head within [2048, 8192]; the launch holds the most
    # chunks a stream up to max_pos can have (32 once max_pos reaches 32 * the
    # floor, 128 at 131071 keys, 256 at 524287)
    assert hswd.num_splits(d, 1) == 2
    assert hswd.num_splits(desc(n_slots=4097), 0, 4096) == 16              # 256 keys
    assert hswd.num_splits(desc(n_slots=8192), 0, 8191) == 32              # 256 keys
    assert hswd.num_splits(desc(n_slots=16385), 0, 16384) == 32            # 512 keys
    assert hswd.num_splits(desc(n_slots=9001), 0, 9000) == 32              # 512: 18, grid 32
    assert hswd.num_splits(desc(n_slots=65537), 0, 65536) == 64            # 1024 keys
    assert hswd.num_splits(desc(n_slots=131073), 0, 131071) == 128         # 1024 keys
    assert hswd.num_splits(desc(n_slots=131073), 0, 131072) == 128         # 2048 keys, 64
    assert hswd.num_splits(desc(n_slots=131073), 0, 5000) == 20            # 256 keys
    assert hswd.num_splits(desc(n_slots=262145), 0, 262144) == 128         # 2048 keys
    assert hswd.num_splits(desc(n_slots=524289), 0, 524287) == 256         # 2048 keys
    assert hswd.num_splits(desc(n_slots=524289), 0, 524288) == 256         # 8192 keys, 64
    assert hswd.num_splits(desc(n_slots=(1 << 20) + 1), 0, 1 << 20) == 256  # 8192: 128
    assert hswd.num_splits(desc(n_slots=(1 << 20) + 1, kv_dtype=3), 0, 1 << 20) == 256
    # fewer kv heads, smaller chunks there: 4096 keys for 4 (256 chunks at
    # 2^20), 2048 for 2 and for 1 (512)
    assert hswd.num_splits(desc(n_slots=(1 << 20) + 1, n_heads=4, n_kv_heads=4), 0, 1 << 20) == 256
    assert hswd.num_splits(desc(n_slots=(1 << 20) + 1, n_heads=2, n_kv_heads=2), 0, 1 << 20) == 512
    assert hswd.num_splits(desc(n_slots=(1 << 20) + 1, n_heads=8, n_kv_heads=1), 0, 1 << 20) == 512
    assert hswd.num_splits(desc(n_slots=4097, head_dim=64), 0, 4096) == 4       # Q = 256
    assert hswd.num_splits(desc(n_slots=4097, kv_dtype=0), 0, 4096) == 32       # f32: Q = 32
    assert hswd.num_splits(desc(n_slots=4097, kv_dtype=3), 0, 4096) == 8        # fp8: Q = 128
    assert hswd.num_splits(desc(kv_dtype=3), 1, 0) == 1
    assert hswd.num_splits(desc(n_slots=4097, keys_per_split=1024), 0, 4096) == 4
    assert hswd.num_splits(desc(n_slots=4097, keys_per_split=128), 0, 4096) == 32
    assert hswd.num_splits(desc(n_slots=4097, chunks_per_workgroup=3), 0, 4096) == 16
    # grouped layers: at least eight quanta (512 keys bf16, 1024 fp8)
    assert hswd.num_splits(desc(n_slots=4097, n_heads=32), 0, 4096) == 8
    assert hswd.num_splits(desc(n_slots=4097, n_heads=32, kv_dtype=3), 0, 4096) == 4
    assert hswd.num_splits(desc(n_heads=16), 1, 0) == 1
    # splits never depend on the batch
    assert hswd.num_splits(desc(batch=1, n_slots=4097), 0, 4096) == \
        hswd.num_splits(desc(batch=64, n_slots=4097), 0, 4096)
    ring = hswd.workspace_bytes(d, 1)
    full = hswd.workspace_bytes(desc(n_slots=4097), 0, 4096)
    assert ring >= 256 + 2 * 8 * 4
    assert full >= 2 * 8 * 8 * (256 + 2) * 4
    assert L.hswd_workspace_bytes(ctypes.byref(desc(head_dim=0)), 1, 0) == 0
    assert L.hswd_num_splits(ctypes.byref(desc(keys_per_split=100)), 1, 0) == -1


def test_groups_up_to_eight_heads_run_in_one_piece():
    """A ring layer with one chunk holds no partials, so its workspace is the
    error word (256 bytes) plus the arrival counters rounded up to 256 bytes:
    one per (stream, kv head) and piece, plus one per (stream, kv head) for
    the entry write when a group runs in pieces.  Groups of 2 to 8 query
    heads per kv head run in one piece; larger ones in pieces of eight."""
    def counters(H, Hkv=8, B=64, dt=2):
        d = desc(batch=B, n_heads=H, n_kv_heads=Hkv, kv_dtype=dt)
        assert hswd.num_splits(d, 1) == 1
        return (hswd.workspace_bytes(d, 1) - 256) // 4
    for dt in (1, 2, 3):
        for H in (16, 24, 32, 40, 48, 56, 64):
            assert counters(H, dt=dt) == 64 * 8, (dt, H)
        assert counters(128, dt=dt) == 64 * 8 * 2 + 64 * 8          # two pieces of 8
        assert counters(96, dt=dt) == 64 * 8 * 2 + 64 * 8           # 12: pieces of 8 and 4
        assert counters(256, Hkv=8, dt=dt) == 64 * 8 * 4 + 64 * 8   # 32: four pieces


@pytest.mark.parametrize("case,kw,want", [
    ("H % Hkv", dict(n_heads=6, n_kv_heads=4), -1),
    ("head_dim", dict(head_dim=96), -6),
    ("head_dim odd", dict(head_dim=7), -1),
    ("dtype", dict(kv_dtype=4), -1),
    ("fp8 head_dim 64", dict(kv_dtype=3, head_dim=64), -6),
    ("fp8 kps quantum", dict(kv_dtype=3, keys_per_split=64), -1),
    ("scale", dict(scale=0.0), -1),
    ("kps", dict(keys_per_split=100), -1),
    ("kps quantum bf16", dict(keys_per_split=96), -1),
    ("kps quantum d128", dict(head_dim=128, keys_per_split=64), -1),
    ("cpw", dict(chunks_per_workgroup=-1), -1),
    ("batch", dict(batch=-1), -1),
    # grouped layers (any H / Hkv > 1) need a 16-bit or fp8 cache and D >= 128
    ("GQA f32", dict(n_heads=16, n_kv_heads=8, kv_dtype=0), -6),
    ("GQA f32 group 8", dict(n_heads=16, n_kv_heads=2, kv_dtype=0), -6),
    ("GQA head_dim 64", dict(n_heads=16, n_kv_heads=8, head_dim=64), -6),
    # a (stream, kv head) block of 4 GiB or more (32-bit offsets in the kernel)
    ("block 4 GiB bf16", dict(n_slots=1 << 23), -6),
    ("block 4 GiB f32", dict(n_slots=1 << 22, kv_dtype=0), -6),
    ("block 4 GiB fp8", dict(n_slots=1 << 24, kv_dtype=3), -6),
])
def test_sliding_rejects_bad_descriptor(case, kw, want):
    L = binding.lib()
    d = desc(**kw)
    st = L.hswd_decode_attn_sliding(A, A, A, A, A, A, A, ctypes.byref(d), A, 1 << 20, None)
    assert st == want, case


def test_attention_host_checks():
    L = binding.lib()
    d = desc()
    big = 1 << 30
    assert L.hswd_decode_attn_sliding(None, A, A, A, A, A, A, ctypes.byref(d), A, big, None) == -1
    assert L.hswd_decode_attn_sliding(A, A, A, A, MIS, A, A, ctypes.byref(d), A, big, None) == -2
    assert L.hswd_decode_attn_sliding(A, A, A, A, A, A, A, ctypes.byref(d), None, big, None) == -3
    assert L.hswd_decode_attn_sliding(A, A, A, A, A, A, A, ctypes.byref(d), A, 16, None) == -3
    assert L.hswd_decode_attn_sliding(A, A, A, A, A, A, A, ctypes.byref(d), MIS, big, None) == -2
    assert L.hswd_decode_attn_sliding(A, A, A, A, A, A, A, None, A, big, None) == -1
    f = desc(n_slots=4097)
    # max_pos + 1 must fit the append capacity
    assert L.hswd_decode_attn_full(A, A, A, A, A, A, A, 4096 + 1, ctypes.byref(f), A, big, None) == -4
    assert L.hswd_decode_attn_full(A, A, A, A, A, A, A, -1, ctypes.byref(f), A, big, None) == -1
    # more than 4096 chunks is refused
    huge = desc(n_slots=1 << 20, keys_per_split=64)
    assert L.hswd_decode_attn_full(A, A, A, A, A, A, A, (1 << 20) - 1, ctypes.byref(huge), A, big,
                                   None) == -1
    need = hswd.workspace_bytes(f, 0, 4096)
    assert L.hswd_decode_attn_full(A, A, A, A, A, A, A, 4096, ctypes.byref(f), A, need - 1,
                                   None) == -3


def test_other_entries_host_checks():
    L = binding.lib()
    d = desc()
    # rope: rot_dim odd / zero / above D, theta <= 0, null q
    assert L.hswd_rope_apply(A, A, A, 2, 8, 8, 256, 255, 1e4, None) == -1
    assert L.hswd_rope_apply(A, A, A, 2, 8, 8, 256, 0, 1e4, None) == -1
    assert L.hswd_rope_apply(A, A, A, 2, 8, 8, 256, 258, 1e4, None) == -1
    assert L.hswd_rope_apply(A, A, A, 2, 8, 8, 256, 64, 0.0, None) == -1
    assert L.hswd_rope_apply(None, A, A, 2, 8, 8, 256, 64, 5e6, None) == -1
    assert L.hswd_rope_apply(A, A, A, 2, 8, 8, 16386, 64, 5e6, None) == -6   # LDS bound
    # kv write
    assert L.hswd_kv_slot_write(A, A, A, A, A, ctypes.byref(d), 1, None, None, None) == -3
    assert L.hswd_kv_slot_write(A, MIS, A, A, A, ctypes.byref(d), 1, None, A, None) == -2
    assert L.hswd_kv_slot_write(A, None, A, A, A, ctypes.byref(d), 1, None, A, None) == -1
    # merge, gate, mask
    assert L.hswd_lse_merge(A, A, A, 2, 8, 256, 0, None) == -1
    assert L.hswd_lse_merge(A, A, A, 2, 8, 256, 2048, None) == -6
    assert L.hswd_head_gate(A, A, None, 2, 8, 256, None) == -1
    assert L.hswd_ring_mask(None, None, A, 2, 511, 1, None) == -1
    assert L.hswd_ring_mask(A, A, A, 2, 0, 1, None) == -1
    # layer step
    assert L.hswd_layer_step(A, A, A, A, A, A, A, A, 1, 255, 1e4, 0, ctypes.byref(d), A,
                             1 << 20, None) == -1
    assert L.hswd_layer_step(A, A, A, A, A, A, A, A, 1, 256, -1.0, 0, ctypes.byref(d), A,
                             1 << 20, None) == -1
    assert L.hswd_workspace_init(None, 64, None) == -3
    assert L.hswd_workspace_init(MIS, 64, None) == -2
    assert L.hswd_check_errors(None, None, None) == -3


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 8, 256)
    with pytest.raises(ValueError):
        hswd.rope_apply(q, None, torch.zeros(1, dtype=torch.int32), 256, 1e4)


def test_empty_batch_is_a_no_op():
    """B = 0: every entry returns OK with null pointers and launches nothing
    (there is no GPU here, so a launch would fail); its other arguments are
    still checked."""
    L = binding.lib()
    d0 = desc(batch=0)
    N = None
    assert L.hswd_ring_mask(N, N, N, 0, 511, 1, N) == 0
    assert L.hswd_ring_mask(N, N, N, 0, 0, 1, N) == -1
    assert L.hswd_rope_apply(N, N, N, 0, 8, 8, 256, 256, 1e4, N) == 0
    assert L.hswd_rope_apply(N, N, N, 0, 8, 8, 256, 255, 1e4, N) == -1
    assert L.hswd_kv_slot_write(N, N, N, N, N, ctypes.byref(d0), 1, N, N, N) == 0
    assert L.hswd_decode_attn_sliding(N, N, N, N, N, N, N, ctypes.byref(d0), N, 0, N) == 0
    assert L.hswd_decode_attn_full(N, N, N, N, N, N, N, 4096, ctypes.byref(d0), N, 0, N) == 0
    assert L.hswd_decode_attn_partials(N, N, N, N, N, N, 1, 0, ctypes.byref(d0), N) == 0
    assert L.hswd_lse_merge(N, N, N, 0, 8, 256, 4, N) == 0
    assert L.hswd_lse_merge(N, N, N, 0, 8, 256, 2048, N) == -6
    assert L.hswd_head_gate(N, N, N, 0, 8, 256, N) == 0
    assert L.hswd_gate_proj(N, N, N, 0, 2048, 8, N) == 0
    assert L.hswd_layer_step(N, N, N, N, N, N, N, N, 1, 256, 1e4, 0, ctypes.byref(d0), N, 0,
                             N) == 0
    assert L.hswd_layer_step(N, N, N, N, N, N, N, N, 1, 256, -1.0, 0, ctypes.byref(d0), N, 0,
                             N) == -1
    assert L.hswd_layer_step_gproj(N, N, N, N, N, N, 2048, N, N, N, 1, 256, 1e4, 0,
                                   ctypes.byref(d0), N, 0, N) == 0
    assert L.hswd_decode_attn_sliding(N, N, N, N, N, N, N, ctypes.byref(desc(batch=0, scale=0.0)),
                                      N, 0, N) == -1
    assert L.hswd_workspace_bytes(ctypes.byref(d0), 1, 0) > 0



def test_binding_covers_every_declared_entry():
    """Every hswd_* entry point the header declares has a ctypes signature and
    a Python function of the same name (without the prefix)."""
    import re
    import hybrid_sliding_window_decode_amd as pkg
    h = open(os.path.join(ROOT, "include", "hswd.h")).read()
    declared = sorted(set(re.findall(r"\b(hswd_[a-z_0-9]+)\s*\(", h)))
    assert len(declared) >= 17
    for name in declared:
        assert name in binding.SIGNATURES, name
        assert hasattr(pkg, name[5:]) or hasattr(binding, name[5:]), name
    # the measurement library: hswd_measure_stream_read -> stream_read
    m = open(os.path.join(ROOT, "include", "hswd_measure.h")).read()
    for name in sorted(set(re.findall(r"\b(hswd_measure_[a-z_0-9]+)\s*\(", m))):
        assert name in binding.MEASURE_SIGNATURES, name
        assert hasattr(pkg, name[len("hswd_measure_"):]), name


def test_binding_refuses_a_descriptor_that_does_not_match_the_tensors():
    """The library addresses every row from the descriptor alone, so the
    binding compares a caller's descriptor with the tensors before anything
    else: a stale one (another batch, cache, head count or type) is refused
    with ValueError.  CPU tensors: a matching descriptor gets as far as the
    device check, which proves the descriptor check came first and passed."""
    import torch
    B, H, Hkv, S, D = 3, 8, 4, 40, 128
    kc = torch.zeros(B, Hkv, S, D, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    q = torch.zeros(B, H, D)
    k = torch.zeros(B, Hkv, D)
    v = torch.zeros(B, Hkv, D)
    g = torch.zeros(B, H)
    pos = torch.zeros(B, dtype=torch.int32)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    good = binding.make_desc(kc, n_heads=H)
    calls = [
        lambda d: hswd.layer_step(q, k, v, g, kc, vc, pos, 0, 32, 5e6, ws, max_pos=10, desc=d),
        lambda d: hswd.bind_layer_step(q, k, v, g, kc, vc, pos, 1, D, 1e4, ws, desc=d),
        lambda d: hswd.decode_attn_full(q, k, v, kc, vc, pos, 10, ws, desc=d),
        lambda d: hswd.decode_attn_sliding(q, k, v, kc, vc, pos, ws, desc=d),
        lambda d: hswd.decode_attn_partials(q, kc, vc, pos, 1, desc=d),
        lambda d: hswd.kv_slot_write(kc, vc, k, v, pos, 1, ws, desc=d),
    ]
    bad = [dict(batch=B + 1), dict(n_heads=2 * H), dict(n_kv_heads=Hkv * 2), dict(head_dim=256),
           dict(n_slots=S + 1), dict(kv_dtype=1)]
    for call in calls:
        with pytest.raises(ValueError, match="CUDA"):
            call(good)
        for change in bad:
            d = binding.make_desc(kc, n_heads=H)
            for key, val in change.items():
                setattr(d, key, val)
            if "n_heads" in change and call is calls[-1]:
                continue            # the entry write has no query heads to compare
            with pytest.raises(ValueError, match="desc"):
                call(d)


def test_default_chunks_fit_the_chunk_limit_on_very_long_caches():
    """Past 2^25 keys the default chunk doubles beyond its 8192-key cap, so
    every cache fits in 4096 chunks; an explicit chunk size that would need
    more is refused by num_splits and gets no workspace size."""
    L = binding.lib()
    for n_slots, dt, D in [((1 << 25) + 2, 3, 128), ((1 << 26) - 1, 2, 64),
                           ((1 << 24) - 1, 3, 128), (1 << 23, 2, 256)]:
        d = desc(n_slots=n_slots, kv_dtype=dt, head_dim=D)
        n = hswd.num_splits(d, 0, n_slots - 1)
        assert 1 <= n <= 4096, (n_slots, dt, D, n)
        assert hswd.workspace_bytes(d, 0, n_slots - 1) > 0
    # a stream's chunk follows its valid keys: 2^25 of them still take
    # 8192-key chunks (4096 of them), one more takes 16384-key chunks; the
    # launch is sized for 4096 chunks from 2^25 keys on
    assert hswd.num_splits(desc(n_slots=1 << 25), 0, (1 << 25) - 1) == 4096
    assert hswd.num_splits(desc(n_slots=(1 << 25) + 1), 0, 1 << 25) == 4096
    assert hswd.num_splits(desc(n_slots=(1 << 25) + 2), 0, (1 << 25) + 1) == 4096
    assert hswd.num_splits(desc(n_slots=(1 << 25) + 1), 0, 5000) == 20
    assert hswd.num_splits(desc(n_slots=1 << 23), 0, (1 << 23) - 1) == 1024
    # an explicit chunk that needs more than 4096 chunks
    big = desc(n_slots=(1 << 20) + 1, keys_per_split=128)
    assert L.hswd_num_splits(ctypes.byref(big), 0, 1 << 20) == -1
    assert hswd.workspace_bytes(big, 0, 1 << 20) == 0
    with pytest.raises(binding.HswdError):
        hswd.num_splits(big, 0, 1 << 20)


def test_noalloc_step_refuses_what_its_array_cannot_hold():
    """hswd_layer_step_noalloc checks, before it touches the device, that the
    call fits the library's 32 MiB array: a call needing more (chunk
    partials of 2 streams of 64 query heads over 2^20-row caches, or more
    arrival counters than its 64 KiB region) returns
    HSWD_ERR_WORKSPACE (on this GPU-less host a device access would have
    returned HSWD_ERR_HIP instead); a misaligned error word is refused."""
    L = binding.lib()
    f = L.hswd_layer_step_noalloc

    def call(d, ring=0, max_pos=0, err=None, rot=64):
        return f(A, A, A, A, None, A, A, A, ring, rot, 5e6, max_pos, ctypes.byref(d), err, None)

    big = desc(batch=2, n_heads=64, n_slots=(1 << 20) + 1)      # 33.8 MB of partials
    assert call(big, max_pos=1 << 20) == -3
    many = desc(batch=2049, n_slots=511)                        # 16392 counters
    assert call(many, ring=1, rot=256) == -3
    assert call(desc(batch=1, n_slots=4097), max_pos=4096, err=ctypes.c_void_p(0x10002)) == -2
    assert call(desc(batch=0, n_slots=4097), max_pos=4096) == 0  # empty batch: nothing to do
    assert call(desc(batch=1, n_slots=4097), max_pos=4097) == -4  # capacity, as layer_step


def test_c_abi_caller_links_and_checks_its_arguments():
    """tests/c_abi/layer_step (the C-ABI caller of the GPU tests) loads the
    library and refuses a wrong argument count before any GPU call."""
    import subprocess
    exe = os.path.join(ROOT, "tests", "c_abi", "layer_step")
    if not os.path.exists(exe):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "hswd_c_abi_build", os.path.join(ROOT, "tests", "c_abi", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
