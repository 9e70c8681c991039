"""CPU tests of the library's host side and its C ABI surface (no GPU):
exported symbols, argument validation, tile layout, store sizing, the
production host Adam against the oracle's, and the seeded weight init."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from layer_streaming_amd import mt
from oracle import step as ostep
from oracle.bf16 import round_bf16

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CFG1 = mt.make_shape(2, 256, 4, 4, 64, 688, 1024)
QWEN7 = mt.make_shape(28, 3584, 28, 4, 128, 18944, 152064)
QWEN14 = mt.make_shape(48, 5120, 40, 8, 128, 13824, 152064)


def _declared_functions():
    names = set()
    for h in ("mt.h", "mt_kernels.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(mt_[a-z_0-9]+)\s*\(", src, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 30
    for n in sorted(names):
        assert hasattr(mt.lib, n), n
    assert names == set(mt.EXPORTED), names ^ set(mt.EXPORTED)


def test_python_mirrors_match_the_abi_structs():
    for which, cls in enumerate((mt.mt_shape, mt.mt_options, mt.mt_stats, mt.mt_tensor_info)):
        assert mt.lib.mt_abi_sizeof(which) == C.sizeof(cls), cls.__name__
    assert mt.lib.mt_abi_sizeof(7) == -1
    # constants the binding mirrors from the header
    hdr = open(os.path.join(ROOT, "include", "mt.h")).read()
    for name in ("MT_MAX_SITES", "MT_MAX_MICRO"):
        assert int(re.search(rf"#define {name} (\d+)", hdr).group(1)) == getattr(mt, name), name


def test_strerror_and_status_codes():
    for s in (mt.MT_OK, mt.MT_E_INVAL, mt.MT_E_NOMEM, mt.MT_E_HIP, mt.MT_E_STATE, mt.MT_E_INTERNAL):
        assert mt.lib.mt_strerror(s)
    assert mt.lib.mt_strerror(-99) == b"unknown status"


def test_tensor_layout_contiguity_and_alignment():
    sh = QWEN7
    d, hq, hkv, f = 3584, 28 * 128, 4 * 128, 18944
    t = [mt.tensor_desc(sh, 0, j) for j in range(9)]
    assert [x["name"] for x in t] == ["g1", "wq", "wk", "wv", "wo", "g2", "wg", "wu", "wd"]
    assert t[2]["offset"] == t[1]["offset"] + hq * d          # wq|wk|wv contiguous
    assert t[3]["offset"] == t[2]["offset"] + hkv * d
    assert t[7]["offset"] == t[6]["offset"] + f * d           # wg|wu contiguous
    for x in t:
        assert x["offset"] % 8 == 0
    for j in (0, 1, 4, 5, 6, 8):
        assert t[j]["offset"] % 128 == 0                      # 256-byte aligned
    assert (t[4]["rows"], t[4]["cols"]) == (d, hq)
    assert (t[8]["rows"], t[8]["cols"]) == (d, f)
    h = [mt.tensor_desc(sh, 28, j) for j in range(2)]
    assert h[1]["name"] == "e_out" and (h[1]["rows"], h[1]["cols"]) == (152064, d)
    assert mt.tensor_desc(sh, 29, 0)["name"] == "e_in"
    assert mt.unit_tensors(sh, 0) == 9 and mt.unit_tensors(sh, 28) == 2 and mt.unit_tensors(sh, 29) == 1
    # no two tensors overlap and the region covers them
    ends = sorted((x["offset"], x["offset"] + x["rows"] * x["cols"]) for x in t)
    for (a0, a1), (b0, b1) in zip(ends, ends[1:]):
        assert a1 <= b0
    assert ends[-1][1] <= mt.unit_elems(sh, 0)


def test_host_store_is_sixteen_bytes_per_parameter():
    o = mt.default_options(max_batch=8, max_seq=1024)
    for sh, n in ((QWEN7, 7_615_487_488), (QWEN14, 14_769_689_600)):
        _, _, store = mt.workspace_bytes(sh, o)
        # padding to 256-byte tensors and 4 KiB tiles adds well under 0.01 %
        assert n * 16 <= store <= n * 16 * 1.0001
    _, _, store = mt.workspace_bytes(QWEN7, o)
    assert abs(store / 1e9 - 121.85) < 0.05                     # the pages' ~122 GB


def test_gpu_working_set_does_not_grow_with_depth():
    o = mt.default_options(max_batch=4, max_seq=2048)
    arenas = set()
    for L in (4, 8, 16, 24):
        sh = mt.make_shape(L, 8192, 64, 8, 128, 28672, 128256)
        a, pinned, _ = mt.workspace_bytes(sh, o)
        arenas.add(a)
    assert len(arenas) == 1
    # with checkpoints kept on the GPU the arena grows with depth instead
    o2 = mt.default_options(max_batch=4, max_seq=2048, ckpt_on_host=0)
    a4 = mt.workspace_bytes(mt.make_shape(4, 8192, 64, 8, 128, 28672, 128256), o2)[0]
    a8 = mt.workspace_bytes(mt.make_shape(8, 8192, 64, 8, 128, 28672, 128256), o2)[0]
    assert a8 > a4


def test_workspace_bytes_deterministic_and_overridable():
    o = mt.default_options(max_batch=8, max_seq=1024)
    a1 = mt.workspace_bytes(QWEN7, o)
    a2 = mt.workspace_bytes(QWEN7, o)
    assert a1 == a2
    o.workspace_bytes_override = a1[0] * 2
    assert mt.workspace_bytes(QWEN7, o)[0] > a1[0]


@pytest.mark.parametrize("field,value", [("d_model", 100), ("head_dim", 96), ("n_kv_heads", 3),
                                         ("vocab", 0), ("n_layers", 0)])
def test_bad_shapes_rejected(field, value):
    sh = mt.make_shape(2, 256, 4, 4, 64, 688, 1024)
    setattr(sh, field, value)
    a, p, h = C.c_uint64(), C.c_uint64(), C.c_uint64()
    o = mt.default_options()
    r = mt.lib.mt_workspace_bytes(C.byref(sh), C.byref(o), C.byref(a), C.byref(p), C.byref(h))
    assert r == mt.MT_E_INVAL
    assert mt.lib.mt_last_error()


@pytest.mark.parametrize("field,value", [("n_weight_slots", 0), ("n_weight_slots", 5), ("n_grad_slabs", 0),
                                         ("slot_mode", 2), ("max_batch", 0), ("beta1", 1.0), ("ckpt_interval", 0),
                                         ("cross_step", 2), ("pin_weights", 2), ("head_vocab_chunk", -2),
                                         ("head_vocab_chunk", 12), ("poison_released", 2),
                                         ("keep_grads", 2), ("keep_grads", -1), ("ckpt_attn", 2)])
def test_bad_options_rejected(field, value):
    o = mt.default_options()
    setattr(o, field, value)
    a, p, h = C.c_uint64(), C.c_uint64(), C.c_uint64()
    assert mt.lib.mt_workspace_bytes(C.byref(CFG1), C.byref(o), C.byref(a), C.byref(p), C.byref(h)) == mt.MT_E_INVAL


def test_option_conflicts_rejected():
    for kw in (dict(ckpt_interval=2, ckpt_on_host=0), dict(pin_weights=1, pin_store=1),
               dict(poison_released=1, slot_mode=1), dict(poison_released=1, resident=1),
               dict(ckpt_attn=1, ckpt_on_host=0), dict(ckpt_attn=1, ckpt_interval=2)):
        o = mt.default_options(**kw)
        a, p, h = C.c_uint64(), C.c_uint64(), C.c_uint64()
        assert mt.lib.mt_workspace_bytes(C.byref(CFG1), C.byref(o), C.byref(a), C.byref(p), C.byref(h)) == mt.MT_E_INVAL


def test_attention_checkpoint_ring_sizes():
    """ckpt_attn adds a second attention buffer pair to the arena (T x Hq*hd
    fp16 and B*S*Hq fp32) and a pinned ring of one such pair per layer; the
    host store does not change."""
    def sizes(**kw):
        o = mt.default_options(max_batch=2, max_seq=64, **kw)
        a, p, h = C.c_uint64(), C.c_uint64(), C.c_uint64()
        assert mt.lib.mt_workspace_bytes(C.byref(CFG1), C.byref(o), C.byref(a), C.byref(p), C.byref(h)) == 0
        return a.value, p.value, h.value
    a0, p0, h0 = sizes()
    a1, p1, h1 = sizes(ckpt_attn=1)
    T, nq, Hq, L = 128, 4 * 64, 4, 2
    al4k = lambda x: (x + 4095) // 4096 * 4096
    assert h1 == h0
    assert p1 - p0 == L * (al4k(T * nq * 2) + al4k(T * Hq * 4))
    assert T * nq * 2 + T * Hq * 4 <= a1 - a0 <= T * nq * 2 + T * Hq * 4 + 1024


def test_vocab_chunked_head_sizes_slots_to_the_decoder_layer():
    """head_vocab_chunk=-1 streams E_out in row chunks no larger than the
    largest decoder layer: at the 7B shape the four slot-sized arena buffers
    and the 14 slot-sized pinned buffers shrink from the head's 1.09 GB to the
    layer's 466 MB (minus the chunked head's own fp32 buffers)."""
    o0 = mt.default_options(max_batch=8, max_seq=1024)
    o1 = mt.default_options(max_batch=8, max_seq=1024, head_vocab_chunk=-1)
    a0, p0, h0 = mt.workspace_bytes(QWEN7, o0)
    a1, p1, h1 = mt.workspace_bytes(QWEN7, o1)
    layer_b = mt.unit_elems(QWEN7, 0) * 2
    head_b = mt.unit_elems(QWEN7, 28) * 2
    assert h1 == h0
    assert abs((p0 - p1) - 14 * (head_b - layer_b)) < 14 * 8192
    assert a1 < a0 - 2 * (head_b - layer_b)


def test_checkpoint_interval_trades_pinned_ring_for_arena_banks():
    """Interval k keeps ceil(L/k) layer inputs in the pinned ring and 2k input
    buffers in the GPU arena (two banks of a block's inputs)."""
    sh = mt.make_shape(6, 256, 4, 4, 64, 688, 1024)
    td = 2 * 64 * 256 * 2  # max_batch 2 x max_seq 64 tokens x d 256, bf16 (a 4 KiB multiple)
    sizes = {}
    for k in (1, 2, 3, 6, 9):
        sizes[k] = mt.workspace_bytes(sh, mt.default_options(max_batch=2, max_seq=64, ckpt_interval=k))
    for k, kk in ((2, 2), (3, 3), (6, 6), (9, 6)):
        a, p, _ = sizes[k]
        assert sizes[1][1] - p == (6 - (6 + kk - 1) // kk) * td  # fewer ring entries
        assert a - sizes[1][0] >= 2 * (kk - 1) * td and a - sizes[1][0] < 2 * (kk - 1) * td + 4 * 4096


def test_init_rejects_null_arena_before_device_work():
    o = mt.default_options(max_batch=1, max_seq=16)
    ptr = C.c_void_p()
    r = mt.lib.mt_init(C.byref(CFG1), C.byref(o), None, 0, None, C.byref(ptr))
    assert r == mt.MT_E_INVAL and not ptr.value


# ------------------------------------------------------------ host Adam ---
@pytest.mark.parametrize("step", [1, 2, 7])
def test_host_adam_matches_oracle(step):
    rng = np.random.default_rng(step)
    n = 100_003
    master = rng.standard_normal(n).astype(np.float32) * 0.05
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32) if step > 1 else np.zeros(n, np.float32)
    v = (np.abs(rng.standard_normal(n)) * 1e-8).astype(np.float32) if step > 1 else np.zeros(n, np.float32)
    g = round_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
    g[:100] = 0.0
    gbits = (g.view(np.uint32) >> 16).astype(np.uint16)
    w = np.zeros(n, np.uint16)
    gst = np.zeros(n, np.uint16)
    pm, pmm, pv = master.copy(), m.copy(), v.copy()
    r = mt.lib.mt_host_adam(w.ctypes.data, gst.ctypes.data, pm.ctypes.data, pmm.ctypes.data, pv.ctypes.data,
                            gbits.ctypes.data, n, step, 1e-4, 0.9, 0.999, 1e-8, 4)
    assert r == mt.MT_OK
    om, omm, ov, ow = ostep.adam_update(master, m, v, g, step, 1e-4, 0.9, 0.999, 1e-8)
    ulp = np.spacing(np.abs(om)).astype(np.float64)
    assert np.all(np.abs(pm.astype(np.float64) - om) <= np.maximum(2 * ulp, 1e-6 * 1e-4))
    # b1*m + (1-b1)*g can cancel: allow ~2 ulp of the operands' scale
    np.testing.assert_allclose(pmm, omm, rtol=2e-6, atol=2e-11)
    np.testing.assert_allclose(pv, ov, rtol=2e-6, atol=2e-15)
    assert np.array_equal(gst, gbits)
    assert np.array_equal((w.astype(np.uint32) << 16).view(np.float32), round_bf16(pm))


@pytest.mark.parametrize("off", [0, 3])
def test_host_adam_vector_path_bit_identical_to_single_elements(off):
    """The host Adam's 8-wide loop against one call per element (which never
    reaches the vector loop), on arrays starting at an unaligned offset, with
    NaN, inf and zero gradients mixed in."""
    rng = np.random.default_rng(11 + off)
    n = 2_051

    def arrays():
        r = np.random.default_rng(5)
        mas = (r.standard_normal(n + off) * 0.05).astype(np.float32)
        mm = (r.standard_normal(n + off) * 1e-4).astype(np.float32)
        vv = (np.abs(r.standard_normal(n + off)) * 1e-8).astype(np.float32)
        return mas, mm, vv, np.zeros(n + off, np.uint16), np.zeros(n + off, np.uint16)

    g = round_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
    g[[5, 17, 100]] = [np.nan, np.inf, 0.0]
    gbits = np.zeros(n + off, np.uint16)
    gbits[off:] = (g.view(np.uint32) >> 16).astype(np.uint16)
    a = arrays()
    b = arrays()
    ptr = lambda x, i=off: x.ctypes.data + i * x.itemsize  # noqa: E731
    assert mt.lib.mt_host_adam(ptr(a[3]), ptr(a[4]), ptr(a[0]), ptr(a[1]), ptr(a[2]), ptr(gbits), n, 3, 1e-4,
                               0.9, 0.999, 1e-8, 3) == mt.MT_OK
    for i in range(n):
        j = off + i
        assert mt.lib.mt_host_adam(ptr(b[3], j), ptr(b[4], j), ptr(b[0], j), ptr(b[1], j), ptr(b[2], j),
                                   ptr(gbits, j), 1, 3, 1e-4, 0.9, 0.999, 1e-8, 1) == mt.MT_OK
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("off", [0, 3])
def test_host_accumulation_matches_oracle_bit_for_bit(off):
    """The production G accumulation of micro-batch steps against the
    oracle's one-rounding BF16 sum: random magnitudes over 60 binades, exact
    ties (half a BF16 unit added to odd and even values), zeros, infinities,
    both signs; an unaligned start exercises the scalar head and tail."""
    rng = np.random.default_rng(40 + off)
    n = 4_099
    a = round_bf16((rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32))
    b = round_bf16((rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32))
    k = np.arange(64, dtype=np.float32)
    a[:64] = round_bf16(np.float32(1.0) + k * np.float32(2.0 ** -7))
    b[:64] = np.where(k % 3 == 0, -2.0 ** -8, 2.0 ** -8).astype(np.float32)
    a[64:70] = [0.0, -0.0, np.inf, -np.inf, 1.0, 3.0]
    b[64:70] = [-0.0, -0.0, 1.0, -2.0, -1.0, -3.0]
    bits = lambda x: (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # noqa: E731
    g = np.zeros(n + off, np.uint16)
    src = np.zeros(n + off, np.uint16)
    g[off:], src[off:] = bits(a), bits(b)
    ptr = lambda x: x.ctypes.data + off * 2  # noqa: E731
    assert mt.lib.mt_host_accum(ptr(g), ptr(src), n, 3) == mt.MT_OK
    want = bits(ostep.accumulate_bf16(a, b))
    assert np.array_equal(g[off:], want)
    assert mt.lib.mt_host_accum(None, ptr(src), n, 1) == mt.MT_E_INVAL


# ------------------------------------------------------------------ init --
def _init_tile(sh, unit, seed, threads):
    n = mt.unit_elems(sh, unit)
    buf = np.zeros(16 * n, np.uint8)
    assert mt.lib.mt_host_init_unit(C.byref(sh), unit, seed, 0.02, threads, buf.ctypes.data, buf.nbytes) == 0
    return buf, n


def test_init_is_deterministic_across_thread_counts_and_statistically_normal():
    b1, n = _init_tile(CFG1, 0, 1234, 1)
    b2, _ = _init_tile(CFG1, 0, 1234, 7)
    assert np.array_equal(b1, b2)
    b3, _ = _init_tile(CFG1, 0, 1235, 2)
    assert not np.array_equal(b1, b3)
    w = b1[: 2 * n].view(np.uint16)
    master = b1[4 * n: 8 * n].view(np.float32)
    assert np.array_equal((w.astype(np.uint32) << 16).view(np.float32), master)   # master = W
    assert np.all(b1[2 * n: 4 * n] == 0) and np.all(b1[8 * n:] == 0)             # G, m, v zero
    for j in range(9):
        t = mt.tensor_desc(CFG1, 0, j)
        x = master[t["offset"]: t["offset"] + t["rows"] * t["cols"]].astype(np.float64)
        if t["rows"] == 1:
            assert np.all(x == 1.0)
        else:
            assert abs(x.mean()) < 3 * 0.02 / np.sqrt(x.size) + 1e-6
            assert abs(x.std() / 0.02 - 1) < 0.02
            # normal, not uniform: kurtosis ~ 3
            k = np.mean((x - x.mean()) ** 4) / x.var() ** 2
            assert abs(k - 3.0) < 0.15


def test_thread_pool_back_to_back_jobs_match_one_thread():
    """The init runs one pool job per tensor, back to back on one pool, so
    workers woken for one job can arrive while the next is being set up.  Many
    such calls with 8 threads give the one-thread tile every time (and, under
    the ThreadSanitizer build, no report)."""
    ref, _ = _init_tile(CFG1, 1, 99, 1)
    for _ in range(40):
        b, _ = _init_tile(CFG1, 1, 99, 8)
        assert np.array_equal(b, ref)


def test_attention_dkdv_split_count_rule():
    """Automatic splits: none once there are 512 key-tile blocks, else enough
    for 512, at most Hq/Hkv; an explicit count is capped by the group."""
    sp = mt.lib.mt_k_attn_dkdv_splits
    assert sp(8, 1024, 28, 4, 128, 0) == 2          # 256 key-tile blocks
    assert sp(4, 2048, 64, 8, 128, 0) == 1          # 512
    assert sp(1, 131072, 28, 4, 128, 0) == 1
    assert sp(1, 100, 7, 1, 128, 0) == 7
    assert sp(1, 100, 7, 1, 128, 9) == 7
    assert sp(1, 100, 4, 4, 128, 0) == 1            # one query head per group
    assert sp(1, 100, 6, 4, 128, 0) == 0            # not a grouping


def test_attention_backward_work_covers_the_automatic_split():
    """The attention backward's scratch holds D and the base-2 log-sum-exp,
    the scaled dO, the partial maxima (32 lines of 256 bytes), when the
    dK/dV pass splits the fp32 partials
    of every split, and for sequences up to 1024 whose dS fits 1 GiB the
    stored dS (B*Hq*Sp^2 fp16, Sp = S rounded up to 128)."""
    al = lambda x: (x + 255) // 256 * 256
    for B, S, Hq, Hkv, hd, has_ds in [(8, 1024, 28, 4, 128, True), (1, 131072, 28, 4, 128, False),
                                      (1, 300, 7, 1, 64, True), (4, 2048, 40, 8, 128, False),
                                      (16, 1024, 32, 8, 128, True), (17, 1024, 32, 8, 128, False),
                                      (1, 1025, 4, 4, 64, False)]:
        T = B * S
        ns = mt.lib.mt_k_attn_dkdv_splits(B, S, Hq, Hkv, hd, 0)
        part = ns * T * 2 * Hkv * hd if ns > 1 else 0
        sp = (S + 127) // 128 * 128
        ds = B * Hq * sp * sp * 2 if has_ds else 0
        want = al(2 * T * Hq * 4) + al(T * Hq * hd * 2) + 8192 + al(part * 4) + al(ds)
        assert mt.lib.mt_k_attn_bwd_work_bytes(B, S, Hq, Hkv, hd) == want, (B, S, Hq)
    assert mt.lib.mt_k_attn_bwd_work_bytes(1, 100, 6, 4, 128) == 0   # not a grouping


def _split_plan(M, N, K, ws):
    nf, sp, kp = C.c_int32(), C.c_int32(), C.c_int32()
    assert mt.lib.mt_k_gemm_split_plan(M, N, K, ws, C.byref(nf), C.byref(sp), C.byref(kp)) == mt.MT_OK
    return nf.value, sp.value, kp.value


def test_gemm_tail_split_plan():
    """The tail split the direct-form GEMM takes: only a partial last round of
    256 x 256 tiles is cut, every K range is non-empty, the partials fit the
    scratch, and at the 7B layer shapes (T = 8192) the long-K products with a
    partial round split while the gate|up forward product (18.5 rounds of short
    K) and grids of whole rounds do not."""
    T, d, F, nqkv = 8192, 3584, 18944, 4608
    ws = 620 << 20
    shapes = {"qkv": (T, nqkv, d), "o": (T, d, d), "gateup": (T, 2 * F, d), "down": (T, d, F),
              "down_dx": (T, F, d), "down_dw": (d, F, T), "gateup_dx": (T, d, 2 * F), "gateup_dw": (2 * F, d, T),
              "o_dw": (d, d, T), "qkv_dw": (nqkv, d, T), "whole_rounds": (8192, 8192, 8192)}
    plans = {k: _split_plan(*v, ws) for k, v in shapes.items()}
    for name, (M, N, K) in shapes.items():
        n_full, splits, kper = plans[name]
        tiles = -(-M // 256) * -(-N // 256)
        nk = -(-K // 64)
        if splits == 1:
            assert n_full == tiles and kper == nk, name
            continue
        assert n_full == tiles - tiles % 256 and tiles % 256, name
        assert (splits - 1) * kper < nk <= splits * kper, name
        assert (tiles - n_full) * splits * 256 * 1024 <= ws, name
    assert plans["gateup"][1] == 1 and plans["whole_rounds"][1] == 1 and plans["o_dw"][1] == 1
    assert plans["gateup_dx"][1] > 1 and plans["gateup_dw"][1] > 1 and plans["down_dw"][1] > 1
    # no scratch, no split; scratch too small for any split, no split
    assert _split_plan(T, d, 2 * F, 0)[1] == 1
    assert _split_plan(T, d, 2 * F, 1 << 20)[1] == 1


def test_bench_refuses_more_than_one_gpu():
    """The benchmark runs on one GPU: --gpus N > 1 exits with status 2 and a
    message before anything touches a GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
