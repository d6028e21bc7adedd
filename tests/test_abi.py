"""The C-ABI library on the CPU: it loads, exports every declared symbol, its struct
layouts match the binding, and host-side argument checks return the documented
status codes before anything is launched (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


@pytest.fixture(scope="module")
def qsa():
    import sparse_attention_ragged_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(qsa):
    names = declared_functions()
    assert set(names) == set(qsa.EXPORTS), names
    raw = ctypes.CDLL(qsa.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_abi_version_and_struct_sizes(qsa):
    assert qsa.lib.qsa_abi_version() == 5
    assert qsa.lib.qsa_struct_size(0) == ctypes.sizeof(qsa._Cache) == 104
    assert qsa.lib.qsa_struct_size(1) == ctypes.sizeof(qsa._Ragged) == 64
    assert qsa.lib.qsa_struct_size(2) == ctypes.sizeof(qsa.LaunchOptions) == 16
    assert qsa.lib.qsa_struct_size(7) == 0


# Host buffers stand in for device pointers: every call below must fail its host checks
# before any launch, so no pointer is ever dereferenced.
BUF = ctypes.create_string_buffer(4096 + 16)
P = (ctypes.addressof(BUF) + 15) & ~15


def cache(**kw):
    from sparse_attention_ragged_amd import _Cache
    d = dict(blocks=P, dtype=1, reserved0=0, num_pages=4, num_planes=2, num_layers=2, page_size=16,
             num_kv_heads=2, head_dim=128, page_stride=-1, lookup_table=P, max_pages=4,
             cache_lengths=P, max_cache_length=10, reserved1=0)
    d.update(kw)
    return _Cache(**d)


def ragged(**kw):
    from sparse_attention_ragged_amd import _Ragged
    d = dict(q=P, dtype=1, reserved0=0, total_q=3, num_q_heads=8, head_dim=128, batch=2,
             input_row_offsets=P, max_prompt_length=2, reserved1=0)
    d.update(kw)
    return _Ragged(**d)


def call_qsa(qsa, q=None, kv=None, layer=0, W=16, out=P, out_dtype=1, ws=None, wsb=0, opts=None,
             scale=0.1, idx=P, counts=P):
    q = q or ragged()
    kv = kv or cache()
    return qsa.lib.qsa_sparse_attention(out, out_dtype, ctypes.byref(q), ctypes.byref(kv), layer, idx, W,
                                        counts, scale, ctypes.byref(opts) if opts else None, ws, wsb, None)


def msg(qsa):
    return qsa.lib.qsa_last_error().decode()


@pytest.mark.parametrize("case,status", [
    (dict(q_kw=dict(dtype=0)), 3),                      # q dtype != cache dtype
    (dict(kv_kw=dict(num_kv_heads=3)), 2),              # 8 q heads not a multiple of 3
    (dict(kv_kw=dict(head_dim=64)), 2),                 # head_dim mismatch
    (dict(layer=2), 2),                                 # layer_idx >= num_layers
    (dict(kv_kw=dict(page_stride=100)), 2),             # stride below a packed page
    (dict(kv_kw=dict(num_planes=1)), 2),                # K/V cache needs two planes
    (dict(kv_kw=dict(blocks=0)), 1),                    # NULL blocks
    (dict(kv_kw=dict(blocks=P + 2)), 2),                # misaligned blocks
    (dict(out=0), 1),                                   # NULL out
    (dict(out_dtype=2), 3),                             # e4m3 output is not offered
    (dict(idx=0), 1),                                   # NULL token_indices
    (dict(W=-1), 2),                                    # negative width
    (dict(scale=float("nan")), 2),                      # non-finite scale
    (dict(q_kw=dict(num_q_heads=48), kv_kw=dict(num_kv_heads=2)), 4),   # group 24 not built
    (dict(q_kw=dict(head_dim=96), kv_kw=dict(head_dim=96)), 4),         # head_dim 96 not built
])
def test_validation_errors(qsa, case, status):
    q = ragged(**case.get("q_kw", {}))
    kv = cache(**case.get("kv_kw", {}))
    args = {k: v for k, v in case.items() if k not in ("q_kw", "kv_kw")}
    assert call_qsa(qsa, q=q, kv=kv, **args) == status, msg(qsa)
    assert msg(qsa)


def test_workspace_checks(qsa):
    q, kv = ragged(), cache()
    n = ctypes.c_size_t(0)
    o = qsa.LaunchOptions(4, 0, 0, 0)
    assert qsa.lib.qsa_sparse_attention_workspace_size(ctypes.byref(q), ctypes.byref(kv), 64,
                                                       ctypes.byref(o), ctypes.byref(n)) == 0
    # 4 splits x 3 rows x 8 heads x (128 acc + 2) fp32, acc padded to 256 bytes
    acc = 4 * 3 * 8 * 128 * 4
    assert n.value == ((acc + 255) // 256) * 256 + 4 * 3 * 8 * 2 * 4
    assert call_qsa(qsa, opts=o, W=64) == 5 and "workspace" in msg(qsa)
    assert call_qsa(qsa, opts=o, W=64, ws=P, wsb=16) == 5
    one = qsa.LaunchOptions(1, 0, 0, 0)
    assert qsa.lib.qsa_sparse_attention_workspace_size(ctypes.byref(q), ctypes.byref(kv), 64,
                                                       ctypes.byref(one), ctypes.byref(n)) == 0
    assert n.value == 0


@pytest.mark.parametrize("opts", [(65, 0, 0, 0), (0, 9, 0, 0), (0, 16, 0, 0), (0, 0, 9, 0), (-1, 0, 0, 0),
                                  (0, 0, 0, 2), (0, 0, 0, 1), (0, 0, 0, -1)])
def test_bad_launch_options(qsa, opts):
    assert call_qsa(qsa, opts=qsa.LaunchOptions(*opts)) == 4, msg(qsa)


def test_ragged_attention_checks(qsa):
    """Dense ragged attention: every bad argument is refused on the host, before any launch."""
    f = qsa.lib.qsa_ragged_attention

    def call(q=None, hkv=2, causal=1, window=-1, opts=None, k=P, v=P, out=P, scale=0.1):
        q = q or ragged()
        return f(out, 1, ctypes.byref(q), k, v, hkv, causal, window, scale,
                 ctypes.byref(opts) if opts else None, None, 0, None)

    assert call(causal=2) == 2                          # causal is 0 or 1
    assert call(window=0) == 2 and call(window=-3) == 2   # -1 (none) or >= 1
    assert call(hkv=3) == 2                             # 8 q heads not a multiple of 3
    assert call(hkv=0) == 2
    assert call(q=ragged(num_q_heads=48), hkv=2) == 4   # group 24 not built here
    assert call(q=ragged(head_dim=96)) == 4             # head_dim 96 not built
    assert call(q=ragged(max_prompt_length=0)) == 2     # the split plan needs the longest sequence
    assert call(k=0) == 1 and call(v=0) == 1 and call(out=0) == 1
    assert call(k=P + 4) == 2                           # 16-byte alignment
    assert call(scale=float("nan")) == 2
    assert call(opts=qsa.LaunchOptions(0, 0, 0, 2)) == 4 and "reserved" in msg(qsa)
    n = ctypes.c_size_t(7)
    assert qsa.lib.qsa_ragged_attention_workspace_size(ctypes.byref(ragged()), 2, 1, -1, None,
                                                       ctypes.byref(n)) == 0
    assert qsa.lib.qsa_ragged_attention_workspace_size(ctypes.byref(ragged()), 2, 5, -1, None,
                                                       ctypes.byref(n)) == 2 and n.value == 0


def test_block_sparse_checks(qsa):
    q, kv = ragged(), cache()
    f = qsa.lib.qsa_block_sparse_attention
    call = lambda **k: f(k.get("out", P), ctypes.byref(k.get("q", q)), ctypes.byref(k.get("kv", kv)),
                         k.get("layer", 0), k.get("idx", P), k.get("topk", 4), k.get("bs", 8), 0.1,
                         None, None, None, None, 0, None)
    assert call(bs=5) == 2            # block size must divide the page size
    assert call(topk=0) == 2
    assert call(q=ragged(dtype=0), kv=cache(dtype=0)) == 3     # fp32 is not offered here
    assert call(idx=0) == 1


def test_latent_checks(qsa):
    q = ragged(num_q_heads=16, head_dim=512)
    swa = cache(num_planes=1, num_kv_heads=1, head_dim=512, num_layers=1)
    comp = cache(num_planes=1, num_kv_heads=1, head_dim=512, num_layers=1)
    f = qsa.lib.qsa_latent_sparse_attention
    call = lambda **k: f(P, 1, ctypes.byref(k.get("q", q)), ctypes.byref(k.get("swa", swa)),
                         ctypes.byref(k.get("comp", comp)), 0, k.get("window", 128), P, 64,
                         k.get("sink", P), 0.1, None, None, 0, None)
    assert call(window=0) == 2
    assert call(swa=cache(num_planes=2, num_kv_heads=1, head_dim=512)) == 2
    assert call(comp=cache(num_planes=1, num_kv_heads=2, head_dim=512, num_layers=1)) == 2
    assert call(sink=0) in (1, 4)     # NULL sink (or an unbuilt shape) is refused


def test_binding_refuses_cpu_tensors(qsa):
    import torch
    q = torch.zeros(2, 4, 64)
    with pytest.raises(ValueError):
        qsa.sparse_attention(q, torch.zeros(2, dtype=torch.int32), None, 0, torch.zeros(2, 4, dtype=torch.int32),
                             torch.zeros(2, dtype=torch.int32), 0.1)


def test_compress_keys_checks(qsa):
    """Key compression: every bad argument is refused on the host, before any launch;
    an empty batch or a zero block bound returns OK without launching anything."""
    f = qsa.lib.qsa_compress_keys
    ind = dict(num_kv_heads=1, max_cache_length=60, max_pages=4, page_size=16)

    def call(kv=None, out=P, max_blocks=16, gamma=P, freqs=P, fdt=0, npos=64, rd=64, counts=P, batch=2,
             layer=0, mpl=4, ratio=4, eps=1e-6):
        kv = kv or cache(**ind)
        return f(out, max_blocks, gamma, freqs, fdt, npos, rd, counts, ctypes.byref(kv), batch, layer, mpl,
                 ratio, eps, None)

    assert call(kv=cache(num_kv_heads=2)) == 2 and "one head" in msg(qsa)
    assert call(kv=cache(dtype=2, **ind)) == 3                       # e4m3 keys are not offered
    assert call(kv=cache(head_dim=96, **ind)) == 4                   # 192-byte rows not built
    assert call(kv=cache(num_planes=1, **ind)) == 2                  # the indexer group has K and V planes
    assert call(layer=2) == 2
    assert call(ratio=0) == 2
    assert call(rd=3) == 2 and call(rd=130) == 2 and call(rd=-2) == 2
    assert call(fdt=2) == 3
    assert call(eps=float("nan")) == 2 and call(eps=-1.0) == 2
    assert call(max_blocks=-1) == 2 and call(batch=-1) == 2
    # blocks up to min(16, (60 + 4) / 4) = 16 start at positions up to 60: the table needs 61 rows
    assert call(npos=60) == 2 and "positions" in msg(qsa)
    assert call(gamma=0) == 1 and call(counts=0) == 1 and call(out=0) == 1
    assert call(freqs=0) == 1                                        # needed when rd > 0
    assert call(out=P + 8) == 2 and call(gamma=P + 4) == 2
    assert call(freqs=P + 2) == 2                                    # fp32 pairs are 8-byte aligned
    # nothing to compute: OK, no launch
    assert call(batch=0) == 0
    assert call(max_blocks=0) == 0
    assert call(kv=cache(num_kv_heads=1, max_cache_length=2, max_pages=4, page_size=16), mpl=1) == 0  # 3 / 4 = 0
    # a max_cache_length of 0 bounds nothing: blocks up to min(16, 64 addressable / 4) = 16
    # start at positions up to 60, so a 60-row table is refused again
    assert call(kv=cache(num_kv_heads=1, max_cache_length=0, max_pages=4, page_size=16), mpl=1, npos=60) == 2


def test_select_blocks_checks(qsa):
    """Block selection: bad arguments are refused on the host before any launch; zero
    rows return OK without launching."""
    f = qsa.lib.qsa_select_blocks
    n = ctypes.c_size_t(0)

    def q(**kw):
        d = dict(num_q_heads=1, head_dim=128, max_prompt_length=1)
        d.update(kw)
        return ragged(**d)

    def call(qd=None, W=2051, idx=P, counts=P, blocks=P, keys=P, max_blocks=64, cl=P, mcl=1000, ratio=4, topk=512,
             ws=P, wsb=1 << 30):
        qd = qd or q()
        return f(idx, W, counts, blocks, ctypes.byref(qd), keys, max_blocks, cl, mcl, ratio, topk, ws, wsb, None)

    assert call(qd=q(num_q_heads=2)) == 2                            # one index query per row
    assert call(qd=q(dtype=2)) == 3                                  # e4m3 not offered
    assert call(qd=q(head_dim=96)) == 4                              # 192-byte rows not built
    assert call(ratio=0) == 2 and call(topk=-1) == 2 and call(max_blocks=-1) == 2
    assert call(W=2050) == 2 and "selection_width" in msg(qsa)      # 512 * 4 + 3 positions
    assert call(max_blocks=40000, mcl=0, qd=q(max_prompt_length=0)) == 4    # over 32768 candidates
    assert call(idx=0) == 1 and call(counts=0) == 1 and call(cl=0) == 1 and call(keys=0) == 1
    assert call(keys=P + 4) == 2
    assert call(ws=0) == 5 and call(wsb=16) == 5 and call(ws=P + 8) == 5
    # workspace: fp32 scores for min(max_blocks, (1000 + 1) / 4) = 64 candidates of 3 rows
    assert qsa.lib.qsa_select_blocks_workspace_size(ctypes.byref(q()), 64, 4, 512, 1000, ctypes.byref(n)) == 0
    assert n.value == 3 * 64 * 4
    assert qsa.lib.qsa_select_blocks_workspace_size(ctypes.byref(q()), 640, 4, 512, 1000, ctypes.byref(n)) == 0
    assert n.value == 3 * 250 * 4
    assert call(qd=q(total_q=0)) == 0                                # nothing to do
    # max_cache_length 0 says nothing about the cache: max_blocks alone bounds the candidates
    assert qsa.lib.qsa_select_blocks_workspace_size(ctypes.byref(q()), 640, 4, 512, 0, ctypes.byref(n)) == 0
    assert n.value == 3 * 640 * 4
    assert call(max_blocks=40000, mcl=0) == 4                        # then max_blocks itself is checked


def test_no_alloc_refuses_plans_beyond_its_scratch(qsa):
    """qsa_sparse_attention_no_alloc checks the plan's split-K partials against the
    library's scratch size on the host and refuses larger plans before touching the
    device (host buffers stand in for device pointers here)."""
    f = qsa.lib.qsa_sparse_attention_no_alloc
    q = ragged(total_q=5000, batch=2)
    # 64 splits x 5000 rows x 8 heads x (128 + 2) fp32 = 1.3 GB of partials
    big = qsa.LaunchOptions(64, 0, 0, 0)
    assert f(P, 1, ctypes.byref(q), ctypes.byref(cache()), 0, P, 2048, P, 0.1, ctypes.byref(big), None) == 5
    assert "scratch" in msg(qsa)
    # the same argument checks as the workspace entry point
    assert f(P, 1, ctypes.byref(q), ctypes.byref(cache()), 5, P, 2048, P, 0.1, None, None) == 2
    assert f(P, 7, ctypes.byref(q), ctypes.byref(cache()), 0, P, 2048, P, 0.1, None, None) == 3
    assert f(P, 1, ctypes.byref(q), ctypes.byref(cache()), 0, P, 2048, P, float("inf"), None, None) == 2
    assert qsa.NO_ALLOC_SCRATCH_BYTES == 16 << 20
    text = open(HEADER).read()
    assert "#define QSA_NO_ALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in text


def test_gather_replay_checks(qsa):
    f = qsa.lib.qsa_gather_replay
    assert f(P, 1 << 20, P, P, 4, 16, 200, 0, P, None) == 2        # row_bytes not a supported size
    assert f(P, 1 << 20, P, P, 4, 0, 256, 0, P, None) == 2         # max_keys >= 1
    assert f(P, 1 << 20, P, P, 4, (1 << 20) + 1, 256, 0, P, None) == 2
    assert f(P, 1 << 20, P, P, 1 << 31, 16, 256, 0, P, None) == 2  # items below 2^31
    assert f(P, 1 << 20, None, P, 4, 16, 256, 0, P, None) == 1
    assert f(P, 1 << 20, P, None, 4, 16, 256, 0, P, None) == 1
    assert f(P, 1 << 20, P, P, 4, 16, 256, 0, None, None) == 1
    assert f(P + 4, 1 << 20, P, P, 4, 16, 256, 0, P, None) == 2    # 16-byte alignment
    assert f(P, 1 << 20, P, P, 4, 16, 256, 8, P, None) == 2        # plane_delta a multiple of 16
    assert f(P, 128, P, P, 4, 16, 256, 0, P, None) == 2            # region holds a row
    assert f(None, 0, None, None, 0, 16, 256, 0, None, None) == 0  # no items: nothing to do


def test_stream_read_checks(qsa):
    f = qsa.lib.qsa_stream_read
    assert f(P, 1024, P, 0, None) == 2                 # grid >= 1
    assert f(P, 1024, P, (1 << 20) + 1, None) == 2
    assert f(P + 4, 1024, P, 8, None) == 2             # 16-byte alignment
    assert f(P, 1000, P, 8, None) == 2                 # whole 16-byte chunks
    assert f(P, 1024, None, 8, None) == 1
    assert f(None, 1024, P, 8, None) == 1
