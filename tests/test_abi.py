"""The C ABI library loads, exports every symbol include/lca.h declares, and
rejects bad arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import long_context_attention_19_amd as lca

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "lca.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_UNSUP, E_WS = 0, -1, -2, -3, -4, -5
FAKE = 0x10000          # an aligned address that validation failures never dereference
MIS = 0x10001           # misaligned


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int32_t|size_t|const char\*)\s+(lca_\w+)\s*\(", txt, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lca._lib, n), n          # ctypes resolves the exported symbol
    assert sorted(lca.EXPORTED) == names        # the binding covers exactly the header


def test_version_and_struct_layout():
    assert lca.abi_version() == 8
    # 4 int32, 10 pointers, 4 window pointers, int32 window (+4 padding), sink pointer,
    # int32 idx_format, int32 kv_format
    assert ctypes.sizeof(lca.LcaLayer) == 16 + 10 * 8 + 4 * 8 + 8 + 8 + 8
    assert lca.LcaLayer.window.offset == 16 + 14 * 8
    assert lca.LcaLayer.sink.offset == 16 + 14 * 8 + 8
    assert lca.LcaLayer.idx_format.offset == 16 + 14 * 8 + 16
    assert lca.LcaLayer.kv_format.offset == 16 + 14 * 8 + 20


def L():
    return lca._lib


def test_kv_compress_validation():
    f = L().lca_kv_compress
    assert f(None, None, 0, 100, 128, 4, None, None, None) == OK       # empty batch: nothing to do
    assert f(FAKE, FAKE, 2, 100, 12, 4, FAKE, FAKE, None) == E_UNSUP   # head_dim % 8
    assert f(FAKE, FAKE, 2, 100, 128, 0, FAKE, FAKE, None) == E_SHAPE  # ratio 0
    assert f(None, FAKE, 2, 100, 128, 4, FAKE, FAKE, None) == E_NULL
    assert f(MIS, FAKE, 2, 100, 128, 4, FAKE, FAKE, None) == E_ALIGN
    assert "aligned" in lca.last_error()


@pytest.mark.parametrize("fn", ["lca_csa_index_select", "lca_csa_index_select_fp4"])
def test_index_select_validation(fn):
    f = getattr(L(), fn)
    # q, q_off, q_pos, k, ent_off, batch, max_q, max_entries, d_idx, c, k, idx, count, n_vis,
    # ws, ws_bytes, stream
    args = [FAKE] * 5 + [2, 32, 1000, 64, 4, 256, FAKE, FAKE, None, None, 0, None]
    bad = list(args); bad[8] = 32
    assert f(*bad) == E_UNSUP                          # d_idx other than 64
    bad = list(args); bad[10] = 0
    assert f(*bad) == E_SHAPE                          # k = 0
    bad = list(args); bad[9] = 0
    assert f(*bad) == E_SHAPE                          # ratio 0
    bad = list(args); bad[3] = None
    assert f(*bad) == E_NULL
    bad = list(args); bad[0] = MIS
    assert f(*bad) == E_ALIGN
    bad = list(args); bad[5] = 0
    assert f(*bad) == OK                               # empty batch: nothing to do
    # decode-sized batches (fewer than 16 query rows per sequence) need the workspace
    need = L().lca_csa_index_select_workspace_bytes(2, 8, 1000, 256)
    assert need > 0
    assert L().lca_csa_index_select_workspace_bytes(2, 32, 1000, 256) == 0   # prefill form
    bad = list(args); bad[6] = 8
    assert f(*bad) == E_WS
    bad[14] = FAKE; bad[15] = need - 1
    assert f(*bad) == E_WS
    bad[15] = need; bad[14] = MIS
    assert f(*bad) == E_ALIGN
    bad = list(args); bad[6] = 8; bad[7] = 2048 * 2048 + 1; bad[14] = FAKE; bad[15] = 1 << 40
    assert f(*bad) == E_UNSUP                          # beyond 4M entries per row


def test_index_select_noalloc_validation():
    """The allocation-free form rejects, before any HIP call, a batch whose workspace
    exceeds its fixed scratch; other argument errors are those of the workspace form."""
    f = L().lca_csa_index_select_noalloc
    cap = 8 << 20
    # q, q_off, q_pos, k, ent_off, batch, max_q, max_entries, d_idx, c, k, idx, count, n_vis,
    # stream
    args = [FAKE] * 5 + [2, 8, 1000, 64, 4, 256, FAKE, FAKE, None, None]
    bad = list(args); bad[8] = 32
    assert f(*bad) == E_UNSUP
    bad = list(args); bad[3] = None
    assert f(*bad) == E_NULL
    bad = list(args); bad[5] = 0
    assert f(*bad) == OK
    # 26 rows of 4M entries fit the 8 MiB scratch, 27 do not
    ws = L().lca_csa_index_select_workspace_bytes
    assert ws(26, 1, 1 << 22, 2048) <= cap < ws(27, 1, 1 << 22, 2048)
    bad = list(args); bad[5] = 27; bad[6] = 1; bad[7] = 1 << 22; bad[10] = 2048
    assert f(*bad) == E_WS
    assert "scratch" in lca.last_error()
    bad[7] = (1 << 22) + 1
    assert f(*bad) == E_UNSUP                          # beyond 4M entries per row


def test_index_select_workspace_bounds_the_candidates():
    """The candidate region holds every row the budget rule allows: for each visible
    count nv in (k, max_n], ceil(nv / 2048) chunks of the rule's slot size."""
    import math

    def slot(nv, k):   # the rule as the header states it
        e = min(2048, -(-k * 2048 // nv))
        sq = math.isqrt(e - 1) + 1
        target = min(2048, e + 6 * sq + 8)
        return min(2048, target + 16)

    f = L().lca_csa_index_select_workspace_bytes
    for max_n, k in [(5000, 256), (262144, 2048), (70001, 2048), (3000, 2048), (2048, 2048)]:
        rows = 3
        need = max((-(-nv // 2048)) * slot(nv, k) for nv in range(k + 1, max_n + 1)) \
            if max_n > k else 0
        nch = max(1, -(-max_n // 2048))
        al = lambda x: (x + 255) // 256 * 256
        expect = al(rows * 4) + al(rows * 16) + al(rows * nch * 4) + al(rows * max(need, 1) * 4)
        assert f(rows, 1, max_n, k) == expect, (max_n, k)
    assert min(slot(nv, 2048) for nv in range(2049, 1 << 22, 997)) >= 31


def test_kv_compress_kv8_validation():
    f = L().lca_kv_compress_kv8
    assert f(None, None, 0, 100, 4, None, None, None) == OK            # empty batch: nothing to do
    assert f(FAKE, FAKE, 2, 3, 4, None, None, None) == OK              # no complete block
    assert f(FAKE, FAKE, 2, 100, 0, FAKE, FAKE, None) == E_SHAPE       # ratio 0
    assert f(FAKE, FAKE, 2, 100, 5000, FAKE, FAKE, None) == E_SHAPE    # ratio above 4096
    assert f(FAKE, FAKE, -1, 100, 4, FAKE, FAKE, None) == E_SHAPE
    assert f(FAKE, FAKE, 2, 100, 4, None, FAKE, None) == E_NULL
    assert f(FAKE, FAKE, 2, 100, 4, MIS, FAKE, None) == E_ALIGN
    assert "aligned" in lca.last_error()


def test_index_score_validation():
    f = L().lca_csa_index_score
    args = [FAKE] * 5 + [2, 1, 1000, 64, 4, FAKE, 1000, FAKE, None, 0, None]
    bad = list(args); bad[8] = 32
    assert f(*bad) == E_UNSUP                          # d_idx != 64
    bad = list(args); bad[11] = 999
    assert f(*bad) == E_SHAPE                          # ld below max_entries
    bad = list(args); bad[0] = None
    assert f(*bad) == E_NULL
    bad = list(args); bad[3] = MIS
    assert f(*bad) == E_ALIGN
    bad = list(args); bad[13] = FAKE; bad[14] = 100
    assert f(*bad) == E_WS                             # fused histogram needs rows * 8 KiB


def test_topk_validation_and_sizes():
    f = L().lca_csa_topk_select
    args = [FAKE, 4096, 4, 4096, FAKE, 256, FAKE, FAKE, FAKE, 1 << 30, 0, None]
    bad = list(args); bad[5] = 0
    assert f(*bad) == E_SHAPE                          # k = 0
    bad = list(args); bad[9] = 16
    assert f(*bad) == E_WS
    bad = list(args); bad[10] = 7
    assert f(*bad) == E_SHAPE                          # unknown flag
    bad = list(args); bad[3] = 1 << 30; bad[1] = 1 << 30
    assert f(*bad) == E_UNSUP                          # beyond the resolver's chunk table
    edge = list(args); edge[3] = 1024 * 4096; edge[1] = 1024 * 4096
    assert f(*edge[:9], 0, 0, None) == E_WS            # the longest row passes the size checks
    edge[3] += 1
    assert f(*edge) == E_UNSUP                         # one entry more does not
    bad = list(args); bad[6] = None
    assert f(*bad) == E_NULL
    n1 = lca.csa_topk_workspace_bytes(4, 262144, 2048)
    n2 = lca.csa_topk_workspace_bytes(4, 2 * 262144, 2048)
    assert 0 < n1 < n2


def test_attention_validation():
    f = L().lca_csa_sparse_attn
    args = [FAKE] * 5 + [4, 1, FAKE, FAKE, 2048, 64, 128, 0.088, 0, FAKE, None, FAKE, 1 << 30, None]
    bad = list(args); bad[11] = 64
    assert f(*bad) == E_UNSUP                          # head_dim 64
    for h in (8, 48, 80):
        bad = list(args); bad[10] = h
        assert f(*bad) == E_UNSUP                      # heads must be 16, 32 or 64k
    bad = list(args); bad[9] = 0
    assert f(*bad) == E_SHAPE
    bad = list(args); bad[7] = None
    assert f(*bad) == E_NULL
    bad = list(args); bad[17] = 10
    assert f(*bad) == E_WS                             # 32 splits need partial buffers
    bad = list(args); bad[12] = float("nan")
    assert f(*bad) == E_SHAPE
    g = L().lca_hca_dense_attn
    gargs = [FAKE] * 6 + [8, 1, 1024, 128, 64, 128, 0.088, 0, FAKE, None, FAKE, 1 << 30, None]
    bad = list(gargs); bad[9] = 0
    assert g(*bad) == E_SHAPE                          # ratio 0
    bad = list(gargs); bad[5] = None
    assert g(*bad) == E_NULL                           # q_pos
    bad = list(gargs); bad[8] = (1 << 24) + 1
    assert g(*bad) == E_UNSUP                          # 32-bit row offsets per sequence
    assert lca.attn_workspace_bytes(4, 64, 1, 0) == lca.attn_workspace_bytes(4, 64, 1, 32)
    assert lca.attn_workspace_bytes(4096, 64, 4096, 0) == 0      # prefill rows are not split


def test_hybrid_validation():
    arr = (lca.LcaLayer * 2)()
    arr[0] = lca.LcaLayer(lca.LCA_LAYER_CSA, 4, 2048, 1000, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          None, FAKE, FAKE)
    arr[1] = lca.LcaLayer(7, 128, 0, 100, FAKE, None, FAKE, FAKE, None, FAKE, FAKE, None, None,
                          None)
    need = lca.hybrid_workspace_bytes(arr, 16, 1, 64)
    assert need > 0
    f = L().lca_hybrid_layer_step
    assert f(arr, 2, FAKE, FAKE, 16, 1, 64, 128, 0.088, FAKE, need, None) == E_SHAPE  # bad kind
    assert f(arr, 2, FAKE, FAKE, 16, 1, 64, 128, 0.088, FAKE, need - 1, None) == E_WS
    arr[1].kind = lca.LCA_LAYER_HCA
    assert f(arr, 2, FAKE, FAKE, 16, 1, 64, 96, 0.088, FAKE, need, None) == E_UNSUP   # head_dim
    arr[0].idx = None
    assert f(arr, 2, FAKE, FAKE, 16, 1, 64, 128, 0.088, FAKE, need, None) == E_NULL


def test_hybrid_timing_validation():
    assert L().lca_hybrid_timing_read(None, 4) == E_NULL


def test_no_oracle_in_product_path():
    # the product package never imports the oracle
    root = os.path.dirname(os.path.abspath(lca.__file__))
    for dp, _, fs in os.walk(root):
        for fn in fs:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dp, fn)).read()
                assert "oracle" not in src.replace("the oracle", ""), fn


def test_window_attn_validation():
    f = L().lca_window_attn
    args = lambda **kw: [kw.get("q", FAKE), kw.get("wk", FAKE), kw.get("wv", FAKE), FAKE, FAKE,
                         FAKE, FAKE, kw.get("B", 2), kw.get("mq", 1), kw.get("win", 128),
                         kw.get("H", 64), kw.get("D", 128), ctypes.c_float(0.088),
                         kw.get("out", FAKE), kw.get("lse", FAKE), None]
    assert f(*args(win=0, q=None, lse=None)) == OK        # no window: nothing to do
    assert f(*args(B=0, q=None)) == OK                     # empty batch
    assert f(*args(D=64)) == E_UNSUP
    assert f(*args(H=48)) == E_UNSUP
    assert f(*args(win=-1)) == E_SHAPE
    assert f(*args(lse=None)) == E_NULL                    # the merge needs the branch's lse
    assert f(*args(wk=None)) == E_NULL
    assert f(*args(wv=MIS)) == E_ALIGN
    assert "aligned" in lca.last_error()


def test_attn_sink_validation():
    f = L().lca_attn_sink
    args = lambda **kw: [kw.get("out", FAKE), kw.get("lse", FAKE), kw.get("sink", FAKE),
                         ctypes.c_int64(kw.get("rows", 4)), kw.get("H", 64), kw.get("D", 128), None]
    assert f(*args(rows=0, out=None)) == OK               # nothing to do
    assert f(*args(D=64)) == E_UNSUP
    assert f(*args(rows=-1)) == E_SHAPE
    assert f(*args(H=0)) == E_SHAPE
    assert f(*args(rows=1 << 22, H=64)) == E_SHAPE        # rows x heads above 2^27
    assert f(*args(lse=None)) == E_NULL
    assert f(*args(sink=None)) == E_NULL
    assert f(*args(out=MIS)) == E_ALIGN
    assert "aligned" in lca.last_error()


def test_index_score_fp4_validation():
    f = L().lca_csa_index_score_fp4
    args = lambda **kw: [kw.get("q", FAKE), FAKE, FAKE, kw.get("k", FAKE), FAKE, kw.get("B", 2),
                         1, 100, kw.get("d", 64), 4, kw.get("s", FAKE), ctypes.c_int64(kw.get("ld", 100)),
                         FAKE, None, 0, None]
    assert f(*args(B=0, q=None)) == OK
    assert f(*args(d=128)) == E_UNSUP
    assert f(*args(ld=98)) == E_SHAPE
    assert f(*args(k=None)) == E_NULL
    assert f(*args(q=MIS)) == E_ALIGN


def test_kv8_attention_validation():
    f = L().lca_hca_dense_attn_kv8
    args = lambda **kw: [FAKE, kw.get("k", FAKE), FAKE, FAKE, FAKE, FAKE, 2, 1, 100, 128,
                         kw.get("H", 64), 128, ctypes.c_float(0.088), 0, FAKE, FAKE, FAKE,
                         1 << 20, None]
    assert f(*args(H=16)) == E_UNSUP                       # 64-head blocks only
    assert "multiple of 64" in lca.last_error()
    assert f(*args(k=None)) == E_NULL
    assert f(*args(k=MIS)) == E_ALIGN
    g = L().lca_csa_sparse_attn_kv8
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1, FAKE, FAKE, 256, 32, 128, ctypes.c_float(0.088),
             0, FAKE, FAKE, FAKE, 1 << 20, None) == E_UNSUP
