"""C-ABI library: symbols, the argument contract and its error texts (CPU only).

The contract and its order come from candle's FlashAttentionVarLen forward as
the error-explainer pages quote it; the expected texts are read from
tests/golden/error_messages.txt (each line cites its page).  No compute call is
made here: fa_varlen_check and fa_varlen_workspace_bytes are pure host code.
"""
import os
import re

import pytest

import varlen_flash_attention_fa_amd as fa
from varlen_flash_attention_fa_amd import desc, FA_DTYPE_BF16, FA_DTYPE_I32

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.lib_path()):
        from varlen_flash_attention_fa_amd import build
        build.build()
    return fa.load()


def golden():
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", "error_messages.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, text, cite = [x.strip() for x in line.split("|")]
        rows.append((int(code), text, cite))
    return rows


def render(template, **vals):
    """Fill a golden template: {name} / {name:?} from vals, bare {:?} in order."""
    seq = list(vals.pop("_seq", []))
    out = template
    for key, val in vals.items():
        out = out.replace("{%s:?}" % key, val).replace("{%s}" % key, val)
    while "{:?}" in out:
        out = out.replace("{:?}", seq.pop(0), 1)
    return out


def tmpl(prefix):
    hits = [g for g in golden() if g[1] == prefix] or [g for g in golden() if g[1].startswith(prefix)]
    assert len(hits) == 1, prefix
    return hits[0]


def check(q, k, v, out=None, batch=2, bt=None, page=0):
    rc = fa.fa_varlen_check(q, k, v, out, batch, bt, page)
    return rc, fa.fa_last_error() if rc else ""


def dl(xs):
    return "[" + ", ".join(str(x) for x in xs) + "]"


# ------------------------------------------------------------------ symbols

def test_exports_every_declared_symbol(lib):
    header = open(os.path.join(ROOT, "include", "fa_varlen.h")).read()
    names = re.findall(r"^(?:int|size_t|const char\*)\s+(fa_\w+)\s*\(", header, re.M)
    assert {"fa_varlen_check", "fa_varlen_workspace_bytes", "fa_varlen_fwd",
            "fa_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_every_golden_text_is_in_the_library_source():
    # the C ABI raises the tensor texts; the offsets arrays reach it as bare
    # pointers, so their layout texts are raised by the binding
    pkg = os.path.join(ROOT, "varlen_flash_attention_fa_amd")
    src = open(os.path.join(pkg, "csrc", "fa_api.cpp")).read() + open(os.path.join(pkg, "__init__.py")).read()
    for code, text, _ in golden():
        fixed = re.split(r"\{[^}]*\}", text)[0].strip()
        assert fixed in src, text


# --------------------------------------------------------------- valid calls

Q = desc([86, 4, 64])
K3 = desc([86, 2, 64])
BT = desc([3, 4], dtype=FA_DTYPE_I32)
KP = desc([10, 32, 2, 64])


def test_valid_nonpaged_and_paged(lib):
    assert check(Q, K3, K3, Q, batch=3)[0] == 0
    assert check(Q, KP, KP, Q, batch=3, bt=BT, page=32)[0] == 0


def test_page_size_without_block_table_is_ignored(lib):
    # page_block_size only matters once a block table makes the call paged
    assert check(Q, K3, K3, Q, batch=3, page=16)[0] == 0


# -------------------------------------------------------- quoted checks, order

def test_rank3_message(lib):
    code, t, _ = tmpl("flash-attn-varlen expects input tensors of rank 3")
    rc, msg = check(desc([2, 86, 4, 64]), K3, K3)
    assert rc == code and msg == render(t, q_rank="4", k_rank="3", v_rank="3")
    rc, msg = check(Q, desc([86, 2, 64]), desc([1, 86, 2, 64]))
    assert rc == code and msg == render(t, q_rank="3", k_rank="3", v_rank="4")
    assert not msg.endswith(")")   # the quoted text has no closing parenthesis


def test_rank4_message_when_paged(lib):
    code, t, _ = tmpl("flash-attn-varlen paged expects")
    rc, msg = check(Q, K3, K3, batch=3, bt=BT, page=32)
    assert rc == code and msg == render(t, k_rank="3", v_rank="3")
    # q of the wrong rank is reported by the rank-3 check first, even when paged
    rc, msg = check(desc([86, 4]), K3, K3, batch=3, bt=BT, page=32)
    assert msg.startswith("flash-attn-varlen expects input tensors of rank 3")


def test_contiguity_messages_in_order(lib):
    qs = desc([86, 4, 64], [512, 128, 2])
    ks = desc([86, 2, 64], [256, 128, 2])
    for name, args, stride in (("q", (qs, ks, ks), [512, 128, 2]), ("k", (Q, ks, ks), [256, 128, 2]),
                               ("v", (Q, K3, ks), [256, 128, 2])):
        code, t, _ = tmpl("the last dim of %s" % name)
        rc, msg = check(*args, batch=3)
        assert rc == code and msg == render(t, **{"%s_stride" % name: dl(stride)})


def test_paged_shape_chain_order(lib):
    # v differs from k -> reported before anything about q or page size
    code, t, _ = tmpl("shape mismatch k")
    v_bad = desc([10, 32, 2, 32])
    rc, msg = check(Q, KP, v_bad, batch=3, bt=BT, page=0)
    assert rc == code and msg == render(t, _seq=[dl([10, 32, 2, 64]), dl([10, 32, 2, 32])])
    # head size of k differs from q -> before the page size checks
    code, t, _ = tmpl("shape mismatch q {:?} and k")
    k_bad = desc([10, 32, 2, 80])
    rc, msg = check(Q, k_bad, k_bad, batch=3, bt=BT, page=0)
    assert rc == code and msg == render(t, _seq=[dl([86, 4, 64]), dl([10, 32, 2, 80])])


def test_missing_page_size(lib):
    code, t, _ = tmpl("paged flash-attn requires page_block_size")
    for page in (0, -32):
        rc, msg = check(Q, KP, KP, batch=3, bt=BT, page=page)
        assert rc == code and msg == t


def test_page_size_mismatch(lib):
    code, t, _ = tmpl("page_block_size {")
    rc, msg = check(Q, KP, KP, batch=3, bt=BT, page=64)
    assert rc == code and msg == render(t, page_block_size_arg="64", _seq=[dl([10, 32, 2, 64])])
    assert "does not match k shape" in msg


def test_page_size_multiple_of_32(lib):
    code, t, _ = tmpl("paged flash-attn requires page_block_size to be")
    for p in (16, 48, 33):
        k = desc([10, p, 2, 64])
        rc, msg = check(Q, k, k, batch=3, bt=BT, page=p)
        assert rc == code and msg == render(t, page_block_size=str(p))
        assert "multiple of 32" in msg
    for p in (32, 64, 96, 128, 256):
        k = desc([10, p, 2, 64])
        assert check(Q, k, k, batch=3, bt=BT, page=p)[0] == 0


def test_paged_head_size_limit(lib):
    code, t, _ = tmpl("paged flash-attn supports head sizes")
    q = desc([5, 2, 520])
    k = desc([4, 32, 1, 520])
    rc, msg = check(q, k, k, batch=3, bt=BT, page=32)
    assert rc == code and msg == render(t, head_size_og="520")
    q = desc([5, 2, 512])
    k = desc([4, 32, 1, 512])
    assert check(q, k, k, batch=3, bt=BT, page=32)[0] == 0


def test_nonpaged_kv_shape(lib):
    code, t, _ = tmpl("shape mismatch q {:?} and k")
    k_bad = desc([86, 2, 32])
    rc, msg = check(Q, k_bad, K3, batch=3)
    assert rc == code and msg == render(t, _seq=[dl([86, 4, 64]), dl([86, 2, 32])])
    code, t, _ = tmpl("shape mismatch q {:?} and v")
    for v_bad in (desc([85, 2, 64]), desc([86, 1, 64]), desc([86, 2, 63])):
        rc, msg = check(Q, K3, v_bad, batch=3)
        assert rc == code and msg == render(t, _seq=[dl([86, 4, 64]), dl(list(v_bad.shape)[:3])])


def test_block_table_checks(lib):
    code, t, _ = tmpl("block_table last dimension")
    bt = desc([3, 4], [8, 2], dtype=FA_DTYPE_I32)
    rc, msg = check(Q, KP, KP, batch=3, bt=bt, page=32)
    assert rc == code and msg == t
    rc, msg = check(Q, KP, KP, batch=2, bt=BT, page=32)
    assert rc == 3 and "block_table" in msg
    rc, msg = check(Q, KP, KP, batch=3, bt=desc([3, 4], dtype=FA_DTYPE_BF16), page=32)
    assert rc == 6


# ------------------------------------------------------------ added checks

def test_dtype_heads_and_out(lib):
    assert check(desc([86, 4, 64], dtype=FA_DTYPE_I32), K3, K3)[0] == 6
    rc, msg = check(desc([86, 3, 64]), K3, K3, batch=3)
    assert rc == 7 and "multiple" in msg
    rc, msg = check(Q, K3, K3, out=desc([86, 4, 32]), batch=3)
    assert rc == 3 and "out" in msg
    rc, msg = check(Q, K3, K3, out=desc([86, 4, 64], [256, 64, 2]), batch=3)
    assert rc == 2 and "out" in msg
    rc, msg = check(desc([5, 2, 600]), desc([5, 1, 600]), desc([5, 1, 600]), batch=1)
    assert rc == 5
    assert check(Q, K3, K3, batch=-1)[0] == 7


def test_quoted_chain_precedes_dtype_check(lib):
    # the dtype rule is not on the pages, so every quoted check wins over it:
    # a rank-4 int32 q reports the rank-3 text, a non-contiguous int32 k the
    # contiguity text, a paged int32 pool of the wrong page size the page text
    I = FA_DTYPE_I32
    code, t, _ = tmpl("flash-attn-varlen expects input tensors of rank 3")
    rc, msg = check(desc([2, 86, 4, 64], dtype=I), K3, K3)
    assert rc == code and msg == render(t, q_rank="4", k_rank="3", v_rank="3")
    rc, msg = check(Q, desc([86, 2, 64], [256, 128, 2], dtype=I), desc([86, 2, 64], dtype=I), batch=3)
    assert msg.startswith("the last dim of k must be contiguous")
    kp = desc([10, 32, 2, 64], dtype=I)
    rc, msg = check(Q, kp, kp, batch=3, bt=BT, page=64)
    assert msg.startswith("page_block_size 64 does not match k shape")
    rc, msg = check(Q, desc([86, 2, 32], dtype=I), desc([86, 2, 32], dtype=I), batch=3)
    assert msg.startswith("shape mismatch q")
    # padded entry: rank, contiguity, shapes, then dtype
    rc, msg = pcheck(q=desc([10, 4, 64], dtype=I))
    assert rc == 1 and "rank 4" in msg
    rc, msg = pcheck(k=desc([2, 9, 2, 64], [2048, 128, 64, 2], dtype=I), v=desc([2, 9, 2, 64], dtype=I))
    assert msg.startswith("the last dim of k must be contiguous")
    rc, msg = pcheck(v=desc([2, 8, 2, 64], dtype=I))
    assert msg.startswith("shape mismatch k")


def test_first_failing_check_wins(lib):
    # several problems at once: rank beats contiguity beats shapes beats page size
    q4 = desc([2, 43, 4, 64], [1, 1, 1, 2])
    assert check(q4, K3, K3)[1].startswith("flash-attn-varlen expects input tensors of rank 3")
    ks = desc([10, 16, 2, 64], [2048, 128, 64, 2])
    msg = check(Q, ks, ks, batch=3, bt=BT, page=0)[1]
    assert msg.startswith("the last dim of k must be contiguous")


def test_workspace_bytes(lib):
    # decode-shaped paged call needs split partials; small prefill needs none
    q = desc([64, 32, 128])
    k = desc([4000, 32, 8, 128])
    bt = desc([64, 128], dtype=FA_DTYPE_I32)
    n = fa.fa_varlen_workspace_bytes(q, k, k, 64, bt, 32)
    assert n > 0 and n % 256 == 0
    # partials: up to ceil(128*32 / split) chunks x tokens x heads x (head_dim + 1) floats
    assert n >= 64 * 32 * 129 * 4 * 2
    small = fa.fa_varlen_workspace_bytes(Q, K3, K3, 3, None, 0)  # work list only
    assert 0 < small < n
    with pytest.raises(fa.FlashAttnError) as e:
        fa.fa_varlen_workspace_bytes(Q, K3, desc([86, 2, 32]), 3, None, 0)
    assert e.value.status == "FA_ERR_SHAPE"


def test_prefill_split_only_for_short_work_lists(lib):
    # the plan cuts prefill keys into chunks (split partials in the workspace)
    # only when the work list cannot fill the GPU: a few row tiles over long keys
    bt_long = desc([2, 313], dtype=FA_DTYPE_I32)                     # up to 20032 keys per sequence
    pool = desc([700, 64, 2, 128])
    short = fa.fa_varlen_workspace_bytes(desc([73, 8, 128]), pool, pool, 2, bt_long, 64)
    assert short >= 73 * 8 * 129 * 4 * 2  # at least two chunks of fp32 partials
    # a 16-sequence chunked prefill over 8k-key caches (about 1.2k work units): no split
    bt_c3 = desc([16, 136], dtype=FA_DTYPE_I32)
    pool3 = desc([2400, 64, 8, 128])
    c3 = fa.fa_varlen_workspace_bytes(desc([4104, 32, 128]), pool3, pool3, 16, bt_c3, 64)
    assert 0 < c3 < 4104 * 32 * 129 * 4


# ------------------------------------------------------------ paged append

KN = desc([6, 2, 64])
KC = desc([10, 32, 2, 64])
BT3 = desc([3, 4], dtype=FA_DTYPE_I32)


def acheck(kn=KN, vn=KN, batch=3, bt=BT3, kc=KC, vc=KC, page=32):
    rc = fa.fa_kv_append_check(kn, vn, batch, bt, kc, vc, page)
    return rc, fa.fa_last_error() if rc else ""


def test_append_valid(lib):
    assert acheck() == (0, "")
    assert acheck(kn=desc([0, 2, 64]), vn=desc([0, 2, 64]))[0] == 0
    assert acheck(batch=0, bt=desc([0, 4], dtype=FA_DTYPE_I32))[0] == 0


def test_append_reuses_paged_page_rules(lib):
    code, t, _ = tmpl("paged flash-attn requires page_block_size")
    assert acheck(page=0) == (code, t)
    code, t, _ = tmpl("page_block_size {")
    assert acheck(page=64) == (code, render(t, page_block_size_arg="64", _seq=[dl([10, 32, 2, 64])]))
    code, t, _ = tmpl("paged flash-attn requires page_block_size to be")
    k = desc([10, 48, 2, 64])
    assert acheck(kc=k, vc=k, page=48) == (code, render(t, page_block_size="48"))
    code, t, _ = tmpl("paged flash-attn supports head sizes")
    kn, kc = desc([6, 1, 520]), desc([4, 32, 1, 520])
    assert acheck(kn=kn, vn=kn, kc=kc, vc=kc) == (code, render(t, head_size_og="520"))
    kn, kc = desc([6, 1, 512]), desc([4, 32, 1, 512])
    assert acheck(kn=kn, vn=kn, kc=kc, vc=kc)[0] == 0


def test_append_shape_rank_dtype_contiguity(lib):
    rank = {v: k for k, v in fa.STATUS.items()}
    assert acheck(kn=desc([6, 2, 64, 1]))[0] == rank["FA_ERR_RANK"]
    assert acheck(kc=desc([10, 32, 128]))[0] == rank["FA_ERR_RANK"]
    assert acheck(kn=desc([6, 2, 64], dtype=FA_DTYPE_I32))[0] == rank["FA_ERR_DTYPE"]
    assert acheck(bt=desc([3, 4]))[0] == rank["FA_ERR_DTYPE"]
    rc, msg = acheck(kn=desc([6, 2, 64], stride=[128, 64, 2]))
    assert rc == rank["FA_ERR_CONTIGUOUS"] and msg.startswith("the last dim of k_new must be contiguous")
    code, t, _ = tmpl("the last dim of k must")
    rc, msg = acheck(kc=desc([10, 32, 2, 64], stride=[8192, 256, 128, 2]))
    assert rc == code and msg == render(t, k_stride=dl([8192, 256, 128, 2]))
    code, t, _ = tmpl("shape mismatch k {:?} and v")
    rc, msg = acheck(vc=desc([11, 32, 2, 64]))
    assert rc == code and msg == render(t, _seq=[dl([10, 32, 2, 64]), dl([11, 32, 2, 64])])
    assert acheck(vn=desc([5, 2, 64]))[0] == rank["FA_ERR_SHAPE"]
    assert acheck(kn=desc([6, 1, 64]), vn=desc([6, 1, 64]))[0] == rank["FA_ERR_SHAPE"]
    assert acheck(bt=desc([2, 4], dtype=FA_DTYPE_I32))[0] == rank["FA_ERR_SHAPE"]
    code, t, _ = tmpl("block_table last dimension")
    assert acheck(bt=desc([3, 4], stride=[8, 2], dtype=FA_DTYPE_I32)) == (code, t)
    assert acheck(batch=-1)[0] == rank["FA_ERR_ARGUMENT"]
    assert acheck(bt=None)[0] == rank["FA_ERR_ARGUMENT"]


def test_append_empty_call_needs_no_gpu(lib):
    """batch 0 or no new tokens: nothing is launched, no device pointer is inspected."""
    assert fa.fa_kv_append(desc([0, 2, 64]), desc([0, 2, 64]), 0, 0, 3, BT3, KC, KC, 32, 0) == 0
    assert fa.fa_kv_append(KN, KN, 0, 0, 0, desc([0, 4], dtype=FA_DTYPE_I32), KC, KC, 32, 0) == 0


# ------------------------------------------------------------ padded entry

QP = desc([2, 5, 4, 64])
KP4 = desc([2, 9, 2, 64])


def pcheck(q=QP, k=KP4, v=KP4, out=None):
    rc = fa.fa_padded_check(q, k, v, out)
    return rc, fa.fa_last_error() if rc else ""


def test_padded_contract(lib):
    code = {v: k for k, v in fa.STATUS.items()}
    assert pcheck() == (0, "")
    assert pcheck(out=QP)[0] == 0
    # head-major views are accepted
    assert pcheck(q=desc([2, 5, 4, 64], stride=[1280, 64, 320, 1]))[0] == 0
    assert pcheck(q=desc([10, 4, 64]))[0] == code["FA_ERR_RANK"]
    assert pcheck(k=desc([2, 9, 2, 64], dtype=FA_DTYPE_I32))[0] == code["FA_ERR_DTYPE"]
    c, t, _ = tmpl("the last dim of q must")
    rc, msg = pcheck(q=desc([2, 5, 4, 64], stride=[2560, 512, 128, 2]))
    assert rc == c and msg == render(t, q_stride=dl([2560, 512, 128, 2]))
    c, t, _ = tmpl("shape mismatch k {:?} and v")
    rc, msg = pcheck(v=desc([2, 8, 2, 64]))
    assert rc == c and msg == render(t, _seq=[dl([2, 9, 2, 64]), dl([2, 8, 2, 64])])
    assert pcheck(k=desc([3, 9, 2, 64]), v=desc([3, 9, 2, 64]))[0] == code["FA_ERR_SHAPE"]
    assert pcheck(k=desc([2, 9, 3, 64]), v=desc([2, 9, 3, 64]))[0] == code["FA_ERR_ARGUMENT"]
    assert pcheck(q=desc([2, 5, 4, 520]), k=desc([2, 9, 2, 520]), v=desc([2, 9, 2, 520]))[0] == code["FA_ERR_HEAD_DIM"]
    assert pcheck(out=desc([2, 5, 4, 32]))[0] == code["FA_ERR_SHAPE"]


def test_padded_workspace_and_empty_call(lib):
    assert fa.fa_padded_workspace_bytes(QP, KP4, KP4) > 0
    # decode-shaped calls split keys: partials make the workspace larger
    big = fa.fa_padded_workspace_bytes(desc([64, 1, 32, 128]), desc([64, 4096, 8, 128]), desc([64, 4096, 8, 128]))
    assert big > 64 * 32 * 128 * 4
    # no batch or no query: nothing is launched, no pointer is inspected
    assert fa.fa_padded_fwd(desc([0, 5, 4, 64]), desc([0, 9, 2, 64]), desc([0, 9, 2, 64]),
                            desc([0, 5, 4, 64]), 0.1, -1, 0, 0, 0, 0, 0) == 0


def test_f16_accepted_and_dtypes_must_match(lib):
    from varlen_flash_attention_fa_amd import FA_DTYPE_F16
    code = {v: k for k, v in fa.STATUS.items()}
    q, k = desc([86, 4, 64], dtype=FA_DTYPE_F16), desc([86, 2, 64], dtype=FA_DTYPE_F16)
    assert check(q, k, k, out=desc([86, 4, 64], dtype=FA_DTYPE_F16))[0] == 0
    # mixed element types are rejected: q/k/v, and out
    assert check(q, K3, K3)[0] == code["FA_ERR_DTYPE"]
    assert check(q, k, K3)[0] == code["FA_ERR_DTYPE"]
    assert check(q, k, k, out=desc([86, 4, 64]))[0] == code["FA_ERR_DTYPE"]
    kn, kc = desc([6, 2, 64], dtype=FA_DTYPE_F16), desc([10, 32, 2, 64], dtype=FA_DTYPE_F16)
    assert acheck(kn=kn, vn=kn, kc=kc, vc=kc)[0] == 0
    assert acheck(kn=kn, vn=kn)[0] == code["FA_ERR_DTYPE"]
    qp, kp = desc([2, 5, 4, 64], dtype=FA_DTYPE_F16), desc([2, 9, 2, 64], dtype=FA_DTYPE_F16)
    assert pcheck(q=qp, k=kp, v=kp)[0] == 0
    assert pcheck(q=qp)[0] == code["FA_ERR_DTYPE"]


def test_alibi_slopes_contract(lib):
    from varlen_flash_attention_fa_amd import FA_DTYPE_F32
    code, t, _ = tmpl("shape mismatch alibi_slopes")
    ok1 = desc([4], dtype=FA_DTYPE_F32)
    ok2 = desc([3, 4], dtype=FA_DTYPE_F32)
    assert fa.fa_varlen_check(Q, K3, K3, None, 3, None, 0, ok1) == 0
    assert fa.fa_varlen_check(Q, K3, K3, None, 3, None, 0, ok2) == 0
    rc = fa.fa_varlen_check(Q, K3, K3, None, 3, None, 0, desc([8], dtype=FA_DTYPE_F32))
    assert rc == code and fa.fa_last_error() == render(t, _seq=[dl([8]), dl([4])])
    rc = fa.fa_varlen_check(Q, K3, K3, None, 3, None, 0, desc([2, 4], dtype=FA_DTYPE_F32))
    assert rc == code and fa.fa_last_error() == render(t, _seq=[dl([2, 4]), dl([3, 4])])
    codes = {v: k for k, v in fa.STATUS.items()}
    assert fa.fa_varlen_check(Q, K3, K3, None, 3, None, 0, desc([4])) == codes["FA_ERR_DTYPE"]
    assert fa.fa_varlen_check(Q, K3, K3, None, 3, None, 0,
                              desc([3, 4], stride=[8, 2], dtype=FA_DTYPE_F32)) == codes["FA_ERR_CONTIGUOUS"]
    # the earlier checks come first
    assert fa.fa_varlen_check(desc([86, 4]), K3, K3, None, 3, None, 0, desc([8])) == codes["FA_ERR_RANK"]
    # padded: (H) or (B, H)
    assert fa.fa_padded_check(QP, KP4, KP4, None, ok1) == 0
    assert fa.fa_padded_check(QP, KP4, KP4, None, desc([2, 4], dtype=FA_DTYPE_F32)) == 0
    assert fa.fa_padded_check(QP, KP4, KP4, None, desc([3, 4], dtype=FA_DTYPE_F32)) == code


# ------------------------------------------------- offsets arrays (binding)

def test_seqlens_layout_texts():
    # the binding rejects strided offsets with the pages' texts before any device
    # work (the tensors here are on the CPU; nothing reaches the C ABI)
    import torch
    q = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    k = torch.zeros(6, 1, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 2, 4], dtype=torch.int32)
    strided = torch.tensor([0, 9, 3, 9, 6, 9], dtype=torch.int32)[::2]
    assert not strided.is_contiguous()
    for args, text in (((strided, cu), "seqlens_q has to be contiguous"),
                       ((cu, strided), "seqlens_k has to be contiguous")):
        c, t, _ = tmpl(text)
        with pytest.raises(fa.FlashAttnError) as e:
            fa.varlen_fwd(q, k, k, *args)
        assert e.value.code == c and str(e.value) == t
    with pytest.raises(fa.FlashAttnError) as e:
        fa.varlen_fwd(q, k, k, cu.long(), cu)
    assert "int32" in str(e.value)
    with pytest.raises(fa.FlashAttnError) as e:
        fa.kv_append(k, k, cu, strided, torch.zeros(2, 1, dtype=torch.int32), k, k)
    assert str(e.value) == "seqlens_k has to be contiguous"
