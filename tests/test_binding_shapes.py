"""CPU tests of the binding's shape checks (binding.check_dense_shapes /
check_csr_shapes): the C ABI takes raw pointers, so the Python layer is the
only one that sees tensor shapes; each mismatch must raise before anything
launches.  CPU tensors stand in for device tensors (the checks look at
shapes, dtypes and strides only)."""
import pytest
import torch

from paged_kv_decode_amd import binding as B

HQ, HKV, D, PS = 8, 2, 64, 16
DT = torch.float16


def desc():
    return B.make_desc(HQ, HKV, D, DT, max_batch=8, max_context_len=4096)


def dense(batch=3, pages=32, cols=8):
    return dict(q=torch.zeros(batch, HQ, D, dtype=DT),
                k_cache=torch.zeros(pages, HKV, PS, D, dtype=DT),
                v_cache=torch.zeros(pages, HKV, PS, D, dtype=DT),
                page_table=torch.zeros(batch, cols, dtype=torch.int32),
                context_lens=torch.full((batch,), 100, dtype=torch.int32),
                out=torch.zeros(batch, HQ, D, dtype=DT),
                lse=torch.zeros(batch, HQ, dtype=torch.float32))


def check_dense(t, max_ctx=100):
    B.check_dense_shapes(desc(), DT, t["q"], t["k_cache"], t["v_cache"], t["page_table"],
                         t["context_lens"], t["out"], t["lse"], max_ctx)


def test_valid_dense_shapes_pass():
    check_dense(dense())
    t = dense()
    t["lse"] = None
    check_dense(t)
    # token-major storage viewed as [pages, Hkv, ps, D]
    t = dense()
    t["k_cache"] = torch.zeros(32, PS, HKV, D, dtype=DT).permute(0, 2, 1, 3)
    t["v_cache"] = torch.zeros(32, PS, HKV, D, dtype=DT).permute(0, 2, 1, 3)
    check_dense(t)
    # empty batch
    t = dense(batch=0)
    check_dense(t, max_ctx=0)


@pytest.mark.parametrize("what,change,exc", [
    ("q heads", lambda t: t.update(q=torch.zeros(3, HQ // 2, D, dtype=DT)), ValueError),
    ("q head_dim", lambda t: t.update(q=torch.zeros(3, HQ, 2 * D, dtype=DT)), ValueError),
    ("q rank", lambda t: t.update(q=torch.zeros(3 * HQ, D, dtype=DT)), ValueError),
    ("q dtype", lambda t: t.update(q=t["q"].float()), TypeError),
    ("out shape", lambda t: t.update(out=torch.zeros(2, HQ, D, dtype=DT)), ValueError),
    ("q not contiguous", lambda t: t.update(q=torch.zeros(HQ, 3, D, dtype=DT).transpose(0, 1)),
     ValueError),
    ("fewer kv heads", lambda t: t.update(k_cache=torch.zeros(32, 1, PS, D, dtype=DT),
                                          v_cache=torch.zeros(32, 1, PS, D, dtype=DT)), ValueError),
    ("more kv heads", lambda t: t.update(k_cache=torch.zeros(32, 4, PS, D, dtype=DT),
                                         v_cache=torch.zeros(32, 4, PS, D, dtype=DT)), ValueError),
    ("page size", lambda t: t.update(k_cache=torch.zeros(32, HKV, 8, D, dtype=DT),
                                     v_cache=torch.zeros(32, HKV, 8, D, dtype=DT)), ValueError),
    ("cache head_dim", lambda t: t.update(k_cache=torch.zeros(32, HKV, PS, 128, dtype=DT),
                                          v_cache=torch.zeros(32, HKV, PS, 128, dtype=DT)), ValueError),
    ("k/v differ", lambda t: t.update(v_cache=torch.zeros(16, HKV, PS, D, dtype=DT)), ValueError),
    ("D not contiguous", lambda t: t.update(
        k_cache=torch.zeros(32, HKV, D, PS, dtype=DT).transpose(2, 3),
        v_cache=torch.zeros(32, HKV, D, PS, dtype=DT).transpose(2, 3)), ValueError),
    ("lse [B]", lambda t: t.update(lse=torch.zeros(3, dtype=torch.float32)), ValueError),
    ("lse [B, Hkv]", lambda t: t.update(lse=torch.zeros(3, HKV, dtype=torch.float32)), ValueError),
    ("lse dtype", lambda t: t.update(lse=torch.zeros(3, HQ, dtype=torch.float16)), TypeError),
    ("page table rows", lambda t: t.update(page_table=torch.zeros(2, 8, dtype=torch.int32)),
     ValueError),
    ("page table too narrow", lambda t: t.update(page_table=torch.zeros(3, 6, dtype=torch.int32)),
     ValueError),
    ("page table dtype", lambda t: t.update(page_table=torch.zeros(3, 8, dtype=torch.int64)),
     TypeError),
    ("page table column-major", lambda t: t.update(
        page_table=torch.zeros(8, 3, dtype=torch.int32).t()), ValueError),
    ("page table view past its storage", lambda t: t.update(
        page_table=torch.zeros(2 * 16 + 8, dtype=torch.int32).as_strided((3, 8), (16, 1))),
     ValueError),
    ("lengths short", lambda t: t.update(context_lens=torch.zeros(2, dtype=torch.int32)),
     ValueError),
    ("lengths dtype", lambda t: t.update(context_lens=torch.zeros(3, dtype=torch.int64)),
     TypeError),
])
def test_dense_mismatch_raises(what, change, exc):
    t = dense()
    change(t)
    with pytest.raises(exc):
        check_dense(t)


def test_page_table_row_stride_inside_storage_passes():
    """A page table whose rows are a slice of wider rows is fine when the
    storage behind every row spans the whole stride."""
    t = dense()
    t["page_table"] = torch.zeros(3, 16, dtype=torch.int32)[:, :8]
    check_dense(t)


def csr(batch=3, nnz=20):
    t = dense(batch)
    del t["page_table"], t["context_lens"]
    t.update(page_indptr=torch.zeros(batch + 1, dtype=torch.int32),
             page_indices=torch.zeros(nnz, dtype=torch.int32),
             last_page_len=torch.ones(batch, dtype=torch.int32), nnz_pages=nnz)
    return t


def check_csr(t):
    B.check_csr_shapes(desc(), DT, t["q"], t["k_cache"], t["v_cache"], t["page_indptr"],
                       t["page_indices"], t["last_page_len"], t["nnz_pages"], t["out"], t["lse"])


def test_valid_csr_shapes_pass():
    check_csr(csr())
    t = csr(nnz=0)
    check_csr(t)


@pytest.mark.parametrize("what,change,exc", [
    ("indptr short", lambda t: t.update(page_indptr=torch.zeros(3, dtype=torch.int32)), ValueError),
    ("last_page_len short", lambda t: t.update(last_page_len=torch.ones(2, dtype=torch.int32)),
     ValueError),
    ("indices short", lambda t: t.update(nnz_pages=21), ValueError),
    ("negative nnz", lambda t: t.update(nnz_pages=-1), ValueError),
    ("indptr int64", lambda t: t.update(page_indptr=torch.zeros(4, dtype=torch.int64)), TypeError),
    ("indices strided", lambda t: t.update(page_indices=torch.zeros(40, dtype=torch.int32)[::2]),
     TypeError),
    ("q heads", lambda t: t.update(q=torch.zeros(3, 4, D, dtype=DT)), ValueError),
    ("lse [B]", lambda t: t.update(lse=torch.zeros(3, dtype=torch.float32)), ValueError),
    ("fewer kv heads", lambda t: t.update(k_cache=torch.zeros(32, 1, PS, D, dtype=DT),
                                          v_cache=torch.zeros(32, 1, PS, D, dtype=DT)), ValueError),
])
def test_csr_mismatch_raises(what, change, exc):
    t = csr()
    change(t)
    with pytest.raises(exc):
        check_csr(t)
