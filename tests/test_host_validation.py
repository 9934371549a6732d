"""Host-side checks of device-resident indices (opt-in with MLA_VALIDATE=1):
slots of an append and the paging of a decode.  They run on CPU tensors."""
import pytest
import torch

from mla_latent_kv_38_amd.ops import check_paging, check_slots


def test_slots_in_range_and_distinct():
    check_slots(torch.tensor([0, 5, 255], dtype=torch.int64), num_pages=4, block_size=64)
    with pytest.raises(ValueError, match="outside"):
        check_slots(torch.tensor([0, 256], dtype=torch.int64), num_pages=4, block_size=64)
    with pytest.raises(ValueError, match="outside"):
        check_slots(torch.tensor([-1], dtype=torch.int64), num_pages=4, block_size=64)
    with pytest.raises(ValueError, match="repeat"):
        check_slots(torch.tensor([3, 3], dtype=torch.int64), num_pages=4, block_size=64)


def test_paging_reads_only_the_used_entries():
    bt = torch.tensor([[2, 0, -1], [1, -7, -7]], dtype=torch.int32)
    # sequence 0: 100 rows = pages 0..1 of its row; sequence 1: 64 rows = page 0
    check_paging(bt, torch.tensor([100, 64], dtype=torch.int32), num_pages=3, block_size=64)
    # a window starting on page 1 of sequence 1 skips the bad entry only if it starts past it
    with pytest.raises(ValueError, match=r"block_table\[1, 1\]"):
        check_paging(bt, torch.tensor([100, 65], dtype=torch.int32), num_pages=3, block_size=64)
    with pytest.raises(ValueError, match=r"block_table\[0, 0\]"):
        check_paging(bt, torch.tensor([100, 64], dtype=torch.int32), num_pages=2, block_size=64)
    with pytest.raises(ValueError, match="seq_lens"):
        check_paging(bt, torch.tensor([193, 0], dtype=torch.int32), num_pages=3, block_size=64)
    # windows: entries before the window's first page are not read
    bt2 = torch.tensor([[-5, 1, 2]], dtype=torch.int32)
    check_paging(bt2, torch.tensor([150], dtype=torch.int32), num_pages=3, block_size=64,
                 seq_starts=torch.tensor([64], dtype=torch.int32))
    with pytest.raises(ValueError, match=r"block_table\[0, 0\]"):
        check_paging(bt2, torch.tensor([150], dtype=torch.int32), num_pages=3, block_size=64,
                     seq_starts=torch.tensor([63], dtype=torch.int32))
    # an empty window reads nothing
    check_paging(bt2, torch.tensor([10], dtype=torch.int32), num_pages=3, block_size=64,
                 seq_starts=torch.tensor([10], dtype=torch.int32))
