"""Host logic of the profile summaries: which dispatches count as a family's batch-8 launch.

Most families are picked by their largest grid. The fused ModUp/inner-product
tile has the same grid at every batch, so its batch-8 dispatches are those that
follow, on the same queue, the batch-8 launch of the kernel before it in a key
switch. These tests build small dispatch tables by hand and a kernel-trace CSV
in a temporary directory; nothing here touches a GPU.
"""

import csv

from key_switching_amd import profiling as P

FUSED = "k_modup_ip<16, 4, 12, false>"
PRED = P.FOLLOWS[FUSED]


def test_largest_grid_for_ordinary_families():
    disp = {1: ("1", "k_md_bconv<16, 6, 3>", 524288), 2: ("1", "k_md_bconv<16, 6, 3>", 65536),
            3: ("1", "k_md_bconv<16, 6, 3>", 524288), 4: ("1", "k_other", 999999999)}
    ids, g = P._batch8_ids(disp, "k_md_bconv<16, 6, 3>")
    assert ids == [1, 3] and g == 524288


def test_fused_tile_follows_its_batch8_predecessor():
    # batch 8: predecessor at its largest grid; batch 1: the same predecessor name
    # at a smaller grid, or another kernel; a second queue interleaved
    disp = {
        10: ("1", PRED, 1048576), 11: ("1", FUSED, 122880),   # batch 8: kept
        12: ("2", PRED, 131072), 13: ("1", "k_other", 1),     # other queue, then a foreign kernel
        14: ("1", FUSED, 122880),                             # after k_other: not kept
        15: ("2", FUSED, 122880),                             # after the small predecessor: not kept
        16: ("1", PRED, 1048576), 17: ("2", "k_x", 5), 18: ("1", FUSED, 122880),  # kept (queue 1)
    }
    ids, g = P._batch8_ids(disp, FUSED)
    assert ids == [11, 18] and g == 122880


def test_missing_family_and_missing_predecessor():
    assert P._batch8_ids({1: ("1", "k_a", 1)}, FUSED) == ([], 0)
    ids, _ = P._batch8_ids({1: ("1", FUSED, 122880), 2: ("1", FUSED, 122880)}, FUSED)
    assert ids == []


def test_family_rows_from_a_trace(tmp_path):
    path = tmp_path / "trace.csv"
    fields = ["Dispatch_Id", "Queue_Id", "Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
              "Start_Timestamp", "End_Timestamp"]
    rows = [
        (1, 1, f"void pc::{PRED}(pc::ModUpArgs)", 1048576, 1, 1, 0, 90000),
        (2, 1, f"void pc::{FUSED}(pc::ModUpIPArgs)", 122880, 1, 1, 90000, 225000),
        (3, 1, "void pc::k_modup_bconv<16, 6, 1>(pc::ModUpArgs)", 131072, 1, 1, 300000, 318000),
        (4, 1, f"void pc::{FUSED}(pc::ModUpIPArgs)", 122880, 1, 1, 318000, 360000),
    ]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(fields)
        w.writerows(rows)
    got, g = P._family_rows(list(csv.DictReader(open(path))), FUSED)
    assert [int(r["Dispatch_Id"]) for r in got] == [2] and g == 122880
