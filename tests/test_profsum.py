"""Host logic of the profile summaries: counter scaling and the source-digest gate."""
import json
import sqlite3
import types

from cnn_backward_pass_amd import profsum


def _db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id int, kernel_name text, "
                "counter_name text, value real)")
    con.executemany("insert into counters_collection values (?,?,?,?)", rows)
    con.commit()
    con.close()


def test_traffic_scaling_and_gate(tmp_path):
    k = "void cbb::conv_dw_kernel<X>(int)"
    fetch = tmp_path / "f.db"
    write = tmp_path / "w.db"
    cf = tmp_path / "cf.db"
    cw = tmp_path / "cw.db"
    # setup pass (act+BN) excluded; two XCD rows of one dispatch are summed
    _db(fetch, [(1, "void cbb::actbn_reduce<1>(int)", "FETCH_SIZE", 999.0),
                (2, k, "FETCH_SIZE", 100.0), (2, k, "FETCH_SIZE", 100.0),
                (3, k, "FETCH_SIZE", 200.0), (4, "at::native::fill", "FETCH_SIZE", 5.0)])
    _db(write, [(2, k, "WRITE_SIZE", 10.0), (3, k, "WRITE_SIZE", 10.0)])
    _db(cf, [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)])
    _db(cw, [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)])
    out = tmp_path / "x_hbm_traffic.md"
    a = types.SimpleNamespace(stage="wl.1.dW", reps=2, fetch=str(fetch), write=str(write),
                              copy_fetch=str(cf), copy_write=str(cw), copy_bytes=1 << 20,
                              out=str(out), cmd=["cmd"])
    profsum.write_traffic(a)
    rec = profsum.load_traffic("wl.1.dW", str(tmp_path))
    assert rec is not None
    assert rec["fetch_bytes"] == 2.0 * 400 * 1024 / 2
    assert rec["write_bytes"] == 20 * 1024 / 2
    assert profsum.load_traffic("wl.0.dW", str(tmp_path)) is None
    # a record taken from other kernel sources is not reported
    text = out.read_text().replace(rec["sources"], "0" * 16)
    out.write_text(text)
    assert profsum.load_traffic("wl.1.dW", str(tmp_path)) is None
    line = [l for l in text.splitlines() if l.startswith(profsum.TRAFFIC_TAG)][0]
    assert json.loads(line[len(profsum.TRAFFIC_TAG):])["stage"] == "wl.1.dW"


def test_mfma_rows_per_kernel(tmp_path):
    """Matrix FLOPs sum over a dispatch's rows (x 512); the busy share divides the summed
    busy cycles by the GPU's active cycles (GRBM_GUI_ACTIVE, read summed over the dies,
    divided by their count) times the SIMD count."""
    k = "void cbb::conv_dx3_s2p<4>(int)"
    db = tmp_path / "m.db"
    _db(db, [(1, k, "SQ_INSTS_VALU_MFMA_MOPS_F32", 1000.0), (1, k, "SQ_INSTS_VALU_MFMA_MOPS_F32", 1000.0),
             (1, k, "SQ_VALU_MFMA_BUSY_CYCLES", 4000.0), (1, k, "GRBM_GUI_ACTIVE", 50.0),
             (1, k, "GRBM_GUI_ACTIVE", 30.0),
             (2, k, "SQ_INSTS_VALU_MFMA_MOPS_F32", 3000.0), (2, k, "SQ_VALU_MFMA_BUSY_CYCLES", 2000.0),
             (2, k, "GRBM_GUI_ACTIVE", 80.0),
             (3, "at::native::fill", "SQ_INSTS_VALU_MFMA_MOPS_F32", 7.0)])
    rows = profsum.mfma_rows(str(db), simds=1000, xcds=8)
    assert list(rows) == ["conv_dx3_s2p<4>"]
    r = rows["conv_dx3_s2p<4>"]
    assert r["dispatches"] == 2
    assert r["mfma_flops"] == (2000.0 + 3000.0) * 512 / 2
    assert abs(r["mfma_busy"] - (0.4 + 0.2) / 2) < 1e-12
    assert r["gui_active_cycles"] == 10.0


def test_lds_rows_per_kernel(tmp_path):
    """LDS instructions average over dispatches; the conflict share divides the summed
    conflict cycles by the summed LDS-busy cycles; kernels without LDS work are left out."""
    k = "void cbb::conv_first_rows<3, false, 0>(int)"
    db = tmp_path / "l.db"
    _db(db, [(1, k, "SQ_INSTS_LDS", 100.0), (1, k, "SQ_INSTS_LDS", 100.0),
             (1, k, "SQ_LDS_BANK_CONFLICT", 30.0), (1, k, "SQ_LDS_IDX_ACTIVE", 100.0),
             (2, k, "SQ_INSTS_LDS", 200.0), (2, k, "SQ_LDS_BANK_CONFLICT", 10.0),
             (2, k, "SQ_LDS_IDX_ACTIVE", 100.0),
             (3, "void cbb::actbn_coef(int)", "SQ_INSTS_LDS", 0.0),
             (3, "void cbb::actbn_coef(int)", "SQ_LDS_BANK_CONFLICT", 0.0),
             (3, "void cbb::actbn_coef(int)", "SQ_LDS_IDX_ACTIVE", 0.0)])
    rows = profsum.lds_rows(str(db))
    assert list(rows) == ["conv_first_rows<3, false, 0>"]
    r = rows["conv_first_rows<3, false, 0>"]
    assert r["dispatches"] == 2 and r["lds_insts"] == 200.0
    assert abs(r["conflict_share"] - 0.2) < 1e-12
    out = tmp_path / "lds.md"
    profsum.main(["lds", "--stage", "wl.0.block", "--db", str(db), "--cmd", "c", "--out",
                  str(out)])
    assert "20.0%" in out.read_text()

