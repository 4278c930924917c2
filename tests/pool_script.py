"""Golden pool-script driver shared by the oracle and library tests."""
import pytest


def run_pool_script(make_pool, script, err_types):
    """Drive a pool object through the golden script.  ``make_pool(N, P,
    free_order)`` returns an object with seq_new / seq_append / seq_fork /
    seq_cow / seq_free / block_tables / stats; ``err_types`` maps the script's
    error names to the exception classes that pool raises."""
    pool = make_pool(script["num_pages"], script["page_size"], script["free_order"])
    for st in script["steps"]:
        op = st["op"]
        if "expect_error" in st:
            before = (pool.stats()[0], pool.stats()[1].tolist())
            with pytest.raises(err_types[st["expect_error"]]):
                if op == "cow":
                    pool.seq_cow(st["seq"], st["logical_page"])
                elif op == "append":
                    pool.seq_append(st["seq"], st["n"])
                elif op == "free":
                    pool.seq_free(st["seq"])
            assert (pool.stats()[0], pool.stats()[1].tolist()) == before, st
            continue
        if op == "seq_new":
            assert pool.seq_new() == st["expect_seq"]
        elif op == "append":
            slots, cow = pool.seq_append(st["seq"], st["n"])
            assert list(slots) == st["expect_slots"], st
            assert (None if cow is None else list(cow)) == st["expect_cow"], st
        elif op == "fork":
            assert pool.seq_fork(st["seq"]) == st["expect_seq"]
        elif op == "cow":
            assert list(pool.seq_cow(st["seq"], st["logical_page"])) == st["expect_pair"]
        elif op == "free":
            pool.seq_free(st["seq"])
        elif op == "tables":
            bt, kv = pool.block_tables(st["seqs"], st["max_pages"])
            assert bt.tolist() == st["expect_bt"] and kv.tolist() == st["expect_len"]
        elif op == "stats":
            nf, ref = pool.stats()
            assert nf == st["expect_free"] and list(ref) == st["expect_ref"]
        else:
            raise AssertionError(op)
    return pool
