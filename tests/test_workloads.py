"""Host-side checks of the workload recipes (no GPU): the whole-schedule decode
workload follows the published layer allocation and holds the published cache
footprint."""
import json
import os

import oracle
from sparse_attention_fp4_cache_amd.workloads import WORKLOADS, published_schedule

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_published_schedule_matches_page_allocation():
    s = GOLD["schedule"]
    modes, m = published_schedule()
    want = ["swa"] * s["encoder"]["swa_only_layers"] + s["encoder"]["group"] * s["encoder"]["groups"]
    want += s["decoder"]["first_group"] + s["decoder"]["group"] * s["decoder"]["groups"]
    assert list(modes) == want
    enc = s["encoder"]["swa_only_layers"] + len(s["encoder"]["group"]) * s["encoder"]["groups"]
    assert all(x == s["encoder"]["m"] for x in m[2:enc]) and all(x == s["decoder"]["m"] for x in m[enc:])
    assert [i for i, md in enumerate(modes) if md == "full"] == GOLD["writer_layers"]["value"]


def test_whole_schedule_workload_footprint():
    sw = WORKLOADS["decode_1m_schedule"]
    assert sw.ctx == GOLD["context_tokens"]["value"]
    # every non-window layer reads the cache of the latest Full layer at or before it
    for li, md in enumerate(sw.modes):
        src = sw.source(li)
        if md == "swa":
            assert src is None
        else:
            assert sw.modes[src] == "full" and sw.m[src] == sw.m[li]
            assert all(sw.modes[j] != "full" for j in range(src + 1, li + 1))
    entries = [int(sw.cache_workload(w).n_entries[0]) for w in sw.writers()]
    assert entries == [524288, 524288, 524288, 1048576]
    per_entry = oracle.entry_bytes(512, 16) + oracle.entry_bytes(128, 32)
    total = sum(entries) * per_entry
    assert total == GOLD["global_bytes_per_token"]["value"] * sw.ctx
    assert round(total / 2**30, 2) == GOLD["global_gib_at_context"]["value"]
    assert len(sw.writers()) == 4 and len(sw.modes) - len(sw.writers()) == 36
