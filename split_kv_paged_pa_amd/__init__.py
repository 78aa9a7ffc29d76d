"""split_kv_paged_pa_amd: paged single-query decode attention for AMD MI355X (gfx950)."""
