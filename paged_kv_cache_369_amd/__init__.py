"""paged_kv_cache_369_amd: paged-KV-cache decode attention for MI355X (gfx950)."""
