"""fp64 CPU oracle of the cross-model KV handoff (test infrastructure only)."""
