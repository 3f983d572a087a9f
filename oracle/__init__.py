"""fp64 CPU oracle for the Muon step: test infrastructure only (see muon_ref)."""
