"""Chunked gated delta-rule forward (KDA / Gated DeltaNet) for MI355X."""
