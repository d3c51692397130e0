"""MX microscaling quantisation and block-scaled GEMMs for MI355X (gfx950)."""
