"""permute_layout for MI355X (gfx950): a C-ABI HIP library and its thin binding."""
