"""MI355X (gfx950) tree-verify MLA attention: a C-ABI HIP library plus a thin binding."""
