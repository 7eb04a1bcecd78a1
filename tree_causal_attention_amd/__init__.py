"""MI355X-native verify step of tree speculative decoding (HIP for gfx950)."""
