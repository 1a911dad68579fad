"""MI355X-native edge-aware attention layer (FlexAttentionGT layer) for gfx950."""
