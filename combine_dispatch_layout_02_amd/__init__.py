"""MI355X-native MoE expert-parallel dispatch / combine (HIP, gfx950)."""
