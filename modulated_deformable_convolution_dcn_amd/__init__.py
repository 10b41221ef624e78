"""MI355X-native modulated deformable conv2d forward (DCNv2)."""
