"""MI355X-native MoE-layer hot path (int4 experts x Q8_0 activations). Binding filled in below."""
