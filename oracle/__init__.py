"""f64 CPU oracle for segmented softmax attention (test infrastructure only)."""
