"""MI355X-native dense row-major GEMM: Python binding over the C-ABI library libmgemm."""
