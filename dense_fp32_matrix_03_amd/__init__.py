"""MI355X single-precision matrix product: Python binding of libsgemm."""
