"""MI355X-native exact attention: tiled online-softmax kernels behind a C ABI."""
