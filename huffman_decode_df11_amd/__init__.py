"""MI355X-native DFloat11 decode: Huffman-coded BF16 exponents decoded on the GPU."""
