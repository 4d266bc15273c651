// Quantize / dequantize with a rotation matrix, d = 256.
#define SRFTQ_D 256
#include "dense_dispatch.inc"
