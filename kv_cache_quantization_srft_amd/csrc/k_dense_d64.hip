// Quantize / dequantize with a rotation matrix, d = 64.
#define SRFTQ_D 64
#include "dense_dispatch.inc"
