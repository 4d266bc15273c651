// Quantize / dequantize with a rotation matrix, d = 128.
#define SRFTQ_D 128
#include "dense_dispatch.inc"
