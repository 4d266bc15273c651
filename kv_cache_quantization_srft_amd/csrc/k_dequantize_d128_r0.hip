// dequantize kernels, d = 128, rotation selector 0.
#define SRFTQ_D 128
#define SRFTQ_PART 1
#define SRFTQ_ROTSEL 0
#include "dispatch.inc"
