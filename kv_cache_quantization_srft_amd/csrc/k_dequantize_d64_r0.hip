// dequantize kernels, d = 64, rotation selector 0.
#define SRFTQ_D 64
#define SRFTQ_PART 1
#define SRFTQ_ROTSEL 0
#include "dispatch.inc"
