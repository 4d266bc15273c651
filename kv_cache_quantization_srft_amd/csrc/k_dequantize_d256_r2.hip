// dequantize kernels, d = 256, rotation selector 2.
#define SRFTQ_D 256
#define SRFTQ_PART 1
#define SRFTQ_ROTSEL 2
#include "dispatch.inc"
