// quantize kernels, d = 256, rotation selector 3.
#define SRFTQ_D 256
#define SRFTQ_PART 0
#define SRFTQ_ROTSEL 3
#include "dispatch.inc"
