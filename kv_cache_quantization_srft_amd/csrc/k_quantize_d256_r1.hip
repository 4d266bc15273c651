// quantize kernels, d = 256, rotation selector 1.
#define SRFTQ_D 256
#define SRFTQ_PART 0
#define SRFTQ_ROTSEL 1
#include "dispatch.inc"
