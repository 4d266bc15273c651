// quantize kernels, d = 256, rotation selector 0.
#define SRFTQ_D 256
#define SRFTQ_PART 0
#define SRFTQ_ROTSEL 0
#include "dispatch.inc"
