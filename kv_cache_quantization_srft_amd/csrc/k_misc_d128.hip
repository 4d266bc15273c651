// misc kernels for d = 128.
#define SRFTQ_D 128
#define SRFTQ_PART 2
#include "dispatch.inc"
