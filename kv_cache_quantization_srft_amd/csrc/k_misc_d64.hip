// misc kernels for d = 64.
#define SRFTQ_D 64
#define SRFTQ_PART 2
#include "dispatch.inc"
