// misc kernels for d = 256.
#define SRFTQ_D 256
#define SRFTQ_PART 2
#include "dispatch.inc"
