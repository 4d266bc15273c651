// Per-lane kernels for d = 96 (SRFT with a radix-3 step).
#define SRFTQ_D 96
#include "lane_dispatch.inc"
