// Decode attention at d = 96 (SRFT with its radix-3 step, or no rotation).
#define SRFTQ_D 96
#include "attn_dispatch.inc"
