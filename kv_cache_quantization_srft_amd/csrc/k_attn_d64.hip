// Decode attention over the quantized cache, d = 64.
#define SRFTQ_D 64
#include "attn_dispatch.inc"
