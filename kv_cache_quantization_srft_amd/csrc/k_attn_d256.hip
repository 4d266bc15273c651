// Decode attention over the quantized cache, d = 256.
#define SRFTQ_D 256
#include "attn_dispatch.inc"
