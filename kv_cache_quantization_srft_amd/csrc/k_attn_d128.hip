// Decode attention over the quantized cache, d = 128.
#define SRFTQ_D 128
#include "attn_dispatch.inc"
