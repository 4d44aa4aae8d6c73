// The decode kernels for rotary widths that are not multiples of 16 (the
// general rotation of nvfp4kv_codec.hpp): the same kernel source, compiled
// once more with the general rotation switched on, behind
// launch_decode_splits_gr.  The reduce, the static workspace and the
// occupancy query live in decode_attn.hip only.
#define NVFP4KV_DECODE_GENERAL_ROPE 1
#include "decode_attn.hip"
