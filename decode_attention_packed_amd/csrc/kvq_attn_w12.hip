// The attention kernels for q4_0 V at head_dim 128 (the column layout of
// single-token decode with 4 grouped query heads per kv head, and the row
// layout of larger query groups such as the verify step's 4 query tokens x 4
// heads), compiled with 12 waves per work-group (3 per SIMD) and 2 ring slots
// each, into namespace kvq::w12.  The third wave per SIMD hides more of the
// MFMA, LDS and exp latency of the tile body than 8 waves with 3 ring slots
// each, once the chunks give every wave 4 tiles or more; the other formats
// keep the 8-wave build (q8_0 V tiles at head_dim 128 would not fit 12 waves
// of 2 slots in the LDS).
#define KVQ_WAVES 12
#define KVQ_NS w12
#define KVQ_Q4_128_ONLY 1
#include "kvq_attn.hip"
