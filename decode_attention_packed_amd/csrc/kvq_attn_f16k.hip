// The attention kernels compiled for fp16 K rows (namespace kvq::f16k): the
// unpacked-K baseline of page 1's comparison, for A/B measurements against
// the packed int8 K of the method.  Six waves per work-group with two ring
// slots each, as an fp16 K tile (8 KB) is twice the packed one.
#define KVQ_KFMT 1
#define KVQ_WAVES 6
#define KVQ_NS f16k
#include "kvq_attn.hip"
