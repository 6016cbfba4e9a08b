// The chunk walks with the layer's input convolution fused in (the kConv
// variants of k_chunk_walk), built as a translation unit of their own so
// that they compile in parallel with the rest of the forward. Everything
// else in the included file is compiled out here.
#define SSD_CONV_TU 1
#include "ssd_fwd.hip"
