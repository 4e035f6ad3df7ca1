// The head_dim 256 instances of the forward kernels (attn_kernel.hip), built
// as a translation unit of their own so that they can take a different
// instruction scheduler from the other head dims.  At head_dim 256 a kernel
// runs one wave per SIMD, so nothing but the wave's own instruction order
// hides its LDS and MFMA latencies; LLVM's iterative ILP scheduler orders
// them further apart (1 x 4096 causal, 16 heads: 212 -> 183 us cold, 203 ->
// 169 us warm), while at the other head dims it measured within +-2 % of the
// default scheduler.
#define ATTNFWD_D256_UNIT 1
#include "attn_kernel.hip"
