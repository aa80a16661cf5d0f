// attn_fwd_d64_full.hip - instantiations of the attention forward kernel and its launches
// for head dim 64, all keys visible (one translation unit per head dim and mask,
// compiled in parallel).
#include "attn_fwd_launch_impl.h"

namespace attn_launch {

template hipError_t launch_dense<64, false>(const attn::Params&, bool, int, bool, bool, bool, hipStream_t);
template hipError_t launch_split<64, false>(const attn::Params&, bool, bool, int, bool, hipStream_t);

}  // namespace attn_launch
