// attn_fwd_launch_impl.h - definitions of the launch templates declared in
// attn_fwd_launch.h; included only by the per-(D, CAUSAL) instantiation units.
#ifndef ATTN_FWD_LAUNCH_IMPL_H
#define ATTN_FWD_LAUNCH_IMPL_H

#include "attn_fwd_launch.h"

namespace attn_launch {

template <int D, bool CAUSAL, bool OF32, int POLY8, bool NEG>
const void* kernel_fn(bool varlen, bool ref) {
  // the reference schedule exists for the hardware exponential and positive scales
  // (validate rejects the other combinations)
  if constexpr (POLY8 == 0 && !NEG) {
    if (ref)
      return varlen ? reinterpret_cast<const void*>(
                          &attn::attn_fwd_kernel<D, Cfg<D>::BC, CAUSAL, OF32, 0, false, true, false, true>)
                    : reinterpret_cast<const void*>(
                          &attn::attn_fwd_kernel<D, Cfg<D>::BC, CAUSAL, OF32, 0, false, false, false, true>);
  }
  return varlen ? reinterpret_cast<const void*>(&attn::attn_fwd_kernel<D, Cfg<D>::BC, CAUSAL, OF32, POLY8, NEG, true>)
                : reinterpret_cast<const void*>(&attn::attn_fwd_kernel<D, Cfg<D>::BC, CAUSAL, OF32, POLY8, NEG, false>);
}

template <int D, bool CAUSAL, bool OF32, int POLY8>
hipError_t launch(const attn::Params& p, bool neg, bool varlen, bool ref, hipStream_t stream) {
  // hipLaunchKernel reports this launch's own error (no sticky state from other calls).
  // A negative scale flips the row maximum of s*c into c * min(s): separate instantiation.
  // One workgroup per compute unit walks its XCD's tile range, so the next tile's
  // loads overlap the current tile's epilogue (causal: in a length-balanced order).
  int per_wg_xcd = p.per_xcd;
  const int slots = cus_per_xcd();
  if (slots > 0 && slots < per_wg_xcd) per_wg_xcd = slots;
  const dim3 grid(per_wg_xcd * p.n_xcd), block(64 * kWaves);
  void* args[] = {const_cast<attn::Params*>(&p)};
  const void* fn =
      neg ? kernel_fn<D, CAUSAL, OF32, POLY8, true>(varlen, ref) : kernel_fn<D, CAUSAL, OF32, POLY8, false>(varlen, ref);
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

template <int D, bool CAUSAL, bool OF32>
hipError_t launch_poly(const attn::Params& p, int poly8, bool neg, bool varlen, bool ref, hipStream_t s) {
  switch (poly8) {
    case 0: return launch<D, CAUSAL, OF32, 0>(p, neg, varlen, ref, s);
    case 4: return launch<D, CAUSAL, OF32, 4>(p, neg, varlen, ref, s);
    default: return launch<D, CAUSAL, OF32, 8>(p, neg, varlen, ref, s);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_dense(const attn::Params& p, bool of32, int poly8, bool neg, bool varlen, bool ref, hipStream_t s) {
  return of32 ? launch_poly<D, CAUSAL, true>(p, poly8, neg, varlen, ref, s)
              : launch_poly<D, CAUSAL, false>(p, poly8, neg, varlen, ref, s);
}

template <int D, bool CAUSAL>
hipError_t launch_split(const attn::Params& p, bool neg, bool of32, int rows_total, bool ref, hipStream_t stream) {
  int per_wg_xcd = p.per_xcd;
  const int slots = cus_per_xcd();
  if (slots > 0 && slots < per_wg_xcd) per_wg_xcd = slots;
  void* args[] = {const_cast<attn::Params*>(&p)};
  const void* fn =
      neg ? reinterpret_cast<const void*>(&attn::attn_fwd_kernel<D, Cfg<D>::BC, CAUSAL, true, 0, true, false, true>)
      : ref ? reinterpret_cast<const void*>(&attn::attn_fwd_kernel<D, Cfg<D>::BC, CAUSAL, true, 0, false, false, true, true>)
            : reinterpret_cast<const void*>(&attn::attn_fwd_kernel<D, Cfg<D>::BC, CAUSAL, true, 0, false, false, true>);
  hipError_t e = hipLaunchKernel(fn, dim3(per_wg_xcd * p.n_xcd), dim3(64 * kWaves), args, 0, stream);
  if (e != hipSuccess) return e;
  int split_keys = p.split_tiles * Cfg<D>::BC;
  void* margs[] = {const_cast<attn::Params*>(&p), &rows_total, &split_keys};
  const void* mfn = of32 ? reinterpret_cast<const void*>(&attn::attn_merge_kernel<D, CAUSAL, true>)
                         : reinterpret_cast<const void*>(&attn::attn_merge_kernel<D, CAUSAL, false>);
  return hipLaunchKernel(mfn, dim3((rows_total + 3) / 4), dim3(256), margs, 0, stream);
}

}  // namespace attn_launch

#endif
