// attn_fwd_launch.h - launch configuration of the gfx950 attention forward
// kernel and the launch entry points, one instantiation per head dim and mask.
// Each (D, CAUSAL) pair is instantiated in its own translation unit
// (attn_fwd_d{64,128}_{full,causal}.hip) so that the kernel variants compile in
// parallel; the host code in attn_fwd.hip calls them through these declarations.
#ifndef ATTN_FWD_LAUNCH_H
#define ATTN_FWD_LAUNCH_H

#include <hip/hip_runtime.h>

#include "attn_fwd_kernel.h"

namespace attn_launch {

// Tile configuration: 8 wavefronts (256 query rows) per workgroup, BC keys per KV tile.
constexpr int kWaves = 8;
constexpr int kRows = 32 * kWaves;  // query rows per workgroup
template <int D> struct Cfg;
template <> struct Cfg<128> { static constexpr int BC = 64; };
template <> struct Cfg<64> { static constexpr int BC = 64; };

// Workgroups per XCD of a persistent launch: one per compute unit of the XCD.
int cus_per_xcd();

// The forward kernel over dense or packed (varlen) rows: o_dtype fp32 or bf16, the
// exponential variant (poly8), negative-scale instantiation, reference schedule.
template <int D, bool CAUSAL>
hipError_t launch_dense(const attn::Params& p, bool of32, int poly8, bool neg, bool varlen, bool ref, hipStream_t s);

// Split keys: the partial kernel (fp32 partial O and LSE per unit into the
// workspace), then the merge kernel, on one stream.
template <int D, bool CAUSAL>
hipError_t launch_split(const attn::Params& p, bool neg, bool of32, int rows_total, bool ref, hipStream_t stream);

}  // namespace attn_launch

#endif
