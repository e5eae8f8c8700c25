// Split merge kernel: 1024 / head_dim query rows of one (request, KV head,
// query tile) group per workgroup, for requests whose key range was split;
// see attn_merge.h for the arithmetic.
#include "attn_merge.h"

namespace d2f {
namespace {

template <int D, typename OutT>
__global__ __launch_bounds__(256) void attn_merge_kernel(const AttnArgs a) {
  constexpr int RPW = 1024 / D;                      // rows per workgroup
  const int slices = (a.qrows + RPW - 1) / RPW;      // workgroups per group
  const int g = blockIdx.x / slices;
  const int slice = blockIdx.x % slices;
  const int ri = find_req_group(a, g);
  if (a.req[ri].nsplit == 1) return;
  const int local = g - a.req[ri].group_base;
  const int qtiles = a.req[ri].qtiles;
  merge_rows<D, OutT>(a, ri, local / qtiles, local % qtiles, slice * RPW);
}

}  // namespace

hipError_t launch_attn_merge(const AttnArgs& a, int head_dim, d2f_dtype_t dt, hipStream_t s) {
  const dim3 grid(a.n_groups * ((a.qrows + 1024 / head_dim - 1) / (1024 / head_dim))),
      block(256);
  if (dt == D2F_BF16) {
    if (head_dim == 128) hipLaunchKernelGGL((attn_merge_kernel<128, __bf16>), grid, block, 0, s, a);
    else if (head_dim == 64) hipLaunchKernelGGL((attn_merge_kernel<64, __bf16>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((attn_merge_kernel<128, float>), grid, block, 0, s, a);
    else if (head_dim == 64) hipLaunchKernelGGL((attn_merge_kernel<64, float>), grid, block, 0, s, a);
    else if (head_dim == 32) hipLaunchKernelGGL((attn_merge_kernel<32, float>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace d2f
