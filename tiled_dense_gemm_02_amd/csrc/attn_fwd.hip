// Instances of the attention-forward kernel: dim 64 / 128, fp16 / bf16, causal or
// not, 128 or 64 queries per workgroup.
#include "attn_fwd.hpp"

namespace tlg {

template <int D, int T, bool NEG, int RT>
static hipError_t launch_attn_s(const AttnParams& p, int causal, hipStream_t stream)
{
    AttnParams args = p;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)(p.nqb * p.H * p.B)), block(256);
    const void* fn = causal ? (const void*)&attn_fwd_kernel<D, T, true, NEG, RT>
                            : (const void*)&attn_fwd_kernel<D, T, false, NEG, RT>;
    return hipLaunchKernel(fn, grid, block, kargs, 0, stream);
}

template <int D, int T, int RT>
static hipError_t launch_attn_r(const AttnParams& p, int causal, hipStream_t stream)
{
    return p.scale_log2 < 0.f ? launch_attn_s<D, T, true, RT>(p, causal, stream)
                              : launch_attn_s<D, T, false, RT>(p, causal, stream);
}

template <int D, int T>
static hipError_t launch_attn_t(const AttnParams& p, int causal, hipStream_t stream)
{
    if (p.block_q == 64) return launch_attn_r<D, T, 1>(p, causal, stream);
    if (p.block_q == 128) return launch_attn_r<D, T, 2>(p, causal, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_attn(const AttnParams& p, int dim, int dtype, int causal, hipStream_t stream)
{
    if (dim == 64)
        return dtype == DT_F16 ? launch_attn_t<64, DT_F16>(p, causal, stream) : launch_attn_t<64, DT_BF16>(p, causal, stream);
    return dtype == DT_F16 ? launch_attn_t<128, DT_F16>(p, causal, stream) : launch_attn_t<128, DT_BF16>(p, causal, stream);
}

}  // namespace tlg
